"""The binding rejects malformed tensors before it reaches the library (CPU:
the shape and dtype checks run before the device check; every case must
raise ValueError or TypeError, never reach a launch)."""
import pytest

from binding_cases import bad_backward_args, bad_forward_args


@pytest.fixture(autouse=True)
def _no_library(monkeypatch):
    import sliding_window_long_amd as sa

    def no_library():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(sa.binding, "load_library", no_library)


@pytest.mark.parametrize("case", range(len(bad_forward_args("cpu"))))
def test_forward_rejects(case):
    import sliding_window_long_amd as sa
    name, a = bad_forward_args("cpu")[case]
    q, k, v = a.pop("q"), a.pop("k"), a.pop("v")
    with pytest.raises((ValueError, TypeError)) as e:
        sa.forward(q, k, v, **a)
    assert "device" not in str(e.value) or name.startswith("k not"), (name, str(e.value))


@pytest.mark.parametrize("case", range(len(bad_backward_args("cpu"))))
def test_backward_rejects(case):
    import sliding_window_long_amd as sa
    name, a = bad_backward_args("cpu")[case]
    with pytest.raises((ValueError, TypeError)) as e:
        sa.backward(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("out"), a.pop("lse"), a.pop("dout"))
    assert "device" not in str(e.value), (name, str(e.value))


def test_cpu_tensors_rejected():
    import torch
    import sliding_window_long_amd as sa
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        sa.forward(q, q[:, :1].contiguous(), q[:, :1].contiguous(), window=8)
