"""Malformed argument sets for the binding's checks (shared by the CPU and
GPU tests): each must raise ValueError or TypeError before the library is
called."""


def bad_forward_args(dev):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    Bt, Hq, Hkv, N, d = 1, 4, 2, 256, 64

    def T(*shape, dtype=bf):
        return torch.zeros(shape, dtype=dtype, device=dev)

    def base():
        return dict(q=T(Bt, Hq, N, d), k=T(Bt, Hkv, N, d), v=T(Bt, Hkv, N, d), window=16)

    cases = []

    def add(name, **kw):
        a = base()
        a.update(kw)
        cases.append((name, a))

    add("k head_dim", k=T(Bt, Hkv, N, 2 * d), v=T(Bt, Hkv, N, 2 * d))
    add("k batch", k=T(2, Hkv, N, d), v=T(2, Hkv, N, d))
    add("v shape", v=T(Bt, Hkv, N - 1, d))
    add("k 3-D", k=T(Hkv, N, d))
    add("fp32 q with bf16 k", q=T(Bt, Hq, N, d, dtype=f32))
    add("v dtype", v=T(Bt, Hkv, N, d, dtype=f32))
    add("k not contiguous", k=T(Bt, N, Hkv, d).transpose(1, 2))
    add("idx_q without idx_k", idx_q=T(Bt, N, 64), token_top_k=8)
    add("token gate without indexer", token_top_k=8)
    add("idx_q dtype", idx_q=T(Bt, N, 64, dtype=f32), idx_k=T(Bt, N, 64), token_top_k=8)
    add("idx_k length", idx_q=T(Bt, N, 64), idx_k=T(Bt, N - 8, 64), token_top_k=8)
    add("idx index dims", idx_q=T(Bt, N, 64), idx_k=T(Bt, N, 32), token_top_k=8)
    add("sink dtype", sink=T(Hq))
    add("sink shape", sink=T(Hq + 1, dtype=f32))
    add("out shape", out=T(Bt, Hq, N, d + 8))
    add("out dtype", out=T(Bt, Hq, N, d, dtype=f32))
    add("lse shape", lse=T(Bt, Hq, N + 1, dtype=f32))
    add("lse dtype", lse=T(Bt, Hq, N))
    return cases


def bad_backward_args(dev):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    Bt, Hq, Hkv, N, d = 1, 4, 2, 256, 64

    def T(*shape, dtype=bf):
        return torch.zeros(shape, dtype=dtype, device=dev)

    def base():
        return dict(q=T(Bt, Hq, N, d), k=T(Bt, Hkv, N, d), v=T(Bt, Hkv, N, d),
                    out=T(Bt, Hq, N, d), lse=T(Bt, Hq, N, dtype=f32), dout=T(Bt, Hq, N, d))

    cases = []

    def add(name, **kw):
        a = base()
        a.update(kw)
        cases.append((name, a))

    add("fp32 inputs", q=T(Bt, Hq, N, d, dtype=f32), k=T(Bt, Hkv, N, d, dtype=f32),
        v=T(Bt, Hkv, N, d, dtype=f32))
    add("dout shape", dout=T(Bt, Hq, N - 1, d))
    add("out shape", out=T(Bt, Hq, N, d - 8))
    add("lse dtype", lse=T(Bt, Hq, N))
    add("k length", k=T(Bt, Hkv, N + 64, d), v=T(Bt, Hkv, N + 64, d))
    return cases
