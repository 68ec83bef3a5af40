"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random tensors
and stores them as bfloat16.  Shapes follow the library's layout:

    AllGather -> GEMM   x [N, m, k]     (sequence shards X_r)
                        w [N, n, k]     (column-parallel weight shards W_r,
                                         one output feature per row)
    GEMM -> ReduceScatter
                        h [N, N*m, k]   (rank r's activation for all T = N*m
                                         tokens, its k = f/N slice)
                        w [N, n, k]     (row-parallel weight shards, stored
                                         one output feature per row)

Distributions: "normal" draws activations from N(0, 1) and weights from
N(0, 0.02^2); "int" draws every element uniformly from {-3, ..., 3}, which
bf16 holds exactly and whose products and sums stay exact in fp32.

Two back ends produce the same kinds of tensors:
  * numpy (CPU): PCG64 streams from SeedSequence(seed).spawn(4) for
    (X, W1, H, W2); float32 draws rounded to bf16 by the bias method below.
  * torch (device): a torch.Generator on the target device, for sizes where
    host generation would be slow; the bf16 cast is torch's (nearest-even).
"""
import numpy as np

ACT_STD = 1.0
WEIGHT_STD = 0.02
INT_LO, INT_HI = -3, 3


def f32_to_bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Bias method on the binary32 bit pattern: add 0x7FFF plus the lowest bit
    that is kept, then drop the low 16 bits.  Inputs must be finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    return ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(seed):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(4)]


def _draw(gen, shape, dist, std):
    if dist == "int":
        return gen.integers(INT_LO, INT_HI + 1, size=shape).astype(np.float32)
    if dist == "normal":
        return (gen.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    raise ValueError("dist must be 'normal' or 'int', got %r" % (dist,))


def ag_inputs(N, m, k, n, dist="normal", seed=0):
    """(x [N,m,k], w [N,n,k]) as uint16 bf16 bit patterns (numpy, CPU)."""
    g = _streams(seed)
    x = f32_to_bf16_bits(_draw(g[0], (N, m, k), dist, ACT_STD))
    w = f32_to_bf16_bits(_draw(g[1], (N, n, k), dist, WEIGHT_STD))
    return x, w


def rs_inputs(N, m, k, n, dist="normal", seed=0):
    """(h [N,N*m,k], w [N,n,k]) as uint16 bf16 bit patterns (numpy, CPU)."""
    g = _streams(seed)
    h = f32_to_bf16_bits(_draw(g[2], (N, N * m, k), dist, ACT_STD))
    w = f32_to_bf16_bits(_draw(g[3], (N, n, k), dist, WEIGHT_STD))
    return h, w


def to_torch_bf16(bits, device="cpu"):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor (bit-identical)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def torch_bf16_to_bits(t):
    """torch.bfloat16 tensor -> numpy uint16 bit patterns (bit-identical)."""
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _torch_draw(shape, dist, std, gen, device):
    import torch
    if dist == "int":
        return torch.randint(INT_LO, INT_HI + 1, shape, generator=gen, device=device).to(torch.bfloat16)
    if dist == "normal":
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return (t * std).to(torch.bfloat16)
    raise ValueError("dist must be 'normal' or 'int', got %r" % (dist,))


def ag_inputs_torch(N, m, k, n, dist="normal", seed=0, device="cuda"):
    """(x [N,m,k], w [N,n,k]) as torch.bfloat16 on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 4 + 0)
    x = _torch_draw((N, m, k), dist, ACT_STD, g, device)
    g.manual_seed(seed * 4 + 1)
    w = _torch_draw((N, n, k), dist, WEIGHT_STD, g, device)
    return x, w


def rs_inputs_torch(N, m, k, n, dist="normal", seed=0, device="cuda"):
    """(h [N,N*m,k], w [N,n,k]) as torch.bfloat16 on `device`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 4 + 2)
    h = _torch_draw((N, N * m, k), dist, ACT_STD, g, device)
    g.manual_seed(seed * 4 + 3)
    w = _torch_draw((N, n, k), dist, WEIGHT_STD, g, device)
    return h, w
