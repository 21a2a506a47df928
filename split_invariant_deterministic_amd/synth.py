"""Seeded synthetic inputs for every workload of the path.

This module only draws random tensors; it contains none of the method's
arithmetic, so both the HIP path (through the tests and the bench) and the
CPU oracle can be fed from it. Every draw uses an explicit torch.Generator
seeded per tensor, so a tensor's values do not depend on which other tensors
were drawn or on the device order of draws:

    seed(tensor) = base_seed * 1000 + tensor_index

Normal draws are float32 N(0, 1) (times a scale), cast to bf16 with torch's
round-to-nearest-even. Small workloads are drawn on the CPU; the large ones
(the LM-head weight, the KV cache, the MoE experts) accept ``device`` so they
can be drawn directly in device memory. Values drawn on different devices
differ (different generators) but each is fixed by its seed.

Workloads (shapes from the pages' model classes; no dataset is involved, the
synthetic draws stand in for the trained weights and prompts the pages use):

* tiny:    x [8, 256], W [512, 256] (N x K storage of the 256 x 512 weight),
           gamma = 1, targets in [0, 512)
* dense:   X [4096, K], W [N, K] * 0.02 for (K, N) in {(4096, 12288),
           (12288, 4096)}; smaller M are row prefixes
* lmhead:  h [4096, 4096], W [151936, 4096] * 0.02, targets in [0, 151936)
* rmsnorm: x [M, 4096], gamma ~ N(1, 0.1)
* attn:    per-sequence lengths uniform in [1, 32768]; q [B, 32, 128],
           K, V [sum L, 8, 128]
* moe:     router logits [T, 128] fp32, x [T, 2048], W1 [128, 1536, 2048] *
           0.02, W2 [128, 2048, 768] * 0.02
* gdn:     packed sequences of the given lengths, q, k, v [T, H, 128] bf16
           N(0, 1), log-decay g [T, H] fp32 uniform in [-0.5, 0], writing
           strength beta [T, H] fp32 uniform in [0, 1]
"""

import torch


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, seed, scale=1.0, dtype=torch.bfloat16, device="cpu", mean=0.0):
    g = _gen(seed, device)
    t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if scale != 1.0:
        t.mul_(scale)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def randint(low, high, shape, seed, device="cpu"):
    g = _gen(seed, device)
    return torch.randint(low, high, shape, generator=g, dtype=torch.int64,
                         device=device).to(torch.int32)


def tiny(seed=0):
    s = seed * 1000
    return {
        "x": randn((8, 256), s + 0),
        "W": randn((512, 256), s + 1, 0.02),
        "gamma": torch.ones(256, dtype=torch.bfloat16),
        "targets": randint(0, 512, (8,), s + 2),
    }


def dense(K, N, M=4096, seed=0, device="cpu"):
    s = seed * 1000 + 10
    return {"X": randn((M, K), s + 0, device=device),
            "W": randn((N, K), s + 1, 0.02, device=device)}


def lmhead(M=4096, H=4096, V=151936, seed=0, device="cpu"):
    s = seed * 1000 + 20
    return {"h": randn((M, H), s + 0, device=device),
            "W": randn((V, H), s + 1, 0.02, device=device),
            "targets": randint(0, V, (M,), s + 2, device=device)}


def rmsnorm(M, H=4096, seed=0, device="cpu"):
    s = seed * 1000 + 30
    return {"x": randn((M, H), s + 0, device=device),
            "gamma": randn((H,), s + 1, 0.1, mean=1.0, device=device)}


def attn_lengths(B=256, Lmax=32768, seed=0):
    return randint(1, Lmax + 1, (B,), seed * 1000 + 40)


def attn(lengths, Hq=32, Hkv=8, D=128, seed=0, device="cpu"):
    """Decode batch: one query row per sequence, at its last position."""
    s = seed * 1000 + 41
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    B = int(lengths.numel())
    total = int(lengths.sum())
    cu = torch.zeros(B + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    return {
        "q": randn((B, Hq, D), s + 0, device=device),
        "k": randn((total, Hkv, D), s + 1, device=device),
        "v": randn((total, Hkv, D), s + 2, device=device),
        "cu_seqlens": cu.to(torch.int32),
        "q_seq": torch.arange(B, dtype=torch.int32),
        "q_pos": (lengths - 1).to(torch.int32),
    }


def moe(T=8192, H=2048, E=128, F=768, seed=0, device="cpu"):
    s = seed * 1000 + 50
    return {
        "logits": randn((T, E), s + 0, dtype=torch.float32, device=device),
        "x": randn((T, H), s + 1, device=device),
        "W1": randn((E, 2 * F, H), s + 2, 0.02, device=device),
        "W2": randn((E, H, F), s + 3, 0.02, device=device),
    }


def gdn(lengths, H=16, seed=0, device="cpu"):
    s = seed * 1000 + 60
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    cu = torch.tensor([0] + lengths, dtype=torch.int64).cumsum(0).to(torch.int32)
    g = torch.rand((T, H), generator=_gen(s + 3, device), device=device) * -0.5
    beta = torch.rand((T, H), generator=_gen(s + 4, device), device=device)
    return {"q": randn((T, H, 128), s + 0, device=device), "k": randn((T, H, 128), s + 1, device=device),
            "v": randn((T, H, 128), s + 2, device=device), "g": g, "beta": beta, "cu_seqlens": cu.to(device)}
