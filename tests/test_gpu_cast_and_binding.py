"""The bf16 boundary cast of the GPU kernels against the oracle's cast, and
the binding's host-side shape checks.

RL-Kernel write-up, section 2: the position of the FP32 -> BF16 conversion is
one of the trigger points of mismatch, so the hardware conversion that every
kernel's epilogue uses (inv_cast_bf16 runs the same device function) is
pinned bit for bit against round-to-nearest-even written from the format's
definition (the oracle's cast, itself pinned against torch's CPU cast).
"""

import numpy as np
import pytest
import torch

from oracle import numerics

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _stratified_f32_bits(n_random=1 << 20, seed=0):
    """Random fp32 patterns plus every sign/exponent/high-mantissa pattern with
    the low half at, next to and away from the rounding midpoint: ties to
    even and odd, subnormals, values rounding to the largest finite bf16 and
    overflowing to inf, infinities and NaNs."""
    rng = np.random.default_rng(seed)
    r = rng.integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    return np.concatenate([r, (hi[:, None] | lows[None, :]).ravel()])


def test_gpu_bf16_cast_bitwise_against_oracle(inv):
    bits = _stratified_f32_bits()
    f = bits.view(np.float32)
    y = inv.cast_bf16(torch.from_numpy(f.copy()).to(DEV)).cpu().view(torch.int16).numpy().view(np.uint16)
    with np.errstate(invalid="ignore"):
        ora = numerics.to_bf16(f.astype(np.float64))
    nan = np.isnan(f)
    got = (y.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(np.isnan(got), nan), "NaN in, NaN out (and nothing else NaN)"
    want = numerics.bf16_bits(ora[~nan])
    bad = y[~nan] != want
    assert not bad.any(), f"{int(bad.sum())} casts differ; first inputs {bits[~nan][bad][:4]}"
    # the interesting classes were present
    fin = f[~nan]
    assert np.any(np.isinf(ora[~nan]) & np.isfinite(fin))       # overflow to inf
    assert np.any((np.abs(fin) < 2.0 ** -126) & (fin != 0))       # subnormal inputs
    assert np.any((bits[~nan] & 0xFFFF) == 0x8000)                # exact ties


def test_binding_rejects_wrong_shapes_before_launch(inv):
    """Wrong-sized buffers raise in the binding, before the C call."""
    c8 = inv.contract(leaves=8)
    A = torch.zeros((16, 256), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((32, 256), dtype=torch.bfloat16, device=DEV)
    Bk = torch.zeros((32, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        inv.gemm(A, Bk, c8)
    with pytest.raises(ValueError):
        inv.gemm_rank(A, Bk, 0, c8)
    with pytest.raises(ValueError):
        inv.gemm_rank(A, B, 0, c8, out=torch.zeros((16, 16), device=DEV))
    with pytest.raises(ValueError):
        inv.gemm_leaves(A, B, 0, 2, c8, out=torch.zeros((1, 16, 32), device=DEV))
    with pytest.raises(ValueError):
        inv.gemm(A, B, c8, out=torch.zeros((16, 16), dtype=torch.bfloat16, device=DEV))
    x = torch.zeros((4, 100), device=DEV)
    t = torch.zeros(3, dtype=torch.int32, device=DEV)
    c4 = inv.contract(leaves=4)
    with pytest.raises(ValueError):
        inv.logprob(x, t, c4)
    with pytest.raises(ValueError):
        inv.logprob(x, torch.zeros(4, dtype=torch.int32, device=DEV), c4, out=torch.zeros(3, device=DEV))
    with pytest.raises(ValueError):
        inv.logprob_partials(x, torch.zeros(4, dtype=torch.int32, device=DEV), 0, 4, c4,
                             stats=torch.zeros((4, 2, 2), device=DEV))
    with pytest.raises(ValueError):
        inv.logprob_combine(torch.zeros((4, 4, 2), device=DEV), torch.zeros(3, device=DEV),
                            torch.zeros(4, dtype=torch.int32, device=DEV), 100, c4)
    with pytest.raises(ValueError):
        inv.rmsnorm(A, torch.zeros(256, dtype=torch.bfloat16, device=DEV), c8, out=torch.zeros_like(A[:8]))
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((10, 2, 128), dtype=torch.bfloat16, device=DEV)
    i2 = torch.zeros(2, dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 5, 10], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        inv.decode_attn(q, kv, kv[:9], cu, i2, i2, inv.contract())
    with pytest.raises(ValueError):
        inv.decode_attn(q, kv, kv, cu, i2[:1], i2, inv.contract())
    Y = torch.zeros((8, 64), device=DEV)
    with pytest.raises(ValueError):
        inv.moe_combine(Y, torch.zeros((2, 4), device=DEV), torch.zeros((2, 8), dtype=torch.int32, device=DEV), c8)
    torch.cuda.synchronize()


def test_attention_workspace_size_is_counted_in_bytes(inv):
    """The attention entry points hand the library the workspace's size in
    bytes whatever its element type: a byte workspace of exactly the size the
    library asks for gives the same output as the default one, one of four
    bytes less is refused by the library's size check, and a host tensor is
    refused before the call."""
    g = torch.Generator().manual_seed(5)
    S, L, Hq, Hkv, D = 2, 300, 8, 2, 128
    q = torch.randn((S, Hq, D), generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn((S * L, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn((S * L, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    cu = torch.tensor([0, L, 2 * L], dtype=torch.int32, device=DEV)
    q_seq = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    q_pos = torch.tensor([L - 1, L - 7], dtype=torch.int32, device=DEV)
    c = inv.contract()
    ref = inv.decode_attn(q, k, v, cu, q_seq, q_pos, c)
    need = inv.workspace_bytes(c, inv.OP_DECODE_ATTN, S, Hq, D)
    assert need > 4
    ws8 = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = inv.decode_attn(q, k, v, cu, q_seq, q_pos, c, ws=ws8)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    with pytest.raises(inv.InvError) as e:
        inv.decode_attn(q, k, v, cu, q_seq, q_pos, c, ws=ws8[: need - 4])
    assert e.value.status == inv.E_WORKSPACE
    with pytest.raises(inv.InvError) as e:
        inv.attn_splits(q, k, v, cu, q_seq, q_pos, 0, c.split_kv, c, ws8[: need - 4])
    assert e.value.status == inv.E_WORKSPACE
    with pytest.raises(inv.InvError) as e:
        inv.attn_combine(ws8[: need - 4], S, Hq, D, c)
    assert e.value.status == inv.E_WORKSPACE
    with pytest.raises(ValueError):
        inv.decode_attn(q, k, v, cu, q_seq, q_pos, c, ws=torch.empty(need, dtype=torch.uint8))
    torch.cuda.synchronize()


def test_elementwise_launches_past_one_grid_pass(inv):
    # More elements than the capped grid covers in one pass (2^20 workgroups
    # x 256 lanes = 2^28): the tree combine and the cast walk the rest by the
    # grid stride, and every element still matches torch's fp32 sum and
    # round-to-nearest-even cast bit for bit.
    M, N = 4099, 65537
    assert M * N > (1 << 28)
    g = torch.Generator(device=DEV).manual_seed(11)
    P = torch.randn((2, M, N), generator=g, device=DEV, dtype=torch.float32)
    out = inv.tree_combine(P, inv.contract(leaves=2, out="bf16"))
    ref = (P[0] + P[1]).to(torch.bfloat16)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    del out, ref
    y = inv.cast_bf16(P[0])
    assert torch.equal(y.view(torch.int16), P[0].to(torch.bfloat16).view(torch.int16))
