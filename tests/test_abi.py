"""Host-side tests of the C-ABI library (no GPU, no kernel launch).

The library loads without a GPU; every symbol that include/inv.h declares is
exported; contract and shape validation runs on the host before any HIP call
and returns the documented status (the IsoExec blog, "Unified execution
contract": a parallel size without a proven-invariance claim is rejected).
Only calls that fail validation or that are empty are made, so nothing is
ever enqueued.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "split_invariant_deterministic_amd", "libinv.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libinv.so not built")


def _inv():
    from split_invariant_deterministic_amd import inv
    return inv


def declared_symbols():
    txt = open(os.path.join(ROOT, "include", "inv.h")).read()
    return sorted(set(re.findall(r"^(?:inv_status|size_t|const char\*)\s+(inv_\w+)\s*\(", txt, re.M)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    decl = declared_symbols()
    assert len(decl) >= 20
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(_inv().EXPORTS) == decl


def test_contract_defaults():
    c = _inv().contract()
    assert (c.leaves, c.ranks, c.split_kv, c.kv_chunk) == (8, 1, 16, 64)
    assert abs(c.eps - 1e-6) < 1e-12
    assert c.struct_size == ctypes.sizeof(c) == 48


@pytest.mark.parametrize("ranks,status", [(1, 0), (2, 0), (4, 0), (8, 0), (3, 3), (5, 3), (6, 3), (16, 3)])
def test_rank_claims(ranks, status):
    inv = _inv()
    c = inv.contract(leaves=8, ranks=ranks)
    assert inv.contract_check(c, inv.OP_GEMM, 4096) == status


def test_contract_violations():
    inv = _inv()
    assert inv.contract_check(inv.contract(leaves=8), inv.OP_GEMM, 4096 + 8) == inv.E_CONTRACT  # K % L
    assert inv.contract_check(inv.contract(leaves=8), inv.OP_GEMM, 8 * 48) == inv.E_CONTRACT    # leaf % 32
    assert inv.contract_check(inv.contract(leaves=6), inv.OP_GEMM, 6 * 64) == inv.E_CONTRACT    # not 2^n
    assert inv.contract_check(inv.contract(leaves=16), inv.OP_GEMM, 16 * 64) == inv.E_UNSUPPORTED
    assert inv.contract_check(inv.contract(accum="bf16"), inv.OP_GEMM, 4096) == inv.E_CONTRACT
    assert inv.contract_check(inv.contract(leaf="bf16"), inv.OP_GEMM, 4096) == inv.E_CONTRACT
    assert inv.contract_check(inv.contract(tree="left_fold"), inv.OP_GEMM, 4096) == inv.E_CONTRACT
    assert inv.contract_check(inv.contract(tree="left_fold"), inv.OP_LOGPROB) == inv.OK
    assert inv.contract_check(inv.contract(split_kv=12), inv.OP_DECODE_ATTN) == inv.E_CONTRACT
    assert inv.contract_check(inv.contract(kv_chunk=48), inv.OP_DECODE_ATTN) == inv.E_CONTRACT
    assert inv.contract_check(inv.contract(eps=float("nan")), inv.OP_RMSNORM) == inv.E_CONTRACT
    c = inv.contract()
    c.struct_size = 40
    assert inv.contract_check(c, inv.OP_GEMM, 4096) == inv.E_ARG
    c = inv.contract()
    c.reserved = 1
    assert inv.contract_check(c, inv.OP_GEMM, 4096) == inv.E_ARG


def test_workspace_sizes():
    inv = _inv()
    assert inv.workspace_bytes(inv.contract(ranks=1), inv.OP_GEMM, 7, 128, 4096) == 0   # stream kernel, M < 8
    assert inv.workspace_bytes(inv.contract(ranks=1), inv.OP_GEMM, 64, 128, 4096) == 8 * 64 * 128 * 4  # 1 tile
    assert inv.workspace_bytes(inv.contract(ranks=1), inv.OP_GEMM, 4096, 12288, 4096) == 0
    # few 128x128 tiles: optional leaf groups (32 tiles x 8 groups at M=128, N=4096)
    assert inv.workspace_bytes(inv.contract(ranks=1), inv.OP_GEMM, 128, 4096, 12288) == 8 * 128 * 4096 * 4
    assert inv.workspace_bytes(inv.contract(ranks=1), inv.OP_GEMM, 512, 4096, 4096) == 2 * 512 * 4096 * 4
    assert inv.workspace_bytes(inv.contract(ranks=1), inv.OP_GEMM, 512, 12288, 4096) == 0  # 384 tiles
    assert inv.workspace_bytes(inv.contract(leaves=2), inv.OP_GEMM, 128, 1024, 4096) == 2 * 128 * 1024 * 4
    assert inv.workspace_bytes(inv.contract(ranks=4), inv.OP_GEMM, 64, 128, 4096) == 4 * 64 * 128 * 4
    assert inv.workspace_bytes(inv.contract(), inv.OP_DECODE_ATTN, 3, 32, 128) == 3 * 32 * 16 * 130 * 4
    assert inv.workspace_bytes(inv.contract(ranks=3), inv.OP_GEMM, 64, 128, 4096) == ctypes.c_size_t(-1).value
    c32 = inv.contract(leaves=8, out="fp32")
    assert inv.workspace_bytes(c32, inv.OP_LMHEAD_LOGPROB, 4096, 151936, 4096) == 4096 * 9496 * 8 + 4096 * 4
    assert inv.workspace_bytes(c32, inv.OP_LOGPROB_BLOCK16, 3, 17, 0) == 3 * 2 * 8 + 3 * 4
    assert inv.workspace_bytes(inv.contract(), inv.OP_LMHEAD_LOGPROB, 8, 512, 256) == ctypes.c_size_t(-1).value
    cg = inv.contract(kv_chunk=64)
    T, H, S = 10240, 16, 5
    assert inv.workspace_bytes(cg, inv.OP_GDN_PREFILL, T, H, S) == \
        (2 * T * H * 128 + T * H + (T // 64 + S) * H * (128 * 128 + 64 * 64 + 128)) * 4 + 16
    assert inv._lib.inv_gdn_cache_bytes(ctypes.byref(cg), 16) == \
        (2 * 16 * 128 * 128 + 64 * 16 * 258 + 16 * (64 * 64 + 128)) * 4


def test_entry_points_reject_before_any_launch():
    inv = _inv()
    lib = inv._lib
    c = inv.contract(ranks=3)
    null = ctypes.c_void_p(0)
    by = ctypes.byref
    assert lib.inv_gemm(by(c), null, null, null, 4, 4, 4096, null, 0, null) == inv.E_TOPOLOGY
    c = inv.contract()
    assert lib.inv_gemm(by(c), null, null, null, 4, 4, 4096, null, 0, null) == inv.E_ARG  # null operands
    assert lib.inv_gemm(by(c), null, null, null, -1, 4, 4096, null, 0, null) == inv.E_ARG
    assert lib.inv_gemm(by(c), null, null, null, 0, 4, 4096, null, 0, null) == inv.OK     # empty: no launch
    c2 = inv.contract(ranks=2)
    # ranks > 1 without workspace: rejected (misaligned pointers are caught first, so use aligned fakes)
    fake = ctypes.c_void_p(1 << 20)
    assert lib.inv_gemm(by(c2), fake, fake, fake, 4, 4, 4096, null, 0, null) == inv.E_WORKSPACE
    # K >= 2^24 would wrap the ring kernel's 32-bit operand offsets: rejected on every GEMM entry point
    kbig = 1 << 24
    assert inv.contract_check(c, inv.OP_GEMM, kbig) == inv.E_UNSUPPORTED
    assert inv.contract_check(c, inv.OP_GEMM, kbig - 256) == inv.OK
    assert lib.inv_gemm(by(c), fake, fake, fake, 4096, 4096, kbig, null, 0, null) == inv.E_UNSUPPORTED
    assert lib.inv_gemm_rank(by(c2), fake, fake, fake, 4096, 4096, kbig, 0, null) == inv.E_UNSUPPORTED
    assert lib.inv_gemm_leaves(by(c), fake, fake, fake, 4096, 4096, kbig, 0, 8, null) == inv.E_UNSUPPORTED
    assert lib.inv_moe_gemm(by(c), fake, 4, null, fake, fake, fake, 4, 2, 64, kbig, null) == inv.E_UNSUPPORTED
    assert lib.inv_moe_gemm_swiglu(by(c), fake, 4, null, fake, fake, fake, 4, 2, 64, kbig, null) \
        == inv.E_UNSUPPORTED
    assert lib.inv_lmhead_logprob(by(inv.contract(out="fp32")), fake, fake, fake, fake, 4, 512, kbig, fake,
                                  1 << 30, null) == inv.E_UNSUPPORTED
    assert lib.inv_gemm_leaves(by(c), fake, fake, fake, 4, 4, 4096, 3, 3, null) == inv.E_ARG
    assert lib.inv_gemm_leaves(by(c), fake, fake, fake, 4, 4, 4096, 0, 9, null) == inv.E_ARG
    assert lib.inv_gemm_rank(by(c2), fake, fake, fake, 4, 4, 4096, 2, null) == inv.E_ARG
    assert lib.inv_tree_combine(by(c), fake, 3, fake, 4, 4, null) == inv.E_UNSUPPORTED
    assert lib.inv_rmsnorm(by(c), fake, fake, fake, 4, 12, null) == inv.E_UNSUPPORTED
    assert lib.inv_rmsnorm(by(c), fake, fake, fake, 4, 16392, null) == inv.E_UNSUPPORTED
    assert lib.inv_rmsnorm(by(c), null, null, null, 0, 4096, null) == inv.OK
    clp = inv.contract(leaves=64)
    assert lib.inv_logprob(by(clp), fake, 10, fake, fake, 4, 32, null) == inv.E_CONTRACT      # C > V
    assert lib.inv_logprob(by(clp), fake, 10, fake, fake, 4, 100, null) == inv.E_ARG          # ldl < V
    assert lib.inv_logprob(by(inv.contract(leaves=1024)), fake, 4096, fake, fake, 4, 4096, null) \
        == inv.E_UNSUPPORTED
    ca = inv.contract()
    assert lib.inv_decode_attn(by(ca), fake, fake, fake, fake, 1, fake, fake, fake, 1, 32, 8, 64, fake,
                               1 << 30, null) == inv.E_UNSUPPORTED                              # D != 128
    assert lib.inv_decode_attn(by(ca), fake, fake, fake, fake, 1, fake, fake, fake, 1, 32, 6, 128, fake,
                               1 << 30, null) == inv.E_UNSUPPORTED                              # Hq % Hkv
    assert lib.inv_decode_attn(by(ca), fake, fake, fake, fake, 1, fake, fake, fake, 1, 32, 8, 128, fake,
                               16, null) == inv.E_WORKSPACE
    assert lib.inv_attn_splits(by(ca), fake, fake, fake, fake, 1, fake, fake, 1, 32, 8, 128, 4, 4, fake,
                               1 << 30, null) == inv.E_ARG
    # a chunk of keys over all kv heads is addressed with 32-bit offsets: 128 x 65536 x 128 x 2 B = 2 GiB
    assert lib.inv_decode_attn(by(inv.contract(kv_chunk=128)), fake, fake, fake, fake, 1, fake, fake, fake, 1,
                               65536, 65536, 128, fake, 1 << 30, null) == inv.E_UNSUPPORTED
    # one workgroup per (row, kv head, split): Tq x Hkv x split_kv < 2^23 (here 65536 x 8 x 16 = 2^23)
    assert lib.inv_decode_attn(by(ca), fake, fake, fake, fake, 1, fake, fake, fake, 65536, 32, 8, 128, fake,
                               1 << 40, null) == inv.E_UNSUPPORTED
    assert lib.inv_attn_splits(by(ca), fake, fake, fake, fake, 1, fake, fake, 65536, 32, 8, 128, 0, 1, fake,
                               1 << 40, null) == inv.E_UNSUPPORTED
    # fp32 workspaces and partials are accessed an element at a time, bf16 outputs likewise: a pointer off
    # its element's alignment is rejected before any launch
    odd2, odd1 = ctypes.c_void_p((1 << 20) + 2), ctypes.c_void_p((1 << 20) + 1)
    assert lib.inv_decode_attn(by(ca), fake, fake, fake, fake, 1, fake, fake, fake, 1, 32, 8, 128, odd2,
                               1 << 30, null) == inv.E_ARG
    assert lib.inv_decode_attn(by(ca), fake, fake, fake, fake, 1, fake, fake, odd1, 1, 32, 8, 128, fake,
                               1 << 30, null) == inv.E_ARG
    assert lib.inv_attn_splits(by(ca), fake, fake, fake, fake, 1, fake, fake, 1, 32, 8, 128, 0, 1, odd2,
                               1 << 30, null) == inv.E_ARG
    assert lib.inv_attn_combine(by(ca), odd2, 1 << 30, fake, 1, 32, 128, null) == inv.E_ARG
    assert lib.inv_attn_combine(by(ca), fake, 1 << 30, odd1, 1, 32, 128, null) == inv.E_ARG
    assert lib.inv_gemm(by(c), fake, fake, fake, 4, 4, 4096, odd2, 1 << 30, null) == inv.E_ARG
    assert lib.inv_gemm(by(c), fake, fake, odd1, 4, 4, 4096, null, 0, null) == inv.E_ARG
    assert lib.inv_gemm(by(inv.contract(out="fp32")), fake, fake, odd2, 4, 4, 4096, null, 0, null) == inv.E_ARG
    assert lib.inv_gemm_rank(by(c2), fake, fake, odd2, 4, 4, 4096, 0, null) == inv.E_ARG
    assert lib.inv_tree_combine(by(c), odd2, 2, fake, 4, 4, null) == inv.E_ARG
    assert lib.inv_tree_combine(by(c), fake, 2, odd1, 4, 4, null) == inv.E_ARG
    cm = inv.contract(leaves=8)
    assert lib.inv_moe_route(by(cm), fake, fake, fake, 4, 300, null) == inv.E_UNSUPPORTED
    assert lib.inv_moe_route(by(cm), fake, fake, fake, 4, 4, null) == inv.E_UNSUPPORTED      # k > E
    assert lib.inv_moe_gemm(by(inv.contract(ranks=2)), fake, 4, fake, fake, fake, fake, 4, 2, 64, 4096,
                            null) == inv.E_TOPOLOGY
    # fused gate/up + SwiGLU: one rank, 16-byte aligned operands, one expert's 2F x K under 4 GiB
    assert lib.inv_moe_gemm_swiglu(by(inv.contract(ranks=2)), fake, 4, fake, fake, fake, fake, 4, 2, 64, 4096,
                                   null) == inv.E_TOPOLOGY
    assert lib.inv_moe_gemm_swiglu(by(cm), fake, 4, fake, fake, fake, fake, 4, 2, 1 << 19, 4096,
                                   null) == inv.E_UNSUPPORTED
    assert lib.inv_moe_gemm_swiglu(by(cm), ctypes.c_void_p((1 << 20) + 2), 4, fake, fake, fake, fake, 4, 2, 64, 4096,
                                   null) == inv.E_ARG
    assert lib.inv_moe_gemm_swiglu(by(cm), null, 0, null, null, null, null, 0, 2, 64, 4096, null) == inv.OK
    assert lib.inv_moe_combine(by(cm), null, null, null, 0, null, 0, 2048, null) == inv.OK
    # fused LM head + logprob: fp32 logits, one rank, V <= 262144, enough aligned workspace
    cl = inv.contract(leaves=8, out="fp32")
    big = 1 << 30
    assert lib.inv_lmhead_logprob(by(inv.contract(leaves=8)), fake, fake, fake, fake, 4, 512, 256, fake, big,
                                  null) == inv.E_CONTRACT
    assert lib.inv_lmhead_logprob(by(inv.contract(leaves=8, ranks=2, out="fp32")), fake, fake, fake, fake, 4, 512,
                                  256, fake, big, null) == inv.E_UNSUPPORTED
    assert lib.inv_lmhead_logprob(by(cl), fake, fake, fake, fake, 4, 262160, 256, fake, big, null) \
        == inv.E_UNSUPPORTED
    assert lib.inv_lmhead_logprob(by(cl), fake, fake, fake, fake, 4, 512, 256, fake, 4 * 32 * 8, null) \
        == inv.E_WORKSPACE
    assert lib.inv_lmhead_logprob(by(cl), fake, fake, fake, fake, 4, 512, 256, ctypes.c_void_p((1 << 20) + 4),
                                  big, null) == inv.E_ARG
    assert lib.inv_lmhead_logprob(by(cl), fake, fake, fake, fake, 0, 512, 256, null, 0, null) == inv.OK
    assert lib.inv_logprob_block16(by(cl), fake, 10, fake, fake, 4, 16, fake, big, null) == inv.E_ARG  # ldl < V
    assert lib.inv_logprob_block16(by(cl), fake, 16, fake, fake, 4, 16, null, 0, null) == inv.E_WORKSPACE
    # CPR Gated DeltaNet: width 128, chunk 32 or 64, one rank, enough aligned workspace
    cg = inv.contract(kv_chunk=64)
    gp = lambda c, D, ws, nbytes, cache=null: lib.inv_gdn_prefill(by(c), fake, fake, fake, fake, fake, fake, 2, 256,
                                                                   16, D, fake, cache, ws, nbytes, null)
    assert gp(cg, 64, fake, big) == inv.E_UNSUPPORTED
    assert gp(inv.contract(kv_chunk=128), 128, fake, big) == inv.E_CONTRACT
    assert gp(inv.contract(kv_chunk=64, ranks=2), 128, fake, big) == inv.E_UNSUPPORTED
    assert gp(cg, 128, fake, 1024) == inv.E_WORKSPACE
    assert gp(cg, 128, ctypes.c_void_p((1 << 20) + 4), big) == inv.E_ARG
    assert gp(cg, 128, fake, big, ctypes.c_void_p((1 << 20) + 8)) == inv.E_ARG  # misaligned cache
    assert lib.inv_gdn_decode(by(cg), fake, fake, fake, fake, fake, fake, 0, 16, 128, fake, fake, null) == inv.OK
    assert lib.inv_gdn_decode(by(cg), fake, fake, fake, fake, fake, fake, 4, 16, 128, fake, null, null) \
        == inv.E_ARG


def test_row_counts_beyond_a_dispatch_are_refused():
    # a dispatch counts workgroups x 256 lanes in 32 bits: one-workgroup-per-row
    # kernels take fewer than 2^24 rows, one-wave-per-row ones fewer than 2^26
    inv = _inv()
    lib = inv._lib
    by = ctypes.byref
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)
    c = inv.contract()
    rows_wg, rows_wave = 1 << 24, 1 << 26
    assert lib.inv_rmsnorm(by(c), fake, fake, fake, rows_wave, 8, null) == inv.E_UNSUPPORTED
    clp = inv.contract(leaves=4)
    assert lib.inv_logprob(by(clp), fake, 16, fake, fake, rows_wg, 16, null) == inv.E_UNSUPPORTED
    assert lib.inv_logprob_partials(by(clp), fake, 16, fake, fake, fake, rows_wg, 16, 0, 4, null) \
        == inv.E_UNSUPPORTED
    assert lib.inv_logprob_combine(by(clp), fake, fake, fake, fake, rows_wg, 16, null) == inv.E_UNSUPPORTED
    assert lib.inv_logprob_block16(by(c), fake, 16, fake, fake, rows_wg, 16, fake, 1 << 40, null) \
        == inv.E_UNSUPPORTED
    assert lib.inv_moe_route(by(c), fake, fake, fake, rows_wave, 128, null) == inv.E_UNSUPPORTED
    assert lib.inv_moe_combine(by(c), fake, fake, fake, 4, fake, 1 << 31, 64, null) == inv.E_UNSUPPORTED


def test_binding_workspace_checked_before_the_call():
    """The binding reports a workspace's size in bytes from its element type
    and refuses a host tensor, before the library sees the pointer."""
    import torch
    inv = _inv()
    assert inv._ws_bytes(None) == 0
    with pytest.raises(ValueError):
        inv._ws_bytes(torch.empty(16, dtype=torch.uint8))
    with pytest.raises(TypeError):
        inv._ws_bytes(16)


def test_status_strings():
    inv = _inv()
    for s in range(7):
        assert inv._lib.inv_status_string(s)
    assert inv._lib.inv_status_string(99) == b"unknown status"


def test_no_atomics_in_kernels():
    """Atomics make accumulation order depend on scheduling ([VeXact] section 3.1)."""
    csrc = os.path.join(ROOT, "split_invariant_deterministic_amd", "csrc")
    for f in os.listdir(csrc):
        txt = open(os.path.join(csrc, f)).read()
        assert not re.search(r"\batomic\w*\s*\(", txt, re.I), f
