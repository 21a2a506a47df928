"""inv_gemm_noalloc against inv_gemm: the no-allocation entry point keeps the
GEMM's partials in the library's fixed per-GPU scratch array and must give
inv_gemm's bits for the same arguments, call after call (the scratch keeps
the previous call's partials), with sizes beyond the scratch rejected before
any launch.
"""

import pytest
import torch

from split_invariant_deterministic_amd import synth
from tests.helpers import bitwise_equal

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _operands(M, N, K, seed):
    return synth.randn((M, K), seed).to(DEV), synth.randn((N, K), seed + 1, 0.02).to(DEV)


def _both(inv, A, B, c):
    out_na = torch.full((A.shape[0], B.shape[0]), float("nan"), device=DEV,
                        dtype=torch.bfloat16 if c.out_dtype == inv.BF16 else torch.float32)
    inv.gemm_noalloc(A, B, c, out_na)
    ref = inv.gemm(A, B, c)   # inv_gemm with the workspace it asks for (allocated by the binding)
    torch.cuda.synchronize()
    return out_na, ref


def test_noalloc_equals_inv_gemm_on_consecutive_calls(inv):
    c8 = inv.contract(leaves=8)
    # 1) leaf groups in the scratch: 64 x 4096 x 12288, G = 8 groups, 8 MiB of partials
    A1, B1 = _operands(64, 4096, 12288, 700)
    assert inv.workspace_bytes(c8, inv.OP_GEMM, 64, 4096, 12288) == 8 * 64 * 4096 * 4
    got, ref = _both(inv, A1, B1, c8)
    assert bitwise_equal(got, ref)
    # 2) a smaller call right after it (the scratch still holds call 1's partials): 9 x 1024 x 2048, fp32 out
    cf = inv.contract(leaves=8, out="fp32")
    A2, B2 = _operands(9, 1024, 2048, 710)
    assert inv.workspace_bytes(cf, inv.OP_GEMM, 9, 1024, 2048) > 0
    got, ref = _both(inv, A2, B2, cf)
    assert bitwise_equal(got, ref)
    # 3) emulated ranks: two rank planes in the scratch
    c2 = inv.contract(leaves=8, ranks=2)
    A3, B3 = _operands(32, 2048, 4096, 720)
    got, ref = _both(inv, A3, B3, c2)
    assert bitwise_equal(got, ref)
    # 4) the largest leaf-group workspace any shape asks for fills the 16 MiB exactly: 1024 x 2048, G = 2
    A4, B4 = _operands(1024, 2048, 1024, 730)
    assert inv.workspace_bytes(c8, inv.OP_GEMM, 1024, 2048, 1024) == 16 << 20
    got, ref = _both(inv, A4, B4, c8)
    assert bitwise_equal(got, ref)
    # 4b) no partials needed (enough tiles): the single pass, no scratch
    A5, B5 = _operands(2048, 2048, 1024, 740)
    assert inv.workspace_bytes(c8, inv.OP_GEMM, 2048, 2048, 1024) == 0
    got, ref = _both(inv, A5, B5, c8)
    assert bitwise_equal(got, ref)
    # 5) more partials than the scratch holds: rejected before any launch, output untouched
    c8r = inv.contract(leaves=8, ranks=8)
    out = torch.full((1024, 2048), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(inv.InvError) as e:
        inv.gemm_noalloc(A4, B4, c8r, out)
    assert e.value.status == inv.E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    # 6) the first shape again, after all of the above
    got, ref = _both(inv, A1, B1, c8)
    assert bitwise_equal(got, ref)
