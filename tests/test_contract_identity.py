"""Serialized execution contract and its SHA-256 identities (host only, no GPU).

IsoExec blog, "Unified execution contract": the contract has cases, a
composition of (region -> implementation + pinned constants), claims of the
proven parallel sizes, and three SHA-256 identities -- semantic,
numerical_policy and deployment -- that two runtimes compare before running.

Pins independent of the library: the FIPS 180 example digests, Python's
hashlib over every padding boundary, and the digests re-derived from the
library's own JSON text with json + hashlib.
"""

import ctypes
import hashlib
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "split_invariant_deterministic_amd", "libinv.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libinv.so not built")


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def path_composition(inv, **over):
    """The whole forward path's composition with the contract defaults."""
    e = {
        "norms.rms": inv.contract(),
        "linear": inv.contract(leaves=8),
        "lm_head": inv.contract(leaves=8, out="fp32"),
        "logprob": inv.contract(leaves=64),
        "attention": inv.contract(split_kv=16, kv_chunk=64),
        "moe.route": inv.contract(leaves=8),
        "moe.experts": inv.contract(leaves=8),
        "moe.combine": inv.contract(leaves=8),
        "lm_head_logprob": inv.contract(leaves=8, out="fp32"),
        "gdn.core": inv.contract(kv_chunk=64),
    }
    e.update(over)
    return e


# ------------------------------------------------------------------ SHA-256

FIPS_VECTORS = [
    (b"abc", "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad"),
    (b"", "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855"),
    (b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq",
     "248d6a61d20638b8e5c026930c3e6039a33ce45964ff2167f6ecedd419db06c1"),
]


@pytest.mark.parametrize("msg,digest", FIPS_VECTORS)
def test_sha256_fips_examples(inv, msg, digest):
    assert inv.sha256(msg).hex() == digest


def test_sha256_against_hashlib_at_padding_boundaries(inv):
    import random
    rng = random.Random(0)
    for n in list(range(0, 130)) + [183, 184, 1000, 4096, 65537]:
        data = bytes(rng.getrandbits(8) for _ in range(n))
        assert inv.sha256(data) == hashlib.sha256(data).digest(), n
    big = b"a" * 1_000_000
    assert inv.sha256(big) == hashlib.sha256(big).digest()


# ------------------------------------------------------------------ JSON and digests

def by_region(d):
    return {c["region"]: c for c in d["composition"]}


def _sections(text):
    d = json.loads(text)["ExecutionContract"]
    dump = lambda o: json.dumps(o, separators=(",", ":"), ensure_ascii=True).encode()
    sem = dump(d["semantic"])
    pol = dump({"cases": d["cases"], "composition": d["composition"], "claims": d["claims"]})
    dep = dump(d["deployment"])
    return d, sem, pol, dep


def test_json_layout_and_identities(inv):
    e = path_composition(inv)
    text = inv.contract_json(e)
    d, sem, pol, dep = _sections(text)
    assert list(d) == ["cases", "composition", "claims", "semantic", "deployment", "identities"]
    # canonical: the library's bytes are exactly the compact dump of what it wrote
    assert json.dumps(json.loads(text), separators=(",", ":")) == text
    regions = [c["region"] for c in d["composition"]]
    assert regions == ["norms.rms", "linear", "lm_head", "logprob", "attention", "moe.route",
                       "moe.experts", "moe.combine", "lm_head_logprob", "gdn.core"]
    assert by_region(d)["lm_head_logprob"]["constants"]["vocab_block"] == 16
    by = {c["region"]: c for c in d["composition"]}
    assert by["linear"]["constants"]["leaves"] == 8 and by["lm_head"]["constants"]["out_dtype"] == "fp32"
    assert by["logprob"]["constants"]["chunks"] == 64
    assert by["attention"]["constants"]["split_kv"] == 16 and by["attention"]["constants"]["kv_chunk"] == 64
    assert all(c["impl"]["arch"] == "gfx950" for c in d["composition"])
    assert d["claims"]["topology"]["linear"]["proven_ranks"] == [1, 2, 4, 8]
    assert d["claims"]["topology"]["logprob"]["proven_ranks"] == [1, 2, 4, 8, 16, 32, 64]
    assert d["semantic"]["constants"]["norms.rms"]["eps_fp32_bits"] == "0x358637bd"  # fp32(1e-6)
    ids = d["identities"]
    assert ids["semantic"] == hashlib.sha256(sem).hexdigest()
    assert ids["numerical_policy"] == hashlib.sha256(pol).hexdigest()
    assert ids["deployment"] == hashlib.sha256(dep).hexdigest()
    assert inv.contract_digest(e, inv.DIGEST_SEMANTIC).hex() == ids["semantic"]
    assert inv.contract_digest(e, inv.DIGEST_NUMERICAL_POLICY).hex() == ids["numerical_policy"]
    assert inv.contract_digest(e, inv.DIGEST_DEPLOYMENT).hex() == ids["deployment"]


def test_entry_order_does_not_matter(inv):
    e = path_composition(inv)
    rev = dict(reversed(list(e.items())))
    assert inv.contract_json(rev) == inv.contract_json(e)


def _digests(inv, e):
    return tuple(inv.contract_digest(e, k) for k in
                 (inv.DIGEST_SEMANTIC, inv.DIGEST_NUMERICAL_POLICY, inv.DIGEST_DEPLOYMENT))


@pytest.mark.parametrize("change,moved", [
    ({"linear": dict(leaves=4)}, "policy"),
    ({"lm_head": dict(leaves=8, out="bf16")}, "policy"),
    ({"logprob": dict(leaves=32)}, "policy"),
    ({"logprob": dict(leaves=64, tree="left_fold")}, "policy"),
    ({"attention": dict(split_kv=8)}, "policy"),
    ({"attention": dict(kv_chunk=128)}, "policy"),
    ({"lm_head_logprob": dict(leaves=4, out="fp32")}, "policy"),
    ({"gdn.core": dict(kv_chunk=32)}, "policy"),
    ({"linear": dict(leaves=8, ranks=4)}, "deployment"),   # a proven rank count: same bits
    ({"logprob": dict(leaves=64, ranks=2)}, "deployment"),
    ({"norms.rms": dict(eps=1e-5)}, "semantic"),           # a different model
])
def test_each_field_moves_exactly_its_digest(inv, change, moved):
    base = _digests(inv, path_composition(inv))
    over = {k: inv.contract(**v) for k, v in change.items()}
    new = _digests(inv, path_composition(inv, **over))
    expect = {"semantic": (False, True, True), "policy": (True, False, True),
              "deployment": (True, True, False)}[moved]
    assert tuple(a == b for a, b in zip(base, new)) == expect


def test_moe_top_k_is_semantic(inv):
    base = _digests(inv, path_composition(inv))
    new = _digests(inv, path_composition(inv, **{"moe.route": inv.contract(leaves=4),
                                                 "moe.combine": inv.contract(leaves=4)}))
    assert base[0] != new[0] and base[1] != new[1]


def test_verify_refuses_a_different_policy(inv):
    e = path_composition(inv)
    mine = inv.contract_digest(e, inv.DIGEST_NUMERICAL_POLICY)
    inv.contract_verify(e, inv.DIGEST_NUMERICAL_POLICY, mine)
    peer = inv.contract_digest(path_composition(inv, linear=inv.contract(leaves=4)), inv.DIGEST_NUMERICAL_POLICY)
    with pytest.raises(inv.InvError) as ex:
        inv.contract_verify(e, inv.DIGEST_NUMERICAL_POLICY, peer)
    assert ex.value.status == inv.E_CONTRACT
    # a peer on another proven rank count still agrees on the policy
    inv.contract_verify(path_composition(inv, linear=inv.contract(leaves=8, ranks=8)),
                        inv.DIGEST_NUMERICAL_POLICY, mine)


def test_invalid_compositions_are_rejected(inv):
    lib = inv._lib
    n = ctypes.c_size_t(0)
    with pytest.raises(inv.InvError) as ex:
        inv.contract_json({"linear": inv.contract(leaves=8, ranks=3)})
    assert ex.value.status == inv.E_TOPOLOGY
    with pytest.raises(inv.InvError) as ex:
        inv.contract_json({"linear": inv.contract(tree="left_fold")})  # the GEMM tree is balanced only
    assert ex.value.status == inv.E_CONTRACT
    with pytest.raises(inv.InvError) as ex:
        inv.contract_json({"lm_head_logprob": inv.contract(leaves=8)})  # logits must stay fp32
    assert ex.value.status == inv.E_CONTRACT
    with pytest.raises(inv.InvError) as ex:
        inv.contract_json({"gdn.core": inv.contract(kv_chunk=128)})  # chunks of 32 or 64
    assert ex.value.status == inv.E_CONTRACT
    with pytest.raises(inv.InvError) as ex:
        inv.contract_json({99: inv.contract()})
    assert ex.value.status == inv.E_ARG
    dup = inv.composition({"linear": inv.contract()})
    two = (inv.RegionContract * 2)(dup[0], dup[0])
    assert lib.inv_contract_json(two, 2, None, 0, ctypes.byref(n)) == inv.E_ARG
    assert lib.inv_contract_json(dup, 0, None, 0, ctypes.byref(n)) == inv.E_ARG
    assert lib.inv_contract_json(dup, 1, None, 0, None) == inv.E_ARG
    assert lib.inv_contract_json(dup, 1, None, 0, ctypes.byref(n)) == inv.OK and n.value > 0
    small = ctypes.create_string_buffer(n.value)  # one byte short of the NUL
    assert lib.inv_contract_json(dup, 1, small, n.value, ctypes.byref(n)) == inv.E_ARG
    assert small.raw == b"\0" * n.value
    d = (ctypes.c_uint8 * 32)()
    assert lib.inv_contract_digest(dup, 1, 7, d) == inv.E_ARG
