"""ctypes binding of libinv.so (declared in include/inv.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch supplies device memory (output and workspace tensors are
allocated here with torch) and the stream (the current torch stream, which is
a hipStream_t on ROCm). Importing this module raises if the library is not
built; there is no fallback of any kind.

Function names follow the C entry points without the ``inv_`` prefix.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m split_invariant_deterministic_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

# ------------------------------------------------------------------ constants
OK, E_ARG, E_CONTRACT, E_TOPOLOGY, E_UNSUPPORTED, E_HIP, E_WORKSPACE = range(7)
BF16, FP32 = 1, 2
BALANCED, LEFT_FOLD = 1, 2
OP_GEMM, OP_TREE_COMBINE, OP_RMSNORM, OP_LOGPROB, OP_DECODE_ATTN, OP_MOE_ROUTE, OP_MOE_GEMM, \
    OP_MOE_COMBINE, OP_LMHEAD_LOGPROB, OP_LOGPROB_BLOCK16, OP_GDN_PREFILL, OP_GDN_DECODE = range(1, 13)
ABI_VERSION = 1

_DT = {"bf16": BF16, "fp32": FP32, BF16: BF16, FP32: FP32}
_TREE = {"balanced": BALANCED, "left_fold": LEFT_FOLD, BALANCED: BALANCED, LEFT_FOLD: LEFT_FOLD}


class Contract(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("abi_version", ctypes.c_uint32),
        ("leaves", ctypes.c_uint32),
        ("ranks", ctypes.c_uint32),
        ("tree", ctypes.c_int32),
        ("accum_dtype", ctypes.c_int32),
        ("leaf_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("split_kv", ctypes.c_uint32),
        ("kv_chunk", ctypes.c_uint32),
        ("eps", ctypes.c_float),
        ("reserved", ctypes.c_uint32),
    ]

    def __repr__(self):
        return ("Contract(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")")


class InvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.inv_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_CP = ctypes.POINTER(Contract)

_SIGS = {
    "inv_contract_default": [_CP],
    "inv_contract_check": [_CP, ctypes.c_int, _I64],
    "inv_gemm": [_CP, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P],
    "inv_gemm_rank": [_CP, _P, _P, _P, _I64, _I64, _I64, _U32, _P],
    "inv_gemm_noalloc": [_CP, _P, _P, _P, _I64, _I64, _I64, _P],
    "inv_gemm_leaves": [_CP, _P, _P, _P, _I64, _I64, _I64, _U32, _U32, _P],
    "inv_tree_combine": [_CP, _P, _U32, _P, _I64, _I64, _P],
    "inv_cast_bf16": [_P, _P, _I64, _P],
    "inv_rmsnorm": [_CP, _P, _P, _P, _I64, _I64, _P],
    "inv_logprob": [_CP, _P, _I64, _P, _P, _I64, _I64, _P],
    "inv_logprob_partials": [_CP, _P, _I64, _P, _P, _P, _I64, _I64, _U32, _U32, _P],
    "inv_logprob_combine": [_CP, _P, _P, _P, _P, _I64, _I64, _P],
    "inv_decode_attn": [_CP, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _I32, _I32, _I32, _P, _SZ, _P],
    "inv_attn_splits": [_CP, _P, _P, _P, _P, _I32, _P, _P, _I64, _I32, _I32, _I32, _U32, _U32, _P,
                        _SZ, _P],
    "inv_attn_combine": [_CP, _P, _SZ, _P, _I64, _I32, _I32, _P],
    "inv_moe_route": [_CP, _P, _P, _P, _I64, _I32, _P],
    "inv_moe_permute": [_CP, _P, _P, _P, _P, _I64, _I32, _P],
    "inv_moe_gemm": [_CP, _P, _I64, _P, _P, _P, _P, _I64, _I32, _I64, _I64, _P],
    "inv_moe_gemm_swiglu": [_CP, _P, _I64, _P, _P, _P, _P, _I64, _I32, _I64, _I64, _P],
    "inv_swiglu": [_CP, _P, _P, _I64, _I64, _P],
    "inv_moe_combine": [_CP, _P, _P, _P, _I64, _P, _I64, _I64, _P],
    "inv_lmhead_logprob": [_CP, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P],
    "inv_logprob_block16": [_CP, _P, _I64, _P, _P, _I64, _I64, _P, _SZ, _P],
    "inv_gdn_prefill": [_CP, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _P, _SZ, _P],
    "inv_gdn_decode": [_CP, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P],
    "inv_bench_mfma_loop": [_I64, _I32, _P, _P, _P],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.inv_workspace_bytes.argtypes = [_CP, ctypes.c_int, _I64, _I64, _I64]
_lib.inv_workspace_bytes.restype = _SZ
_lib.inv_gdn_cache_bytes.argtypes = [_CP, _I32]
_lib.inv_gdn_cache_bytes.restype = _SZ
_lib.inv_status_string.argtypes = [ctypes.c_int]
_lib.inv_status_string.restype = ctypes.c_char_p


class RegionContract(ctypes.Structure):
    _fields_ = [("region", ctypes.c_int32), ("reserved", ctypes.c_uint32), ("contract", Contract)]


REGIONS = {"norms.rms": 1, "linear": 2, "lm_head": 3, "logprob": 4, "attention": 5, "moe.route": 6,
           "moe.experts": 7, "moe.combine": 8, "lm_head_logprob": 9, "gdn.core": 10}
DIGEST_SEMANTIC, DIGEST_NUMERICAL_POLICY, DIGEST_DEPLOYMENT = 1, 2, 3
_RCP = ctypes.POINTER(RegionContract)
_D32 = ctypes.c_uint8 * 32
for _name, _args in {
    "inv_contract_json": [_RCP, _SZ, ctypes.c_char_p, _SZ, ctypes.POINTER(_SZ)],
    "inv_contract_digest": [_RCP, _SZ, ctypes.c_int, _D32],
    "inv_contract_verify": [_RCP, _SZ, ctypes.c_int, _D32],
    "inv_sha256": [ctypes.c_char_p, _SZ, _D32],
}.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int

EXPORTS = sorted(list(_SIGS) + ["inv_workspace_bytes", "inv_status_string", "inv_gdn_cache_bytes", "inv_contract_json",
                                "inv_contract_digest", "inv_contract_verify", "inv_sha256"])


def _call(name, *args):
    st = getattr(_lib, name)(*args)
    if st != OK:
        raise InvError(st, name)


# ------------------------------------------------------------------ contract

def contract(leaves=8, ranks=1, tree="balanced", out="bf16", split_kv=16, kv_chunk=64, eps=1e-6,
             accum="fp32", leaf="fp32"):
    """A filled inv_contract (defaults from inv_contract_default, then overrides)."""
    c = Contract()
    _call("inv_contract_default", ctypes.byref(c))
    c.leaves = leaves
    c.ranks = ranks
    c.tree = _TREE[tree]
    c.out_dtype = _DT[out]
    c.accum_dtype = _DT[accum]
    c.leaf_dtype = _DT[leaf]
    c.split_kv = split_kv
    c.kv_chunk = kv_chunk
    c.eps = eps
    return c


def contract_check(c, op, K=0):
    """Host-only validation; returns the status code (0 = ok)."""
    return _lib.inv_contract_check(ctypes.byref(c), op, K)


def workspace_bytes(c, op, d0, d1, d2):
    return _lib.inv_workspace_bytes(ctypes.byref(c), op, d0, d1, d2)


# ------------------------------------------------------------------ identities

def composition(entries):
    """A C array of inv_region_contract from {region name: Contract}."""
    arr = (RegionContract * len(entries))()
    for i, (name, c) in enumerate(entries.items()):
        arr[i].region = REGIONS[name] if isinstance(name, str) else int(name)
        arr[i].contract = c
    return arr


def contract_json(entries):
    """Canonical JSON text of the composition (inv_contract_json)."""
    arr = composition(entries)
    n = _SZ(0)
    _call("inv_contract_json", arr, len(arr), None, 0, ctypes.byref(n))
    buf = ctypes.create_string_buffer(n.value + 1)
    _call("inv_contract_json", arr, len(arr), buf, n.value + 1, ctypes.byref(n))
    return buf.value.decode("ascii")


def contract_digest(entries, kind):
    """32-byte SHA-256 identity `kind` of the composition (inv_contract_digest)."""
    arr = composition(entries)
    d = _D32()
    _call("inv_contract_digest", arr, len(arr), kind, d)
    return bytes(d)


def contract_verify(entries, kind, expected):
    """Raises InvError (status E_CONTRACT) if the peer's digest differs."""
    arr = composition(entries)
    if len(expected) != 32:
        raise ValueError("a digest is 32 bytes")
    _call("inv_contract_verify", arr, len(arr), kind, _D32(*expected))


def sha256(data):
    d = _D32()
    _call("inv_sha256", bytes(data), len(data), d)
    return bytes(d)


# ------------------------------------------------------------------ helpers

def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {t.dim()}")
    return t


def _ws_bytes(ws, name="ws"):
    """Size in bytes of a workspace tensor, 0 for None.

    The library checks this size against what the call needs, so it must be
    the tensor's real size whatever its element type, and the pointer must be
    a device allocation the kernels can write from its start onwards."""
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if ws.device.type != "cuda":
        raise ValueError(f"{name}: expected a device tensor, got {ws.device}")
    if not ws.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ws.numel() * ws.element_size()


def _shape(t, shape, name):
    """Raises before any launch if t's shape is not ``shape`` (a wrong-sized
    buffer would be read or written out of bounds by the kernels)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _out_torch_dtype(c):
    return torch.bfloat16 if c.out_dtype == BF16 else torch.float32


# ------------------------------------------------------------------ GEMM

def gemm(A, B, c, out=None, ws=None, use_ws=True):
    """C [M,N] = tree over K leaves of A [M,K] . B[N,K]^T (inv_gemm).

    The workspace the library asks for is allocated unless ``ws`` is given;
    with ranks == 1 it is optional (``use_ws=False`` runs without it)."""
    _need(A, torch.bfloat16, "A", 2)
    _need(B, torch.bfloat16, "B", 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=_out_torch_dtype(c), device=A.device)
    _need(out, _out_torch_dtype(c), "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    nbytes = workspace_bytes(c, OP_GEMM, M, N, K)
    if ws is None and nbytes > 0 and (use_ws or c.ranks > 1):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=A.device)
    wsz = _ws_bytes(ws)
    _call("inv_gemm", ctypes.byref(c), _ptr(A), _ptr(B), _ptr(out), M, N, K, _ptr(ws), wsz, _stream())
    return out


def gemm_noalloc(A, B, c, out):
    """inv_gemm_noalloc: inv_gemm with the partials in the library's fixed
    per-GPU scratch; the caller passes the output, nothing is allocated."""
    _need(A, torch.bfloat16, "A", 2)
    _need(B, torch.bfloat16, "B", 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    _need(out, _out_torch_dtype(c), "out", 2)
    _shape(out, (M, N), "out")
    _call("inv_gemm_noalloc", ctypes.byref(c), _ptr(A), _ptr(B), _ptr(out), M, N, K, _stream())
    return out


def gemm_rank(A, B, rank, c, out=None):
    """P_r [M,N] fp32: the balanced subtree of emulated rank `rank` (inv_gemm_rank)."""
    _need(A, torch.bfloat16, "A", 2)
    _need(B, torch.bfloat16, "B", 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _need(out, torch.float32, "out", 2)
    _shape(out, (M, N), "out")
    _call("inv_gemm_rank", ctypes.byref(c), _ptr(A), _ptr(B), _ptr(out), M, N, K, rank, _stream())
    return out


def gemm_leaves(A, B, leaf_lo, leaf_hi, c, out=None):
    """P [hi-lo, M, N] fp32 per-leaf partials (inv_gemm_leaves)."""
    _need(A, torch.bfloat16, "A", 2)
    _need(B, torch.bfloat16, "B", 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if out is None:
        out = torch.empty((leaf_hi - leaf_lo, M, N), dtype=torch.float32, device=A.device)
    _need(out, torch.float32, "out", 3)
    _shape(out, (leaf_hi - leaf_lo, M, N), "out")
    _call("inv_gemm_leaves", ctypes.byref(c), _ptr(A), _ptr(B), _ptr(out), M, N, K, leaf_lo, leaf_hi,
          _stream())
    return out


def tree_combine(P, c, out=None):
    """C = cast(tree(P[0..count-1])) for P [count, M, N] fp32 (inv_tree_combine)."""
    _need(P, torch.float32, "P", 3)
    cnt, M, N = P.shape
    if out is None:
        out = torch.empty((M, N), dtype=_out_torch_dtype(c), device=P.device)
    _need(out, _out_torch_dtype(c), "out", 2)
    _shape(out, (M, N), "out")
    _call("inv_tree_combine", ctypes.byref(c), _ptr(P), cnt, _ptr(out), M, N, _stream())
    return out


def cast_bf16(x, out=None):
    _need(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    _shape(out, x.shape, "out")
    _call("inv_cast_bf16", _ptr(x), _ptr(out), x.numel(), _stream())
    return out


# ------------------------------------------------------------------ RMSNorm

def rmsnorm(x, gamma, c, out=None):
    _need(x, torch.bfloat16, "x", 2)
    _need(gamma, torch.bfloat16, "gamma", 1)
    M, H = x.shape
    if gamma.shape[0] != H:
        raise ValueError("gamma has the wrong length")
    if out is None:
        out = torch.empty_like(x)
    _need(out, torch.bfloat16, "out", 2)
    _shape(out, (M, H), "out")
    _call("inv_rmsnorm", ctypes.byref(c), _ptr(x), _ptr(gamma), _ptr(out), M, H, _stream())
    return out


# ------------------------------------------------------------------ logprob

def _logits_ld(logits):
    if logits.device.type != "cuda" or logits.dtype != torch.float32 or logits.dim() != 2:
        raise TypeError("logits: expected a 2-D fp32 device tensor")
    if logits.stride(1) != 1 or logits.stride(0) < logits.shape[1]:
        raise ValueError("logits: rows must be contiguous with stride >= V")
    return logits.stride(0)


def logprob(logits, target, c, out=None):
    ldl = _logits_ld(logits)
    M, V = logits.shape
    _need(target, torch.int32, "target", 1)
    _shape(target, (M,), "target")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=logits.device)
    _need(out, torch.float32, "out", 1)
    _shape(out, (M,), "out")
    _call("inv_logprob", ctypes.byref(c), _ptr(logits), ldl, _ptr(target), _ptr(out), M, V, _stream())
    return out


def logprob_partials(logits, target, chunk_lo, chunk_hi, c, stats=None, tlogit=None):
    ldl = _logits_ld(logits)
    M, V = logits.shape
    _need(target, torch.int32, "target", 1)
    if stats is None:
        stats = torch.full((M, c.leaves, 2), float("nan"), dtype=torch.float32, device=logits.device)
    if tlogit is None:
        tlogit = torch.full((M,), float("nan"), dtype=torch.float32, device=logits.device)
    _need(stats, torch.float32, "stats", 3)
    _need(tlogit, torch.float32, "tlogit", 1)
    _shape(target, (M,), "target")
    _shape(stats, (M, c.leaves, 2), "stats")
    _shape(tlogit, (M,), "tlogit")
    _call("inv_logprob_partials", ctypes.byref(c), _ptr(logits), ldl, _ptr(target), _ptr(stats),
          _ptr(tlogit), M, V, chunk_lo, chunk_hi, _stream())
    return stats, tlogit


def logprob_combine(stats, tlogit, target, V, c, out=None):
    _need(stats, torch.float32, "stats", 3)
    _need(tlogit, torch.float32, "tlogit", 1)
    _need(target, torch.int32, "target", 1)
    M = stats.shape[0]
    _shape(stats, (M, c.leaves, 2), "stats")
    _shape(tlogit, (M,), "tlogit")
    _shape(target, (M,), "target")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=stats.device)
    _need(out, torch.float32, "out", 1)
    _shape(out, (M,), "out")
    _call("inv_logprob_combine", ctypes.byref(c), _ptr(stats), _ptr(tlogit), _ptr(target), _ptr(out), M, V,
          _stream())
    return out


# ------------------------------------------------------------------ attention

def block16_workspace(M, V, device):
    """Workspace of the 16-column block schedule: stats [M, nb, 2] then tlogit [M]."""
    nb = (V + 15) // 16
    return torch.empty(M * nb * 2 + M, dtype=torch.float32, device=device)


def block16_views(ws, M, V):
    """(stats [M, nb, 2], tlogit [M]) views of a block16 workspace."""
    nb = (V + 15) // 16
    return ws[:M * nb * 2].view(M, nb, 2), ws[M * nb * 2:M * nb * 2 + M]


def lmhead_logprob(h, W, target, c, out=None, ws=None):
    """Fused LM head + selected-token logprob (inv_lmhead_logprob): lp [M] fp32."""
    _need(h, torch.bfloat16, "h", 2)
    _need(W, torch.bfloat16, "W", 2)
    _need(target, torch.int32, "target", 1)
    M, K = h.shape
    V = W.shape[0]
    if W.shape[1] != K or target.shape[0] != M:
        raise ValueError("h, W and target disagree")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=h.device)
    _need(out, torch.float32, "out", 1)
    _shape(out, (M,), "out")
    if ws is None:
        ws = block16_workspace(M, V, h.device)
    _call("inv_lmhead_logprob", ctypes.byref(c), _ptr(h), _ptr(W), _ptr(target), _ptr(out), M, V, K, _ptr(ws),
          _ws_bytes(ws), _stream())
    return out


def logprob_block16(logits, target, c, out=None, ws=None):
    """The 16-column block schedule from stored fp32 logits (inv_logprob_block16)."""
    _need(target, torch.int32, "target", 1)
    ldl = _logits_ld(logits)
    M, V = logits.shape
    _shape(target, (M,), "target")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=logits.device)
    _need(out, torch.float32, "out", 1)
    _shape(out, (M,), "out")
    if ws is None:
        ws = block16_workspace(M, V, logits.device)
    _call("inv_logprob_block16", ctypes.byref(c), _ptr(logits), ldl, _ptr(target), _ptr(out), M, V, _ptr(ws),
          _ws_bytes(ws), _stream())
    return out


# ------------------------------------------------------------------ Gated DeltaNet (CPR)

def gdn_cache(c, S, H, device):
    """Zeroed decode caches for S sequences (the state of empty sequences)."""
    n = _lib.inv_gdn_cache_bytes(ctypes.byref(c), H)
    if n == ctypes.c_size_t(-1).value:
        raise InvError(E_CONTRACT, "inv_gdn_cache_bytes")
    return torch.zeros(S * n // 4, dtype=torch.float32, device=device)


def gdn_prefill(q, k, v, g, beta, cu_seqlens, c, out=None, cache=None, ws=None):
    """CPR Gated DeltaNet over packed sequences (inv_gdn_prefill): out [T, H, 128]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n, 3)
    _need(g, torch.float32, "g", 2)
    _need(beta, torch.float32, "beta", 2)
    _need(cu_seqlens, torch.int32, "cu_seqlens", 1)
    T, H, D = q.shape
    S = cu_seqlens.shape[0] - 1
    _shape(k, q.shape, "k")
    _shape(v, q.shape, "v")
    _shape(g, (T, H), "g")
    _shape(beta, (T, H), "beta")
    if out is None:
        out = torch.empty((T, H, D), dtype=_out_torch_dtype(c), device=q.device)
    _need(out, _out_torch_dtype(c), "out", 3)
    _shape(out, (T, H, D), "out")
    if cache is not None:
        _need(cache, torch.float32, "cache", 1)
        if cache.numel() * 4 < S * _lib.inv_gdn_cache_bytes(ctypes.byref(c), H):
            raise ValueError("cache: smaller than S decode caches")
    if ws is None:
        ws = torch.empty(workspace_bytes(c, OP_GDN_PREFILL, T, H, S), dtype=torch.uint8, device=q.device)
    _call("inv_gdn_prefill", ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), S,
          T, H, D, _ptr(out), _ptr(cache), _ptr(ws), _ws_bytes(ws), _stream())
    return out


def gdn_decode(q, k, v, g, beta, pos, cache, c, out=None):
    """One decode token per sequence (inv_gdn_decode); cache is updated in place."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n, 3)
    _need(g, torch.float32, "g", 2)
    _need(beta, torch.float32, "beta", 2)
    _need(pos, torch.int32, "pos", 1)
    B, H, D = q.shape
    _shape(k, q.shape, "k")
    _shape(v, q.shape, "v")
    _shape(g, (B, H), "g")
    _shape(beta, (B, H), "beta")
    _shape(pos, (B,), "pos")
    _need(cache, torch.float32, "cache", 1)
    if cache.numel() * 4 < B * _lib.inv_gdn_cache_bytes(ctypes.byref(c), H):
        raise ValueError("cache: smaller than B decode caches")
    if out is None:
        out = torch.empty((B, H, D), dtype=_out_torch_dtype(c), device=q.device)
    _need(out, _out_torch_dtype(c), "out", 3)
    _shape(out, (B, H, D), "out")
    _call("inv_gdn_decode", ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(pos), B, H, D,
          _ptr(out), _ptr(cache), _stream())
    return out


def bench_mfma_loop(iters, groups, device="cuda"):
    """Measurement helper (inv_bench_mfma_loop): returns (clk [groups, 2]
    int64 cycles / 100 MHz ticks, flops) of a register-only MFMA loop."""
    clk = torch.zeros((groups, 2), dtype=torch.int64, device=device)
    sink = torch.empty(groups * 512, dtype=torch.float32, device=device)
    _call("inv_bench_mfma_loop", iters, groups, _ptr(clk), _ptr(sink), _stream())
    return clk, float(groups) * 8 * 8 * iters * 16384


def _attn_args(q, k, v, cu_seqlens, q_seq, q_pos):
    _need(q, torch.bfloat16, "q", 3)
    _need(k, torch.bfloat16, "k", 3)
    _need(v, torch.bfloat16, "v", 3)
    _need(cu_seqlens, torch.int32, "cu_seqlens", 1)
    _need(q_seq, torch.int32, "q_seq", 1)
    _need(q_pos, torch.int32, "q_pos", 1)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape[2] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k and v disagree on the head width, or k and v differ in shape")
    _shape(q_seq, (Tq,), "q_seq")
    _shape(q_pos, (Tq,), "q_pos")
    return Tq, Hq, Hkv, D, cu_seqlens.shape[0] - 1


def attn_workspace(q, c):
    Tq, Hq, D = q.shape
    n = workspace_bytes(c, OP_DECODE_ATTN, Tq, Hq, D)
    return torch.empty(max(n // 4, 1), dtype=torch.float32, device=q.device)


def decode_attn(q, k, v, cu_seqlens, q_seq, q_pos, c, ws=None, out=None):
    Tq, Hq, Hkv, D, S = _attn_args(q, k, v, cu_seqlens, q_seq, q_pos)
    if ws is None:
        ws = attn_workspace(q, c)
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out", 3)
    _shape(out, q.shape, "out")
    _call("inv_decode_attn", ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), S, _ptr(q_seq),
          _ptr(q_pos), _ptr(out), Tq, Hq, Hkv, D, _ptr(ws), _ws_bytes(ws), _stream())
    return out


def attn_splits(q, k, v, cu_seqlens, q_seq, q_pos, split_lo, split_hi, c, ws):
    Tq, Hq, Hkv, D, S = _attn_args(q, k, v, cu_seqlens, q_seq, q_pos)
    _call("inv_attn_splits", ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), S, _ptr(q_seq),
          _ptr(q_pos), Tq, Hq, Hkv, D, split_lo, split_hi, _ptr(ws), _ws_bytes(ws), _stream())
    return ws


def attn_combine(ws, Tq, Hq, D, c, out=None, device=None):
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=torch.bfloat16, device=ws.device)
    _need(out, torch.bfloat16, "out", 3)
    _shape(out, (Tq, Hq, D), "out")
    _call("inv_attn_combine", ctypes.byref(c), _ptr(ws), _ws_bytes(ws), _ptr(out), Tq, Hq, D, _stream())
    return out


# ------------------------------------------------------------------ MoE

def moe_route(logits, c):
    _need(logits, torch.float32, "logits", 2)
    T, E = logits.shape
    ids = torch.empty((T, c.leaves), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, c.leaves), dtype=torch.float32, device=logits.device)
    _call("inv_moe_route", ctypes.byref(c), _ptr(logits), _ptr(ids), _ptr(w), T, E, _stream())
    return ids, w


def moe_permute(ids, E, c):
    _need(ids, torch.int32, "ids", 2)
    T = ids.shape[0]
    offsets = torch.empty(E + 1, dtype=torch.int32, device=ids.device)
    rows = torch.empty(max(T * c.leaves, 1), dtype=torch.int32, device=ids.device)
    slot = torch.empty((T, c.leaves), dtype=torch.int32, device=ids.device)
    _call("inv_moe_permute", ctypes.byref(c), _ptr(ids), _ptr(offsets), _ptr(rows), _ptr(slot), T, E, _stream())
    return offsets, rows[:T * c.leaves], slot


def moe_gemm(X, rows, offsets, W, R, c, out=None):
    """Y [R, N]: grouped K-leaf GEMM of (gathered) X rows against W[e] (inv_moe_gemm)."""
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 3)
    _need(offsets, torch.int32, "offsets", 1)
    if rows is not None:
        _need(rows, torch.int32, "rows", 1)
    E, N, K = W.shape
    if X.shape[1] != K:
        raise ValueError("X and W disagree on K")
    _shape(offsets, (E + 1,), "offsets")
    if out is None:
        out = torch.empty((R, N), dtype=_out_torch_dtype(c), device=X.device)
    _need(out, _out_torch_dtype(c), "out", 2)
    _shape(out, (R, N), "out")
    if rows is not None and rows.shape[0] < R:
        raise ValueError("rows: fewer entries than grouped rows R")
    _call("inv_moe_gemm", ctypes.byref(c), _ptr(X), X.shape[0], _ptr(rows), _ptr(offsets), _ptr(W), _ptr(out), R,
          E, N, K, _stream())
    return out


def moe_gemm_swiglu(X, rows, offsets, W, R, c, out=None):
    """A [R, F]: the gate/up grouped GEMM (W [E, 2F, K], gate rows then up rows)
    with the SwiGLU in its epilogue (inv_moe_gemm_swiglu); bitwise
    swiglu(moe_gemm(...)) with a bf16 gate/up output."""
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 3)
    _need(offsets, torch.int32, "offsets", 1)
    if rows is not None:
        _need(rows, torch.int32, "rows", 1)
    E, N2, K = W.shape
    if X.shape[1] != K or N2 % 2:
        raise ValueError("X and W disagree on K, or W has an odd number of rows")
    F = N2 // 2
    _shape(offsets, (E + 1,), "offsets")
    if out is None:
        out = torch.empty((R, F), dtype=torch.bfloat16, device=X.device)
    _need(out, torch.bfloat16, "out", 2)
    _shape(out, (R, F), "out")
    if rows is not None and rows.shape[0] < R:
        raise ValueError("rows: fewer entries than grouped rows R")
    _call("inv_moe_gemm_swiglu", ctypes.byref(c), _ptr(X), X.shape[0], _ptr(rows), _ptr(offsets), _ptr(W), _ptr(out),
          R, E, F, K, _stream())
    return out


def swiglu(GU, c, out=None):
    _need(GU, torch.bfloat16, "GU", 2)
    R, F2 = GU.shape
    if F2 % 2:
        raise ValueError("GU: odd number of columns")
    F = F2 // 2
    if out is None:
        out = torch.empty((R, F), dtype=torch.bfloat16, device=GU.device)
    _need(out, torch.bfloat16, "out", 2)
    _shape(out, (R, F), "out")
    _call("inv_swiglu", ctypes.byref(c), _ptr(GU), _ptr(out), R, F, _stream())
    return out


def moe_combine(Y, w, slot, c, out=None):
    _need(Y, torch.float32, "Y", 2)
    _need(w, torch.float32, "w", 2)
    _need(slot, torch.int32, "slot", 2)
    T = w.shape[0]
    H = Y.shape[1]
    _shape(w, (T, c.leaves), "w")
    _shape(slot, (T, c.leaves), "slot")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=Y.device)
    _need(out, torch.bfloat16, "out", 2)
    _shape(out, (T, H), "out")
    _call("inv_moe_combine", ctypes.byref(c), _ptr(Y), _ptr(w), _ptr(slot), Y.shape[0], _ptr(out), T, H,
          _stream())
    return out


def moe_layer(x, logits, W1, W2, c_gemm, c_route, out_stage=None):
    """The whole MoE layer: route, group, gate/up GEMM with the SwiGLU fused in
    its epilogue, down GEMM, combine.

    c_gemm pins the expert GEMMs' K leaves; c_route.leaves is the top-k and
    the combine's leaf count. Returns out [T, H] bf16 (and the stage tensors
    in ``out_stage`` if a dict is passed).
    """
    T = x.shape[0]
    E = W1.shape[0]
    ids, w = moe_route(logits, c_route)
    offsets, rows, slot = moe_permute(ids, E, c_route)
    R = T * c_route.leaves
    cg = Contract.from_buffer_copy(c_gemm)
    cg.out_dtype = BF16
    A = moe_gemm_swiglu(x, rows, offsets, W1, R, cg)
    cd = Contract.from_buffer_copy(c_gemm)
    cd.out_dtype = FP32
    Y = moe_gemm(A, None, offsets, W2, R, cd)
    out = moe_combine(Y, w, slot, c_route)
    if out_stage is not None:  # the unfused gate/up output too, for inspection
        GU = moe_gemm(x, rows, offsets, W1, R, cg)
        out_stage.update(ids=ids, w=w, offsets=offsets, rows=rows, slot=slot, GU=GU, A=A, Y=Y)
    return out
