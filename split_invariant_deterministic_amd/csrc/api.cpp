// C-ABI layer of libinv: contract and shape validation (host only, before any
// HIP call), workspace sizing, and dispatch to the gfx950 kernel launchers.
//
// The contract mirrors the execution contract of the IsoExec blog ("Unified
// execution contract"): every constant that can move a rounding is explicit.
// The topology claim of that section -- a parallel size is accepted only if
// it has been proven invariant -- becomes the rank check here: ranks must be
// a power of two dividing the leaf count, because then each rank owns an
// aligned block of leaves, which is a subtree of the balanced tree, and its
// local sum is a node of the same tree.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <new>

#include "../../include/inv.h"
#include "launch.h"

namespace {

bool is_pow2(uint64_t v) { return v != 0 && (v & (v - 1)) == 0; }

inv_status hip_status(hipError_t e) { return e == hipSuccess ? INV_OK : INV_E_HIP; }

// Common contract checks; op-specific limits follow in each entry point.
inv_status check_contract(const inv_contract* c) {
  if (!c) return INV_E_ARG;
  if (c->struct_size != sizeof(inv_contract) || c->abi_version != INV_ABI_VERSION) return INV_E_ARG;
  if (c->reserved != 0) return INV_E_ARG;
  if (c->accum_dtype != INV_FP32 || c->leaf_dtype != INV_FP32) return INV_E_CONTRACT;
  if (c->out_dtype != INV_BF16 && c->out_dtype != INV_FP32) return INV_E_CONTRACT;
  if (c->tree != INV_TREE_BALANCED && c->tree != INV_TREE_LEFT_FOLD) return INV_E_CONTRACT;
  if (!is_pow2(c->leaves)) return INV_E_CONTRACT;
  if (!is_pow2(c->ranks) || c->ranks > c->leaves || c->leaves % c->ranks != 0) return INV_E_TOPOLOGY;
  return INV_OK;
}

inv_status check_gemm_contract(const inv_contract* c, int64_t K) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (c->tree != INV_TREE_BALANCED) return INV_E_CONTRACT;  // the in-kernel tree is balanced only
  if (c->leaves > 8) return INV_E_UNSUPPORTED;
  if (K < 0) return INV_E_ARG;
  // the ring kernel addresses a tile's 128 operand rows by 32-bit byte
  // offsets (row * K * 2): K < 2^24 keeps every one of them in range
  if (K >= ((int64_t)1 << 24)) return INV_E_UNSUPPORTED;
  if (K % c->leaves != 0) return INV_E_CONTRACT;
  if ((K / c->leaves) % 32 != 0) return INV_E_CONTRACT;
  if (K == 0) return INV_E_CONTRACT;
  return INV_OK;
}

inv_status check_attn_contract(const inv_contract* c) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (!is_pow2(c->split_kv) || c->split_kv > 32) return INV_E_CONTRACT;
  if (c->kv_chunk != 32 && c->kv_chunk != 64 && c->kv_chunk != 128) return INV_E_CONTRACT;
  if (c->out_dtype != INV_BF16) return INV_E_CONTRACT;
  return INV_OK;
}

inv_status check_gdn_contract(const inv_contract* c) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (c->kv_chunk != 32 && c->kv_chunk != 64) return INV_E_CONTRACT;
  if (c->ranks != 1) return INV_E_UNSUPPORTED;
  return INV_OK;
}

size_t gdn_prefill_ws_bytes(int64_t T, int64_t H, int64_t S, int64_t C) {
  return ((size_t)2 * T * H * 128 + (size_t)T * H + (size_t)(T / C + S) * H * (128 * 128 + C * C + 2 * C)) *
         sizeof(float);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// fp32 and bf16 buffers are read and written at least one element at a time
bool aligned_to(const void* p, unsigned bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1u)) == 0; }

inv_status check_logprob_contract(const inv_contract* c, int64_t V) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (c->leaves > 512) return INV_E_UNSUPPORTED;
  if (V > 0 && (int64_t)c->leaves > V) return INV_E_CONTRACT;  // every chunk non-empty
  return INV_OK;
}

bool out_is_bf16(const inv_contract* c) { return c->out_dtype == INV_BF16; }

// A dispatch counts its work-items (workgroups x 256 lanes here) in 32 bits.
// Kernels with one 256-lane workgroup per row therefore take fewer than 2^24
// rows per launch, and those with four rows (one wave each) per workgroup
// fewer than 2^26; more is refused before any launch.
constexpr int64_t kMaxRowsWg = (int64_t)1 << 24;
constexpr int64_t kMaxRowsWave = (int64_t)1 << 26;

// Leaf groups for the single-rank GEMM when 128 x 128 tiles alone leave
// compute units idle (M >= 8; below 8 rows the stream kernel reads the
// weights fastest in one pass): G aligned subtrees of L/G leaves each are
// reduced by separate workgroups into a workspace and the top log2(G) tree
// levels finish the sum. Every subtree is a node of the same balanced tree,
// so the bits equal the single-pass kernel's. A tile's time is set by its K
// chain, so G is the largest power of two with tiles * G <= 256 (one
// workgroup per compute unit on MI355X); measured best on 4096-12288 wide
// projections.
int gemm_split_groups(const inv_contract* c, int64_t M, int64_t N) {
  if (c->ranks != 1 || M < 8) return 1;
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int G = 1;
  while (G < (int)c->leaves && tiles * G * 2 <= 256) G *= 2;
  return G;
}

}  // namespace

extern "C" {

inv_status inv_contract_default(inv_contract* c) {
  if (!c) return INV_E_ARG;
  std::memset(c, 0, sizeof(*c));
  c->struct_size = sizeof(inv_contract);
  c->abi_version = INV_ABI_VERSION;
  c->leaves = 8;
  c->ranks = 1;
  c->tree = INV_TREE_BALANCED;
  c->accum_dtype = INV_FP32;
  c->leaf_dtype = INV_FP32;
  c->out_dtype = INV_BF16;
  c->split_kv = 16;
  c->kv_chunk = 64;
  c->eps = 1e-6f;
  c->reserved = 0;
  return INV_OK;
}

inv_status inv_contract_check(const inv_contract* c, int op, int64_t K) {
  switch (op) {
    case INV_OP_GEMM:
    case INV_OP_MOE_GEMM:
      return check_gemm_contract(c, K);
    case INV_OP_TREE_COMBINE:
    case INV_OP_MOE_COMBINE:
    case INV_OP_MOE_ROUTE:
      return check_contract(c);
    case INV_OP_RMSNORM: {
      inv_status s = check_contract(c);
      if (s != INV_OK) return s;
      if (!(c->eps >= 0.0f) || !std::isfinite(c->eps)) return INV_E_CONTRACT;
      return INV_OK;
    }
    case INV_OP_LOGPROB:
      return check_logprob_contract(c, 0);
    case INV_OP_DECODE_ATTN:
      return check_attn_contract(c);
    case INV_OP_LMHEAD_LOGPROB: {
      inv_status s = check_gemm_contract(c, K);
      if (s != INV_OK) return s;
      if (c->out_dtype != INV_FP32) return INV_E_CONTRACT;
      return c->ranks == 1 ? INV_OK : INV_E_UNSUPPORTED;
    }
    case INV_OP_LOGPROB_BLOCK16:
      return check_contract(c);
    case INV_OP_GDN_PREFILL:
    case INV_OP_GDN_DECODE:
      return check_gdn_contract(c);
    default:
      return INV_E_ARG;
  }
}

size_t inv_workspace_bytes(const inv_contract* c, int op, int64_t d0, int64_t d1, int64_t d2) {
  if (d0 < 0 || d1 < 0 || d2 < 0) return (size_t)-1;
  switch (op) {
    case INV_OP_GEMM: {
      if (check_gemm_contract(c, d2) != INV_OK) return (size_t)-1;
      if (c->ranks > 1) return (size_t)c->ranks * (size_t)d0 * (size_t)d1 * sizeof(float);
      const int G = gemm_split_groups(c, d0, d1);
      return G > 1 ? (size_t)G * (size_t)d0 * (size_t)d1 * sizeof(float) : 0;
    }
    case INV_OP_DECODE_ATTN:
      if (check_attn_contract(c) != INV_OK) return (size_t)-1;
      return (size_t)d0 * (size_t)d1 * (size_t)c->split_kv * (size_t)(d2 + 2) * sizeof(float);
    case INV_OP_GDN_PREFILL:
      if (check_gdn_contract(c) != INV_OK || d1 < 1 || d2 < 1) return (size_t)-1;
      return gdn_prefill_ws_bytes(d0, d1, d2, c->kv_chunk) + 16;
    case INV_OP_LMHEAD_LOGPROB:
    case INV_OP_LOGPROB_BLOCK16:
      if (inv_contract_check(c, op, d2) != INV_OK || d1 <= 0 || (d1 + 15) / 16 > 16384) return (size_t)-1;
      return (size_t)d0 * (size_t)((d1 + 15) / 16) * 8u + (size_t)d0 * 4u;
    default:
      if (inv_contract_check(c, op, d2) != INV_OK) return (size_t)-1;
      return 0;
  }
}

const char* inv_status_string(inv_status s) {
  switch (s) {
    case INV_OK: return "ok";
    case INV_E_ARG: return "invalid argument";
    case INV_E_CONTRACT: return "contract constant not implemented";
    case INV_E_TOPOLOGY: return "rank count outside the proven set";
    case INV_E_UNSUPPORTED: return "shape outside the implemented range";
    case INV_E_HIP: return "HIP launch or query failed";
    case INV_E_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------ GEMM

static inv::GemmLaunch gemm_launch(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                   int kl, int leaf_lo, int nl, int groups, bool out_bf16) {
  inv::GemmLaunch g;
  g.A = A;
  g.B = B;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.c_group_stride = M * N;
  g.kl = kl;
  g.leaf_lo = leaf_lo;
  g.nl = nl;
  g.groups = groups;
  g.out_bf16 = out_bf16;
  g.rows = nullptr;
  g.offsets = nullptr;
  g.E = 0;
  g.a_rows = M;
  g.b_expert_stride = 0;
  return g;
}

static inv_status gemm_shape_check(const void* A, const void* B, const void* C, unsigned c_elem, int64_t M,
                                   int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0) return INV_E_ARG;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 31) return INV_E_UNSUPPORTED;
  if (M > 0 && N > 0 && (!A || !B || !C)) return INV_E_ARG;
  // 16-byte vector loads along K
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15u) return INV_E_ARG;
  if (!aligned_to(C, c_elem)) return INV_E_ARG;
  return INV_OK;
}

inv_status inv_gemm(const inv_contract* c, const void* A, const void* B, void* C, int64_t M, int64_t N,
                    int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
  inv_status s = check_gemm_contract(c, K);
  if (s != INV_OK) return s;
  if ((s = gemm_shape_check(A, B, C, out_is_bf16(c) ? 2u : 4u, M, N, K)) != INV_OK) return s;
  if (!aligned_to(ws, 4u)) return INV_E_ARG;  // fp32 partial planes
  if (M == 0 || N == 0) return INV_OK;
  const int L = (int)c->leaves, R = (int)c->ranks;
  const int kl = (int)(K / L);
  if (R == 1) {
    const int G = gemm_split_groups(c, M, N);
    const size_t need_g = (size_t)G * (size_t)M * (size_t)N * sizeof(float);
    if (G == 1 || !ws || ws_bytes < need_g)  // the workspace is optional here
      return hip_status(inv::launch_gemm(gemm_launch(A, B, C, M, N, K, kl, 0, L, 1, out_is_bf16(c)), stream));
    hipError_t e = inv::launch_gemm(gemm_launch(A, B, ws, M, N, K, kl, 0, L / G, G, false), stream);
    if (e != hipSuccess) return INV_E_HIP;
    return hip_status(inv::launch_tree_combine(static_cast<const float*>(ws), G, M * N, C, out_is_bf16(c), false,
                                               stream));
  }
  const size_t need = (size_t)R * (size_t)M * (size_t)N * sizeof(float);
  if (!ws || ws_bytes < need) return INV_E_WORKSPACE;
  // every emulated rank reduces its aligned subtree into its own fp32 plane ...
  hipError_t e = inv::launch_gemm(gemm_launch(A, B, ws, M, N, K, kl, 0, L / R, R, false), stream);
  if (e != hipSuccess) return INV_E_HIP;
  // ... and the top log2(R) levels of the same tree finish the sum
  return hip_status(inv::launch_tree_combine(static_cast<const float*>(ws), R, M * N, C, out_is_bf16(c), false,
                                             stream));
}

inv_status inv_gemm_noalloc(const inv_contract* c, const void* A, const void* B, void* C, int64_t M, int64_t N,
                            int64_t K, hipStream_t stream) {
  inv_status s = check_gemm_contract(c, K);
  if (s != INV_OK) return s;
  if ((s = gemm_shape_check(A, B, C, out_is_bf16(c) ? 2u : 4u, M, N, K)) != INV_OK) return s;
  if (M == 0 || N == 0) return INV_OK;
  const int L = (int)c->leaves, R = (int)c->ranks;
  const int kl = (int)(K / L);
  // the partials inv_gemm keeps in its workspace: R rank planes, or (one rank)
  // the G leaf groups it uses when given enough workspace
  const int G = R > 1 ? R : gemm_split_groups(c, M, N);
  if (G == 1) return hip_status(inv::launch_gemm(gemm_launch(A, B, C, M, N, K, kl, 0, L, 1, out_is_bf16(c)), stream));
  const size_t need = (size_t)G * (size_t)M * (size_t)N * sizeof(float);
  if (need > inv::kScratchBytes) return INV_E_WORKSPACE;  // more partials than the fixed scratch holds
  void* ws = nullptr;
  if (inv::scratch_device_ptr(&ws) != hipSuccess) return INV_E_HIP;
  // every partial plane is written in full before the combine reads it: nothing needs clearing
  hipError_t e = inv::launch_gemm(gemm_launch(A, B, ws, M, N, K, kl, 0, L / G, G, false), stream);
  if (e != hipSuccess) return INV_E_HIP;
  return hip_status(
      inv::launch_tree_combine(static_cast<const float*>(ws), G, M * N, C, out_is_bf16(c), false, stream));
}

inv_status inv_gemm_rank(const inv_contract* c, const void* A, const void* B, float* P_r, int64_t M, int64_t N,
                         int64_t K, uint32_t rank, hipStream_t stream) {
  inv_status s = check_gemm_contract(c, K);
  if (s != INV_OK) return s;
  if ((s = gemm_shape_check(A, B, P_r, 4u, M, N, K)) != INV_OK) return s;
  if (rank >= c->ranks) return INV_E_ARG;
  if (M == 0 || N == 0) return INV_OK;
  const int L = (int)c->leaves, R = (int)c->ranks;
  const int nl = L / R;
  return hip_status(
      inv::launch_gemm(gemm_launch(A, B, P_r, M, N, K, (int)(K / L), (int)rank * nl, nl, 1, false), stream));
}

inv_status inv_gemm_leaves(const inv_contract* c, const void* A, const void* B, float* P, int64_t M, int64_t N,
                           int64_t K, uint32_t leaf_lo, uint32_t leaf_hi, hipStream_t stream) {
  inv_status s = check_gemm_contract(c, K);
  if (s != INV_OK) return s;
  if ((s = gemm_shape_check(A, B, P, 4u, M, N, K)) != INV_OK) return s;
  if (leaf_lo >= leaf_hi || leaf_hi > c->leaves) return INV_E_ARG;
  if (M == 0 || N == 0) return INV_OK;
  const int L = (int)c->leaves;
  return hip_status(inv::launch_gemm(
      gemm_launch(A, B, P, M, N, K, (int)(K / L), (int)leaf_lo, 1, (int)(leaf_hi - leaf_lo), false), stream));
}

inv_status inv_tree_combine(const inv_contract* c, const float* P, uint32_t count, void* C, int64_t M, int64_t N,
                            hipStream_t stream) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (M < 0 || N < 0) return INV_E_ARG;
  if (!is_pow2(count) || count > 64) return INV_E_UNSUPPORTED;
  if (M == 0 || N == 0) return INV_OK;
  if (!P || !C) return INV_E_ARG;
  if (!aligned_to(P, 4u) || !aligned_to(C, out_is_bf16(c) ? 2u : 4u)) return INV_E_ARG;
  return hip_status(inv::launch_tree_combine(P, (int)count, M * N, C, out_is_bf16(c), c->tree == INV_TREE_LEFT_FOLD,
                                             stream));
}

inv_status inv_cast_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream) {
  if (n < 0) return INV_E_ARG;
  if (n == 0) return INV_OK;
  if (!x || !y) return INV_E_ARG;
  return hip_status(inv::launch_cast_bf16(x, y, n, stream));
}

// --------------------------------------------------------------- RMSNorm

inv_status inv_rmsnorm(const inv_contract* c, const void* x, const void* gamma, void* y, int64_t M, int64_t H,
                       hipStream_t stream) {
  inv_status s = inv_contract_check(c, INV_OP_RMSNORM, 0);
  if (s != INV_OK) return s;
  if (M < 0 || H < 0) return INV_E_ARG;
  if (H % 8 != 0 || H > 16384 || (H > 0 && H < 8)) return INV_E_UNSUPPORTED;
  if (M >= kMaxRowsWave) return INV_E_UNSUPPORTED;
  if (M == 0 || H == 0) return INV_OK;
  if (!x || !gamma || !y) return INV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(gamma) | reinterpret_cast<uintptr_t>(y)) & 15u)
    return INV_E_ARG;
  if (c->out_dtype != INV_BF16) return INV_E_CONTRACT;
  return hip_status(inv::launch_rmsnorm(x, gamma, y, M, H, c->eps, stream));
}

// --------------------------------------------------------------- logprob

inv_status inv_logprob(const inv_contract* c, const float* logits, int64_t ldl, const int32_t* target, float* out,
                       int64_t M, int64_t V, hipStream_t stream) {
  inv_status s = check_logprob_contract(c, V);
  if (s != INV_OK) return s;
  if (M < 0 || V <= 0 || ldl < V) return INV_E_ARG;
  if (M >= kMaxRowsWg) return INV_E_UNSUPPORTED;
  if (M == 0) return INV_OK;
  if (!logits || !target || !out) return INV_E_ARG;
  return hip_status(inv::launch_logprob(logits, ldl, target, out, nullptr, nullptr, M, V, (int)c->leaves, 0,
                                        (int)c->leaves, c->tree == INV_TREE_LEFT_FOLD, false, stream));
}

// ------------------------------------------------------- Gated DeltaNet (CPR)

size_t inv_gdn_cache_bytes(const inv_contract* c, int32_t H) {
  if (check_gdn_contract(c) != INV_OK || H <= 0) return (size_t)-1;
  return (size_t)inv::gdn_cache_floats(H, (int)c->kv_chunk) * sizeof(float);
}

inv_status inv_gdn_prefill(const inv_contract* c, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu_seqlens, int32_t S, int64_t T, int32_t H, int32_t D,
                           void* out, void* cache, void* ws, size_t ws_bytes, hipStream_t stream) {
  inv_status s = check_gdn_contract(c);
  if (s != INV_OK) return s;
  if (D != 128) return INV_E_UNSUPPORTED;
  if (S < 1 || T < 0 || H < 1) return INV_E_ARG;
  if (T / (int64_t)c->kv_chunk + S > ((int64_t)1 << 31) - 1 || H > 65535) return INV_E_UNSUPPORTED;
  if (!cu_seqlens) return INV_E_ARG;
  if (T > 0 && (!q || !k || !v || !g || !beta || !out)) return INV_E_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(cache) || !aligned16(ws))
    return INV_E_ARG;
  const size_t need = gdn_prefill_ws_bytes(T, H, S, c->kv_chunk);
  if (!ws || ws_bytes < need) return INV_E_WORKSPACE;
  inv::GdnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.S = S;
  a.T = T;
  a.H = H;
  a.out = out;
  a.cache = cache;
  float* w = static_cast<float*>(ws);
  a.qh = w;
  a.kh = w + T * H * 128;
  a.alpha = w + 2 * T * H * 128;
  // boundary states and chunk coefficients start on 16-byte boundaries
  const int64_t slots = T / c->kv_chunk + S, C = c->kv_chunk;
  a.bstates = w + ((2 * T * H * 128 + T * H + 3) / 4) * 4;
  a.coef = a.bstates + slots * H * 128 * 128;
  if (reinterpret_cast<char*>(a.coef + slots * H * (C * C + 2 * C)) > static_cast<char*>(ws) + ws_bytes)
    return INV_E_WORKSPACE;
  return hip_status(inv::launch_gdn_prefill(a, (int)c->kv_chunk, out_is_bf16(c), stream));
}

inv_status inv_gdn_decode(const inv_contract* c, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* pos, int32_t B, int32_t H, int32_t D, void* out,
                          void* cache, hipStream_t stream) {
  inv_status s = check_gdn_contract(c);
  if (s != INV_OK) return s;
  if (D != 128) return INV_E_UNSUPPORTED;
  if (B < 0 || H < 1 || H > 65535) return INV_E_ARG;
  if (B == 0) return INV_OK;
  if (!q || !k || !v || !g || !beta || !pos || !out || !cache) return INV_E_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(cache)) return INV_E_ARG;
  inv::GdnDecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.g = g;
  a.beta = beta;
  a.pos = pos;
  a.B = B;
  a.H = H;
  a.out = out;
  a.cache = cache;
  return hip_status(inv::launch_gdn_decode(a, (int)c->kv_chunk, out_is_bf16(c), stream));
}

// ------------------------------------------------------- LM head + logprob

namespace {
constexpr int64_t kMaxBlocks16 = 16384;  // 16-column blocks per row: V <= 262144

size_t block16_ws_bytes(int64_t M, int64_t V) {
  const int64_t nb = (V + 15) / 16;
  return (size_t)M * (size_t)nb * 8u + (size_t)M * 4u;
}

inv_status check_block16(const inv_contract* c, int64_t M, int64_t V, void* ws, size_t ws_bytes) {
  if (M < 0 || V <= 0) return INV_E_ARG;
  if ((V + 15) / 16 > kMaxBlocks16 || M >= kMaxRowsWg) return INV_E_UNSUPPORTED;
  if (M > 0 && (!ws || ws_bytes < block16_ws_bytes(M, V))) return INV_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 7u) return INV_E_ARG;  // (m, s) pairs are read as float2
  (void)c;
  return INV_OK;
}
}  // namespace

inv_status inv_lmhead_logprob(const inv_contract* c, const void* h, const void* W, const int32_t* target,
                              float* out, int64_t M, int64_t V, int64_t K, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  inv_status s = check_gemm_contract(c, K);
  if (s != INV_OK) return s;
  if (c->out_dtype != INV_FP32) return INV_E_CONTRACT;  // logits are never rounded below fp32
  if (c->ranks != 1) return INV_E_UNSUPPORTED;
  if ((s = gemm_shape_check(h, W, out, 4u, M, V, K)) != INV_OK) return s;
  if ((s = check_block16(c, M, V, ws, ws_bytes)) != INV_OK) return s;
  if (M == 0) return INV_OK;
  if (!target) return INV_E_ARG;
  float* stats = static_cast<float*>(ws);
  float* tlogit = stats + 2 * M * ((V + 15) / 16);
  inv::GemmLaunch g = gemm_launch(h, W, nullptr, M, V, K, (int)(K / c->leaves), 0, (int)c->leaves, 1, false);
  g.lp_stats = stats;
  g.lp_tlogit = tlogit;
  g.lp_target = target;
  hipError_t e = inv::launch_gemm(g, stream);
  if (e != hipSuccess) return INV_E_HIP;
  return hip_status(inv::launch_block16_merge(stats, tlogit, target, out, M, V, false, stream));
}

inv_status inv_logprob_block16(const inv_contract* c, const float* logits, int64_t ldl, const int32_t* target,
                               float* out, int64_t M, int64_t V, void* ws, size_t ws_bytes, hipStream_t stream) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (ldl < V) return INV_E_ARG;
  if ((s = check_block16(c, M, V, ws, ws_bytes)) != INV_OK) return s;
  if (M == 0) return INV_OK;
  if (!logits || !target || !out) return INV_E_ARG;
  float* stats = static_cast<float*>(ws);
  float* tlogit = stats + 2 * M * ((V + 15) / 16);
  hipError_t e = inv::launch_block16_stats(logits, ldl, target, stats, tlogit, M, V, stream);
  if (e != hipSuccess) return INV_E_HIP;
  return hip_status(
      inv::launch_block16_merge(stats, tlogit, target, out, M, V, c->tree == INV_TREE_LEFT_FOLD, stream));
}

inv_status inv_logprob_partials(const inv_contract* c, const float* logits, int64_t ldl, const int32_t* target,
                                float* stats, float* tlogit, int64_t M, int64_t V, uint32_t chunk_lo,
                                uint32_t chunk_hi, hipStream_t stream) {
  inv_status s = check_logprob_contract(c, V);
  if (s != INV_OK) return s;
  if (M < 0 || V <= 0 || ldl < V) return INV_E_ARG;
  if (chunk_lo >= chunk_hi || chunk_hi > c->leaves) return INV_E_ARG;
  if (M >= kMaxRowsWg) return INV_E_UNSUPPORTED;
  if (M == 0) return INV_OK;
  if (!logits || !target || !stats || !tlogit) return INV_E_ARG;
  return hip_status(inv::launch_logprob(logits, ldl, target, nullptr, stats, tlogit, M, V, (int)c->leaves,
                                        (int)chunk_lo, (int)chunk_hi, false, true, stream));
}

inv_status inv_logprob_combine(const inv_contract* c, const float* stats, const float* tlogit,
                               const int32_t* target, float* out, int64_t M, int64_t V, hipStream_t stream) {
  inv_status s = check_logprob_contract(c, V);
  if (s != INV_OK) return s;
  if (M < 0 || V <= 0) return INV_E_ARG;
  if (M >= kMaxRowsWg) return INV_E_UNSUPPORTED;
  if (M == 0) return INV_OK;
  if (!stats || !tlogit || !target || !out) return INV_E_ARG;
  return hip_status(inv::launch_logprob_combine(stats, tlogit, target, out, M, V, (int)c->leaves,
                                                c->tree == INV_TREE_LEFT_FOLD, stream));
}

// ------------------------------------------------------------- attention

static inv_status attn_check(const inv_contract* c, const void* q, const void* k, const void* v,
                             const int32_t* cu, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                             int64_t Tq, int32_t Hq, int32_t Hkv, int32_t D) {
  inv_status s = check_attn_contract(c);
  if (s != INV_OK) return s;
  if (Tq < 0 || Hq <= 0 || Hkv <= 0 || num_seqs < 0) return INV_E_ARG;
  if (D != 128) return INV_E_UNSUPPORTED;
  if (Hq % Hkv != 0 || Hq / Hkv > 16) return INV_E_UNSUPPORTED;
  // a chunk's keys of all kv heads are addressed with 32-bit offsets
  if ((int64_t)Hkv * D * 2 * c->kv_chunk >= ((int64_t)1 << 31)) return INV_E_UNSUPPORTED;
  // one workgroup of up to 512 threads per (row, kv head, split): the grid's
  // threads must fit 32 bits, and the kernel indexes items in 32 bits
  if (Tq > (((int64_t)1 << 23) - 1) / ((int64_t)Hkv * c->split_kv)) return INV_E_UNSUPPORTED;
  if (Tq > 0 && (!q || !k || !v || !cu || !q_seq || !q_pos || num_seqs == 0)) return INV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15u)
    return INV_E_ARG;
  return INV_OK;
}

static inv::AttnLaunch attn_launch(const inv_contract* c, const void* q, const void* k, const void* v,
                                   const int32_t* cu, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                                   int64_t Tq, int32_t Hq, int32_t Hkv, int32_t D, uint32_t lo, uint32_t hi,
                                   void* ws) {
  inv::AttnLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_seqlens = cu;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.Tq = Tq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.num_seqs = num_seqs;
  a.split_kv = (int)c->split_kv;
  a.kv_chunk = (int)c->kv_chunk;
  a.split_lo = (int)lo;
  a.split_hi = (int)hi;
  a.ws = static_cast<float*>(ws);
  return a;
}

inv_status inv_decode_attn(const inv_contract* c, const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                           void* out, int64_t Tq, int32_t Hq, int32_t Hkv, int32_t D, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  inv_status s = attn_check(c, q, k, v, cu_seqlens, num_seqs, q_seq, q_pos, Tq, Hq, Hkv, D);
  if (s != INV_OK) return s;
  if (Tq == 0) return INV_OK;
  if (!out) return INV_E_ARG;
  const size_t need = inv_workspace_bytes(c, INV_OP_DECODE_ATTN, Tq, Hq, D);
  if (!ws || ws_bytes < need) return INV_E_WORKSPACE;
  if (!aligned_to(ws, 4u) || !aligned_to(out, 2u)) return INV_E_ARG;  // fp32 split states, bf16 output
  hipError_t e = inv::launch_attn_splits(
      attn_launch(c, q, k, v, cu_seqlens, num_seqs, q_seq, q_pos, Tq, Hq, Hkv, D, 0, c->split_kv, ws), stream);
  if (e != hipSuccess) return INV_E_HIP;
  return hip_status(inv::launch_attn_combine(static_cast<const float*>(ws), out, Tq, Hq, D, (int)c->split_kv,
                                             c->tree == INV_TREE_LEFT_FOLD, stream));
}

inv_status inv_attn_splits(const inv_contract* c, const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* q_seq, const int32_t* q_pos,
                           int64_t Tq, int32_t Hq, int32_t Hkv, int32_t D, uint32_t split_lo, uint32_t split_hi,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  inv_status s = attn_check(c, q, k, v, cu_seqlens, num_seqs, q_seq, q_pos, Tq, Hq, Hkv, D);
  if (s != INV_OK) return s;
  if (split_lo >= split_hi || split_hi > c->split_kv) return INV_E_ARG;
  if (Tq == 0) return INV_OK;
  const size_t need = inv_workspace_bytes(c, INV_OP_DECODE_ATTN, Tq, Hq, D);
  if (!ws || ws_bytes < need) return INV_E_WORKSPACE;
  if (!aligned_to(ws, 4u)) return INV_E_ARG;
  return hip_status(inv::launch_attn_splits(
      attn_launch(c, q, k, v, cu_seqlens, num_seqs, q_seq, q_pos, Tq, Hq, Hkv, D, split_lo, split_hi, ws), stream));
}

inv_status inv_attn_combine(const inv_contract* c, const void* ws, size_t ws_bytes, void* out, int64_t Tq,
                            int32_t Hq, int32_t D, hipStream_t stream) {
  inv_status s = check_attn_contract(c);
  if (s != INV_OK) return s;
  if (Tq < 0 || Hq <= 0) return INV_E_ARG;
  if (D != 128) return INV_E_UNSUPPORTED;
  if (Tq == 0) return INV_OK;
  if (!out) return INV_E_ARG;
  const size_t need = inv_workspace_bytes(c, INV_OP_DECODE_ATTN, Tq, Hq, D);
  if (!ws || ws_bytes < need) return INV_E_WORKSPACE;
  if (!aligned_to(ws, 4u) || !aligned_to(out, 2u)) return INV_E_ARG;
  return hip_status(inv::launch_attn_combine(static_cast<const float*>(ws), out, Tq, Hq, D, (int)c->split_kv,
                                             c->tree == INV_TREE_LEFT_FOLD, stream));
}

// ----------------------------------------------------------- measurement

inv_status inv_bench_mfma_loop(int64_t iters, int32_t groups, uint64_t* clk, float* sink, hipStream_t stream) {
  if (iters < 0 || groups < 0 || groups > (1 << 20)) return INV_E_ARG;
  if (iters == 0 || groups == 0) return INV_OK;
  if (!clk || !sink) return INV_E_ARG;
  return hip_status(inv::launch_mfma_loop(iters, groups, clk, sink, stream));
}

// ------------------------------------------------------------------- MoE

inv_status inv_moe_route(const inv_contract* c, const float* logits, int32_t* ids, float* w, int64_t T, int32_t E,
                         hipStream_t stream) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (T < 0 || E <= 0) return INV_E_ARG;
  if (E > 256 || (int64_t)c->leaves > E || c->leaves > 32) return INV_E_UNSUPPORTED;
  if (T >= kMaxRowsWave) return INV_E_UNSUPPORTED;  // (16 lanes per token: within the bound)
  if (T == 0) return INV_OK;
  if (!logits || !ids || !w) return INV_E_ARG;
  return hip_status(inv::launch_moe_route(logits, ids, w, T, E, (int)c->leaves, stream));
}

inv_status inv_moe_permute(const inv_contract* c, const int32_t* ids, int32_t* offsets, int32_t* rows,
                           int32_t* slot, int64_t T, int32_t E, hipStream_t stream) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (T < 0 || E <= 0) return INV_E_ARG;
  if (E > 256 || (int64_t)c->leaves > E || c->leaves > 32) return INV_E_UNSUPPORTED;
  if (T * (int64_t)c->leaves > ((int64_t)1 << 31) - 1) return INV_E_UNSUPPORTED;
  if (!offsets) return INV_E_ARG;
  if (T > 0 && (!ids || !rows || !slot)) return INV_E_ARG;
  return hip_status(inv::launch_moe_permute(ids, offsets, rows, slot, T, E, (int)c->leaves, stream));
}

inv_status inv_moe_gemm(const inv_contract* c, const void* X, int64_t x_rows, const int32_t* rows,
                        const int32_t* offsets, const void* W, void* Y, int64_t R, int32_t E, int64_t N, int64_t K,
                        hipStream_t stream) {
  inv_status s = check_gemm_contract(c, K);
  if (s != INV_OK) return s;
  if (c->ranks != 1) return INV_E_TOPOLOGY;
  if (R < 0 || N < 0 || E <= 0 || x_rows < 0) return INV_E_ARG;
  if (E > 65536 || R > ((int64_t)1 << 31) - 1) return INV_E_UNSUPPORTED;
  // gathered rows are addressed by 32-bit byte offsets from the start of X
  if (rows && x_rows * K * 2 > ((int64_t)1 << 32) - 1) return INV_E_UNSUPPORTED;
  if (R == 0 || N == 0) return INV_OK;
  if (!X || !offsets || !W || !Y) return INV_E_ARG;
  if (!rows && x_rows < R) return INV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W)) & 15u) return INV_E_ARG;
  inv::GemmLaunch g = gemm_launch(X, W, Y, R, N, K, (int)(K / c->leaves), 0, (int)c->leaves, 1, out_is_bf16(c));
  g.rows = rows;
  g.offsets = offsets;
  g.E = E;
  g.a_rows = x_rows;
  g.b_expert_stride = N * K;
  return hip_status(inv::launch_gemm(g, stream));
}

inv_status inv_moe_gemm_swiglu(const inv_contract* c, const void* X, int64_t x_rows, const int32_t* rows,
                               const int32_t* offsets, const void* W, void* Aout, int64_t R, int32_t E, int64_t F,
                               int64_t K, hipStream_t stream) {
  inv_status s = check_gemm_contract(c, K);
  if (s != INV_OK) return s;
  if (c->ranks != 1) return INV_E_TOPOLOGY;
  if (R < 0 || F < 0 || E <= 0 || x_rows < 0) return INV_E_ARG;
  if (E > 65536 || R > ((int64_t)1 << 31) - 1) return INV_E_UNSUPPORTED;
  if (rows && x_rows * K * 2 > ((int64_t)1 << 32) - 1) return INV_E_UNSUPPORTED;
  // one expert's [gate; up] rows are addressed by 32-bit byte offsets
  if (2 * F * K * 2 > ((int64_t)1 << 32) - 1) return INV_E_UNSUPPORTED;
  if (R == 0 || F == 0) return INV_OK;
  if (!X || !offsets || !W || !Aout) return INV_E_ARG;
  if (!rows && x_rows < R) return INV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W)) & 15u) return INV_E_ARG;
  inv::GemmLaunch g = gemm_launch(X, W, Aout, R, 2 * F, K, (int)(K / c->leaves), 0, (int)c->leaves, 1, true);
  g.rows = rows;
  g.offsets = offsets;
  g.E = E;
  g.a_rows = x_rows;
  g.b_expert_stride = 2 * F * K;
  g.swiglu = true;
  return hip_status(inv::launch_gemm(g, stream));
}

inv_status inv_swiglu(const inv_contract* c, const void* GU, void* Aout, int64_t R, int64_t F, hipStream_t stream) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (R < 0 || F < 0) return INV_E_ARG;
  if (R == 0 || F == 0) return INV_OK;
  if (!GU || !Aout) return INV_E_ARG;
  return hip_status(inv::launch_swiglu(GU, Aout, R, F, stream));
}

inv_status inv_moe_combine(const inv_contract* c, const float* Y, const float* w, const int32_t* slot,
                           int64_t y_rows, void* out, int64_t T, int64_t H, hipStream_t stream) {
  inv_status s = check_contract(c);
  if (s != INV_OK) return s;
  if (c->leaves > 32) return INV_E_UNSUPPORTED;
  if (T < 0 || H < 0 || y_rows < 0) return INV_E_ARG;
  if (T > ((int64_t)1 << 31) - 1) return INV_E_UNSUPPORTED;  // tokens index the grid's second dimension
  if (T == 0 || H == 0) return INV_OK;
  if (!Y || !w || !slot || !out) return INV_E_ARG;
  if (c->out_dtype != INV_BF16) return INV_E_CONTRACT;
  return hip_status(inv::launch_moe_combine(Y, w, slot, y_rows, out, T, H, (int)c->leaves,
                                            c->tree == INV_TREE_LEFT_FOLD, stream));
}

}  // extern "C"
