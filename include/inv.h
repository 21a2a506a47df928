/*
 * inv.h -- C ABI of the split-invariant forward kernels for MI355X (gfx950).
 *
 * The library computes the forward of an LLM's selected-token log-probability
 * so that every output bit is independent of the batch size M, of how the
 * K dimension of a GEMM is partitioned across (emulated) ranks, of how the
 * vocabulary or the key range is cut into chunks and splits, and of prefill
 * versus decode. It follows the idea of an execution contract: every choice
 * that can move a rounding (leaf count, tree shape, accumulation and boundary
 * dtypes, split-KV count) is an explicit constant passed with each call.
 *
 *   Sources (cited by page title and section):
 *   [IsoExec]  vllm.ai blog "IsoExec: Unified Execution to Eliminate
 *              Trainer-Inference Mismatch in SkyRL"
 *   [NovaSky]  alphasignal.ai "NovaSky's IsoExec Fixes the Hidden Math Bug
 *              Corrupting AI Training Runs"
 *   [RLK]      "Reinforcement Learning Post-Training for Large Models: How
 *              RL-Kernel Completely Eliminates Train-Inference LogP
 *              Discrepancy"
 *   [VeXact]   arXiv 2605.14220 "Diagnosing Training Inference Mismatch in
 *              LLM Reinforcement Learning"
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The
 *     library never allocates, frees or synchronises; all work is enqueued on
 *     the caller's `stream` (NULL = the default stream) and is asynchronous.
 *   - bf16 tensors are passed as raw 16-bit storage (uint16_t bit patterns).
 *   - Tensors are dense and row-major unless a leading dimension is given.
 *   - Before any HIP call, the contract and every shape are validated on the
 *     host; a violation returns INV_E_ARG / INV_E_CONTRACT / INV_E_TOPOLOGY /
 *     INV_E_UNSUPPORTED / INV_E_WORKSPACE and enqueues nothing. A failed
 *     launch returns INV_E_HIP. No C++ exception crosses this boundary.
 *   - Device-side data errors (a target id outside [0, V), an expert id
 *     outside [0, E)) do not fault: the affected output row becomes NaN.
 *   - The library holds no mutable global state; calls on different streams
 *     may run concurrently if their output buffers do not overlap.
 *   - Integer sizes are int64_t; every size must be >= 0, and an empty call
 *     (a zero extent) returns INV_OK without launching anything.
 */
#ifndef INV_H_
#define INV_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define INV_ABI_VERSION 1u

typedef enum inv_status {
  INV_OK = 0,
  INV_E_ARG = 1,         /* null pointer, negative size, bad stride, range   */
  INV_E_CONTRACT = 2,    /* a contract constant the kernels do not implement */
  INV_E_TOPOLOGY = 3,    /* rank count outside the proven set for the leaves */
  INV_E_UNSUPPORTED = 4, /* a shape outside the implemented range            */
  INV_E_HIP = 5,         /* a HIP launch or query failed                     */
  INV_E_WORKSPACE = 6    /* workspace missing or smaller than required       */
} inv_status;

typedef enum inv_dtype { INV_BF16 = 1, INV_FP32 = 2 } inv_dtype;

/* Combine schedule over leaves / chunks / splits.
 * BALANCED: recursive halving over a power-of-two count n, adjacent pairs
 *   first: for n = 8, ((x0+x1)+(x2+x3)) + ((x4+x5)+(x6+x7)). Every aligned
 *   block of 2^j consecutive items is a subtree, which is what lets a rank
 *   that owns such a block reduce it locally ([IsoExec] "Parallelism-invariant
 *   kernels": rank-to-leaf mapping and binary schedule fixed by the contract;
 *   [RLK] section 6, fixed balanced tree for TP 1/2/4/8).
 * LEFT_FOLD: (((x0+x1)+x2)+...)+x_{n-1}. Only the partial-buffer combines
 *   accept it; it exists so tests can show that a different schedule does
 *   change bits ([RLK] section 2, the two orders of a+b+c+d). */
typedef enum inv_tree { INV_TREE_BALANCED = 1, INV_TREE_LEFT_FOLD = 2 } inv_tree;

/* The execution contract of one region ([IsoExec] "Unified execution
 * contract": the composition pins accumulation and boundary dtypes and the
 * split-K / split-KV partition counts of each region). Fill it with
 * inv_contract_default() and override per region. */
typedef struct inv_contract {
  uint32_t struct_size; /* = sizeof(inv_contract)                               */
  uint32_t abi_version; /* = INV_ABI_VERSION                                    */
  uint32_t leaves;      /* GEMM: K leaves; logprob: vocabulary chunks;
                           MoE combine: routed experts per token (top-k).
                           Must be a power of two.                              */
  uint32_t ranks;       /* emulated ranks owning contiguous leaves; a power of
                           two that divides `leaves` (the proven set)           */
  int32_t tree;         /* inv_tree                                             */
  int32_t accum_dtype;  /* must be INV_FP32                                     */
  int32_t leaf_dtype;   /* dtype of partials between stages: must be INV_FP32   */
  int32_t out_dtype;    /* boundary dtype of the region's output                */
  uint32_t split_kv;    /* attention: number of key splits (power of two)       */
  uint32_t kv_chunk;    /* attention: key chunk size, a multiple of 32          */
  float eps;            /* RMSNorm epsilon                                      */
  uint32_t reserved;    /* must be 0                                            */
} inv_contract;

/* Fills the defaults: leaves 8, ranks 1, balanced tree, fp32 accumulation and
 * leaves, bf16 output, split_kv 16, kv_chunk 64, eps 1e-6. Returns INV_E_ARG
 * if c is NULL. Host only. */
inv_status inv_contract_default(inv_contract* c);

/* Operation ids for validation and workspace queries. */
typedef enum inv_op {
  INV_OP_GEMM = 1,
  INV_OP_TREE_COMBINE = 2,
  INV_OP_RMSNORM = 3,
  INV_OP_LOGPROB = 4,
  INV_OP_DECODE_ATTN = 5,
  INV_OP_MOE_ROUTE = 6,
  INV_OP_MOE_GEMM = 7,
  INV_OP_MOE_COMBINE = 8,
  INV_OP_LMHEAD_LOGPROB = 9,
  INV_OP_LOGPROB_BLOCK16 = 10,
  INV_OP_GDN_PREFILL = 11,
  INV_OP_GDN_DECODE = 12
} inv_op;

/* Host-only contract validation for `op`; the same check every entry point
 * runs first. K is the contraction length (GEMM ops; else ignored). */
inv_status inv_contract_check(const inv_contract* c, int op, int64_t K);

/* Workspace bytes `op` needs for the given sizes (0 if none):
 *   INV_OP_GEMM:        d0 = M, d1 = N, d2 = K  -> ranks*M*N*4 when ranks > 1;
 *                       with ranks == 1 the optional leaf-group size (or 0)
 *   INV_OP_DECODE_ATTN: d0 = Tq, d1 = Hq, d2 = D -> Tq*Hq*split_kv*(D+2)*4
 *   INV_OP_LMHEAD_LOGPROB, INV_OP_LOGPROB_BLOCK16: d0 = M, d1 = V, d2 = K
 *                       -> M*ceil(V/16)*8 + M*4
 *   INV_OP_GDN_PREFILL: d0 = T tokens, d1 = H heads, d2 = S sequences
 *                       -> (2*T*H*128 + T*H + (T/C + S)*H*(128*128 + C*C + 2C))*4 + 16
 * Returns (size_t)-1 if the contract is invalid. Host only. */
size_t inv_workspace_bytes(const inv_contract* c, int op, int64_t d0, int64_t d1, int64_t d2);

/* Static text for a status code; never NULL. */
const char* inv_status_string(inv_status s);

/* ------------------------------------------------------------------------
 * Serialized contract and identity digests ([IsoExec] "Unified execution
 * contract": cases, a composition mapping each region to an implementation
 * and its pinned constants, claims of the proven parallel sizes, and SHA-256
 * identities -- semantic (the logical model), numerical_policy (every choice
 * that can move a bit) and deployment (settings proven not to move bits).
 * Two runtimes exchange the digests and refuse to run on a mismatch of the
 * semantic or numerical_policy digest). Host only; nothing is launched.
 * ------------------------------------------------------------------------ */

/* Regions of the forward path a composition can pin. */
typedef enum inv_region {
  INV_REGION_NORM = 1,        /* RMSNorm                                   */
  INV_REGION_LINEAR = 2,      /* dense projections (inv_gemm)              */
  INV_REGION_LM_HEAD = 3,     /* LM-head logits (inv_gemm, fp32 boundary)  */
  INV_REGION_LOGPROB = 4,     /* selected-token log-softmax                */
  INV_REGION_ATTENTION = 5,   /* split-KV attention                        */
  INV_REGION_MOE_ROUTE = 6,   /* top-k routing                             */
  INV_REGION_MOE_EXPERTS = 7, /* grouped expert GEMMs                      */
  INV_REGION_MOE_COMBINE = 8, /* fixed-order combine                       */
  INV_REGION_LMHEAD_LOGPROB = 9, /* fused LM head + logprob (16-col blocks) */
  INV_REGION_GDN = 10            /* CPR Gated DeltaNet (gdn.core)         */
} inv_region;

/* One composition entry: a region and the contract pinned for it. */
typedef struct inv_region_contract {
  int32_t region;       /* inv_region                                        */
  uint32_t reserved;    /* must be 0                                         */
  inv_contract contract;
} inv_region_contract;

typedef enum inv_digest_kind {
  INV_DIGEST_SEMANTIC = 1,
  INV_DIGEST_NUMERICAL_POLICY = 2,
  INV_DIGEST_DEPLOYMENT = 3
} inv_digest_kind;

/* Canonical JSON of a composition of n >= 1 entries (each region at most
 * once, in any order; written sorted by region): compact, fixed key order, integers
 * and ASCII strings only, floats as IEEE-754 bit patterns, so one
 * composition has one byte sequence. Layout:
 *   {"ExecutionContract":{"cases":[..],"composition":[..],"claims":{..},
 *    "semantic":{..},"deployment":{..},"identities":{"semantic":hex,
 *    "numerical_policy":hex,"deployment":hex}}}
 * The digests are SHA-256 of: the "semantic" value; the text
 * {"cases":..,"composition":..,"claims":..}; the "deployment" value.
 * Ranks are deployment (each proven rank count gives the same bits); leaves,
 * chunks, splits, tree, dtypes and implementation ids are numerical policy;
 * the region set, RMSNorm eps and the MoE top-k are semantic.
 * *len receives the text length without the terminating NUL. buf == NULL is
 * a size query; cap < *len + 1 returns INV_E_ARG and writes nothing. Each
 * entry's contract is validated as its entry point would (INV_E_CONTRACT /
 * INV_E_TOPOLOGY); an unknown or repeated region is INV_E_ARG. */
inv_status inv_contract_json(const inv_region_contract* entries, size_t n, char* buf, size_t cap,
                             size_t* len);

/* The SHA-256 digest `kind` of the composition into digest[32]. */
inv_status inv_contract_digest(const inv_region_contract* entries, size_t n, int kind,
                               uint8_t digest[32]);

/* INV_OK if the composition's digest `kind` equals expected[32] (a peer's),
 * INV_E_CONTRACT if it differs: the caller refuses to run. */
inv_status inv_contract_verify(const inv_region_contract* entries, size_t n, int kind,
                               const uint8_t expected[32]);

/* SHA-256 (FIPS 180-4) of `bytes` bytes of host memory. */
inv_status inv_sha256(const void* data, size_t bytes, uint8_t digest[32]);

/* ------------------------------------------------------------------------
 * GEMM with K leaves  ([IsoExec] "Parallelism-invariant kernels";
 * [NovaSky] "Making kernels parallelism-invariant"; [RLK] section 7, GEMM
 * merged in FP32 then written as BF16)
 *
 *   C[m,n] = round_out( tree_l P_l[m,n] ),
 *   P_l[m,n] = sum over k in leaf l of A[m,k] * B[n,k]   (fp32, from +0.0)
 *
 * A [M,K] bf16, B [N,K] bf16 (the weight, K contiguous: logical K x N),
 * C [M,N] out_dtype (bf16 by round-to-nearest-even, or fp32).
 * Leaf l covers k in [l*K/L, (l+1)*K/L); K % L == 0 and (K/L) % 32 == 0;
 * K < 2^24 (else INV_E_UNSUPPORTED; this holds for every GEMM entry point).
 * Inside a leaf the sum runs in ascending steps of 32 k on one fixed MFMA
 * instruction (v_mfma_f32_16x16x32_bf16) with one fixed k-to-lane map, for
 * every M, N, tile shape and rank split; the leaves are then combined by the
 * balanced tree in fp32. The bits of row m depend only on A[m,:] and B.
 * ranks > 1 emulates tensor parallelism on one GPU: rank r reduces the
 * subtree of leaves [r*L/R, (r+1)*L/R) into a workspace of R fp32 [M,N]
 * partials (ws_bytes >= inv_workspace_bytes(INV_OP_GEMM)), and the top
 * log2(R) tree levels finish the sum. The result is bitwise identical for
 * every proven R. tree must be BALANCED.
 * ranks == 1: the workspace is optional. For M >= 8 with too few 128 x 128
 * output tiles to fill the chip (tiles * G <= 256), inv_workspace_bytes
 * reports G*M*N*4 bytes; given that much, G aligned subtrees are reduced in
 * parallel and combined by the same tree (bitwise the same result as without
 * the workspace).
 * A and B are 16-byte aligned, C is aligned to its element (2 bytes bf16, 4
 * fp32) and ws, when given, is 4-byte aligned; else INV_E_ARG.
 * ------------------------------------------------------------------------ */
inv_status inv_gemm(const inv_contract* c, const void* A, const void* B, void* C,
                    int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* inv_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument, and the call allocates nothing. The fp32 partials that
 * inv_gemm would keep in a caller workspace (the R rank planes when
 * ranks > 1; the leaf groups of a single rank when M >= 8 and the 128 x 128
 * tiles alone would leave compute units idle) go to a library-owned scratch
 * array of 16 MiB per GPU, allocated when the library is loaded on that GPU
 * and held until the process ends. Every single-rank shape fits; with
 * ranks > 1 a call needing R*M*N*4 bytes above 16 MiB returns
 * INV_E_WORKSPACE before any launch. The result is bitwise inv_gemm's for
 * the same arguments (same kernels, same tree). All calls on one GPU share
 * that GPU's scratch and each call leaves its partials there: calls that
 * overlap in time on one GPU (concurrent streams, or host threads) race and
 * must be serialised by the caller. The first call on a device looks up the
 * scratch address for it (hipGetSymbolAddress); a failure there returns
 * INV_E_HIP. */
inv_status inv_gemm_noalloc(const inv_contract* c, const void* A, const void* B, void* C,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* One rank's share of inv_gemm: P_r [M,N] fp32 = the balanced subtree over
 * leaves [rank*L/R, (rank+1)*L/R). A and B are the full operands; only the
 * rank's K slice is read. */
inv_status inv_gemm_rank(const inv_contract* c, const void* A, const void* B, float* P_r,
                         int64_t M, int64_t N, int64_t K, uint32_t rank, hipStream_t stream);

/* Per-leaf partials: P [leaf_hi-leaf_lo, M, N] fp32, P[i] = P_{leaf_lo+i}.
 * Bitwise equal to the leaf sums inside inv_gemm (same instruction chain). */
inv_status inv_gemm_leaves(const inv_contract* c, const void* A, const void* B, float* P,
                           int64_t M, int64_t N, int64_t K, uint32_t leaf_lo,
                           uint32_t leaf_hi, hipStream_t stream);

/* Combine `count` fp32 partials P [count, M, N] with the contract's tree
 * and cast to out_dtype: C = round_out(tree(P[0..count-1])). count is a power
 * of two; with BALANCED, combining the R rank partials of inv_gemm_rank, or
 * the L leaf partials of inv_gemm_leaves, reproduces inv_gemm bit for bit.
 * P is 4-byte aligned and C aligned to its element, else INV_E_ARG. */
inv_status inv_tree_combine(const inv_contract* c, const float* P, uint32_t count, void* C,
                            int64_t M, int64_t N, hipStream_t stream);

/* Boundary cast: y[i] = bf16 round-to-nearest-even of x[i] (NaN stays NaN).
 * The same conversion every kernel uses at its output boundary ([RLK]
 * section 2, the FP32 to BF16 conversion position as a trigger point). */
inv_status inv_cast_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t stream);

/* ------------------------------------------------------------------------
 * RMSNorm over the hidden dimension ([RLK] section 4, reduction class over
 * the hidden dimension; [VeXact] section 3.1, batch-invariant RMSNorm)
 *
 *   r = 1 / sqrt( ss * (1/H) + eps ),   y[m,h] = bf16( (x[m,h] * r) * g[h] )
 *
 * x, y [M,H] bf16; gamma [H] bf16; all math fp32. ss = sum of x^2 in a fixed
 * order that depends on H only: element h goes to lane (h/8) % 64 of a
 * 64-lane group; each lane runs fused multiply-adds over its elements in
 * ascending h; the 64 lane sums are combined by an xor butterfly with
 * offsets 32, 16, 8, 4, 2, 1. H % 8 == 0, 8 <= H <= 16384. eps = c->eps.
 * M < 2^26 (one wave per row; else INV_E_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
inv_status inv_rmsnorm(const inv_contract* c, const void* x, const void* gamma, void* y,
                       int64_t M, int64_t H, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Selected-token log-probability ([RLK] section 4: LSE definition, its
 * max-shifted form and the two-block merge; [RLK] section 7, per-shard
 * statistics merged in a fixed vocabulary-tile order; [VeXact] Eq. (1))
 *
 *   lp[m] = x[m, t_m] - LSE(x[m, :])
 *
 * logits [M, V] fp32 with row stride ldl >= V (elements); target [M] int32;
 * out [M] fp32. The vocabulary is cut into C = c->leaves chunks, chunk j =
 * [floor(j*V/C), floor((j+1)*V/C)), 1 <= C <= V, C a power of two.
 * Per chunk: m_j = max (exact), s_j = sum of exp2((x - m_j) * log2e) with
 * element e of the chunk on lane e % 64, each lane summing in ascending e and
 * the lanes combined by an xor butterfly 32..1. The (m_j, s_j) are merged by
 * the contract's tree with m = max(m1,m2), s = s1*exp(m1-m) + s2*exp(m2-m);
 * LSE = m + log(s). A target outside [0, V) gives NaN. M < 2^24 (one
 * workgroup per row) here and in every logprob entry point below, else
 * INV_E_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
inv_status inv_logprob(const inv_contract* c, const float* logits, int64_t ldl,
                       const int32_t* target, float* out, int64_t M, int64_t V,
                       hipStream_t stream);

/* Vocabulary-shard share of inv_logprob: for chunks [chunk_lo, chunk_hi)
 * writes stats[m*C + j] = (m_j, s_j) as float pairs (stats is [M, C, 2]
 * fp32) and, for rows whose target lies in the shard's vocabulary range,
 * tlogit[m] = x[m, t_m]. Other entries are left untouched. */
inv_status inv_logprob_partials(const inv_contract* c, const float* logits, int64_t ldl,
                                const int32_t* target, float* stats, float* tlogit,
                                int64_t M, int64_t V, uint32_t chunk_lo, uint32_t chunk_hi,
                                hipStream_t stream);

/* Finishes inv_logprob from the full stats [M, C, 2] and tlogit [M]:
 * out[m] = tlogit[m] - (m + log s) over the contract's tree; bitwise equal to
 * inv_logprob when the partials came from any set of disjoint shards that
 * covers all chunks. target is read only to turn out-of-range ids into NaN. */
inv_status inv_logprob_combine(const inv_contract* c, const float* stats, const float* tlogit,
                               const int32_t* target, float* out, int64_t M, int64_t V,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Split-KV attention with a pinned split rule and combine ([IsoExec]
 * "Unified execution contract": split-KV partition counts are contract
 * constants; [RLK] section 4, LSE merge over visible keys; [RLK] section 7,
 * fixed block partition, chunk order and rescale-merge order)
 *
 * q [Tq, Hq, D] bf16; k, v [sumL, Hkv, D] bf16 packed by sequence, sequence
 * s occupying rows [cu_seqlens[s], cu_seqlens[s+1]); query row i belongs to
 * sequence q_seq[i] and sees keys at positions [0, q_pos[i]] of it.
 * out [Tq, Hq, D] bf16. Query head h reads kv head h / (Hq/Hkv).
 * D == 128; Hq % Hkv == 0; Hq/Hkv <= 16; kv_chunk keys of all kv heads
 * (kv_chunk * Hkv * D * 2 bytes) < 2 GiB; Tq * Hkv * split_kv < 2^23 (one
 * workgroup per row, kv head and split); else INV_E_UNSUPPORTED. q, k, v
 * 16-byte aligned, else INV_E_ARG.
 * For a row with L = q_pos+1 visible keys: keys form chunks of kv_chunk from
 * position 0, n = ceil(L/kv_chunk); split j (of S = split_kv) owns chunks
 * [floor(j*n/S), floor((j+1)*n/S)), processed in ascending order with an
 * online-softmax update per chunk: scores = (q.k) * (1/sqrt(D)) in fp32,
 * p = exp2((score - m) * log2e) split into bf16 parts p_hi = bf16(p) and
 * p_lo = bf16(p - p_hi), row sum and P.V taken from the same p_hi + p_lo
 * (two chained MFMAs per step, high part first). Empty splits are the identity (m = -inf, l = 0, o = 0).
 * The S split states are merged by the contract's tree (o scaled like l) and
 * out = bf16(o / l). Every row's bits depend only on its own q, its visible
 * keys and L, so a decode row equals the same position's prefill row.
 * Workspace: ws_bytes >= inv_workspace_bytes(INV_OP_DECODE_ATTN, Tq, Hq, D),
 * else INV_E_WORKSPACE; ws 4-byte aligned and out 2-byte aligned, else
 * INV_E_ARG (the same for the two calls below).
 * ------------------------------------------------------------------------ */
inv_status inv_decode_attn(const inv_contract* c, const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* q_seq,
                           const int32_t* q_pos, void* out, int64_t Tq, int32_t Hq,
                           int32_t Hkv, int32_t D, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* The split states of splits [split_lo, split_hi) into ws (layout
 * [Tq, Hq, split_kv, D+2] fp32: o[0..D-1], m, l), as a context-parallel rank
 * owning those splits would compute them. */
inv_status inv_attn_splits(const inv_contract* c, const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens, int32_t num_seqs, const int32_t* q_seq,
                           const int32_t* q_pos, int64_t Tq, int32_t Hq, int32_t Hkv,
                           int32_t D, uint32_t split_lo, uint32_t split_hi, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Merges the split states in ws with the contract's tree and writes out. */
inv_status inv_attn_combine(const inv_contract* c, const void* ws, size_t ws_bytes, void* out,
                            int64_t Tq, int32_t Hq, int32_t D, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Mixture-of-experts layer ([IsoExec] "Unified model": deterministic routing
 * and combination; [IsoExec] "Parallelism-invariant kernels": a token's
 * expert results are summed in an order set by the routing, independent of
 * which rank computed them; [IsoExec] "Unified
 * execution contract", the moe.combine entry with 8 fp32 leaves; [RLK]
 * section 7, packed gate/up GEMM, SwiGLU and down GEMM as separate stages)
 * ------------------------------------------------------------------------ */

/* Top-k routing: for each token the k = c->leaves largest of E router logits
 * (fp32; ties go to the lower expert id), emitted in ascending expert id;
 * w = softmax over the k selected logits in fp32 (max-shifted, exp2 form,
 * denominator summed in ascending expert id). logits [T, E] fp32,
 * ids [T, k] int32, w [T, k] fp32. E <= 256, k <= E, T < 2^26, else
 * INV_E_UNSUPPORTED. */
inv_status inv_moe_route(const inv_contract* c, const float* logits, int32_t* ids, float* w,
                         int64_t T, int32_t E, hipStream_t stream);

/* Groups the T*k (token, expert) pairs by expert, stable in token id:
 * offsets [E+1] (offsets[e] = first grouped row of expert e), rows [T*k]
 * (token id of each grouped row), slot [T, k] (grouped row of pair (t, j)).
 * Deterministic without atomics. */
inv_status inv_moe_permute(const inv_contract* c, const int32_t* ids, int32_t* offsets,
                           int32_t* rows, int32_t* slot, int64_t T, int32_t E,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Fused LM head + selected-token log-probability.
 *
 * [RLK] section 4: the log-probability of the selected token is its logit
 * minus the LSE over the vocabulary, and vocabulary blocks carry local
 * (m_j, s_j) statistics merged in an order the contract fixes; section 7:
 * logits stay fp32. Here the vocabulary block is 16 columns -- the columns
 * of one 16x16 MFMA output block -- so the GEMM reduces each block while the
 * fp32 logits are still in registers and never writes the [M, V] logits.
 *   block b = columns [16b, min(16b+16, V)), nb = ceil(V/16);
 *   m_b = max over the block; s_b = sum of exp2((x - m_b) * log2e) by the
 *     xor butterfly 1, 2, 4, 8 over the 16 columns (a balanced tree over the
 *     column index; columns past V contribute nothing);
 *   (m, s) = balanced tree over b, padded with (-inf, 0) to a power of two
 *     (the merge of the pages, exact on the padding);
 *   LSE = m + log2(s) * ln2; lp = x[t] - LSE, NaN when t is outside [0, V).
 * The logits x are bitwise inv_gemm's fp32 output, so the fused result is
 * bitwise inv_logprob_block16 applied to inv_gemm's logits, for every M.
 * This schedule differs from inv_logprob's C-chunk schedule (a separate
 * contract: same mathematics, other rounding).
 * ------------------------------------------------------------------------ */

/* out[m] = lp of target[m] for rows h [M, K] bf16 against W [V, K] bf16
 * (logits = inv_gemm with c->leaves K-leaves and fp32 boundary dtype:
 * c->out_dtype must be INV_FP32, c->tree BALANCED, c->ranks 1).
 * target [M] int32, out [M] fp32. Workspace: ws_bytes >=
 * inv_workspace_bytes(INV_OP_LMHEAD_LOGPROB, M, V, K), 8-byte aligned; on
 * return it holds the block statistics [M, nb, 2] fp32 followed by the
 * target logits [M]. V <= 262144. */
inv_status inv_lmhead_logprob(const inv_contract* c, const void* h, const void* W, const int32_t* target,
                              float* out, int64_t M, int64_t V, int64_t K, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* The same 16-column block schedule from stored fp32 logits [M, ldl]
 * (ldl >= V): the unfused counterpart of inv_lmhead_logprob. c->tree may be
 * LEFT_FOLD (the merge over blocks left to right) as the contrasting
 * schedule. Workspace and layout as for inv_lmhead_logprob. */
inv_status inv_logprob_block16(const inv_contract* c, const float* logits, int64_t ldl, const int32_t* target,
                               float* out, int64_t M, int64_t V, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gated DeltaNet under the chunkwise-parallel recurrent (CPR) schedule.
 *
 * [IsoExec] "Chunkwise-parallel recurrent (CPR) GDN" ([NovaSky] "Solving the
 * linear-attention headache"). The token recurrence defines the layer.
 * Prefill obtains the state at each multiple of C with a separate boundary
 * pass and evaluates the chunks' tokens independently, each chunk from its
 * opening state; decode steps the recurrence and, when a chunk completes,
 * swaps its running state for the boundary state. Prefill, training forward
 * and decode thus round identically. The
 * layer (the gated delta rule, restated; the pages give no formulas), per
 * head with key and value width D = 128:
 *   k^ = k / sqrt(sum k^2 + 1e-6), q^ = q / sqrt(sum q^2 + 1e-6) / sqrt(128)
 *   alpha = exp(g) (g <= 0 the log-decay), beta in [0, 1]
 *   S_t = alpha_t (S_{t-1} - beta_t k^_t (k^_t^T S_{t-1})) + beta_t k^_t v_t^T,
 *   S_0 = 0, o_t = S_t^T q^_t   (S is D x D fp32)
 * Boundaries at multiples of C = c->kv_chunk (32 or 64) from each sequence's
 * first token; a boundary state is the previous one advanced by the
 * chunkwise closed form of the recurrence (gamma = running product of alpha
 * inside the chunk; w = M r with M = (I + diag(beta) A)^-1 diag(beta) by
 * forward substitution, A[t][s] = (gamma_t/gamma_s)(k^_s . k^_t) for s < t,
 * r_t = v_t - gamma_t S_0^T k^_t; S_C = gamma_C S_0 + sum_s (gamma_C /
 * gamma_s) k^_s w_s^T); every output comes from the token-by-token
 * recurrence started at its chunk's boundary state.
 * The same device functions run in both entry points, so a sequence
 * prefilled to any length and continued by decode gives, token for token,
 * the bits of one prefill of the whole sequence. c->ranks must be 1;
 * c->out_dtype is the output's dtype (bf16 or fp32).
 * ------------------------------------------------------------------------ */

/* Bytes of one sequence's decode cache: the running state and the last
 * boundary state [H][128][128] fp32 each, then the open chunk's k^ and v
 * [C][H][128] fp32 and alpha, beta [C][H] fp32, then [H][C*C + 2C] fp32 of
 * scratch for the chunk-closing step. A fresh sequence's cache is all zeros.
 * (size_t)-1 if the contract is invalid. */
size_t inv_gdn_cache_bytes(const inv_contract* c, int32_t H);

/* Prefill / training forward of S packed sequences (cu_seqlens [S+1] int32,
 * T = cu_seqlens[S] tokens): q, k, v [T, H, D] bf16, g, beta [T, H] fp32,
 * out [T, H, D] out_dtype. D must be 128. If cache is not NULL it receives,
 * per sequence, the decode cache after the sequence's last token (cache
 * [S] x inv_gdn_cache_bytes). Workspace: ws_bytes >=
 * inv_workspace_bytes(INV_OP_GDN_PREFILL, T, H, S), 16-byte aligned; it holds
 * k^, q^, alpha, every boundary state and every chunk's M, gamma and gamma
 * ratios. */
inv_status inv_gdn_prefill(const inv_contract* c, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu_seqlens, int32_t S, int64_t T, int32_t H,
                           int32_t D, void* out, void* cache, void* ws, size_t ws_bytes, hipStream_t stream);

/* One decode token for each of B sequences: q, k, v [B, H, D] bf16, g, beta
 * [B, H] fp32, pos [B] int32 = the number of tokens the sequence already has
 * (this token's position), out [B, H, D] out_dtype, cache [B] decode caches
 * (updated in place: the token joins the open chunk; when it closes the
 * chunk, the boundary state advances and the running state resynchronises
 * to it). The caller advances pos. */
inv_status inv_gdn_decode(const inv_contract* c, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* pos, int32_t B, int32_t H, int32_t D, void* out,
                          void* cache, hipStream_t stream);

/* Grouped GEMM: for expert e, grouped rows r in [offsets[e], offsets[e+1]):
 * Y[r, :] = inv_gemm row of A = X[rows[r], :] (or X[r, :] if rows is NULL)
 * against B = W[e] [N, K]. Same leaves, tree and instruction chain as
 * inv_gemm, so each row is bitwise what inv_gemm gives for it alone.
 * X [x_rows, K] bf16, W [E, N, K] bf16, Y [R, N] out_dtype, offsets [E+1]
 * int32 non-decreasing with offsets[E] <= R (as inv_moe_permute writes it).
 * Offsets are clamped to [0, R] and a gathered index outside [0, x_rows)
 * reads a zero row, so malformed tables cannot address outside the buffers.
 * ranks must be 1. */
inv_status inv_moe_gemm(const inv_contract* c, const void* X, int64_t x_rows, const int32_t* rows,
                        const int32_t* offsets, const void* W, void* Y, int64_t R, int32_t E,
                        int64_t N, int64_t K, hipStream_t stream);

/* Gate/up grouped GEMM with the SwiGLU fused into its epilogue (the
 * pages' MoE FFN: packed gate/up projection, SwiGLU, down projection; the
 * elementwise step is done where the GEMM holds its outputs, so the [R, 2F]
 * gate/up tensor never reaches memory). W [E, 2F, K] bf16 holds each
 * expert's gate rows then its up rows; Aout [R, F] bf16. Aout is bitwise
 * inv_swiglu of what inv_moe_gemm would write for the same arguments with
 * N = 2F and a bf16 out_dtype (the contract's out_dtype is not used): every
 * gate and up value is rounded to bf16 first. Rows, offsets, the contract
 * and the clamping of malformed tables are as for inv_moe_gemm; one
 * expert's 2F x K weights must span fewer than 2^32 bytes. ranks must be 1. */
inv_status inv_moe_gemm_swiglu(const inv_contract* c, const void* X, int64_t x_rows, const int32_t* rows,
                               const int32_t* offsets, const void* W, void* Aout, int64_t R, int32_t E,
                               int64_t F, int64_t K, hipStream_t stream);

/* SwiGLU on a packed [gate | up] row: a = bf16( silu(g) * u ) with
 * silu(g) = g / (1 + exp(-g)), g and u read as bf16, math fp32.
 * GU [R, 2F] bf16, Aout [R, F] bf16. */
inv_status inv_swiglu(const inv_contract* c, const void* GU, void* Aout, int64_t R, int64_t F,
                      hipStream_t stream);

/* Combine: out[t, :] = bf16( tree over j of w[t,j] * Y[slot[t,j], :] ) with
 * the k = c->leaves leaves in ascending expert id (the order inv_moe_route
 * emits), fp32 products and the contract's fp32 tree (balanced; left fold
 * only as the contrasting schedule). Y [y_rows, H] fp32, w [T, k] fp32,
 * slot [T, k] int32, out [T, H] bf16. A slot outside [0, y_rows) makes that
 * token's row NaN. T < 2^31, else INV_E_UNSUPPORTED. */
inv_status inv_moe_combine(const inv_contract* c, const float* Y, const float* w,
                           const int32_t* slot, int64_t y_rows, void* out, int64_t T, int64_t H,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not a step of the forward path): the MFMA ceiling of
 * the chip and the shader clock it runs at, as context for the GEMMs'
 * fraction of the published peak.
 *
 * Launches `groups` workgroups of 8 waves; every wave runs `iters` steps of
 * 8 independent v_mfma_f32_16x16x32_bf16 accumulator chains on register
 * operands (no memory traffic): groups * 8 * 8 * iters * 16384 flops.
 * clk [groups, 2] uint64 (device) receives, per workgroup, the elapsed
 * shader-clock cycles and the elapsed ticks of the constant 100 MHz
 * real-time counter over the loop; sink [groups * 512] fp32 (device)
 * receives values that keep the results live. groups <= 2^20; zero iters or
 * groups returns INV_OK without a launch.
 * ------------------------------------------------------------------------ */
inv_status inv_bench_mfma_loop(int64_t iters, int32_t groups, uint64_t* clk, float* sink,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* INV_H_ */
