// Internal launcher interface between the C-ABI layer (api.cpp) and the HIP
// kernels. Arguments here are already validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace inv {

// Workgroups of a grid-stride elementwise launch: enough to cover n items at
// `per` items per workgroup, at most 2^20 (so the dispatch's work-item count,
// workgroups times 256 lanes, stays below 2^32 whatever n is; the kernels
// walk the rest by the grid stride).
inline unsigned stride_grid(int64_t n, int64_t per) {
  const int64_t g = (n + per - 1) / per;
  return (unsigned)(g < ((int64_t)1 << 20) ? (g > 0 ? g : 1) : ((int64_t)1 << 20));
}

// ---- GEMM -----------------------------------------------------------------
// One launch reduces, for every output element, `groups` independent balanced
// subtrees of `nl` consecutive leaves each: group z covers leaves
// [leaf_lo + z*nl, leaf_lo + (z+1)*nl) and writes C + z*c_group_stride.
struct GemmLaunch {
  const void* A;           // [rows, K] bf16
  const void* B;           // [N, K] bf16 (grouped: [E, N, K])
  void* C;                 // [M, N] out dtype (per group)
  int64_t M, N, K;
  int64_t c_group_stride;  // elements between groups' outputs
  int kl;                  // leaf length (multiple of 32)
  int leaf_lo;             // first leaf of group 0
  int nl;                  // leaves per group (power of two, <= 8)
  int groups;              // number of groups (grid z)
  bool out_bf16;           // else fp32
  // grouped (MoE) mode: offsets != nullptr
  const int32_t* rows;     // gather of A rows (nullable)
  const int32_t* offsets;  // [E+1] grouped row ranges per expert
  int E;
  int64_t a_rows;          // rows of A (gathered indices outside [0, a_rows) read as zero rows)
  int64_t b_expert_stride; // elements between experts' B
  // LM-head statistics mode (lp_stats != nullptr, groups == 1, not grouped):
  // C is not written; per row and 16-column vocabulary block the (m, s) pair
  // goes to lp_stats [M, ceil(N/16), 2] and the target's logit to lp_tlogit.
  float* lp_stats = nullptr;
  float* lp_tlogit = nullptr;
  const int32_t* lp_target = nullptr;
  // Fused SwiGLU (grouped only): B = W [E, N, K] holds [gate; up] rows
  // (N = 2F); C is A [M, F] bf16 with A[r, f] = bf16(silu_mul(bf16 g, bf16 u)),
  // g and u being what the unfused GEMM would store at columns f and F + f.
  bool swiglu = false;
};
hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s);

// C = cast(tree(P[0..count-1])), P [count, plane] fp32.
hipError_t launch_tree_combine(const float* P, int count, int64_t plane, void* C, bool out_bf16,
                               bool left_fold, hipStream_t s);

hipError_t launch_cast_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s);

// ---- RMSNorm ----------------------------------------------------------------
hipError_t launch_rmsnorm(const void* x, const void* gamma, void* y, int64_t M, int64_t H,
                          float eps, hipStream_t s);

// ---- logprob ----------------------------------------------------------------
// mode 0: full logprob -> out; mode 1: partial stats for chunks [lo, hi).
hipError_t launch_logprob(const float* logits, int64_t ldl, const int32_t* target, float* out,
                          float* stats, float* tlogit, int64_t M, int64_t V, int C, int chunk_lo,
                          int chunk_hi, bool left_fold, bool partial, hipStream_t s);
// LM-head logprob from 16-column block statistics: per row, the balanced
// tree (or left fold) over ceil(V/16) blocks padded with (-inf, 0) to a power
// of two, then lp = tlogit - LSE. stats [M, nb, 2], nb = ceil(V/16).
hipError_t launch_block16_merge(const float* stats, const float* tlogit, const int32_t* target, float* out,
                                int64_t M, int64_t V, bool left_fold, hipStream_t s);
// The same block statistics computed from stored fp32 logits [M, ldl].
hipError_t launch_block16_stats(const float* logits, int64_t ldl, const int32_t* target, float* stats,
                                float* tlogit, int64_t M, int64_t V, hipStream_t s);
hipError_t launch_logprob_combine(const float* stats, const float* tlogit, const int32_t* target,
                                  float* out, int64_t M, int64_t V, int C, bool left_fold,
                                  hipStream_t s);

// ---- attention --------------------------------------------------------------
struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_seqlens;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int64_t Tq;
  int Hq, Hkv, D;
  int num_seqs;
  int split_kv, kv_chunk;
  int split_lo, split_hi;
  float* ws;  // [Tq, Hq, split_kv, D+2]
};
hipError_t launch_attn_splits(const AttnLaunch& a, hipStream_t s);
hipError_t launch_attn_combine(const float* ws, void* out, int64_t Tq, int Hq, int D, int split_kv,
                               bool left_fold, hipStream_t s);

// ---- Gated DeltaNet (CPR) ---------------------------------------------------
// Floats of one sequence's decode cache: running state and last boundary
// state [H][128][128] each, then the open chunk's k^, v [C][H][128] and
// alpha, beta [C][H], then per head the closing chunk's coefficients
// [H][C*C + 2C] (scratch of the chunk-closing decode step).
__host__ __device__ inline int64_t gdn_cache_floats(int H, int C) {
  return 2LL * H * 128 * 128 + (int64_t)C * H * (2 * 128 + 2) + (int64_t)H * (C * C + 2 * C);
}
struct GdnArgs {
  const uint16_t* q;      // [T, H, 128] bf16
  const uint16_t* k;
  const uint16_t* v;
  const float* g;         // [T, H] log-decay
  const float* beta;      // [T, H]
  const int32_t* cu;      // [S+1]
  int S;
  int64_t T;
  int H;
  void* out;              // [T, H, 128]
  void* cache;            // [S] decode caches, nullable
  float* qh;              // workspace: [T, H, 128]
  float* kh;              // [T, H, 128]
  float* alpha;           // [T, H]
  float* bstates;         // [T/C + S, H, 128, 128] boundary states
  float* coef;            // [T/C + S, H, C*C + 2C] per-chunk M (row-major), gamma, gamma_last/gamma
};
struct GdnDecodeArgs {
  const uint16_t* q;      // [B, H, 128] bf16
  const uint16_t* k;
  const uint16_t* v;
  const float* g;         // [B, H]
  const float* beta;
  const int32_t* pos;     // [B] position of this token in its sequence
  int B;
  int H;
  void* out;              // [B, H, 128]
  void* cache;            // [B] decode caches
};
hipError_t launch_gdn_prefill(const GdnArgs& a, int C, bool out_bf16, hipStream_t s);
hipError_t launch_gdn_decode(const GdnDecodeArgs& a, int C, bool out_bf16, hipStream_t s);

// ---- library-owned scratch (no-allocation entry points) -------------------------
// Bytes of the per-device scratch array: the largest leaf-group workspace any
// single-rank GEMM asks for (G * M * N fp32 with tiles * G <= 256 tiles of
// 128 x 128) is 256 * 128 * 128 * 4 bytes = 16 MiB.
constexpr size_t kScratchBytes = size_t{16} << 20;
// The current device's address of the scratch array (looked up once per
// device with that device current).
hipError_t scratch_device_ptr(void** out);

// ---- measurement ---------------------------------------------------------------
// groups workgroups of 8 waves, each wave 8 independent MFMA chains of iters
// steps; clk [groups, 2]: shader-clock cycles and 100 MHz ticks of the loop;
// sink [groups * 512] keeps the results live.
hipError_t launch_mfma_loop(int64_t iters, int groups, uint64_t* clk, float* sink, hipStream_t s);

// ---- MoE --------------------------------------------------------------------
hipError_t launch_moe_route(const float* logits, int32_t* ids, float* w, int64_t T, int E, int k,
                            hipStream_t s);
hipError_t launch_moe_permute(const int32_t* ids, int32_t* offsets, int32_t* rows, int32_t* slot,
                              int64_t T, int E, int k, hipStream_t s);
hipError_t launch_swiglu(const void* gu, void* a, int64_t R, int64_t F, hipStream_t s);
hipError_t launch_moe_combine(const float* Y, const float* w, const int32_t* slot, int64_t y_rows,
                              void* out, int64_t T, int64_t H, int k, bool left_fold, hipStream_t s);

}  // namespace inv
