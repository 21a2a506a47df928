// Selected-token log-probability with a pinned chunk tree, for gfx950.
//
// RL-Kernel write-up, section 4: LSE(x) = m + log sum exp(x - m); the
// log-probability of the selected token is its logit minus the LSE over the
// whole vocabulary; vocabulary blocks carry local (m_j, s_j) merged as
// m = max(m1, m2), s = s1 e^(m1-m) + s2 e^(m2-m), in an order the contract
// fixes. Section 7 of the same write-up: each TP shard computes local
// statistics, merged in a fixed vocabulary-tile order.
//
// Pinned schedule (depends on V and C only, never on M or the launch):
//   chunk j = [floor(jV/C), floor((j+1)V/C));
//   m_j = max over the chunk (exact);
//   s_j: element e of the chunk on lane e % 64, each lane summing
//        exp2((x - m_j) * log2e) over its elements in ascending e, lanes
//        combined by the xor butterfly 32..1;
//   (m, s) = tree over j of the merge above (balanced, or left fold for
//        the contrasting schedule), LSE = m + log2(s) * ln2;
//   lp = x[t] - LSE, NaN when t is outside [0, V).
// One workgroup per row; a wave owns whole chunks, so the chunk-to-wave
// assignment never changes a chunk's arithmetic. Logits are read once.
#include "common.h"
#include "launch.h"

namespace inv {
namespace {

constexpr int kMaxChunks = 512;
constexpr int kRegPerLane = 40;  // chunk elements cached per lane (chunks up to 2560)

// Statistics of one chunk [lo, hi) of row x, computed by one wave.
__device__ __forceinline__ MS chunk_stats(const float* __restrict__ x, int64_t lo, int64_t hi, int lane) {
  const int64_t len = hi - lo;
  if (len <= 64 * kRegPerLane) {
    float v[kRegPerLane];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kRegPerLane; ++i) {
      const int64_t e = lane + 64 * i;
      v[i] = e < len ? __builtin_nontemporal_load(x + lo + e) : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kRegPerLane; ++i) {
      const int64_t e = lane + 64 * i;
      if (e < len) s = s + exp_shifted(v[i], m);
    }
    return MS{m, wave_sum_butterfly(s)};
  }
  // Long chunks: two passes over memory with the same per-lane order.
  float m = -INFINITY;
  for (int64_t e = lane; e < len; e += 64) m = fmaxf(m, x[lo + e]);
  m = wave_max(m);
  float s = 0.0f;
  for (int64_t e = lane; e < len; e += 64) s = s + exp_shifted(x[lo + e], m);
  return MS{m, wave_sum_butterfly(s)};
}

// Tree over st[0..C) in LDS; returns the root in every thread. C is a power
// of two. Balanced: adjacent pairs level by level. Fold: left to right.
__device__ __forceinline__ MS chunk_tree(MS* st, int C, bool fold) {
  if (fold) {
    __shared__ MS root;
    if (threadIdx.x == 0) {
      MS a = st[0];
      for (int j = 1; j < C; ++j) a = lse_merge(a, st[j]);
      root = a;
    }
    __syncthreads();
    return root;
  }
  // C <= 512 = 2 * blockDim: one pair per thread per level
  for (int n = C; n > 1; n >>= 1) {
    const int j = threadIdx.x;
    MS r{0.f, 0.f};
    if (j < n / 2) r = lse_merge(st[2 * j], st[2 * j + 1]);
    __syncthreads();
    if (j < n / 2) st[j] = r;
    __syncthreads();
  }
  return st[0];
}

__global__ __launch_bounds__(256) void logprob_kernel(const float* __restrict__ logits, int64_t ldl,
                                                      const int32_t* __restrict__ target,
                                                      float* __restrict__ out, float* __restrict__ stats,
                                                      float* __restrict__ tlogit, int64_t V, int C,
                                                      int chunk_lo, int chunk_hi, int fold, int partial) {
  __shared__ MS st[kMaxChunks];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const float* x = logits + row * ldl;
  for (int j = chunk_lo + wave; j < chunk_hi; j += 4) {
    const int64_t lo = ((int64_t)j * V) / C, hi = ((int64_t)(j + 1) * V) / C;
    const MS r = chunk_stats(x, lo, hi, lane);
    if (lane == 0) {
      if (partial) {
        stats[(row * C + j) * 2 + 0] = r.m;
        stats[(row * C + j) * 2 + 1] = r.s;
      } else {
        st[j] = r;
      }
    }
  }
  const int32_t t = target[row];
  if (partial) {
    const int64_t vlo = ((int64_t)chunk_lo * V) / C, vhi = ((int64_t)chunk_hi * V) / C;
    if (threadIdx.x == 0 && t >= vlo && t < vhi) tlogit[row] = x[t];
    return;
  }
  __syncthreads();
  const MS root = chunk_tree(st, C, fold != 0);
  if (threadIdx.x == 0) {
    const float lse = root.m + log2_hw(root.s) * kLn2;
    out[row] = (t >= 0 && t < V) ? x[t] - lse : __builtin_nanf("");
  }
}

__global__ __launch_bounds__(256) void logprob_combine_kernel(const float* __restrict__ stats,
                                                              const float* __restrict__ tlogit,
                                                              const int32_t* __restrict__ target,
                                                              float* __restrict__ out, int64_t V, int C,
                                                              int fold) {
  __shared__ MS st[kMaxChunks];
  const int64_t row = blockIdx.x;
  for (int j = threadIdx.x; j < C; j += blockDim.x)
    st[j] = MS{stats[(row * C + j) * 2 + 0], stats[(row * C + j) * 2 + 1]};
  __syncthreads();
  const MS root = chunk_tree(st, C, fold != 0);
  if (threadIdx.x == 0) {
    const int32_t t = target[row];
    const float lse = root.m + log2_hw(root.s) * kLn2;
    out[row] = (t >= 0 && t < V) ? tlogit[row] - lse : __builtin_nanf("");
  }
}

// ---------------------------------------------------------------- 16-column blocks
//
// The LM-head schedule: vocabulary block b = columns [16b, min(16b+16, V)),
// one 16x16 MFMA output block wide, so the GEMM epilogue that produces the
// logits can reduce a block where the logits sit in registers (every GEMM
// kernel, at every M, holds a block's 16 columns on the 16 lanes of a lane
// group). block16_stats fixes the block's arithmetic; the blocks are then
// merged by the balanced tree over the block index, padded with the exact
// identity (-inf, 0) to a power of two.

// Statistics from stored fp32 logits, one row per workgroup: 4096-column
// panels are read coalesced into LDS (block b of the panel at row b of a
// 17-float-stride table), then thread b reduces block b in registers with the
// same block16_stats as the GEMM epilogue.
__global__ __launch_bounds__(256) void block16_stats_kernel(const float* __restrict__ logits, int64_t ldl,
                                                            const int32_t* __restrict__ target,
                                                            float* __restrict__ stats, float* __restrict__ tlogit,
                                                            int64_t V) {
  __shared__ float buf[256 * 17];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* x = logits + row * ldl;
  const int32_t t = target[row];
  const int64_t nb = (V + 15) / 16;
  for (int64_t p0 = 0; p0 < V; p0 += 4096) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int e = tid + 256 * k;
      const int64_t col = p0 + e;
      buf[(e >> 4) * 17 + (e & 15)] = col < V ? __builtin_nontemporal_load(x + col) : 0.0f;
    }
    __syncthreads();
    const int64_t c0 = p0 + 16 * tid;
    float v[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] = buf[tid * 17 + c];
    const int nvalid = (int)min(max(V - c0, (int64_t)0), (int64_t)16);
    const MS st = block16_stats(v, nvalid);
    if (nvalid > 0) {
      stats[2 * (row * nb + c0 / 16) + 0] = st.m;
      stats[2 * (row * nb + c0 / 16) + 1] = st.s;
    }
    if ((int64_t)t >= c0 && (int64_t)t < c0 + nvalid) tlogit[row] = buf[tid * 17 + (int)(t - c0)];
    __syncthreads();
  }
}

// Balanced tree over the B blocks [j0, j0+B) (identity past nb), in registers.
template <int B>
__device__ __forceinline__ MS block_subtree(const float* __restrict__ st, int64_t j0, int64_t nb) {
  MS v[B];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int64_t j = j0 + i;
    if (j < nb) {
      const float2 q = *reinterpret_cast<const float2*>(st + 2 * j);
      v[i] = MS{q.x, q.y};
    } else {
      v[i] = MS{-INFINITY, 0.0f};
    }
  }
#pragma unroll
  for (int w = B; w > 1; w /= 2)
#pragma unroll
    for (int k = 0; k < w / 2; ++k) v[k] = lse_merge(v[2 * k], v[2 * k + 1]);
  return v[0];
}

// One workgroup per row. P = 2^ceil(log2 nb) leaves; thread t reduces the
// aligned block of B = max(1, P/256) leaves, then an LDS tree joins the
// T = P/B thread results pairwise, level by level: together one balanced
// tree over the P leaves.
template <int B>
__global__ __launch_bounds__(256) void block16_merge_kernel(const float* __restrict__ stats,
                                                            const float* __restrict__ tlogit,
                                                            const int32_t* __restrict__ target,
                                                            float* __restrict__ out, int64_t V, int T, int fold) {
  __shared__ MS part[256];
  const int64_t row = blockIdx.x;
  const int64_t nb = (V + 15) / 16;
  const float* st = stats + 2 * row * nb;
  MS root;
  if (fold) {
    __shared__ MS r0;
    if (threadIdx.x == 0) {
      MS a{st[0], st[1]};
      for (int64_t j = 1; j < nb; ++j) a = lse_merge(a, MS{st[2 * j], st[2 * j + 1]});
      r0 = a;
    }
    __syncthreads();
    root = r0;
  } else {
    if ((int)threadIdx.x < T) part[threadIdx.x] = block_subtree<B>(st, (int64_t)threadIdx.x * B, nb);
    __syncthreads();
    for (int n = T; n > 1; n >>= 1) {
      const int j = threadIdx.x;
      MS r{0.f, 0.f};
      if (j < n / 2) r = lse_merge(part[2 * j], part[2 * j + 1]);
      __syncthreads();
      if (j < n / 2) part[j] = r;
      __syncthreads();
    }
    root = part[0];
  }
  if (threadIdx.x == 0) {
    const int32_t t = target[row];
    const float lse = root.m + log2_hw(root.s) * kLn2;
    out[row] = (t >= 0 && t < V) ? tlogit[row] - lse : __builtin_nanf("");
  }
}

}  // namespace

hipError_t launch_block16_stats(const float* logits, int64_t ldl, const int32_t* target, float* stats,
                                float* tlogit, int64_t M, int64_t V, hipStream_t s) {
  hipLaunchKernelGGL(block16_stats_kernel, dim3((unsigned)M), dim3(256), 0, s, logits, ldl, target, stats, tlogit,
                     V);
  return hipGetLastError();
}

hipError_t launch_block16_merge(const float* stats, const float* tlogit, const int32_t* target, float* out,
                                int64_t M, int64_t V, bool left_fold, hipStream_t s) {
  const int64_t nb = (V + 15) / 16;
  int64_t P = 1;
  while (P < nb) P *= 2;
  const int64_t B = P >= 256 ? P / 256 : 1;
  const int T = (int)(P / B);
  const dim3 grid((unsigned)M), block(256);
  const int f = left_fold ? 1 : 0;
  switch (B) {
    case 1: hipLaunchKernelGGL((block16_merge_kernel<1>), grid, block, 0, s, stats, tlogit, target, out, V, T, f); break;
    case 2: hipLaunchKernelGGL((block16_merge_kernel<2>), grid, block, 0, s, stats, tlogit, target, out, V, T, f); break;
    case 4: hipLaunchKernelGGL((block16_merge_kernel<4>), grid, block, 0, s, stats, tlogit, target, out, V, T, f); break;
    case 8: hipLaunchKernelGGL((block16_merge_kernel<8>), grid, block, 0, s, stats, tlogit, target, out, V, T, f); break;
    case 16: hipLaunchKernelGGL((block16_merge_kernel<16>), grid, block, 0, s, stats, tlogit, target, out, V, T, f); break;
    case 32: hipLaunchKernelGGL((block16_merge_kernel<32>), grid, block, 0, s, stats, tlogit, target, out, V, T, f); break;
    case 64: hipLaunchKernelGGL((block16_merge_kernel<64>), grid, block, 0, s, stats, tlogit, target, out, V, T, f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_logprob(const float* logits, int64_t ldl, const int32_t* target, float* out, float* stats,
                          float* tlogit, int64_t M, int64_t V, int C, int chunk_lo, int chunk_hi, bool left_fold,
                          bool partial, hipStream_t s) {
  if (C > kMaxChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(logprob_kernel, dim3((unsigned)M), dim3(256), 0, s, logits, ldl, target, out, stats, tlogit,
                     V, C, chunk_lo, chunk_hi, left_fold ? 1 : 0, partial ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_logprob_combine(const float* stats, const float* tlogit, const int32_t* target, float* out,
                                  int64_t M, int64_t V, int C, bool left_fold, hipStream_t s) {
  if (C > kMaxChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(logprob_combine_kernel, dim3((unsigned)M), dim3(256), 0, s, stats, tlogit, target, out, V, C,
                     left_fold ? 1 : 0);
  return hipGetLastError();
}

}  // namespace inv
