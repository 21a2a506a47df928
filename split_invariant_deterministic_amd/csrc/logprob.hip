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

}  // namespace

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
