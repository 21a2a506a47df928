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
//
// Chunks of up to 64 * kRegPerLane elements are held in registers, ROWS
// 64-element rows per chunk: one buffer descriptor over the chunk, the lane's
// offset one VGPR and the row a scalar, so the loads need no 64-bit
// addresses and no exec branches (elements past the chunk read 0).
// The logit loads stream (kNT): each logit is read once; under graph replay
// the 4096 x 151936 pass takes 365 us with the hint and 411 us without.
template <int ROWS>
struct ChunkRegs {
  float v[ROWS];
};

template <int ROWS>
__device__ __forceinline__ void chunk_issue(const float* __restrict__ x, int64_t lo, int n, int lane,
                                            ChunkRegs<ROWS>& c) {
  const buf_rsrc r = make_rsrc(x + lo, (uint32_t)n * 4u);
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
    c.v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)lane * 4u,
                                                                            (uint32_t)(256 * i), kNT));
}

// ROWS = ceil(ceil(V / C) / 64). Every chunk is floor(V / C) or ceil(V / C)
// long, and 64 (ROWS - 1) <= ceil(V / C) - 1 <= floor(V / C), so rows
// 0 .. ROWS-2 are whole in every chunk: only the last row needs a mask.
// Lane l adds its elements l + 64 i in ascending i.
template <int ROWS>
__device__ __forceinline__ MS chunk_reduce(const ChunkRegs<ROWS>& c, int n, int lane) {
  const bool last_ok = lane + 64 * (ROWS - 1) < n;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < ROWS - 1; ++i) m = fmaxf(m, c.v[i]);
  if (last_ok) m = fmaxf(m, c.v[ROWS - 1]);
  m = wave_max(m);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < ROWS - 1; ++i) s = s + exp_shifted(c.v[i], m);
  const float e = exp_shifted(c.v[ROWS - 1], m);
  if (last_ok) s = s + e;
  s = wave_sum_butterfly(s);
  // A chunk whose logits are all -inf (a masked vocabulary range) is the
  // merge identity (-inf, 0): its exp terms would be exp2(-inf - -inf) = NaN.
  return MS{m, m == -INFINITY ? 0.0f : s};
}

// Longer chunks: two passes over memory with the same per-lane order.
__device__ __forceinline__ MS chunk_stats_long(const float* __restrict__ x, int64_t lo, int64_t hi, int lane) {
  const int64_t len = hi - lo;
  float m = -INFINITY;
  for (int64_t e = lane; e < len; e += 64) m = fmaxf(m, x[lo + e]);
  m = wave_max(m);
  float s = 0.0f;
  for (int64_t e = lane; e < len; e += 64) s = s + exp_shifted(x[lo + e], m);
  s = wave_sum_butterfly(s);
  return MS{m, m == -INFINITY ? 0.0f : s};  // an all -inf chunk is the identity
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

// ROWS = 0: chunks longer than 64 * kRegPerLane (two passes over memory).
template <int ROWS>
__global__ __launch_bounds__(256) void logprob_kernel(const float* __restrict__ logits, int64_t ldl,
                                                      const int32_t* __restrict__ target,
                                                      float* __restrict__ out, float* __restrict__ stats,
                                                      float* __restrict__ tlogit, int64_t V, int C,
                                                      int chunk_lo, int chunk_hi, int fold, int partial) {
  __shared__ MS st[kMaxChunks];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // chunk bounds stay scalar
  const int64_t row = blockIdx.x;
  const float* x = logits + row * ldl;
  auto put = [&](int j, const MS& r) {
    if (lane == 0) {
      if (partial) {
        stats[(row * C + j) * 2 + 0] = r.m;
        stats[(row * C + j) * 2 + 1] = r.s;
      } else {
        st[j] = r;
      }
    }
  };
  auto lo_of = [&](int j) { return ((int64_t)j * V) / C; };
  if constexpr (ROWS > 0) {
    // The wave's chunks j, j+4, ...: the next chunk's loads are issued before
    // the current chunk is reduced (two register sets, alternating).
    int j = chunk_lo + wave;
    if (j < chunk_hi) {
      ChunkRegs<ROWS> a, b;
      int64_t lo = lo_of(j);
      int n = (int)(lo_of(j + 1) - lo);
      chunk_issue(x, lo, n, lane, a);
      for (;;) {
        const bool more = j + 4 < chunk_hi;
        int64_t lo2 = 0;
        int n2 = 0;
        if (more) {
          lo2 = lo_of(j + 4);
          n2 = (int)(lo_of(j + 5) - lo2);
          chunk_issue(x, lo2, n2, lane, b);
        }
        put(j, chunk_reduce(a, n, lane));
        if (!more) break;
        j += 4;
        const bool more2 = j + 4 < chunk_hi;
        if (more2) {
          lo = lo_of(j + 4);
          n = (int)(lo_of(j + 5) - lo);
          chunk_issue(x, lo, n, lane, a);
        }
        put(j, chunk_reduce(b, n2, lane));
        if (!more2) break;
        j += 4;
      }
    }
  } else {
    for (int j = chunk_lo + wave; j < chunk_hi; j += 4) put(j, chunk_stats_long(x, lo_of(j), lo_of(j + 1), lane));
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

// One workgroup per row. P = 2^ceil(log2 nb) leaves; thread t reduces the
// aligned block of B = max(1, P/256) leaves [tB, tB+B) by the balanced tree
// over it, then an LDS tree joins the T = P/B thread results pairwise, level
// by level: together one balanced tree over the P leaves, leaves past nb
// being the merge identity (-inf, 0).
//
// The leaves reach the threads through LDS in pieces of PB = min(B, 16)
// leaves per thread, so that the global reads are whole 128-byte lines
// (16 lanes read one thread's 16 consecutive (m, s) pairs) instead of one
// 8-byte pair per lane 8B bytes apart. In LDS, leaf i of thread t's piece
// sits at i * S + t (S odd, at least the threads in use), so the staging
// writes spread over the banks and each thread's reads are consecutive
// across the wave. A thread's B leaves are NP = B / PB aligned pieces: the
// subtree over each piece, then the balanced tree over the pieces, is the
// balanced tree over the B leaves.
constexpr int kMergePiece = 16;
constexpr int kMergeStride = 257;  // odd, >= 256 threads

template <int B>
__global__ __launch_bounds__(256) void block16_merge_kernel(const float* __restrict__ stats,
                                                            const float* __restrict__ tlogit,
                                                            const int32_t* __restrict__ target,
                                                            float* __restrict__ out, int64_t V, int T, int fold) {
  constexpr int PB = B < kMergePiece ? B : kMergePiece;
  constexpr int NP = B / PB;
  __shared__ MS part[256];
  __shared__ float2 stage[PB * kMergeStride];
  const int64_t row = blockIdx.x;
  const int64_t nb = (V + 15) / 16;
  const float* st = stats + 2 * row * nb;
  const int tid = threadIdx.x;
  MS root;
  if (fold) {
    __shared__ MS r0;
    if (tid == 0) {
      MS a{st[0], st[1]};
      for (int64_t j = 1; j < nb; ++j) a = lse_merge(a, MS{st[2 * j], st[2 * j + 1]});
      r0 = a;
    }
    __syncthreads();
    root = r0;
  } else {
    // threads holding at least one real leaf; the rest reduce identities only
    const int TU = (int)((nb + B - 1) / B);
    // Every piece's global loads are issued up front (at most 16 pairs per
    // thread per piece: TU * PB <= 256 * 16), so a lone row pays one memory
    // latency, not one per piece.
    float2 ld[NP][kMergePiece];
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int r = 0; r < kMergePiece; ++r) {
        const int e = tid + 256 * r;
        const int t = e / PB, i = e % PB;
        const int64_t j = (int64_t)t * B + q * PB + i;
        ld[q][r] = make_float2(-INFINITY, 0.0f);
        if (e < TU * PB && j < nb) ld[q][r] = *reinterpret_cast<const float2*>(st + 2 * j);
      }
    MS pv[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      if (q > 0) __syncthreads();  // every thread has read the previous piece
#pragma unroll
      for (int r = 0; r < kMergePiece; ++r) {
        const int e = tid + 256 * r;
        if (e < TU * PB) stage[(e % PB) * kMergeStride + e / PB] = ld[q][r];
      }
      __syncthreads();
      MS v[PB];
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        if (tid < TU) {
          const float2 f = stage[i * kMergeStride + tid];
          v[i] = MS{f.x, f.y};
        } else {
          v[i] = MS{-INFINITY, 0.0f};
        }
      }
#pragma unroll
      for (int w = PB; w > 1; w /= 2)
#pragma unroll
        for (int k = 0; k < w / 2; ++k) v[k] = lse_merge(v[2 * k], v[2 * k + 1]);
      pv[q] = v[0];
    }
#pragma unroll
    for (int w = NP; w > 1; w /= 2)
#pragma unroll
      for (int k = 0; k < w / 2; ++k) pv[k] = lse_merge(pv[2 * k], pv[2 * k + 1]);
    if (tid < T) part[tid] = pv[0];
    __syncthreads();
    for (int n = T; n > 1; n >>= 1) {
      const int j = tid;
      MS r{0.f, 0.f};
      if (j < n / 2) r = lse_merge(part[2 * j], part[2 * j + 1]);
      __syncthreads();
      if (j < n / 2) part[j] = r;
      __syncthreads();
    }
    root = part[0];
  }
  if (tid == 0) {
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
  const int64_t rows = ((V + C - 1) / C + 63) / 64;
  const int r = rows <= kRegPerLane ? (int)rows : 0;
  switch (r) {
#define INV_LP_ROWS(R_)                                                                                            \
  case R_:                                                                                                         \
    hipLaunchKernelGGL((logprob_kernel<R_>), dim3((unsigned)M), dim3(256), 0, s, logits, ldl, target, out, stats, \
                       tlogit, V, C, chunk_lo, chunk_hi, left_fold ? 1 : 0, partial ? 1 : 0);                    \
    break;
    INV_LP_ROWS(0) INV_LP_ROWS(1) INV_LP_ROWS(2) INV_LP_ROWS(3) INV_LP_ROWS(4) INV_LP_ROWS(5) INV_LP_ROWS(6)
    INV_LP_ROWS(7) INV_LP_ROWS(8) INV_LP_ROWS(9) INV_LP_ROWS(10) INV_LP_ROWS(11) INV_LP_ROWS(12) INV_LP_ROWS(13)
    INV_LP_ROWS(14) INV_LP_ROWS(15) INV_LP_ROWS(16) INV_LP_ROWS(17) INV_LP_ROWS(18) INV_LP_ROWS(19) INV_LP_ROWS(20)
    INV_LP_ROWS(21) INV_LP_ROWS(22) INV_LP_ROWS(23) INV_LP_ROWS(24) INV_LP_ROWS(25) INV_LP_ROWS(26) INV_LP_ROWS(27)
    INV_LP_ROWS(28) INV_LP_ROWS(29) INV_LP_ROWS(30) INV_LP_ROWS(31) INV_LP_ROWS(32) INV_LP_ROWS(33) INV_LP_ROWS(34)
    INV_LP_ROWS(35) INV_LP_ROWS(36) INV_LP_ROWS(37) INV_LP_ROWS(38) INV_LP_ROWS(39) INV_LP_ROWS(40)
#undef INV_LP_ROWS
    default: return hipErrorInvalidValue;
  }
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
