// K-leaf GEMM for gfx950: C = cast( tree_l P_l ), P_l = sum_{k in leaf l} A[m,k] B[n,k].
//
// IsoExec blog, "Parallelism-invariant kernels" (and the NovaSky write-up,
// "Making kernels parallelism-invariant"): K is cut into contiguous leaves,
// each accumulated in FP32, and the leaf partials are combined by a binary
// schedule the contract fixes. RL-Kernel write-up, section 7: on ROCm a
// custom MFMA GEMM with a fixed chunk order merges in FP32 and writes BF16.
//
// Per output element the arithmetic is one fixed chain, whatever the kernel,
// tile shape, M, N or rank split:
//   P_l = 0; for each 32-wide k block of leaf l in ascending order:
//            P_l = v_mfma_f32_16x16x32_bf16(A block, B block, P_l)
//   C   = balanced fp32 tree over the leaves, then one cast.
// Row m of the MFMA output depends only on row m of its A operand, so the
// kernels are free to choose tiles by M; padding rows are zero-filled.
//
// Kernels
//   gemm_tile_kernel    LDS-staged 2x2-wave tile (128 x 128) for large M; the
//                       balanced subtree of up to 8 leaves is evaluated in
//                       registers in post-order (log2(nl)+1 live sets).
//   gemm_stream_kernel  small M (<= 64): each wave owns whole leaves of one
//                       16FM x 16 tile and streams its K range straight from
//                       HBM into MFMA fragments; the waves' subtrees are then
//                       combined through LDS with the same balanced tree.
//   tree_combine_kernel fp32 tree over a partial buffer (ranks, leaves).
#include "common.h"
#include "launch.h"

namespace inv {
namespace {

constexpr int kPad = 40;  // staged row stride in bf16 (32 k + 8 pad: conflict-free b128 reads)

template <int FM, int FN>
struct AccT {
  f32x4 v[FM][FN];
};

template <int FM, int FN>
__device__ __forceinline__ void acc_zero(AccT<FM, FN>& a) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) a.v[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int FM, int FN>
__device__ __forceinline__ void acc_add(AccT<FM, FN>& a, const AccT<FM, FN>& b) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) a.v[i][j][r] = a.v[i][j][r] + b.v[i][j][r];
}

// Balanced subtree over NL consecutive leaves in post-order: left subtree,
// right subtree, one fp32 add per element.
template <int NL, class Ctx>
__device__ __forceinline__ void run_tree(Ctx& c, typename Ctx::Acc& out) {
  if constexpr (NL == 1) {
    c.leaf(out);
  } else {
    run_tree<NL / 2>(c, out);
    typename Ctx::Acc right;
    run_tree<NL / 2>(c, right);
    acc_add(out, right);
  }
}

struct TileParams {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int64_t M, N, K;
  int64_t c_group_stride;
  int kl, leaf_lo, nl;
  const int32_t* rows;
  const int32_t* offsets;
  int E;
  int64_t a_rows;
  int64_t b_expert_stride;
};

// ---------------------------------------------------------------- tile kernel

template <int FM, int FN>
struct TileCtx {
  static constexpr int BM = 32 * FM, BN = 32 * FN;
  static constexpr int CHUNKS = (BM + BN) * 4;  // 16-byte chunks per 32-k stage
  static constexpr int CPT = CHUNKS / 256;
  using Acc = AccT<FM, FN>;

  uint16_t* lds;  // [2][(BM+BN) * kPad]
  const uint16_t* src[CPT];
  int dst[CPT];
  u32x4 stage[CPT];
  int64_t kbase;   // first k of the WG's leaf range
  int g;           // next stage to compute (global within the range)
  int total;       // stages in the range
  int spl;         // stages per leaf
  int lane, wm, wn;

  __device__ __forceinline__ void gload(int st) {
    const int64_t k = kbase + (int64_t)st * 32;
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      stage[u] = src[u] ? *reinterpret_cast<const u32x4*>(src[u] + k) : u32x4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void lstore(int buf) {
    uint16_t* base = lds + buf * ((BM + BN) * kPad);
#pragma unroll
    for (int u = 0; u < CPT; ++u) *reinterpret_cast<u32x4*>(base + dst[u]) = stage[u];
  }
  __device__ __forceinline__ void compute(int buf, Acc& acc) {
    const uint16_t* base = lds + buf * ((BM + BN) * kPad);
    const int col = 8 * (lane >> 4);
    bf16x8 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(base + (wm * 16 * FM + 16 * i + (lane & 15)) * kPad + col);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(base + (BM + wn * 16 * FN + 16 * j + (lane & 15)) * kPad + col);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc.v[i][j] = mfma16(af[i], bfr[j], acc.v[i][j]);
  }
  // One leaf: acc starts at +0 and takes the leaf's stages in ascending k.
  __device__ __forceinline__ void leaf(Acc& acc) {
    acc_zero(acc);
    for (int s = 0; s < spl; ++s) {
      const bool more = (g + 1) < total;
      if (more) gload(g + 1);
      compute(g & 1, acc);
      if (more) lstore((g + 1) & 1);
      __syncthreads();
      ++g;
    }
  }
};

template <int FM, int FN, int NL, bool OUT_BF16, bool GROUPED>
__global__ __launch_bounds__(256) void gemm_tile_kernel(TileParams p) {
  using Ctx = TileCtx<FM, FN>;
  constexpr int BM = Ctx::BM, BN = Ctx::BN;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * kPad];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  int64_t m0, m_end;
  const uint16_t* B = p.B;
  if constexpr (GROUPED) {
    // Tile slot -> (expert, rows): experts own consecutive runs of tiles of
    // ceil(count_e / BM) each, in expert order.
    const int t = blockIdx.y;
    int e = 0, tstart = 0;
    int64_t r0 = 0, r1 = 0;
    bool found = false;
    for (; e < p.E; ++e) {
      // offsets come from device memory: clamp so a malformed table can
      // never address rows outside [0, M)
      r0 = min(max((int64_t)p.offsets[e], (int64_t)0), p.M);
      r1 = min(max((int64_t)p.offsets[e + 1], r0), p.M);
      const int nt = (int)((r1 - r0 + BM - 1) / BM);
      if (t < tstart + nt) {
        found = true;
        break;
      }
      tstart += nt;
    }
    if (!found) return;  // slot past the last tile: uniform exit before any barrier
    m0 = r0 + (int64_t)(t - tstart) * BM;
    m_end = r1;
    B += (int64_t)e * p.b_expert_stride;
  } else {
    m0 = (int64_t)blockIdx.y * BM;
    m_end = p.M;
  }
  const int z = blockIdx.z;
  const int leaf0 = p.leaf_lo + z * NL;

  Ctx c;
  c.lds = lds;
  c.lane = lane;
  c.wm = wave >> 1;
  c.wn = wave & 1;
  c.kbase = (int64_t)leaf0 * p.kl;
  c.spl = p.kl / 32;
  c.total = c.spl * NL;
  c.g = 0;
#pragma unroll
  for (int u = 0; u < Ctx::CPT; ++u) {
    const int ch = tid + 256 * u;
    const int cc = ch & 3;
    if (ch < BM * 4) {
      const int r = ch >> 2;
      const int64_t row = m0 + r;
      const uint16_t* ptr = nullptr;
      if (row < m_end) {
        const int64_t arow = (GROUPED && p.rows) ? (int64_t)p.rows[row] : row;
        if (arow >= 0 && arow < p.a_rows) ptr = p.A + arow * p.K + cc * 8;
      }
      c.src[u] = ptr;
      c.dst[u] = r * kPad + cc * 8;
    } else {
      const int r = (ch >> 2) - BM;
      const int64_t col = n0 + r;
      c.src[u] = (col < p.N) ? B + col * p.K + cc * 8 : nullptr;
      c.dst[u] = (BM + r) * kPad + cc * 8;
    }
  }
  c.gload(0);
  c.lstore(0);
  __syncthreads();

  typename Ctx::Acc acc;
  run_tree<NL>(c, acc);

  // Epilogue: lane holds rows 4*(lane/16)+r of each 16x16 block, column lane%16.
  const int64_t rbase = m0 + c.wm * 16 * FM + 4 * (lane >> 4);
  const int64_t cbase = n0 + c.wn * 16 * FN + (lane & 15);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = rbase + 16 * i + r;
        const int64_t col = cbase + 16 * j;
        if (row < m_end && col < p.N) {
          const int64_t off = (int64_t)z * p.c_group_stride + row * p.N + col;
          if constexpr (OUT_BF16)
            reinterpret_cast<uint16_t*>(p.C)[off] = f32_to_bf16_bits(acc.v[i][j][r]);
          else
            reinterpret_cast<float*>(p.C)[off] = acc.v[i][j][r];
        }
      }
}

// -------------------------------------------------------------- stream kernel

template <int FM>
struct StreamCtx {
  using Acc = AccT<FM, 1>;
  const uint16_t* arow[FM];  // this lane's A row per m block (clamped)
  bool avalid[FM];
  const uint16_t* brow;
  bool bvalid;
  int64_t k;    // next k to load for this wave
  int spl;
  int lane;

  __device__ __forceinline__ void load(int64_t kk, bf16x8 (&a)[FM], bf16x8& b) {
    const int off = 8 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      u32x4 v = *reinterpret_cast<const u32x4*>(arow[i] + kk + off);
      if (!avalid[i]) v = u32x4{0u, 0u, 0u, 0u};
      a[i] = __builtin_bit_cast(bf16x8, v);
    }
    u32x4 v = *reinterpret_cast<const u32x4*>(brow + kk + off);
    if (!bvalid) v = u32x4{0u, 0u, 0u, 0u};
    b = __builtin_bit_cast(bf16x8, v);
  }
  __device__ __forceinline__ void mma(const bf16x8 (&a)[FM], const bf16x8& b, Acc& acc) {
#pragma unroll
    for (int i = 0; i < FM; ++i) acc.v[i][0] = mfma16(a[i], b, acc.v[i][0]);
  }
  // One leaf of spl 32-k blocks, two blocks per iteration so the next loads
  // are in flight while the current MFMAs run.
  __device__ __forceinline__ void leaf(Acc& acc) {
    acc_zero(acc);
    bf16x8 a0[FM], a1[FM], b0, b1;
    load(k, a0, b0);
    int s = 0;
    for (; s + 2 <= spl; s += 2) {
      load(k + 32, a1, b1);
      mma(a0, b0, acc);
      if (s + 2 < spl) load(k + 64, a0, b0);
      mma(a1, b1, acc);
      k += 64;
    }
    if (s < spl) {  // odd block count
      mma(a0, b0, acc);
      k += 32;
    }
  }
};

template <int FM, int NW, bool OUT_BF16>
__global__ __launch_bounds__(64 * NW) void gemm_stream_kernel(TileParams p) {
  using Ctx = StreamCtx<FM>;
  __shared__ float xch[NW > 1 ? NW : 1][FM * 4 * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * FM;
  const int z = blockIdx.z;
  const int leaf = p.leaf_lo + z * NW + w;  // one leaf per wave

  Ctx c;
  c.lane = lane;
  c.spl = p.kl / 32;
  c.k = (int64_t)leaf * p.kl;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = m0 + 16 * i + (lane & 15);
    c.avalid[i] = row < p.M;
    c.arow[i] = p.A + (c.avalid[i] ? row : 0) * p.K;
  }
  {
    const int64_t col = n0 + (lane & 15);
    c.bvalid = col < p.N;
    c.brow = p.B + (c.bvalid ? col : 0) * p.K;
  }
  typename Ctx::Acc acc;
  c.leaf(acc);

  // Balanced tree across the waves' leaves: adjacent pairs first.
#pragma unroll
  for (int step = 1; step < NW; step *= 2) {
    if ((w % (2 * step)) == step) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) xch[w][(i * 4 + r) * 64 + lane] = acc.v[i][0][r];
    }
    __syncthreads();
    if ((w % (2 * step)) == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc.v[i][0][r] = acc.v[i][0][r] + xch[w + step][(i * 4 + r) * 64 + lane];
    }
    __syncthreads();
  }
  if (w != 0) return;
  const int64_t col = n0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + 16 * i + 4 * (lane >> 4) + r;
      if (row < p.M && col < p.N) {
        const int64_t off = (int64_t)z * p.c_group_stride + row * p.N + col;
        if constexpr (OUT_BF16)
          reinterpret_cast<uint16_t*>(p.C)[off] = f32_to_bf16_bits(acc.v[i][0][r]);
        else
          reinterpret_cast<float*>(p.C)[off] = acc.v[i][0][r];
      }
    }
}

// ------------------------------------------------------------- tree combine

template <int CNT, bool OUT_BF16, bool FOLD>
__global__ __launch_bounds__(256) void tree_combine_kernel(const float* __restrict__ P, int64_t plane,
                                                           void* __restrict__ C) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= plane) return;
  float v[CNT];
#pragma unroll
  for (int j = 0; j < CNT; ++j) v[j] = P[(int64_t)j * plane + i];
  float s;
  if constexpr (FOLD) {
    s = v[0];
#pragma unroll
    for (int j = 1; j < CNT; ++j) s = s + v[j];
  } else {
#pragma unroll
    for (int w = CNT; w > 1; w /= 2)
#pragma unroll
      for (int j = 0; j < w / 2; ++j) v[j] = v[2 * j] + v[2 * j + 1];
    s = v[0];
  }
  if constexpr (OUT_BF16)
    reinterpret_cast<uint16_t*>(C)[i] = f32_to_bf16_bits(s);
  else
    reinterpret_cast<float*>(C)[i] = s;
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y,
                                                        int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = f32_to_bf16_bits(x[i]);
}

// ------------------------------------------------------------------ dispatch

// Wave tile per subtree size: up to 4 leaves keep 64x64 per wave (<= 3 live
// accumulator sets); 8 leaves need 4 live sets and use 64x32 per wave.
inline int tile_bn(int nl) { return nl >= 8 ? 64 : 128; }

template <bool OUT_BF16, bool GROUPED>
hipError_t tile_dispatch(const TileParams& p, dim3 grid, int nl, hipStream_t s) {
  switch (nl) {
    case 1: hipLaunchKernelGGL((gemm_tile_kernel<4, 4, 1, OUT_BF16, GROUPED>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_tile_kernel<4, 4, 2, OUT_BF16, GROUPED>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_tile_kernel<4, 4, 4, OUT_BF16, GROUPED>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_tile_kernel<4, 2, 8, OUT_BF16, GROUPED>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FM, bool OUT_BF16>
hipError_t stream_dispatch_nw(const TileParams& p, dim3 grid, int nw, hipStream_t s) {
  switch (nw) {
    case 1: hipLaunchKernelGGL((gemm_stream_kernel<FM, 1, OUT_BF16>), grid, dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_stream_kernel<FM, 2, OUT_BF16>), grid, dim3(128), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_stream_kernel<FM, 4, OUT_BF16>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_stream_kernel<FM, 8, OUT_BF16>), grid, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool OUT_BF16>
hipError_t stream_dispatch(const TileParams& p, int fm, dim3 grid, int nw, hipStream_t s) {
  switch (fm) {
    case 1: return stream_dispatch_nw<1, OUT_BF16>(p, grid, nw, s);
    case 2: return stream_dispatch_nw<2, OUT_BF16>(p, grid, nw, s);
    case 3: return stream_dispatch_nw<3, OUT_BF16>(p, grid, nw, s);
    case 4: return stream_dispatch_nw<4, OUT_BF16>(p, grid, nw, s);
    default: return hipErrorInvalidValue;
  }
}

template <int CNT>
hipError_t combine_cnt(const float* P, int64_t plane, void* C, bool out_bf16, bool fold, hipStream_t s) {
  dim3 grid((unsigned)((plane + 255) / 256));
  if (out_bf16) {
    if (fold) hipLaunchKernelGGL((tree_combine_kernel<CNT, true, true>), grid, dim3(256), 0, s, P, plane, C);
    else hipLaunchKernelGGL((tree_combine_kernel<CNT, true, false>), grid, dim3(256), 0, s, P, plane, C);
  } else {
    if (fold) hipLaunchKernelGGL((tree_combine_kernel<CNT, false, true>), grid, dim3(256), 0, s, P, plane, C);
    else hipLaunchKernelGGL((tree_combine_kernel<CNT, false, false>), grid, dim3(256), 0, s, P, plane, C);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s) {
  TileParams p;
  p.A = static_cast<const uint16_t*>(g.A);
  p.B = static_cast<const uint16_t*>(g.B);
  p.C = g.C;
  p.M = g.M;
  p.N = g.N;
  p.K = g.K;
  p.c_group_stride = g.c_group_stride;
  p.kl = g.kl;
  p.leaf_lo = g.leaf_lo;
  p.nl = g.nl;
  p.rows = g.rows;
  p.offsets = g.offsets;
  p.E = g.E;
  p.a_rows = g.a_rows;
  p.b_expert_stride = g.b_expert_stride;

  if (g.offsets) {  // grouped: tile slots = an upper bound on sum_e ceil(count_e / 128)
    const int64_t slots = g.M / 128 + g.E;
    const int bn = tile_bn(g.nl);
    dim3 grid((unsigned)((g.N + bn - 1) / bn), (unsigned)slots, (unsigned)g.groups);
    return g.out_bf16 ? tile_dispatch<true, true>(p, grid, g.nl, s) : tile_dispatch<false, true>(p, grid, g.nl, s);
  }
  if (g.M <= 64) {
    const int fm = (int)((g.M + 15) / 16);
    // each wave owns one leaf; groups of nl leaves become nl waves per WG
    dim3 grid((unsigned)((g.N + 15) / 16), 1u, (unsigned)g.groups);
    return g.out_bf16 ? stream_dispatch<true>(p, fm, grid, g.nl, s) : stream_dispatch<false>(p, fm, grid, g.nl, s);
  }
  const int bn = tile_bn(g.nl);
  dim3 grid((unsigned)((g.N + bn - 1) / bn), (unsigned)((g.M + 127) / 128), (unsigned)g.groups);
  return g.out_bf16 ? tile_dispatch<true, false>(p, grid, g.nl, s) : tile_dispatch<false, false>(p, grid, g.nl, s);
}

hipError_t launch_tree_combine(const float* P, int count, int64_t plane, void* C, bool out_bf16, bool left_fold,
                               hipStream_t s) {
  switch (count) {
    case 1: return combine_cnt<1>(P, plane, C, out_bf16, left_fold, s);
    case 2: return combine_cnt<2>(P, plane, C, out_bf16, left_fold, s);
    case 4: return combine_cnt<4>(P, plane, C, out_bf16, left_fold, s);
    case 8: return combine_cnt<8>(P, plane, C, out_bf16, left_fold, s);
    case 16: return combine_cnt<16>(P, plane, C, out_bf16, left_fold, s);
    case 32: return combine_cnt<32>(P, plane, C, out_bf16, left_fold, s);
    case 64: return combine_cnt<64>(P, plane, C, out_bf16, left_fold, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_cast_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

}  // namespace inv
