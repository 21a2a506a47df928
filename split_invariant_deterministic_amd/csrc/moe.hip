// Mixture-of-experts stages around the K-leaf grouped GEMM, for gfx950.
//
// IsoExec blog, "Unified model": MoE routing and combination are made
// deterministic; "Parallelism-invariant kernels": the summation order of a
// token's expert results follows the routing, not the producing rank; "Unified execution
// contract": the moe.combine region is a leaf tree of 8 fp32 leaves.
// RL-Kernel write-up, sections 6 and 7: packed gate/up GEMM, SwiGLU and down
// GEMM run as separate fixed stages.
//
// Every stage is per token (route, combine) or per grouped row (SwiGLU), so
// a token's bits never depend on which other tokens share the launch; the
// grouping of tokens by expert uses counts and prefix sums, never atomics.
#include "common.h"
#include "launch.h"

namespace inv {
namespace {

// ------------------------------------------------------------------ routing
//
// Sixteen lanes per token. k rounds of an argmax over the token's experts
// (larger logit wins, equal logits go to the lower id)
// select the top k; NaN logits are never selected, and a round without a
// candidate leaves id -1 and weight NaN (a data error marks the token).
// The selection is then written in ascending expert id, and the weights are
// the softmax over the selected logits: e_j = exp2((z_j - max) * log2e),
// denominator summed over j in ascending id, w_j = e_j / denominator.
//
// The argmax runs on 64-bit keys whose unsigned order is the selection order:
// high word the logit mapped monotonically to an unsigned integer (-0 taken
// as +0, since the two compare equal), low word 0xFFFF - id. NaN logits,
// experts past E and taken experts have key 0. A round is a branch-free
// maximum over the lane's keys, then over the token's 16 lanes by four DPP
// steps (VALU only).
constexpr int kRouteMaxK = 32;

__device__ __forceinline__ uint32_t route_key_hi(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (hi, lo) <- the larger of itself and (ohi, olo), unsigned 64-bit order
__device__ __forceinline__ void key_take_max(uint32_t& hi, uint32_t& lo, uint32_t ohi, uint32_t olo) {
  const bool t = ohi > hi || (ohi == hi && olo > lo);
  hi = t ? ohi : hi;
  lo = t ? olo : lo;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Maximum key over each row of 16 lanes, left in every lane of the row:
// quad pairs (xor 1, xor 2), then the half-row and row mirrors. The maximum
// of a set does not depend on the order it is taken in.
__device__ __forceinline__ void row_key_max(uint32_t& hi, uint32_t& lo) {
  key_take_max(hi, lo, dpp_u32<0xB1>(hi), dpp_u32<0xB1>(lo));
  key_take_max(hi, lo, dpp_u32<0x4E>(hi), dpp_u32<0x4E>(lo));
  key_take_max(hi, lo, dpp_u32<0x141>(hi), dpp_u32<0x141>(lo));
  key_take_max(hi, lo, dpp_u32<0x140>(hi), dpp_u32<0x140>(lo));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sixteen lanes per token, four tokens per wave: lane l of a row holds
// experts l, l + 16, ..., l + 16 (NQ - 1) (NQ = ceil(E / 16) rounded up to
// 4, 8 or 16).
template <int NQ>
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                        float* __restrict__ w, int64_t T, int E, int k) {
  __shared__ float ez[16][kRouteMaxK];
  const int lane = threadIdx.x & 63, l16 = lane & 15, row = threadIdx.x >> 4;  // row: token of the block
  const int64_t t = (int64_t)blockIdx.x * 16 + row;
  const bool live = t < T;  // no early return: the block meets at a barrier below

  float z[NQ];
  uint32_t khi[NQ], klo[NQ];
  bool taken[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = l16 + 16 * q;
    z[q] = (live && e < E) ? logits[t * E + e] : -INFINITY;
    const bool cand = live && e < E && !__builtin_isnan(z[q]);
    khi[q] = cand ? route_key_hi(z[q]) : 0u;
    klo[q] = cand ? 0xFFFFu - (uint32_t)e : 0u;
    taken[q] = false;
  }
  int found = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t hi = khi[0], lo = klo[0];
#pragma unroll
    for (int q = 1; q < NQ; ++q) key_take_max(hi, lo, khi[q], klo[q]);
    row_key_max(hi, lo);  // this token's best remaining key, in all 16 lanes
    if (__ballot(lo != 0u) == 0) break;  // wave-uniform: no token of the wave has a candidate left
    found += lo != 0u;
    const int bid = lo != 0u ? (int)(0xFFFFu - lo) : -1;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const bool hit = bid == l16 + 16 * q;
      taken[q] = taken[q] || hit;
      khi[q] = hit ? 0u : khi[q];
      klo[q] = hit ? 0u : klo[q];
    }
  }
  // position of each selected expert in ascending id order within the token
  const int sh = 16 * ((threadIdx.x >> 4) & 3);
  int before = 0;
  int pos[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const uint32_t bits = (uint32_t)(__ballot(taken[q]) >> sh) & 0xFFFFu;
    pos[q] = before + __popc(bits & ((1u << l16) - 1u));
    before += __popc(bits);
  }
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    if (taken[q]) m = fmaxf(m, z[q]);
  m = fmaxf(m, dpp_f32<0xB1>(m));
  m = fmaxf(m, dpp_f32<0x4E>(m));
  m = fmaxf(m, dpp_f32<0x141>(m));
  m = fmaxf(m, dpp_f32<0x140>(m));
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    if (taken[q]) ez[row][pos[q]] = exp_shifted(z[q], m);
  __syncthreads();
  float den = 0.0f;
  for (int j = 0; j < found; ++j) den = den + ez[row][j];
  if (!live) return;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    if (taken[q]) {
      ids[t * k + pos[q]] = l16 + 16 * q;
      w[t * k + pos[q]] = ez[row][pos[q]] / den;
    }
  for (int j = found + l16; j < k; j += 16) {  // rounds that found no candidate
    ids[t * k + j] = -1;
    w[t * k + j] = __builtin_nanf("");
  }
}

// ------------------------------------------------------------ grouping
//
// Pairs p = t*k + j are grouped by expert id, stable in p (so in token id,
// since a token lists each expert once). Three launches, no atomics:
//   count  : block e counts pairs with id e -> offsets[e+1]; block 0 also
//            marks pairs with an id outside [0, E) as slot -1;
//   scan   : offsets[0] = 0, offsets[e+1] += offsets[e] (one thread);
//   scatter: block (e, s) owns slice s of the pairs; it counts expert e's
//            pairs in the earlier slices (its base), each wave counts its
//            quarter of the slice, and the waves then hand out consecutive
//            grouped rows in ascending p with ballots.

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ off) << 2, v);
  return v;
}

// Matches of id e in pairs [lo, hi), summed over the calling threads
// (stride = number of threads taking part, t = this thread's index). Integer
// counts are exact in any order. The aligned middle is read as int4, eight
// loads in flight per thread; the few ids before and after it one by one.
__device__ __forceinline__ int count_matches(const int32_t* __restrict__ ids, int64_t lo, int64_t hi, int e, int t,
                                             int stride) {
  int cnt = 0;
  if ((reinterpret_cast<uintptr_t>(ids) & 15u) == 0 && hi - lo >= 8) {
    const int64_t a0 = (lo + 3) & ~(int64_t)3, a1 = hi & ~(int64_t)3;
    for (int64_t p = lo + t; p < a0; p += stride) cnt += ids[p] == e;
    for (int64_t p = a1 + t; p < hi; p += stride) cnt += ids[p] == e;
    const int4* v = reinterpret_cast<const int4*>(ids + a0);
    const int64_t n4 = (a1 - a0) / 4;
    auto m4 = [e](const int4 x) { return (x.x == e) + (x.y == e) + (x.z == e) + (x.w == e); };
    int64_t q = t;
    for (; q + 7 * (int64_t)stride < n4; q += 8 * (int64_t)stride) {
      int4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = v[q + u * (int64_t)stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) cnt += m4(x[u]);
    }
    for (; q < n4; q += stride) cnt += m4(v[q]);
    return cnt;
  }
  int64_t p = lo + t;
  for (; p + 3 * (int64_t)stride < hi; p += 4 * (int64_t)stride) {
    const int32_t a = ids[p], b = ids[p + stride], c = ids[p + 2 * stride], d = ids[p + 3 * stride];
    cnt += (a == e) + (b == e) + (c == e) + (d == e);
  }
  for (; p < hi; p += stride) cnt += (ids[p] == e);
  return cnt;
}

// One workgroup per expert counts its pairs; pairs with an id outside
// [0, E) get slot -1, each workgroup marking its own 1/E of the pairs.
__global__ __launch_bounds__(256) void moe_count_kernel(const int32_t* __restrict__ ids, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ slot, int64_t P, int E) {
  __shared__ int part[4];
  const int e = blockIdx.x;
  for (int64_t p = (P * e) / E + threadIdx.x; p < (P * (e + 1)) / E; p += 256) {
    const int32_t id = ids[p];
    if (id < 0 || id >= E) slot[p] = -1;
  }
  const int cnt = wave_sum_int(count_matches(ids, 0, P, e, threadIdx.x, 256));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) offsets[e + 1] = part[0] + part[1] + part[2] + part[3];
}

// Exclusive prefix of the E <= 256 counts in offsets[1..E]: one load per
// thread, an inclusive Hillis-Steele scan in LDS, one store per thread.
__global__ __launch_bounds__(256) void moe_scan_kernel(int32_t* __restrict__ offsets, int E) {
  __shared__ int c[2][256];
  const int t = threadIdx.x;
  int cur = 0;
  c[0][t] = t < E ? offsets[t + 1] : 0;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    c[cur ^ 1][t] = c[cur][t] + (t >= d ? c[cur][t - d] : 0);
    cur ^= 1;
    __syncthreads();
  }
  if (t < E) offsets[t + 1] = c[cur][t];
  if (t == 0) offsets[0] = 0;
}

constexpr int kScatterSlices = 8;

__global__ __launch_bounds__(256) void moe_scatter_kernel(const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ rows, int32_t* __restrict__ slot,
                                                          int64_t P, int k) {
  __shared__ int part[2][4];
  const int e = blockIdx.x, sidx = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t s0 = (P * sidx) / kScatterSlices, s1 = (P * (sidx + 1)) / kScatterSlices;
  const int64_t q0 = s0 + ((s1 - s0) * w) / 4, q1 = s0 + ((s1 - s0) * (w + 1)) / 4;  // this wave's quarter
  // expert e's pairs before this slice, and in this wave's quarter
  const int before = wave_sum_int(count_matches(ids, 0, s0, e, threadIdx.x, 256));
  const int mine = wave_sum_int(count_matches(ids, q0, q1, e, lane, 64));
  if (lane == 0) {
    part[0][w] = before;
    part[1][w] = mine;
  }
  __syncthreads();
  int next = offsets[e] + part[0][0] + part[0][1] + part[0][2] + part[0][3];
  for (int v = 0; v < w; ++v) next += part[1][v];
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int64_t base = q0; base < q1; base += 256) {
    int32_t id[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = base + 64 * j + lane;
      id[j] = p < q1 ? ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = base + 64 * j + lane;
      const bool f = id[j] == e;
      const uint64_t bal = __ballot(f);
      if (f) {
        const int r = next + __popcll(bal & lt);
        rows[r] = (int32_t)(p / k);
        slot[p] = r;
      }
      next += __popcll(bal);
    }
  }
}

// ------------------------------------------------------------------ SwiGLU
//
// a = bf16( silu_mul(g, u) ) (common.h) for the bf16 halves of a packed
// [gate | up] row; the gate/up GEMM's fused epilogue calls the same function.

// Scalar form (any F).
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ gu, uint16_t* __restrict__ a,
                                                     int64_t R, int64_t F) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < R * F; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / F, f = i - r * F;
    const float g = bf16_bits_to_f32(gu[r * 2 * F + f]);
    const float u = bf16_bits_to_f32(gu[r * 2 * F + F + f]);
    a[i] = f32_to_bf16_bits(silu_mul(g, u));
  }
}

// F % 8 == 0: 8 outputs per thread with 16-byte accesses (same per-element math).
__global__ __launch_bounds__(256) void swiglu8_kernel(const uint16_t* __restrict__ gu, uint16_t* __restrict__ a,
                                                      int64_t R, int64_t F) {
  const int64_t F8 = F >> 3;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < R * F8; v += (int64_t)gridDim.x * 256) {
    const int64_t r = v / F8, f = (v - r * F8) * 8;  // 8-element group v
    const u32x4 g = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gu + r * 2 * F + f));
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gu + r * 2 * F + F + f));
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack_bf16x2(silu_mul(bf16_lo(g[q]), bf16_lo(u[q])), silu_mul(bf16_hi(g[q]), bf16_hi(u[q])));
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a + r * F + f));
  }
}

// ----------------------------------------------------------------- combine
//
// out[t, h] = bf16( tree_j fp32(w[t,j] * Y[slot[t,j], h]) ), j over the k
// experts of token t in ascending expert id, balanced tree (adjacent pairs
// first) or left fold. A slot outside [0, y_rows) makes the row NaN.
template <int KK, bool FOLD>
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ Y, const float* __restrict__ w,
                                                          const int32_t* __restrict__ slot, int64_t y_rows,
                                                          uint16_t* __restrict__ out, int64_t H) {
  const int64_t t = blockIdx.y;
  const int64_t h = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  const int nv = (int)min((int64_t)4, H - h);
  float v[KK][4];
  bool bad = false;
  const bool vec = H % 4 == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
  if (vec) {
    // rows 16-byte aligned and h < H a multiple of 4: one float4 per expert
    // row, all KK loads in flight (a row past the table reads row 0 and the
    // token becomes NaN below); the rows are read once, so the loads stream
    // past the caches
    f32x4 y[KK];
    float wj[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      const int32_t s = slot[t * KK + j];
      wj[j] = w[t * KK + j];
      const bool ok = s >= 0 && s < y_rows;
      bad |= !ok;
      y[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + (ok ? (int64_t)s : 0) * H + h));
    }
#pragma unroll
    for (int j = 0; j < KK; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[j][q] = wj[j] * y[j][q];
  } else {
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      const int32_t s = slot[t * KK + j];
      const float wj = w[t * KK + j];
      const bool ok = s >= 0 && s < y_rows;
      bad |= !ok;
      const float* yr = Y + (ok ? (int64_t)s : 0) * H + h;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[j][q] = (q < nv && ok) ? wj * yr[q] : 0.0f;
    }
  }
  float r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float s;
    if constexpr (FOLD) {
      s = v[0][q];
#pragma unroll
      for (int j = 1; j < KK; ++j) s = s + v[j][q];
    } else {
#pragma unroll
      for (int n = KK; n > 1; n /= 2)
#pragma unroll
        for (int j = 0; j < n / 2; ++j) v[j][q] = v[2 * j][q] + v[2 * j + 1][q];
      s = v[0][q];
    }
    r[q] = bad ? __builtin_nanf("") : s;
  }
  if (vec && (reinterpret_cast<uintptr_t>(out) & 7) == 0) {  // the four bf16 as one 8-byte store
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    *reinterpret_cast<u32x2*>(out + t * H + h) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < nv) out[t * H + h + q] = f32_to_bf16_bits(r[q]);
  }
}

template <int KK>
hipError_t combine_k(const float* Y, const float* w, const int32_t* slot, int64_t y_rows, void* out, int64_t T,
                     int64_t H, bool fold, hipStream_t s) {
  dim3 grid((unsigned)((H + 1023) / 1024), (unsigned)T);
  auto O = static_cast<uint16_t*>(out);
  if (fold) hipLaunchKernelGGL((moe_combine_kernel<KK, true>), grid, dim3(256), 0, s, Y, w, slot, y_rows, O, H);
  else hipLaunchKernelGGL((moe_combine_kernel<KK, false>), grid, dim3(256), 0, s, Y, w, slot, y_rows, O, H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_route(const float* logits, int32_t* ids, float* w, int64_t T, int E, int k, hipStream_t s) {
  if (k > kRouteMaxK || E > 256) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((T + 15) / 16));
  if (E <= 64) hipLaunchKernelGGL(moe_route_kernel<4>, grid, dim3(256), 0, s, logits, ids, w, T, E, k);
  else if (E <= 128) hipLaunchKernelGGL(moe_route_kernel<8>, grid, dim3(256), 0, s, logits, ids, w, T, E, k);
  else hipLaunchKernelGGL(moe_route_kernel<16>, grid, dim3(256), 0, s, logits, ids, w, T, E, k);
  return hipGetLastError();
}

hipError_t launch_moe_permute(const int32_t* ids, int32_t* offsets, int32_t* rows, int32_t* slot, int64_t T, int E,
                              int k, hipStream_t s) {
  const int64_t P = T * k;
  hipLaunchKernelGGL(moe_count_kernel, dim3((unsigned)E), dim3(256), 0, s, ids, offsets, slot, P, E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(256), 0, s, offsets, E);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3((unsigned)E, kScatterSlices), dim3(256), 0, s, ids, offsets, rows, slot,
                     P, k);
  return hipGetLastError();
}

hipError_t launch_swiglu(const void* gu, void* a, int64_t R, int64_t F, hipStream_t s) {
  auto G = static_cast<const uint16_t*>(gu);
  auto O = static_cast<uint16_t*>(a);
  const bool vec = F % 8 == 0 && ((reinterpret_cast<uintptr_t>(gu) | reinterpret_cast<uintptr_t>(a)) & 15u) == 0;
  if (vec) {
    const int64_t n = R * (F / 8);
    hipLaunchKernelGGL(swiglu8_kernel, dim3(stride_grid(n, 256)), dim3(256), 0, s, G, O, R, F);
  } else {
    const int64_t n = R * F;
    hipLaunchKernelGGL(swiglu_kernel, dim3(stride_grid(n, 256)), dim3(256), 0, s, G, O, R, F);
  }
  return hipGetLastError();
}

hipError_t launch_moe_combine(const float* Y, const float* w, const int32_t* slot, int64_t y_rows, void* out,
                              int64_t T, int64_t H, int k, bool left_fold, hipStream_t s) {
  switch (k) {
    case 1: return combine_k<1>(Y, w, slot, y_rows, out, T, H, left_fold, s);
    case 2: return combine_k<2>(Y, w, slot, y_rows, out, T, H, left_fold, s);
    case 4: return combine_k<4>(Y, w, slot, y_rows, out, T, H, left_fold, s);
    case 8: return combine_k<8>(Y, w, slot, y_rows, out, T, H, left_fold, s);
    case 16: return combine_k<16>(Y, w, slot, y_rows, out, T, H, left_fold, s);
    case 32: return combine_k<32>(Y, w, slot, y_rows, out, T, H, left_fold, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace inv
