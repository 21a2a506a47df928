// Mixture-of-experts stages around the K-leaf grouped GEMM, for gfx950.
//
// IsoExec blog, "Unified model": MoE routing and combination are made
// deterministic; "Parallelism-invariant kernels": expert outputs are combined
// in a fixed routing order instead of rank order; "Unified execution
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
// One wave per token. Lane l holds experts l, l+64, l+128, l+192. k rounds of
// a wave-wide argmax (larger logit wins, equal logits go to the lower id)
// select the top k; NaN logits are never selected, and a round without a
// candidate leaves id -1 and weight NaN (a data error marks the token).
// The selection is then written in ascending expert id, and the weights are
// the softmax over the selected logits: e_j = exp2((z_j - max) * log2e),
// denominator summed over j in ascending id, w_j = e_j / denominator.
constexpr int kRouteMaxK = 32;

__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                        float* __restrict__ w, int64_t T, int E, int k) {
  __shared__ float ez[4][kRouteMaxK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  const bool live = t < T;  // no early return: the block meets at a barrier below

  float z[4];
  bool taken[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    z[q] = (live && e < E) ? logits[t * E + e] : -INFINITY;
    taken[q] = false;
  }
  int found = 0;
  for (int r = 0; r < k; ++r) {
    // this lane's best untaken candidate
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E && !taken[q] && (z[q] > bv || (z[q] == bv && e < bid))) {
        bv = z[q];
        bid = e;
      }
    }
    // wave argmax, same comparison
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = shfl_xor(bv, off);
      const int oid = __builtin_amdgcn_ds_bpermute((lane ^ off) << 2, bid);
      if (ov > bv || (ov == bv && oid < bid)) {
        bv = ov;
        bid = oid;
      }
    }
    if (bid == 0x7fffffff) break;  // wave-uniform: nothing selectable left
    ++found;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (bid == lane + 64 * q) taken[q] = true;
  }
  // position of each selected expert in ascending id order
  int before = 0;
  int pos[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t bal = __ballot(taken[q]);
    pos[q] = before + __popcll(bal & ((1ull << lane) - 1ull));
    before += __popcll(bal);
  }
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (taken[q]) m = fmaxf(m, z[q]);
  m = wave_max(m);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (taken[q]) ez[wave][pos[q]] = exp_shifted(z[q], m);
  __syncthreads();
  float den = 0.0f;
  for (int j = 0; j < found; ++j) den = den + ez[wave][j];
  if (!live) return;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (taken[q]) {
      ids[t * k + pos[q]] = lane + 64 * q;
      w[t * k + pos[q]] = ez[wave][pos[q]] / den;
    }
  if (lane >= found && lane < k) {  // rounds that found no candidate
    ids[t * k + lane] = -1;
    w[t * k + lane] = __builtin_nanf("");
  }
}

// ------------------------------------------------------------ grouping
//
// Pairs p = t*k + j are grouped by expert id, stable in p (so in token id,
// since a token lists each expert once). Three launches, no atomics:
//   count  : block e counts pairs with id e -> offsets[e+1]; block 0 also
//            marks pairs with an id outside [0, E) as slot -1;
//   scan   : offsets[0] = 0, offsets[e+1] += offsets[e] (one thread);
//   scatter: block e walks the pairs in ascending p, 1024 per round, and
//            gives its pairs consecutive grouped rows from offsets[e].

__global__ __launch_bounds__(256) void moe_count_kernel(const int32_t* __restrict__ ids, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ slot, int64_t P, int E) {
  __shared__ int part[4];
  const int e = blockIdx.x;
  int cnt = 0;
  for (int64_t p = threadIdx.x; p < P; p += 256) {
    const int32_t id = ids[p];
    cnt += (id == e);
    if (e == 0 && (id < 0 || id >= E)) slot[p] = -1;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ off) << 2, cnt);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) offsets[e + 1] = part[0] + part[1] + part[2] + part[3];
}

__global__ void moe_scan_kernel(int32_t* __restrict__ offsets, int E) {
  if (threadIdx.x != 0) return;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
}

__global__ __launch_bounds__(256) void moe_scatter_kernel(const int32_t* __restrict__ ids,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ rows, int32_t* __restrict__ slot,
                                                          int64_t P, int k) {
  __shared__ int scan[256];
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t next = offsets[e];
  for (int64_t base = 0; base < P; base += 1024) {
    bool f[4];
    int c = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t p = base + 4 * tid + u;
      f[u] = p < P && ids[p] == e;
      c += f[u];
    }
    // inclusive Hillis-Steele scan of the per-thread counts (integers: exact)
    scan[tid] = c;
    __syncthreads();
#pragma unroll
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    int r = (int)next + scan[tid] - c;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (f[u]) {
        const int64_t p = base + 4 * tid + u;
        rows[r] = (int32_t)(p / k);
        slot[p] = r;
        ++r;
      }
    }
    next += scan[255];
    __syncthreads();  // scan[] is rewritten next round
  }
}

// ------------------------------------------------------------------ SwiGLU
//
// a = bf16( silu(g) * u ), silu(g) = g / (1 + exp(-g)), g and u the bf16
// halves of a packed [gate | up] row, math in fp32 (exp as exp2(-g*log2e)).
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ gu, uint16_t* __restrict__ a,
                                                     int64_t R, int64_t F) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * F) return;
  const int64_t r = i / F, f = i - r * F;
  const float g = bf16_bits_to_f32(gu[r * 2 * F + f]);
  const float u = bf16_bits_to_f32(gu[r * 2 * F + F + f]);
  const float t = -g * kLog2e;
  const float den = 1.0f + exp2_hw(t);
  const float s = g / den;
  a[i] = f32_to_bf16_bits(s * u);
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
    if (bad) s = __builtin_nanf("");
    if (q < nv) out[t * H + h + q] = f32_to_bf16_bits(s);
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
  hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, ids, w, T, E, k);
  return hipGetLastError();
}

hipError_t launch_moe_permute(const int32_t* ids, int32_t* offsets, int32_t* rows, int32_t* slot, int64_t T, int E,
                              int k, hipStream_t s) {
  const int64_t P = T * k;
  hipLaunchKernelGGL(moe_count_kernel, dim3((unsigned)E), dim3(256), 0, s, ids, offsets, slot, P, E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(64), 0, s, offsets, E);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3((unsigned)E), dim3(256), 0, s, ids, offsets, rows, slot, P, k);
  return hipGetLastError();
}

hipError_t launch_swiglu(const void* gu, void* a, int64_t R, int64_t F, hipStream_t s) {
  const int64_t n = R * F;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(gu), static_cast<uint16_t*>(a), R, F);
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
