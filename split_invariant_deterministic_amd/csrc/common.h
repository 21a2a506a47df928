// Internal device helpers shared by the gfx950 kernels of libinv.
//
// Numerics pinned here and used by every kernel:
//   * one MFMA instruction for every bf16 contraction: v_mfma_f32_16x16x32_bf16
//     with the k-to-lane map "lane group g = lane/16 holds k = 8g .. 8g+7 of the
//     32-wide block, element e = k - 8g"; A rows / B columns sit on lane % 16;
//   * exp as exp2((x - m) * log2e) on the hardware exp2 (v_exp_f32), with the
//     product rounded to fp32 before the exp2;
//   * bf16 boundary casts by round-to-nearest-even (v_cvt_pk_bf16_f32);
//   * no contraction of a*b+c into FMA unless written as __builtin_fmaf
//     (the library is built with -ffp-contract=off).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace inv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr float kLog2e = 1.44269504088896340736f;  // fp32 rounding of log2(e)
constexpr float kLn2 = 0.693147180559945309417f;    // fp32 rounding of ln(2)

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer loads: a 128-bit descriptor (base, size in bytes, gfx9 raw
// format word 0x00020000: byte addressing, no stride or swizzle) in SGPRs, a
// per-lane 32-bit offset in one VGPR and a wave-uniform offset in an SGPR.
// Callers keep every access inside the described range.
// Cache policy for data read once (buffer and direct-to-LDS loads): nt,
// bit 1 of the gfx950 cache-policy field.
constexpr int kNT = 2;

typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(buf_rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// exp(x - m) in the pinned form. x - m is rounded, then the product with log2e.
__device__ __forceinline__ float exp_shifted(float x, float m) {
  float d = x - m;
  float t = d * kLog2e;
  return exp2_hw(t);
}

// SwiGLU of one element: silu(g) * u with silu(g) = g / (1 + exp(-g)), in
// fp32, exp as exp2(-g * log2e). The MoE SwiGLU kernels and the gate/up
// GEMM's fused epilogue both call this, so the two paths agree bit for bit.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float t = -g * kLog2e;
  const float den = 1.0f + exp2_hw(t);
  const float s = g / den;
  return s * u;
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Cross-lane exchange inside a 64-lane wave (ds_bpermute based shuffle).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  int lane = threadIdx.x & 63;
  int src = lane ^ mask;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

// Sum over the 64 lanes by the xor butterfly 32, 16, 8, 4, 2, 1. Every lane
// ends with the same bits (each step adds the same two values in either
// operand order, and fp32 addition is commutative).
__device__ __forceinline__ float wave_sum_butterfly(float v) {
  v = v + shfl_xor(v, 32);
  v = v + shfl_xor(v, 16);
  v = v + shfl_xor(v, 8);
  v = v + shfl_xor(v, 4);
  v = v + shfl_xor(v, 2);
  v = v + shfl_xor(v, 1);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, shfl_xor(v, 32));
  v = fmaxf(v, shfl_xor(v, 16));
  v = fmaxf(v, shfl_xor(v, 8));
  v = fmaxf(v, shfl_xor(v, 4));
  v = fmaxf(v, shfl_xor(v, 2));
  v = fmaxf(v, shfl_xor(v, 1));
  return v;
}

// The pinned two-block LSE merge: m = max(m1, m2); s = s1 e^(m1-m) + s2 e^(m2-m).
// (-inf, 0) is the identity and two empty blocks stay empty (no -inf - -inf).
struct MS {
  float m, s;
};

__device__ __forceinline__ MS lse_merge(MS a, MS b) {
  float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MS{-INFINITY, 0.0f};
  float fa = exp_shifted(a.m, m);
  float fb = exp_shifted(b.m, m);
  float s = a.s * fa + b.s * fb;
  return MS{m, s};
}

// Statistics of one 16-column vocabulary block held by one lane (v[c] is
// column c of the block; columns c >= nvalid lie past the vocabulary):
// m = max over the valid columns (exact); s = sum of exp2((v[c] - m) * log2e)
// over them by the balanced tree over the column index, adjacent pairs first:
// ((e0+e1)+(e2+e3))+((e4+e5)+(e6+e7)) + (the same over columns 8..15).
// Columns past the vocabulary contribute +0. A NaN logit makes s NaN.
__device__ __forceinline__ MS block16_stats(const float (&v)[16], int nvalid) {
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < 16; ++c)
    if (c < nvalid) m = fmaxf(m, v[c]);
  float e[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) e[c] = (c < nvalid && v[c] != -INFINITY) ? exp_shifted(v[c], m) : 0.0f;
#pragma unroll
  for (int w = 16; w > 1; w /= 2)
#pragma unroll
    for (int k = 0; k < w / 2; ++k) e[k] = e[2 * k] + e[2 * k + 1];
  return MS{m, e[0]};
}

}  // namespace inv
