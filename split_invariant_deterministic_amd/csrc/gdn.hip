// Gated DeltaNet under the chunkwise-parallel recurrent (CPR) schedule, gfx950.
//
// IsoExec blog, "Chunkwise-parallel recurrent (CPR) GDN" (and the NovaSky
// write-up, "Solving the linear-attention headache"). The token recurrence
// defines the layer. Prefill obtains the state at each multiple of C with a
// separate boundary pass and then evaluates all chunks' tokens independently,
// each from its own opening state; decode steps the recurrence and, whenever
// a chunk completes, swaps its running state for that chunk's boundary
// state. Both paths run the same device functions below (rec_step for a
// token, chunk_coeffs and chunk_state for a boundary) on the same thread
// layouts, so they round identically.
//
// Layer (gated delta rule, one head, width 128, restated):
//   k^ = k / sqrt(sum k^2 + eps), q^ = q / sqrt(sum q^2 + eps) * 128^(-1/2)
//   alpha = exp(g); S_t = alpha (S - beta k^ (k^T S)) + beta k^ v^T; o_t = S_t^T q^
// Boundary states use the chunkwise closed form of the same recurrence:
//   gamma_t = alpha_0 ... alpha_t (running product inside the chunk)
//   w = M r, M = (I + diag(beta) A)^(-1) diag(beta), A[t][s] = (gamma_t/gamma_s)(k^_s.k^_t)
//       for s < t, r_t = v_t - gamma_t S0^T k^_t
//   S_C = gamma_{C-1} S0 + sum_s (gamma_{C-1}/gamma_s) k^_s w_s^T
// M, gamma and the ratios do not depend on the state, so in a prefill they
// are computed for every chunk in parallel; only r, w and S_C stay serial.
//
// Thread layouts. The recurrence (256 threads): thread (ti, tj), ti = lane %
// 16, tj = 4 * wave + lane / 16, holds S[8ti .. 8ti+8)[8tj .. 8tj+8) in
// registers; a reduction over the state rows (S^T x) is, per column, a
// sequential fma chain over 8 rows, then a balanced tree over the 16 row
// groups (the 16 lanes of a DPP row share the column: an in-register
// butterfly). The chunk update: a wave owns 16 value columns of the state,
// all 128 rows, as eight fp32 MFMA accumulators (16x16 blocks); the chunk's
// three products (P = K^ S, w = M r, and the rank-C state update) are fp32
// MFMA chains over those blocks. Columns never mix, so the bits of a column
// do not depend on which wave or workgroup holds it.
#include "common.h"
#include "launch.h"

namespace inv {
namespace {

constexpr int kD = 128;              // key = value width
constexpr float kGdnEps = 1e-6f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // fp32(128^-1/2)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                               true));
}

// Sum over the 16 lanes of a DPP row, pairing xor 1, 2, 4, 8 (a balanced tree
// over the lane index). 0xB1 / 0x4E: quad_perm [1,0,3,2] / [2,3,0,1]; after
// two steps a quad is uniform, so row_half_mirror (0x141) reads the xor-4
// partner's value, and then row_mirror (0x140) the xor-8 partner's.
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp<0xB1>(v);
  v = v + dpp<0x4E>(v);
  v = v + dpp<0x141>(v);
  v = v + dpp<0x140>(v);
  return v;
}

struct Tl {
  int tid, lane, ti, tj;
};
__device__ __forceinline__ Tl thread_layout() {
  Tl t;
  t.tid = threadIdx.x;
  t.lane = t.tid & 63;
  t.ti = t.lane & 15;
  t.tj = 4 * (t.tid >> 6) + (t.lane >> 4);
  return t;
}

// norms.l2 + gating for one (token, head), one wave: lane l holds elements 2l
// and 2l+1 of q and k (bf16 pairs). Sum of squares: a*a then fma(b, b, .) per
// lane, then the xor butterfly 32..1.
__device__ __forceinline__ float2 l2norm_pair(uint32_t bits, float scale) {
  const float a = bf16_lo(bits), b = bf16_hi(bits);
  float ss = a * a;
  ss = __builtin_fmaf(b, b, ss);
  ss = wave_sum_butterfly(ss);
  const float r = 1.0f / __builtin_sqrtf(ss + kGdnEps);
  return make_float2((a * r) * scale, (b * r) * scale);
}

__device__ __forceinline__ float gate_alpha(float g) { return exp2_hw(g * kLog2e); }

// One token of the recurrence on the thread's 8x8 block. k8 / q8: the
// thread's 8 rows of k^ and q^; v8: its 8 columns of v.
__device__ __forceinline__ void rec_step(float (&S)[8][8], const float (&k8)[8], const float (&q8)[8],
                                         const float (&v8)[8], float a, float b, float (&o8)[8]) {
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    float u = 0.0f;
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) u = __builtin_fmaf(S[ii][jj], k8[ii], u);
    u = row16_sum(u);
    const float d = b * (v8[jj] - a * u);
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) S[ii][jj] = __builtin_fmaf(k8[ii], d, a * S[ii][jj]);
  }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    float o = 0.0f;
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) o = __builtin_fmaf(S[ii][jj], q8[ii], o);
    o8[jj] = row16_sum(o);
  }
}

// The coefficient phase: a workgroup of 256 threads per chunk; the layout
// below only numbers the threads.
constexpr int kKStride = kD + 1;  // odd row stride: lanes reading different rows hit different banks

struct Tc {
  int tid, lane, ti, tc;
};
__device__ __forceinline__ Tc col_layout() {
  Tc t;
  t.tid = threadIdx.x;
  t.lane = t.tid & 63;
  t.ti = t.lane & 15;
  t.tc = 4 * (t.tid >> 6) + (t.lane >> 4);
  return t;
}

// LDS of one chunk's coefficient phase. K: k^ of the chunk's C tokens (all
// 128 rows); MT: M transposed (MT[s][t] = M[t][s]); gates and their running
// products; A: the scaled Gram matrix.
template <int C>
struct alignas(16) ChunkLds {
  float K[C][kKStride];
  float MT[C][C];
  float alpha[C], beta[C], gamma[C], cf[C];
  union {
    float A[C][C];
  } u;
};

// Coefficients of a chunk, independent of the state: gamma_t = alpha_0 ...
// alpha_t (one thread, ascending), cf_s = gamma_last / gamma_s, the strictly
// lower A[t][s] = (gamma_t / gamma_s) (k^_s . k^_t), and
// M = (I + diag(beta) A)^(-1) diag(beta), lower triangular, column c by
// forward substitution: M[t][c] = -beta_t (sum_{s<t} A[t][s] M[s][c] - [t == c])
// (s ascending from 0): signed zeros above the diagonal, beta_c on it.
// Needs K, alpha, beta; writes gamma, cf, MT (A is scratch).
template <int C>
__device__ void chunk_coeffs(ChunkLds<C>& L, const Tc& T) {
  if (T.tid == 0) {
    float gm = 1.0f;  // 1 * alpha_0 = alpha_0 exactly
#pragma unroll
    for (int t0 = 0; t0 < C; t0 += 16) {
      float al[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) al[q] = L.alpha[t0 + q];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        gm = gm * al[q];
        L.gamma[t0 + q] = gm;
      }
    }
  }
  __syncthreads();
  if (T.tid < C) L.cf[T.tid] = L.gamma[C - 1] / L.gamma[T.tid];
  // Gram entries: each dot a sequential fma over the width in ascending order,
  // in register tiles of 4 x 4 (per step 4 + 4 reads, 16 fmas)
  static_assert(C % 16 == 0 && (C / 4) * (C / 4) <= 256, "chunk shape");
  if (T.tid < (C / 4) * (C / 4)) {
    const int t0 = 4 * (T.tid / (C / 4)), s0 = 4 * (T.tid % (C / 4));
    if (s0 <= t0) {
      float dot[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) dot[a][b] = 0.0f;
      for (int i = 0; i < kD; ++i) {
        float kt[4], ks[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) kt[a] = L.K[t0 + a][i];
#pragma unroll
        for (int b = 0; b < 4; ++b) ks[b] = L.K[s0 + b][i];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) dot[a][b] = __builtin_fmaf(kt[a], ks[b], dot[a][b]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          L.u.A[t0 + a][s0 + b] = s0 + b < t0 + a ? (L.gamma[t0 + a] / L.gamma[s0 + b]) * dot[a][b] : 0.0f;
    }
  }
  __syncthreads();
  // M column c on thread c, in registers. Rows go in blocks of 16: the block's
  // 16 sums over the earlier blocks run as interleaved independent chains
  // (A read four entries at a time), then the in-block terms in order; every
  // entry keeps its single ascending-s chain.
  if (T.tid < C) {
    const int c = T.tid;
    float m[C];
#pragma unroll
    for (int b0 = 0; b0 < C; b0 += 16) {
      float acc[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
#pragma unroll
      for (int s4 = 0; s4 < b0; s4 += 4)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float4 a4 = *reinterpret_cast<const float4*>(&L.u.A[b0 + q][s4]);
          acc[q] = __builtin_fmaf(a4.x, m[s4], acc[q]);
          acc[q] = __builtin_fmaf(a4.y, m[s4 + 1], acc[q]);
          acc[q] = __builtin_fmaf(a4.z, m[s4 + 2], acc[q]);
          acc[q] = __builtin_fmaf(a4.w, m[s4 + 3], acc[q]);
        }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = b0 + q;
#pragma unroll
        for (int s = b0; s < t; ++s) acc[q] = __builtin_fmaf(L.u.A[t][s], m[s], acc[q]);
        // right-hand side e_c: m_t = -beta_t (acc_t - [t == c]); above the
        // diagonal acc is +0 and m_t a signed zero, on it m_c = beta_c exactly
        m[t] = -L.beta[t] * (acc[q] - (t == c ? 1.0f : 0.0f));
      }
#pragma unroll
      for (int q = 0; q < 16; q += 4)
        *reinterpret_cast<float4*>(&L.MT[c][b0 + q]) = make_float4(m[b0 + q], m[b0 + q + 1], m[b0 + q + 2],
                                                                     m[b0 + q + 3]);
    }
  }
  __syncthreads();
}

// State phase of a chunk update: a wave owns the 16 value columns c0 .. c0+15
// of the state, all 128 rows, as 8 fp32 MFMA accumulators: lane l holds
// S[16 ib + 4 (l / 16) + r][c0 + l % 16] in S[ib][r] (v_mfma_f32_16x16x4f32:
// A[l % 16][l / 16], B[l / 16][l % 16], D[4 (l / 16) + r][l % 16]). With that
// layout the state feeds the next product directly: k-step q of a 16-row
// block takes register q as the B operand (rows 16 ib + 4 g + q for the four
// lane groups g) and the matching A columns, so nothing is transposed.
constexpr int kWC = 16;                      // state columns per wave
constexpr int kStateWaves = 4;               // waves per state workgroup: with two, pairs of
                                             // waves could share a SIMD's MFMA unit
constexpr int kSB = kWC * kStateWaves;       // state columns per workgroup
constexpr int kSKStride = kD + 4;            // K rows: 16-byte aligned, 16 rows cover the 64 banks
template <int C>
struct alignas(16) StateLds {
  float K[C][kSKStride];  // k^ of the chunk's tokens
  float M[C][C + 4];      // M[t][s]
  float gamma[C], cf[C];
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// S (b_j on entry) becomes b_{j+1}:
//   P_t = S0^T k^_t: per 16-token block, MFMA k-steps over row blocks ib
//        ascending, k-step q taking rows 16 ib + 4 g + q;
//   r_t = v_t - gamma_t P_t;
//   w_t = sum_s M[t][s] r_s: k-steps over token blocks sb ascending, q as
//        above (s over the whole chunk; M is +0 above the diagonal);
//   S_C = gamma_last S0 + sum_s (cf_s k^_s) w_s^T: S0 scaled first, then
//        k-steps over sb ascending; A entries cf_s * k^_s[i] rounded once.
// v: this lane's v_t (t = 16 tb + 4 g + r).
template <int C>
__device__ __forceinline__ void chunk_state(f32x4 (&S)[8], const StateLds<C>& L, const float (&v)[C / 16][4],
                                            int lane) {
  constexpr int TB = C / 16;
  const int g = lane >> 4, c16 = lane & 15;
  f32x4 P[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) P[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Each P[tb] is its own chain over (ib, q) ascending; the TB chains are
  // interleaved so that consecutive MFMAs never wait on each other.
#pragma unroll
  for (int ib = 0; ib < 8; ++ib) {
    f32x4 k4[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) k4[tb] = *reinterpret_cast<const f32x4*>(&L.K[16 * tb + c16][16 * ib + 4 * g]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) P[tb] = mfma4(k4[tb][q], S[ib][q], P[tb]);
  }
  f32x4 R[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) R[tb][r] = v[tb][r] - L.gamma[16 * tb + 4 * g + r] * P[tb][r];
  f32x4 W[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) W[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sb = 0; sb < TB; ++sb) {
    f32x4 m4[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) m4[tb] = *reinterpret_cast<const f32x4*>(&L.M[16 * tb + c16][16 * sb + 4 * g]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) W[tb] = mfma4(m4[tb][q], R[sb][q], W[tb]);
  }
  const float glast = L.gamma[C - 1];
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[ib][r] = glast * S[ib][r];
#pragma unroll
  for (int sb = 0; sb < TB; ++sb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* krow = &L.K[16 * sb + 4 * g + q][c16];
      const float cf = L.cf[16 * sb + 4 * g + q];
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) S[ib] = mfma4(cf * krow[16 * ib], W[sb][q], S[ib]);
    }
}

// Buffer accesses: a descriptor over one array range (uniform), the lane's
// part of the byte offset in one VGPR and the rest a scalar offset, so a
// loop over blocks keeps no per-load 64-bit address.
__device__ __forceinline__ float bload(buf_rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ f32x4 bload4(buf_rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ void bstore(float v, buf_rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}

// The wave's state columns <-> one global state [128][128] fp32 (row-major).
__device__ __forceinline__ void load_cols(f32x4 (&S)[8], const float* __restrict__ g, int c0, int lane) {
  const buf_rsrc r = make_rsrc(g, kD * kD * 4);
  const uint32_t vo = (uint32_t)((4 * (lane >> 4) * kD + c0 + (lane & 15)) * 4);
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int q = 0; q < 4; ++q) S[ib][q] = bload(r, vo, (uint32_t)((16 * ib + q) * kD * 4));
}
__device__ __forceinline__ void store_cols(const f32x4 (&S)[8], float* __restrict__ g, int c0, int lane) {
  const buf_rsrc r = make_rsrc(g, kD * kD * 4);
  const uint32_t vo = (uint32_t)((4 * (lane >> 4) * kD + c0 + (lane & 15)) * 4);
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int q = 0; q < 4; ++q) bstore(S[ib][q], r, vo, (uint32_t)((16 * ib + q) * kD * 4));
}

// One chunk's state-phase inputs. K (k^: C token rows of 128 fp32 at kbase,
// tok_stride floats apart), M (row-major) and the gates' products go to LDS,
// every global load issued before the first LDS write; the lane's own v
// (C token rows at vbase, tok_stride elements apart, bf16 or fp32) goes to
// registers. coef: the chunk's [M (C x C) | gamma (C) | cf (C)].
template <int C>
struct StateRegs {
  static constexpr int NT = 64 * kStateWaves;
  static constexpr int PK = C * kD / 4 / NT, PM = C * C / 4 / NT;
  f32x4 kr[PK], mr[PM];
  float v[C / 16][4];
  float gc;
};

// Issue the chunk's loads into registers (nothing waits for them here).
template <int C, typename VT>
__device__ __forceinline__ void state_load(StateRegs<C>& R, const float* __restrict__ coef,
                                           const float* __restrict__ kbase, const VT* __restrict__ vbase,
                                           int64_t tok_stride, int tid, int c0) {
  constexpr int NT = StateRegs<C>::NT, PK = StateRegs<C>::PK, PM = StateRegs<C>::PM;
  static_assert(NT % (kD / 4) == 0, "a thread keeps its k^ column across loads");
  static_assert(NT >= 2 * C, "one thread per gamma and cf entry");
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const uint32_t ts = (uint32_t)tok_stride;
  const buf_rsrc rk = make_rsrc(kbase, (uint32_t)(((C - 1) * tok_stride + kD) * 4));
  const buf_rsrc rc = make_rsrc(coef, (uint32_t)((C * C + 2 * C) * 4));
  const buf_rsrc rv = make_rsrc(vbase, (uint32_t)(((C - 1) * tok_stride + kD) * sizeof(VT)));
  const int tk = tid / (kD / 4), i4 = 4 * (tid % (kD / 4));  // token row and column of load u = 0
#pragma unroll
  for (int u = 0; u < PK; ++u)
    R.kr[u] = bload4(rk, (uint32_t)((tk * ts + i4) * 4), (uint32_t)(u * (NT / (kD / 4)) * ts * 4));
#pragma unroll
  for (int u = 0; u < PM; ++u) R.mr[u] = bload4(rc, (uint32_t)(tid * 16), (uint32_t)(u * NT * 16));
  const uint32_t vo = (uint32_t)((4 * g * ts + c0 + c16) * sizeof(VT));
#pragma unroll
  for (int tb = 0; tb < C / 16; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t so = (uint32_t)((16 * tb + r) * ts * sizeof(VT));
      if constexpr (sizeof(VT) == 2)
        R.v[tb][r] = bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rv, vo, so, 0));
      else
        R.v[tb][r] = bload(rv, vo, so);
    }
  R.gc = 0.0f;
  if (tid < 2 * C) R.gc = bload(rc, (uint32_t)((C * C + tid) * 4), 0u);  // gamma then cf
}

// Publish loaded inputs in LDS: k^ rows, M, gamma and cf.
template <int C>
__device__ __forceinline__ void state_commit(StateLds<C>& L, const StateRegs<C>& R, int tid) {
  constexpr int NT = StateRegs<C>::NT, PK = StateRegs<C>::PK, PM = StateRegs<C>::PM;
  const int tk = tid / (kD / 4), i4 = 4 * (tid % (kD / 4));
  __syncthreads();  // every wave is done with the previous chunk's LDS
#pragma unroll
  for (int u = 0; u < PK; ++u) *reinterpret_cast<f32x4*>(&L.K[tk + u * (NT / (kD / 4))][i4]) = R.kr[u];
#pragma unroll
  for (int u = 0; u < PM; ++u) {
    const int e = tid + NT * u;
    *reinterpret_cast<f32x4*>(&L.M[e / (C / 4)][4 * (e % (C / 4))]) = R.mr[u];
  }
  if (tid < C) L.gamma[tid] = R.gc;
  else if (tid < 2 * C) L.cf[tid - C] = R.gc;
  __syncthreads();
}

template <int C, typename VT>
__device__ __forceinline__ void state_inputs(StateLds<C>& L, const float* __restrict__ coef,
                                             const float* __restrict__ kbase, const VT* __restrict__ vbase,
                                             int64_t tok_stride, float (&v)[C / 16][4], int tid, int c0) {
  StateRegs<C> R;
  state_load<C>(R, coef, kbase, vbase, tok_stride, tid, c0);
  state_commit<C>(L, R, tid);
#pragma unroll
  for (int tb = 0; tb < C / 16; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) v[tb][r] = R.v[tb][r];
}

// The coefficient phase's inputs into LDS: every global load issued before
// the first LDS write, so the memory latency is paid once. K: all 128 rows of
// k^ for the chunk's C tokens; the gates.
template <int C, typename KAt, typename GAt>
__device__ __forceinline__ void fill_chunk(ChunkLds<C>& L, const Tc& T, KAt kat, GAt gat) {
  constexpr int PK = C * kD / 256;
  float kr[PK];
#pragma unroll
  for (int u = 0; u < PK; ++u) {
    const int e = T.tid + 256 * u;
    kr[u] = kat(e / kD, e % kD);
  }
  float al = 0.0f, be = 0.0f;
  if (T.tid < C) gat(T.tid, al, be);
#pragma unroll
  for (int u = 0; u < PK; ++u) {
    const int e = T.tid + 256 * u;
    L.K[e / kD][e % kD] = kr[u];
  }
  if (T.tid < C) {
    L.alpha[T.tid] = al;
    L.beta[T.tid] = be;
  }
  __syncthreads();
}

// State block <-> global [128][128] fp32 (row-major), thread's 8x8 block.
__device__ __forceinline__ void load_state(float (&S)[8][8], const float* __restrict__ g, const Tl& T) {
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    const float4* r = reinterpret_cast<const float4*>(g + (8 * T.ti + ii) * kD + 8 * T.tj);
    const float4 x = r[0], y = r[1];
    S[ii][0] = x.x; S[ii][1] = x.y; S[ii][2] = x.z; S[ii][3] = x.w;
    S[ii][4] = y.x; S[ii][5] = y.y; S[ii][6] = y.z; S[ii][7] = y.w;
  }
}
__device__ __forceinline__ void store_state(const float (&S)[8][8], float* __restrict__ g, const Tl& T) {
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    float4* r = reinterpret_cast<float4*>(g + (8 * T.ti + ii) * kD + 8 * T.tj);
    r[0] = make_float4(S[ii][0], S[ii][1], S[ii][2], S[ii][3]);
    r[1] = make_float4(S[ii][4], S[ii][5], S[ii][6], S[ii][7]);
  }
}

// Decode cache of one sequence (fp32): running state, last boundary state,
// and the tokens of the open chunk (k^, v, alpha, beta per slot).
struct CacheView {
  float* srun;  // [H][128][128]
  float* sb;    // [H][128][128]
  float* kbuf;  // [C][H][128]
  float* vbuf;  // [C][H][128]
  float* abuf;  // [C][H]
  float* bbuf;  // [C][H]
  float* coef;  // [H][C*C + 2C] the closing chunk's M (row-major), gamma, ratios (decode scratch)
};
__device__ __forceinline__ CacheView cache_view(void* base, int64_t seq, int H, int C) {
  const int64_t per = gdn_cache_floats(H, C);
  float* p = static_cast<float*>(base) + seq * per;
  CacheView v;
  v.srun = p;
  v.sb = p + (int64_t)H * kD * kD;
  v.kbuf = v.sb + (int64_t)H * kD * kD;
  v.vbuf = v.kbuf + (int64_t)C * H * kD;
  v.abuf = v.vbuf + (int64_t)C * H * kD;
  v.bbuf = v.abuf + (int64_t)C * H;
  v.coef = v.bbuf + (int64_t)C * H;
  return v;
}

// ------------------------------------------------------------------ kernels

// Prep: one wave per (token, head): k^, q^ (fp32) and alpha.
__global__ __launch_bounds__(256) void gdn_prep_kernel(const uint32_t* __restrict__ q, const uint32_t* __restrict__ k,
                                                       const float* __restrict__ g, float* __restrict__ qh,
                                                       float* __restrict__ kh, float* __restrict__ alpha,
                                                       int64_t TH) {
  const int lane = threadIdx.x & 63;
  // one wave per (token, head), the grid striding over the rest (uniform per
  // wave; no block-wide barrier below)
  for (int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); th < TH; th += (int64_t)gridDim.x * 4) {
    const float2 kk = l2norm_pair(k[th * 64 + lane], 1.0f);
    const float2 qq = l2norm_pair(q[th * 64 + lane], kInvSqrtD);
    reinterpret_cast<float2*>(kh)[th * 64 + lane] = kk;
    reinterpret_cast<float2*>(qh)[th * 64 + lane] = qq;
    if (lane == 0) alpha[th] = gate_alpha(g[th]);
  }
}

// Sequence bounds from the device table, clamped to [0, T] so that a
// malformed table can never address outside the buffers (its outputs are
// then meaningless, but every index stays in range).
__device__ __forceinline__ int64_t cu_at(const GdnArgs& a, int s) {
  return min(max((int64_t)a.cu[s], (int64_t)0), a.T);
}
// First boundary-state slot of sequence s: floor(cu[s] / C) + s. Slot
// base(s) + j holds boundary j of sequence s; slots never collide for a
// well-formed table and stay below T/C + S for any table.
__device__ __forceinline__ int64_t boundary_base(const GdnArgs& a, int s, int C) { return cu_at(a, s) / C + s; }

// Coefficients of every full chunk, independent of the state, all chunks in
// parallel: one workgroup per (chunk slot, head). Slot c of sequence s is
// chunk j = c - boundary_base(s).
template <int C>
__global__ __launch_bounds__(256, 2) void gdn_coef_kernel(GdnArgs a) {
  __shared__ ChunkLds<C> L;
  const Tc T = col_layout();
  const int64_t c = blockIdx.x;
  const int h = blockIdx.y;
  int lo = 0, hi = a.S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (boundary_base(a, mid, C) <= c) lo = mid;
    else hi = mid - 1;
  }
  const int s = lo;
  const int64_t t0 = cu_at(a, s), len = max(cu_at(a, s + 1) - t0, (int64_t)0);
  const int64_t j = c - boundary_base(a, s, C);
  if (j < 0 || (j + 1) * C > len) return;  // not a full chunk (uniform)
  const int64_t tc0 = t0 + j * C;
  fill_chunk<C>(
      L, T, [&](int t, int i) { return a.kh[((tc0 + t) * a.H + h) * kD + i]; },
      [&](int t, float& al, float& be) {
        al = a.alpha[(tc0 + t) * a.H + h];
        be = a.beta[(tc0 + t) * a.H + h];
      });
  chunk_coeffs<C>(L, T);
  float* dst = a.coef + (c * a.H + h) * (int64_t)(C * C + 2 * C);
  for (int e = T.tid; e < C * C; e += 256) dst[e] = L.MT[e % C][e / C];  // M[t][s], row-major
  if (T.tid < C) {
    dst[C * C + T.tid] = L.gamma[T.tid];
    dst[C * C + C + T.tid] = L.cf[T.tid];
  }
}

// First pass, the state-dependent part: one workgroup per (sequence, head,
// 32-column block), a wave per 16 columns, the chunks in order, each chunk's
// coefficients read from the coefficient pass.
template <int C>
__global__ __launch_bounds__(64 * kStateWaves) __attribute__((amdgpu_waves_per_eu(2))) void gdn_boundary_kernel(GdnArgs a) {
  __shared__ StateLds<C> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int c0 = kSB * (int)blockIdx.z + kWC * (tid >> 6);
  const int s = blockIdx.x, h = blockIdx.y;
  const int64_t t0 = cu_at(a, s), len = max(cu_at(a, s + 1) - t0, (int64_t)0);
  const int64_t n = len / C;
  const int64_t base = boundary_base(a, s, C);
  const int64_t plane = (int64_t)kD * kD;
  f32x4 S[8];
#pragma unroll
  for (int ib = 0; ib < 8; ++ib) S[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
  store_cols(S, a.bstates + (base * a.H + h) * plane, c0, lane);
  // Chunk j+1's inputs are loaded into registers while chunk j is computed.
  auto load = [&](StateRegs<C>& R, int64_t j) {
    const int64_t tc0 = t0 + j * C;
    state_load<C>(R, a.coef + ((base + j) * a.H + h) * (int64_t)(C * C + 2 * C), a.kh + (tc0 * a.H + h) * kD,
                  a.v + (tc0 * a.H + h) * kD, (int64_t)a.H * kD, tid, c0);
  };
  StateRegs<C> nx;
  if (n > 0) load(nx, 0);
  for (int64_t j = 0; j < n; ++j) {
    state_commit<C>(L, nx, tid);
    float v[C / 16][4];
#pragma unroll
    for (int tb = 0; tb < C / 16; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[tb][r] = nx.v[tb][r];
    if (j + 1 < n) load(nx, j + 1);
    chunk_state<C>(S, L, v, lane);
    store_cols(S, a.bstates + ((base + j + 1) * a.H + h) * plane, c0, lane);
  }
  if (a.cache) {
    const CacheView cv = cache_view(a.cache, s, a.H, C);
    store_cols(S, cv.sb + h * plane, c0, lane);
    if (len % C == 0) store_cols(S, cv.srun + h * plane, c0, lane);
  }
}

// One token's inputs for the thread: k^ and q^ rows, v columns, gates.
struct TokIn {
  float k8[8], q8[8], v8[8], a, b;
};
__device__ __forceinline__ void load_tok(TokIn& x, const GdnArgs& a, int64_t tok, int h, const Tl& T) {
  const int64_t r = (tok * a.H + h) * kD;
  const float4* kp = reinterpret_cast<const float4*>(a.kh + r + 8 * T.ti);
  const float4* qp = reinterpret_cast<const float4*>(a.qh + r + 8 * T.ti);
  const float4 k0 = kp[0], k1 = kp[1], q0 = qp[0], q1 = qp[1];
  x.k8[0] = k0.x; x.k8[1] = k0.y; x.k8[2] = k0.z; x.k8[3] = k0.w;
  x.k8[4] = k1.x; x.k8[5] = k1.y; x.k8[6] = k1.z; x.k8[7] = k1.w;
  x.q8[0] = q0.x; x.q8[1] = q0.y; x.q8[2] = q0.z; x.q8[3] = q0.w;
  x.q8[4] = q1.x; x.q8[5] = q1.y; x.q8[6] = q1.z; x.q8[7] = q1.w;
  const u32x4 vv = *reinterpret_cast<const u32x4*>(a.v + r + 8 * T.tj);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x.v8[2 * e] = bf16_lo(vv[e]);
    x.v8[2 * e + 1] = bf16_hi(vv[e]);
  }
  x.a = a.alpha[tok * a.H + h];
  x.b = a.beta[tok * a.H + h];
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_out(void* out, int64_t row, const float (&o8)[8], const Tl& T) {
  if (T.ti != 0) return;
  if constexpr (OUT_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(o8[2 * e], o8[2 * e + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + row + 8 * T.tj) = u32x4{w[0], w[1], w[2], w[3]};
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + row + 8 * T.tj);
    p[0] = make_float4(o8[0], o8[1], o8[2], o8[3]);
    p[1] = make_float4(o8[4], o8[5], o8[6], o8[7]);
  }
}

// Second pass: one workgroup per (chunk slot, head); chunk slot c of sequence
// s is c - boundary_base(s). Runs the recurrence from the chunk's boundary.
template <int C, bool OUT_BF16>
__global__ __launch_bounds__(256) void gdn_output_kernel(GdnArgs a) {
  const Tl T = thread_layout();
  const int64_t c = blockIdx.x;
  const int h = blockIdx.y;
  // the sequence owning slot c: largest s with base(s) <= c (uniform search)
  int lo = 0, hi = a.S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (boundary_base(a, mid, C) <= c) lo = mid;
    else hi = mid - 1;
  }
  const int s = lo;
  const int64_t t0 = cu_at(a, s), len = max(cu_at(a, s + 1) - t0, (int64_t)0);
  const int64_t j = c - boundary_base(a, s, C);
  if (j < 0 || j * C >= len) return;  // a slot with no tokens
  const int64_t plane = (int64_t)kD * kD;
  float S[8][8];
  load_state(S, a.bstates + (c * a.H + h) * plane, T);
  const int64_t ta = t0 + j * C, tb = min(t0 + (j + 1) * C, t0 + len);
  // Two token buffers in turn (the loop is unrolled by two), each loaded one
  // token ahead: no register copies between steps.
  TokIn ta_in, tb_in;
  load_tok(ta_in, a, ta, h, T);
  for (int64_t t = ta; t < tb; t += 2) {
    if (t + 1 < tb) load_tok(tb_in, a, t + 1, h, T);
    float o8[8];
    rec_step(S, ta_in.k8, ta_in.q8, ta_in.v8, ta_in.a, ta_in.b, o8);
    store_out<OUT_BF16>(a.out, (t * a.H + h) * kD, o8, T);
    if (t + 1 >= tb) break;
    if (t + 2 < tb) load_tok(ta_in, a, t + 2, h, T);
    rec_step(S, tb_in.k8, tb_in.q8, tb_in.v8, tb_in.a, tb_in.b, o8);
    store_out<OUT_BF16>(a.out, ((t + 1) * a.H + h) * kD, o8, T);
  }
  // the open chunk of the last slot continues in decode
  if (a.cache && tb == t0 + len && len % C != 0) {
    const CacheView cv = cache_view(a.cache, s, a.H, C);
    store_state(S, cv.srun + h * plane, T);
    for (int64_t t = ta; t < tb; ++t) {
      const int slot = (int)(t - ta);
      const int64_t r = (t * a.H + h) * kD;
      for (int e = T.tid; e < kD; e += 256) {
        cv.kbuf[((int64_t)slot * a.H + h) * kD + e] = a.kh[r + e];
        cv.vbuf[((int64_t)slot * a.H + h) * kD + e] = bf16_bits_to_f32(a.v[r + e]);
      }
      if (T.tid == 0) {
        cv.abuf[(int64_t)slot * a.H + h] = a.alpha[t * a.H + h];
        cv.bbuf[(int64_t)slot * a.H + h] = a.beta[t * a.H + h];
      }
    }
  }
}

// Decode, part 1: one token per sequence, one workgroup per (sequence, head).
// Wave 0 prepares the token exactly as gdn_prep_kernel does; the recurrence
// step then runs from the cached running state. The token joins the open
// chunk's buffer at slot pos % C.
template <int C, bool OUT_BF16>
__global__ __launch_bounds__(256) void gdn_decode_step_kernel(GdnDecodeArgs a) {
  __shared__ float kq[2][kD];
  __shared__ float ab[2];
  const Tl T = thread_layout();
  const int bseq = blockIdx.x, h = blockIdx.y;
  const int64_t pos = a.pos[bseq];
  const int64_t r = ((int64_t)bseq * a.H + h) * kD;
  if (pos < 0) {  // a data error: NaN output, the cache untouched (uniform exit)
    const float nan8[8] = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                           __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    store_out<OUT_BF16>(a.out, r, nan8, T);
    return;
  }
  const int slot = (int)(pos % C);
  const CacheView cv = cache_view(a.cache, bseq, a.H, C);
  const int64_t plane = (int64_t)kD * kD;
  // the state and v loads go out first, so their latency overlaps the token's preparation
  float S[8][8];
  load_state(S, cv.srun + h * plane, T);
  float k8[8], q8[8], v8[8], o8[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) v8[jj] = bf16_bits_to_f32(a.v[r + 8 * T.tj + jj]);
  if (T.tid < 64) {
    const float2 kk = l2norm_pair(reinterpret_cast<const uint32_t*>(a.k)[r / 2 + T.lane], 1.0f);
    const float2 qq = l2norm_pair(reinterpret_cast<const uint32_t*>(a.q)[r / 2 + T.lane], kInvSqrtD);
    kq[0][2 * T.lane] = kk.x;
    kq[0][2 * T.lane + 1] = kk.y;
    kq[1][2 * T.lane] = qq.x;
    kq[1][2 * T.lane + 1] = qq.y;
    if (T.lane == 0) {
      ab[0] = gate_alpha(a.g[(int64_t)bseq * a.H + h]);
      ab[1] = a.beta[(int64_t)bseq * a.H + h];
    }
  }
  __syncthreads();
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    k8[ii] = kq[0][8 * T.ti + ii];
    q8[ii] = kq[1][8 * T.ti + ii];
  }
  rec_step(S, k8, q8, v8, ab[0], ab[1], o8);
  store_out<OUT_BF16>(a.out, r, o8, T);
  store_state(S, cv.srun + h * plane, T);
  for (int e = T.tid; e < kD; e += 256) {
    cv.kbuf[((int64_t)slot * a.H + h) * kD + e] = kq[0][e];
    cv.vbuf[((int64_t)slot * a.H + h) * kD + e] = bf16_bits_to_f32(a.v[r + e]);
  }
  if (T.tid == 0) {
    cv.abuf[(int64_t)slot * a.H + h] = ab[0];
    cv.bbuf[(int64_t)slot * a.H + h] = ab[1];
  }
}

// Decode, part 2: where the token closed a chunk, the chunk's coefficients
// (one workgroup per (sequence, head)) ...
template <int C>
__global__ __launch_bounds__(256, 2) void gdn_decode_coef_kernel(GdnDecodeArgs a) {
  __shared__ ChunkLds<C> L;
  const Tc T = col_layout();
  const int bseq = blockIdx.x, h = blockIdx.y;
  const int64_t pos = a.pos[bseq];
  if (pos < 0 || (pos + 1) % C != 0) return;  // uniform
  const CacheView cv = cache_view(a.cache, bseq, a.H, C);
  fill_chunk<C>(
      L, T, [&](int t, int i) { return cv.kbuf[((int64_t)t * a.H + h) * kD + i]; },
      [&](int t, float& al, float& be) {
        al = cv.abuf[(int64_t)t * a.H + h];
        be = cv.bbuf[(int64_t)t * a.H + h];
      });
  chunk_coeffs<C>(L, T);
  float* dst = cv.coef + (int64_t)h * (C * C + 2 * C);
  for (int e = T.tid; e < C * C; e += 256) dst[e] = L.MT[e % C][e / C];  // M[t][s], row-major
  if (T.tid < C) {
    dst[C * C + T.tid] = L.gamma[T.tid];
    dst[C * C + C + T.tid] = L.cf[T.tid];
  }
}

// ... then the boundary state advanced by the same chunk_state as the first
// pass (one workgroup per 32 columns, a wave per 16), and the running state
// resynchronised to it.
template <int C>
__global__ __launch_bounds__(64 * kStateWaves) __attribute__((amdgpu_waves_per_eu(2))) void gdn_decode_resync_kernel(GdnDecodeArgs a) {
  __shared__ StateLds<C> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int c0 = kSB * (int)blockIdx.z + kWC * (tid >> 6);
  const int bseq = blockIdx.x, h = blockIdx.y;
  const int64_t pos = a.pos[bseq];
  if (pos < 0 || (pos + 1) % C != 0) return;  // uniform
  const CacheView cv = cache_view(a.cache, bseq, a.H, C);
  const float* coef = cv.coef + (int64_t)h * (C * C + 2 * C);
  const int64_t plane = (int64_t)kD * kD;
  f32x4 S[8];
  load_cols(S, cv.sb + h * plane, c0, lane);
  float v[C / 16][4];
  state_inputs<C>(L, coef, cv.kbuf + (int64_t)h * kD, cv.vbuf + (int64_t)h * kD, (int64_t)a.H * kD, v, tid, c0);
  chunk_state<C>(S, L, v, lane);
  store_cols(S, cv.sb + h * plane, c0, lane);
  store_cols(S, cv.srun + h * plane, c0, lane);
}

}  // namespace

hipError_t launch_gdn_prefill(const GdnArgs& a, int C, bool out_bf16, hipStream_t s) {
  const int64_t TH = a.T * a.H;
  if (TH > 0) {
    hipLaunchKernelGGL(gdn_prep_kernel, dim3(stride_grid(TH, 4)), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(a.q), reinterpret_cast<const uint32_t*>(a.k), a.g, a.qh, a.kh,
                       a.alpha, TH);
  }
  const dim3 gb((unsigned)a.S, (unsigned)a.H, (unsigned)(kD / kSB));
  const dim3 go((unsigned)(a.T / C + a.S), (unsigned)a.H);
  switch (C) {
    case 32:
      hipLaunchKernelGGL(gdn_coef_kernel<32>, go, dim3(256), 0, s, a);
      hipLaunchKernelGGL(gdn_boundary_kernel<32>, gb, dim3(64 * kStateWaves), 0, s, a);
      if (out_bf16) hipLaunchKernelGGL((gdn_output_kernel<32, true>), go, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gdn_output_kernel<32, false>), go, dim3(256), 0, s, a);
      break;
    case 64:
      hipLaunchKernelGGL(gdn_coef_kernel<64>, go, dim3(256), 0, s, a);
      hipLaunchKernelGGL(gdn_boundary_kernel<64>, gb, dim3(64 * kStateWaves), 0, s, a);
      if (out_bf16) hipLaunchKernelGGL((gdn_output_kernel<64, true>), go, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gdn_output_kernel<64, false>), go, dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gdn_decode(const GdnDecodeArgs& a, int C, bool out_bf16, hipStream_t s) {
  const dim3 grid((unsigned)a.B, (unsigned)a.H);
  const dim3 grid_r((unsigned)a.B, (unsigned)a.H, (unsigned)(kD / kSB));
  switch (C) {
    case 32:
      if (out_bf16) hipLaunchKernelGGL((gdn_decode_step_kernel<32, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gdn_decode_step_kernel<32, false>), grid, dim3(256), 0, s, a);
      hipLaunchKernelGGL(gdn_decode_coef_kernel<32>, grid, dim3(256), 0, s, a);
      hipLaunchKernelGGL(gdn_decode_resync_kernel<32>, grid_r, dim3(64 * kStateWaves), 0, s, a);
      break;
    case 64:
      if (out_bf16) hipLaunchKernelGGL((gdn_decode_step_kernel<64, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gdn_decode_step_kernel<64, false>), grid, dim3(256), 0, s, a);
      hipLaunchKernelGGL(gdn_decode_coef_kernel<64>, grid, dim3(256), 0, s, a);
      hipLaunchKernelGGL(gdn_decode_resync_kernel<64>, grid_r, dim3(64 * kStateWaves), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace inv
