// Split-KV attention with a pinned split rule and merge order, for gfx950.
//
// IsoExec blog, "Unified execution contract": the split-KV partition count is
// a pinned constant of the composition. RL-Kernel write-up, section 4: the
// softmax over the visible keys is an LSE reduction whose block maxima, sums
// and merge order must be fixed; section 7 (optional ROCm path): fixed block
// partition, chunk order and rescale-merge order.
//
// Schedule for a query row with L visible keys (depends on L only):
//   keys form chunks of CH from position 0, n = ceil(L / CH) chunks;
//   split j of S owns chunks [floor(j n / S), floor((j+1) n / S));
//   per chunk, in ascending order (online softmax, all fp32):
//     s     = (q . k) * (1/sqrt(D))      q.k: 4 chained MFMAs over d from +0
//     m'    = max(m, max_chunk s)
//     alpha = exp2((m - m') * log2e)
//     p     = exp2((s - m') * log2e), masked keys give 0, split into two
//             bf16 parts p_hi = bf16(p), p_lo = bf16(p - p_hi) so that the
//             P.V MFMAs see p to about 16 bits instead of bf16's 8
//     l'    = l * alpha + sum_chunk (p_hi + p_lo)  (lane sums in (block,
//                                        row) order, then xor 16, 32)
//     o'    = MFMA chain of P.V over the chunk's 32-key steps, started from
//             o * alpha; per step the p_hi MFMA, then the p_lo MFMA
//   empty splits are (m, l, o) = (-inf, 0, 0).
// The S split states are then merged by the contract's tree with
// m = max(m1,m2), l = l1 f1 + l2 f2, o = o1 f1 + o2 f2 (f = exp2((m_i - m)
// log2e)), and out = bf16(o / l).
//
// One wave computes one (row, kv head, split) for the whole GQA group of
// query heads (rows of the MFMA tile), so a row's bits depend only on its q,
// its visible keys and L: a decode row equals the same position's row in a
// multi-row (prefill) launch. Scores are produced transposed (keys x heads):
// each lane then holds the 8 probabilities of one head that the P.V MFMA
// takes as its A operand. V rows go straight from HBM into LDS (direct
// loads) and the P.V B operand is read back transposed with the gfx950
// transpose read, holding the same 8 keys in the same slots.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace inv {
namespace {

constexpr int kD = 128;

template <int CH>
struct AttnCfg {
  static constexpr int KB = CH / 16;        // 16-key blocks per chunk
  static constexpr int PV = CH / 32;        // 32-key MFMA steps per chunk
  static constexpr int ROWB = kD * 2;       // bytes per staged V row (one key)
  static constexpr int VDMA = CH / 4;       // 1 KB (4-key) direct loads per chunk
};

// V rows are staged in LDS in their own layout (key-major, d contiguous),
// 16-byte chunk c of key k stored at chunk c ^ (2 * (k % 4)). The P.V MFMA
// needs V transposed (keys along the operand's k slots); the gfx950
// transpose read ds_read_b64_tr_b16 delivers that: within each 16-lane group
// the 16 four-element reads are concatenated and lane l receives elements
// l, l+16, l+32, l+48, so source lane q + 4m reading 8 bytes of key key0+m at
// d = 16 db + 4q hands lane n the values V[key0 + m][16 db + n], m = 0..3.
// With the swizzle the 16 lanes of a group touch 128 distinct bytes.
__device__ __forceinline__ int vswz(int key, int chunk) { return chunk ^ ((key & 3) << 1); }

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) uint8_t*)p));
#else
  (void)p;
  return s16x4{0, 0, 0, 0};
#endif
}

// s_waitcnt vmcnt(N) (N < 64), expcnt and lgkmcnt not waited on, through
// the builtin: the compiler then knows which loads have landed (in
// particular the direct-to-LDS loads older than the last N), and does not
// add a wait for every outstanding load before the LDS reads that follow.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

template <int CH>
__global__ __launch_bounds__(64) void attn_split_kernel(AttnLaunch a, float scale) {
  using Cfg = AttnCfg<CH>;
  __shared__ __attribute__((aligned(1024))) uint8_t vs[CH * Cfg::ROWB];

  const int lane = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int nsplit = a.split_hi - a.split_lo;
  int64_t idx = blockIdx.x;
  const int j = a.split_lo + (int)(idx % nsplit);
  idx /= nsplit;
  const int kvh = (int)(idx % a.Hkv);
  const int64_t row = idx / a.Hkv;
  const int grp = a.Hq / a.Hkv;
  const int S = a.split_kv;

  // Row indices come from device memory: a sequence id outside [0, num_seqs)
  // or a position outside that sequence makes the row's state NaN (the
  // combine then returns NaN) instead of reading outside the key buffers.
  const int seq = a.q_seq[row];
  bool valid = seq >= 0 && seq < a.num_seqs;
  int64_t start = 0, L = 1;
  if (valid) {
    start = a.cu_seqlens[seq];
    const int64_t len = (int64_t)a.cu_seqlens[seq + 1] - start;
    const int64_t p = a.q_pos[row];
    valid = p >= 0 && p < len;
    L = p + 1;
  }
  if (!valid) {  // uniform over the block (one wave, one row)
    float* ws = a.ws;
    const int64_t hb = row * a.Hq + (int64_t)kvh * grp;
    for (int h = 0; h < grp; ++h) {
      float* st = ws + ((hb + h) * S + j) * (kD + 2);
      st[lane] = __builtin_nanf("");
      st[lane + 64] = __builtin_nanf("");
      if (lane < 2) st[kD + lane] = __builtin_nanf("");
    }
    return;
  }
  const int64_t n = (L + CH - 1) / CH;
  const int64_t c0 = ((int64_t)j * n) / S, c1 = ((int64_t)(j + 1) * n) / S;

  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint8_t* Vb = static_cast<const uint8_t*>(a.v);
  const int64_t kv_row = (int64_t)a.Hkv * kD;  // elements between consecutive keys

  // Q^T as the B operand: column = head c16 of the group, k = d.
  bf16x8 qf[4];
  {
    const bool hv = c16 < grp;
    const uint16_t* qp = Q + (row * a.Hq + (int64_t)kvh * grp + (hv ? c16 : 0)) * kD;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + ds * 32 + 8 * g4);
      if (!hv) v = u32x4{0u, 0u, 0u, 0u};
      qf[ds] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // transpose-read lane roles: source lane s = q + 4m of each 16-lane group
  const int tr_m = (lane & 15) >> 2, tr_q = lane & 3;

  float m_run = -INFINITY, l_run = 0.0f;  // per head c16 (identical in the 4 lanes of a head)
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads of chunk c + 1 are issued while chunk c computes: its K fragments
  // right after the score MFMAs have read chunk c's (same registers), its V
  // rows right after the P.V reads of chunk c's (same LDS buffer). Keys past
  // L read a clamped valid key: score row j of the MFMA below depends only
  // on key row j, and those rows' scores are set to -inf; a clamped V row's
  // p is exactly 0 and its values are finite cache data. K and V are read
  // once per (sequence, kv head, split). V's direct loads (1 KB of whole
  // lines each) stream past the caches; K's fragment loads take 64 bytes of
  // each 128-byte line per instruction, the other half one instruction
  // later, so they keep the default policy and the second half hits.
  bf16x8 kf[Cfg::KB][4];
  auto load_k = [&](int64_t cc) {
#pragma unroll
    for (int kb = 0; kb < Cfg::KB; ++kb) {
      const int64_t pos = min(cc * CH + kb * 16 + c16, L - 1);
      const uint16_t* kp = K + (start + pos) * kv_row + (int64_t)kvh * kD + 8 * g4;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        kf[kb][ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + ds * 32));
    }
  };
  auto load_v = [&](int64_t cc) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int i = 0; i < Cfg::VDMA; ++i) {
      const int key = 4 * i + (lane >> 4);
      const int slot = lane & 15;
      const int64_t pos = min(cc * CH + key, L - 1);
      const uint8_t* src = Vb + ((start + pos) * kv_row + (int64_t)kvh * kD) * 2 + vswz(key, slot) * 16;
      __builtin_amdgcn_global_load_lds(src, &vs[i * 1024], 16, 0, kNT);
    }
#else
    (void)cc;
#endif
  };
  // ---- S^T = K Q^T: lane holds keys kb*16 + 4*g4 + r for head c16
  f32x4 st[Cfg::KB];
  auto scores = [&]() {
    // The fragments pass through an empty asm statement, so that the score
    // MFMAs are not scheduled above the wait that precedes this call.
#pragma unroll
    for (int kb = 0; kb < Cfg::KB; ++kb)
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) asm volatile("" : "+v"(kf[kb][ds]));
#pragma unroll
    for (int kb = 0; kb < Cfg::KB; ++kb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) acc = mfma16(kf[kb][ds], qf[ds], acc);
      st[kb] = acc;
    }
  };
  // The loop is rotated and its last chunk peeled: a chunk with a successor
  // loads that successor's K fragments at its start and its V rows once the
  // P.V reads are done, then turns the fragments into the successor's
  // scores. No register load is then carried across the back edge and the
  // loop body has no branch, so the only waits are the explicit ones below;
  // the compiler otherwise waited for every outstanding load at the loop
  // head, the V rows just prefetched into LDS included.
  if (c0 < c1) {
    load_k(c0);
    load_v(c0);
    wait_vm<Cfg::VDMA>();  // the K fragments, issued before the V rows
    scores();
  }
  auto chunk = [&](int64_t c, auto has_next) {
    constexpr bool MORE = decltype(has_next)::value;
    const int64_t kbase = c * CH;  // position of the chunk's first key
    if constexpr (MORE) load_k(c + 1);
    float cmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < Cfg::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t pos = kbase + kb * 16 + 4 * g4 + r;
        float s = st[kb][r] * scale;
        if (pos >= L) s = -INFINITY;
        st[kb][r] = s;
        cmax = fmaxf(cmax, s);
      }
    cmax = fmaxf(cmax, shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = exp_shifted(m_run, m_new);
    float psum = 0.0f;
    uint32_t pw[Cfg::KB][2];  // bf16 high parts of p, packed pairs
    uint32_t pl[Cfg::KB][2];  // bf16 low parts: p - high, rounded
#pragma unroll
    for (int kb = 0; kb < Cfg::KB; ++kb) {
      float ph[4], plo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp_shifted(st[kb][r], m_new);
        ph[r] = bf16_bits_to_f32(f32_to_bf16_bits(p));
        plo[r] = bf16_bits_to_f32(f32_to_bf16_bits(p - ph[r]));  // p - ph is exact in fp32
        psum = psum + (ph[r] + plo[r]);                          // exact: at most 16 significant bits
      }
      pw[kb][0] = pack_bf16x2(ph[0], ph[1]);
      pw[kb][1] = pack_bf16x2(ph[2], ph[3]);
      pl[kb][0] = pack_bf16x2(plo[0], plo[1]);
      pl[kb][1] = pack_bf16x2(plo[2], plo[3]);
    }
    psum = psum + shfl_xor(psum, 16);
    psum = psum + shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // ---- o = P V, started from o * alpha. Output rows = heads 4*g4 + r.
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((4 * g4 + r) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[db][r] = o[db][r] * al[r];
    // this wave's V rows of chunk c are in LDS once at most the next chunk's
    // K loads (issued after them) are outstanding
    wait_vm<MORE ? Cfg::KB * 4 : 0>();
#pragma unroll
    for (int t = 0; t < Cfg::PV; ++t) {
      // A operand: head c16, keys {32t + 4 g4 + e} (e < 4) and {32t + 16 + 4 g4 + e - 4}
      u32x4 pa, pb;
      pa[0] = pw[2 * t][0];
      pa[1] = pw[2 * t][1];
      pa[2] = pw[2 * t + 1][0];
      pa[3] = pw[2 * t + 1][1];
      pb[0] = pl[2 * t][0];
      pb[1] = pl[2 * t][1];
      pb[2] = pl[2 * t + 1][0];
      pb[3] = pl[2 * t + 1][1];
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pa);
      const bf16x8 pfl = __builtin_bit_cast(bf16x8, pb);
      // B operand: the same keys for d = 16 db + c16, by two transpose reads
      const int k0 = 32 * t + 4 * g4 + tr_m, k1 = k0 + 16;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int ch = 2 * db + (tr_q >> 1), byte = (tr_q & 1) * 8;
        const s16x4 lo = lds_read_tr16(&vs[k0 * Cfg::ROWB + vswz(k0, ch) * 16 + byte]);
        const s16x4 hi = lds_read_tr16(&vs[k1 * Cfg::ROWB + vswz(k1, ch) * 16 + byte]);
        u32x4 vb;
        vb[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
        vb[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
        vb[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
        vb[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, vb);
        o[db] = mfma16(pf, vf, o[db]);   // high parts first,
        o[db] = mfma16(pfl, vf, o[db]);  // then the low parts, in this fixed order
      }
    }
    if constexpr (MORE) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V reads done before the next chunk's rows land
      load_v(c + 1);
      wait_vm<Cfg::VDMA>();  // chunk c + 1's K fragments, issued before its V rows
      scores();
    }
  };
  for (int64_t c = c0; c + 1 < c1; ++c) chunk(c, std::true_type{});
  if (c0 < c1) chunk(c1 - 1, std::false_type{});

  // ---- split state: o (rows = heads 4 g4 + r, col d = 16 db + c16), m, l (head c16)
  float* ws = a.ws;
  const int64_t hbase = row * a.Hq + (int64_t)kvh * grp;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g4 + r;
    if (h < grp) {
      float* st = ws + ((hbase + h) * S + j) * (kD + 2);
#pragma unroll
      for (int db = 0; db < 8; ++db) st[db * 16 + c16] = o[db][r];
    }
  }
  if (g4 == 0 && c16 < grp) {
    float* st = ws + ((hbase + c16) * S + j) * (kD + 2);
    st[kD] = m_run;
    st[kD + 1] = l_run;
  }
}

struct AttnState {
  float m, l, o0, o1;
};

__device__ __forceinline__ AttnState attn_merge(const AttnState& a, const AttnState& b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return a;
  const float fa = exp_shifted(a.m, m);
  const float fb = exp_shifted(b.m, m);
  AttnState r;
  r.m = m;
  r.l = a.l * fa + b.l * fb;
  r.o0 = a.o0 * fa + b.o0 * fb;
  r.o1 = a.o1 * fa + b.o1 * fb;
  return r;
}

// One wave per (row, head); lane owns d = lane and lane + 64.
template <int S, bool FOLD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ ws, uint16_t* __restrict__ out,
                                                           int64_t rows_heads) {
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= rows_heads) return;
  const int lane = threadIdx.x & 63;
  const float* base = ws + rh * S * (kD + 2);
  AttnState st[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const float* p = base + j * (kD + 2);
    st[j] = AttnState{p[kD], p[kD + 1], p[lane], p[lane + 64]};
  }
  AttnState r;
  if constexpr (FOLD) {
    r = st[0];
#pragma unroll
    for (int j = 1; j < S; ++j) r = attn_merge(r, st[j]);
  } else {
#pragma unroll
    for (int w = S; w > 1; w /= 2)
#pragma unroll
      for (int j = 0; j < w / 2; ++j) st[j] = attn_merge(st[2 * j], st[2 * j + 1]);
    r = st[0];
  }
  out[rh * kD + lane] = f32_to_bf16_bits(r.o0 / r.l);
  out[rh * kD + lane + 64] = f32_to_bf16_bits(r.o1 / r.l);
}

template <int S>
hipError_t combine_s(const float* ws, void* out, int64_t rh, bool fold, hipStream_t s) {
  dim3 grid((unsigned)((rh + 3) / 4));
  auto O = static_cast<uint16_t*>(out);
  if (fold) hipLaunchKernelGGL((attn_combine_kernel<S, true>), grid, dim3(256), 0, s, ws, O, rh);
  else hipLaunchKernelGGL((attn_combine_kernel<S, false>), grid, dim3(256), 0, s, ws, O, rh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_splits(const AttnLaunch& a, hipStream_t s) {
  const float scale = 1.0f / __builtin_sqrtf((float)a.D);
  const int64_t wgs = a.Tq * a.Hkv * (int64_t)(a.split_hi - a.split_lo);
  if (wgs <= 0) return hipSuccess;
  dim3 grid((unsigned)wgs), block(64);
  switch (a.kv_chunk) {
    case 32: hipLaunchKernelGGL(attn_split_kernel<32>, grid, block, 0, s, a, scale); break;
    case 64: hipLaunchKernelGGL(attn_split_kernel<64>, grid, block, 0, s, a, scale); break;
    case 128: hipLaunchKernelGGL(attn_split_kernel<128>, grid, block, 0, s, a, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const float* ws, void* out, int64_t Tq, int Hq, int D, int split_kv, bool left_fold,
                               hipStream_t s) {
  (void)D;
  const int64_t rh = Tq * Hq;
  if (rh <= 0) return hipSuccess;
  switch (split_kv) {
    case 1: return combine_s<1>(ws, out, rh, left_fold, s);
    case 2: return combine_s<2>(ws, out, rh, left_fold, s);
    case 4: return combine_s<4>(ws, out, rh, left_fold, s);
    case 8: return combine_s<8>(ws, out, rh, left_fold, s);
    case 16: return combine_s<16>(ws, out, rh, left_fold, s);
    case 32: return combine_s<32>(ws, out, rh, left_fold, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace inv
