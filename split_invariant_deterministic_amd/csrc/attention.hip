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
//     l'    = l * alpha + sum_chunk (p_hi + p_lo)  (per lane: a balanced
//             pairwise tree over a 16-key block's 4 keys, then over the
//             chunk's blocks in ascending order, then xor 16, xor 32)
//     o'    = MFMA chain of P.V over the chunk's 32-key steps, started from
//             o * alpha; per step the p_hi MFMA, then the p_lo MFMA
//   empty splits are (m, l, o) = (-inf, 0, 0).
// The S split states are then merged by the contract's tree with
// m = max(m1,m2), l = l1 f1 + l2 f2, o = o1 f1 + o2 f2 (f = exp2((m_i - m)
// log2e)), and out = bf16(o / l).
//
// One workgroup of NW waves computes one (row, kv head, split) for the whole
// GQA group of query heads (columns of the score MFMA), so a row's bits
// depend only on its q, its visible keys and L: a decode row equals the same
// position's row in a multi-row (prefill) launch, and a batch of one row
// equals its row in a batch of 256. Scores are produced transposed (keys x
// heads): each lane then holds the probabilities of one head, which the P.V
// MFMA takes as its B operand; its A operand is V^T, read back from an LDS
// stage of V with the gfx950 transpose read, holding the same keys in the
// same slots. The output is thus O^T (d x heads), so a lane rescales its
// column by its own head's alpha.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace inv {
namespace {

constexpr int kD = 128;

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

// v + v[lane ^ 16], then that + its value at lane ^ 32: the same two sums as
// two xor shuffles, by the gfx950 row and half swaps (VALU, no LDS round
// trip). Swapping two copies of v leaves each lane holding its own value and
// its partner's, in one order or the other; fp32 addition is commutative, so
// the bits equal the shuffle form. Inline asm with the swap's two wait
// states, because the compiler's builtin for it folds two copies of one value.
__device__ __forceinline__ float xor_sum_16_32(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  v = a + b;
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

// The maximum of a set of values, three at a time by the hardware's
// three-input max. fmaxf would first quiet each operand loaded from LDS (a
// signalling NaN is not a maximum); the values here are scores or maxima of
// scores, so any NaN among them is already quiet. A max over a set does not
// depend on the grouping.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
template <int N>
__device__ __forceinline__ float max_of(const float (&v)[N]) {
  if constexpr (N == 1) {
    return v[0];
  } else {
    constexpr int M = (N + 2) / 3;
    float u[M];
#pragma unroll
    for (int i = 0; i < M; ++i)
      u[i] = vmax3(v[3 * i], v[3 * i + 1 < N ? 3 * i + 1 : 3 * i], v[3 * i + 2 < N ? 3 * i + 2 : 3 * i]);
    return max_of<M>(u);
  }
}

// Two floats rounded to bf16 (nearest even) as one packed word, element 0 in
// the low half.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

// Work split inside the workgroup of NW = 2 NWS waves. The NWS score waves
// load K, compute the scores and probabilities of the chunk's 16-key blocks
// [w KBW, (w+1) KBW) and their part of the probability sum; the first of them
// also keeps the running sum l. The NWS V waves load V and stage it in LDS.
// All waves then multiply P by V for the output's 16-wide d blocks
// [w DBW, (w+1) DBW). Block maxima, the packed probabilities and the sum's
// parts pass through LDS; the chunk loop below is software-pipelined to one
// barrier per chunk. The order of every reduction is that of the schedule
// above, whichever wave holds the operands: the chunk max is a max over the
// same set (exact, and a zero max is made +0), the sum's tree does not depend
// on which wave adds which node, and each output d block sees the schedule's
// MFMA chain. Several waves per item keep the chip busy at decode batches of
// a few rows (16 splits x 8 kv heads are 128 items at one row), where a
// chunk's dependent steps, not the bytes, set the time.
//
// K and V are read through buffer descriptors whose range ends at the chunk's
// last visible key, so keys past L read as zero without a per-lane clamp and
// a chunk's addressing is one scalar base; offsets are 32-bit, so CH keys of
// all kv heads must span less than 2 GiB (checked by the host). V goes
// through registers into a double-buffered LDS stage: every outstanding load
// is then a register load whose count the compiler tracks exactly, and the
// next chunk's loads stay in flight across the exchange reads.
template <int CH>
struct AttnCfg {
  static constexpr int KB = CH / 16;           // 16-key blocks per chunk
  static constexpr int NWS = KB < 4 ? KB : 4;  // score waves: K loads, scores, probabilities
  static constexpr int KBW = KB / NWS;         // 16-key blocks per score wave
  static constexpr int NW = 2 * NWS;           // waves per item: the score waves, then as many V waves
  static constexpr int VLD = CH / 4 / NWS;     // 1 KB (4-key) V loads per V wave per chunk
  static constexpr int DBW = 8 / NW;           // 16-wide output d blocks per wave
  static constexpr int PV = CH / 32;           // 32-key MFMA steps per chunk
  static constexpr int NLD = KBW * 4;          // 16-byte loads per lane per chunk, either role
  static_assert(NLD == VLD, "score and V waves load the same number of registers");
};

template <int CH>
__global__ __launch_bounds__(AttnCfg<CH>::NW * 64) void attn_split_kernel(AttnLaunch a, float scale) {
  using Cfg = AttnCfg<CH>;
  constexpr int NWS = Cfg::NWS, KBW = Cfg::KBW, DBW = Cfg::DBW, VLD = Cfg::VLD, NLD = Cfg::NLD;
  __shared__ __attribute__((aligned(1024))) uint8_t vs[2][CH * kD * 2];
  // per chunk parity, 32-key MFMA step and lane: the P.V operand words, p_hi
  // in pexh and p_lo in pexl (block 2t's two pairs, then block 2t+1's)
  __shared__ u32x4 pexh[2][Cfg::PV][64], pexl[2][Cfg::PV][64];
  __shared__ __attribute__((aligned(16))) float mex[2][16][NWS][4];  // per parity and head: max of each score wave's lane group
  __shared__ float psx[2][NWS][64];  // per parity, score wave and lane: that wave's part of the probability sum

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const bool sw = wave < NWS;             // a score wave (else a V wave)
  const int sv = sw ? wave : wave - NWS;  // its index within its role
  const int g4 = lane >> 4, c16 = lane & 15;
  const int nsplit = a.split_hi - a.split_lo;
  int64_t idx = blockIdx.x;
  const int j = a.split_lo + (int)(idx % nsplit);
  idx /= nsplit;
  const int kvh = (int)(idx % a.Hkv);
  int64_t row = idx / a.Hkv;
  const int grp = a.Hq / a.Hkv;
  const int S = a.split_kv;

  bool valid;
  int64_t start = 0, L = 1;
  if (a.Tq >= 2 && a.Tq <= 64) {
    // A few rows of unequal length: the workgroups take the rows in order of
    // decreasing chunk count (ties by row index), so the longest rows are
    // dispatched first and the launch does not end on a long row that was
    // dispatched last. Which workgroup computes an item does not change its
    // arithmetic. Lane i holds row i's bounds; every wave ranks the rows alike.
    const int nr = (int)a.Tq;
    int si = -1, pi = -1, s0 = 0, len = 0;
    if (lane < nr) {
      si = a.q_seq[lane];
      pi = a.q_pos[lane];
    }
    const bool sok = si >= 0 && si < a.num_seqs;
    if (sok) {
      s0 = a.cu_seqlens[si];
      len = a.cu_seqlens[si + 1] - s0;
    }
    const bool vi = sok && pi >= 0 && pi < len;
    const int ni = vi ? (int)(((int64_t)pi + CH) / CH) : 0;  // chunks of the row's visible keys
    int rank = 0;
    for (int q = 0; q < nr; ++q) {
      const int nq = __builtin_amdgcn_readlane(ni, q);
      rank += (nq > ni || (nq == ni && q < lane)) ? 1 : 0;
    }
    const int r = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < nr && rank == (int)row));
    row = r;
    valid = __builtin_amdgcn_readlane((int)vi, r) != 0;
    start = __builtin_amdgcn_readlane(s0, r);
    L = (int64_t)__builtin_amdgcn_readlane(pi, r) + 1;
  } else {
    const int seq = a.q_seq[row];
    valid = seq >= 0 && seq < a.num_seqs;
    if (valid) {
      start = a.cu_seqlens[seq];
      const int64_t len = (int64_t)a.cu_seqlens[seq + 1] - start;
      const int64_t p = a.q_pos[row];
      valid = p >= 0 && p < len;
      L = p + 1;
    }
  }
  if (!valid) {  // uniform over the block
    if (wave == 0) {
      float* ws = a.ws;
      const int64_t hb = row * a.Hq + (int64_t)kvh * grp;
      for (int h = 0; h < grp; ++h) {
        float* st = ws + ((hb + h) * S + j) * (kD + 2);
        st[lane] = __builtin_nanf("");
        st[lane + 64] = __builtin_nanf("");
        if (lane < 2) st[kD + lane] = __builtin_nanf("");
      }
    }
    return;
  }
  const int64_t n = (L + CH - 1) / CH;
  const int64_t c0 = ((int64_t)j * n) / S, c1 = ((int64_t)(j + 1) * n) / S;

  const int64_t rowB = (int64_t)a.Hkv * kD * 2;  // bytes between consecutive keys
  const uint32_t rb = (uint32_t)rowB;
  const uint8_t* Kh = static_cast<const uint8_t*>(a.k) + (start * a.Hkv + kvh) * (kD * 2);
  const uint8_t* Vh = static_cast<const uint8_t*>(a.v) + (start * a.Hkv + kvh) * (kD * 2);
  // chunk cc of this head's keys, as a range that ends with the chunk's last visible key
  auto chunk_rsrc = [&](const uint8_t* base, int64_t cc) {
    const int64_t rem = L - cc * CH;  // visible keys from the chunk's first (>= 1)
    const uint32_t bytes = rem >= CH ? (uint32_t)(CH * rowB) : (uint32_t)((rem - 1) * rowB + kD * 2);
    return make_rsrc(base + cc * CH * rowB, bytes);
  };

  bf16x8 qf[4];
  if (sw) {
    const bool hv = c16 < grp;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (row * a.Hq + (int64_t)kvh * grp + (hv ? c16 : 0)) * kD;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + ds * 32 + 8 * g4);
      if (!hv) v = u32x4{0u, 0u, 0u, 0u};
      qf[ds] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const int tr_m = (lane & 15) >> 2, tr_q = lane & 3;
  const uint32_t kvo = (uint32_t)c16 * rb + 16u * g4;  // K: key c16 of a block, d = 8 g4 (+ 32 ds)
  const uint32_t vvo = (uint32_t)g4 * rb + 16u * c16;  // V: key g4 of a 4-key group, 16-byte slot c16
  const int vlds = g4 * (kD * 2) + vswz(g4, c16) * 16;  // that slot's place in the stage

  // A score wave's K fragments or a V wave's V rows of one chunk: the same
  // registers and the same number of loads in both roles.
  u32x4 ld[NLD];
  auto load_next = [&](int64_t cc) {
    if (sw) {
      const buf_rsrc r = chunk_rsrc(Kh, cc);
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        const uint32_t so = (uint32_t)((sv * KBW + kb) * 16) * rb;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) ld[kb * 4 + ds] = buf_load16(r, kvo + 64u * ds, so);
      }
    } else {
      const buf_rsrc r = chunk_rsrc(Vh, cc);
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const uint32_t so = (uint32_t)(4 * (sv * VLD + i)) * rb;
        ld[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vvo, so, kNT));
      }
    }
  };
  f32x4 st[KBW];
  auto scores = [&]() {  // score waves: the chunk in ld
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) acc = mfma16(__builtin_bit_cast(bf16x8, ld[kb * 4 + ds]), qf[ds], acc);
      st[kb] = acc;
    }
  };
  auto store_v = [&](int buf) {  // V waves: the chunk in ld into LDS buffer buf
#pragma unroll
    for (int i = 0; i < VLD; ++i) *reinterpret_cast<u32x4*>(&vs[buf][(sv * VLD + i) * 1024 + vlds]) = ld[i];
  };
  // score waves: scaled (and, in a split's last chunk, masked) scores of
  // chunk cc and their maxima per lane group
  auto block_max = [&](int64_t cc, auto last) {
    float bmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = st[kb][r] * scale;
        if constexpr (decltype(last)::value) {  // only a split's last chunk can hold keys past L
          const int64_t pos = cc * CH + (sv * KBW + kb) * 16 + 4 * g4 + r;
          if (pos >= L) s = -INFINITY;
        }
        st[kb][r] = s;
        bmax = fmaxf(bmax, s);
      }
    mex[cc & 1][c16][sv][g4] = bmax;
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[DBW];
#pragma unroll
  for (int db = 0; db < DBW; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // all waves: chunk cc's running max and alpha; score waves: its packed
  // probabilities into pexh / pexl[cc & 1]. Returns alpha.
  auto softmax = [&](int64_t cc) {
    float mv[4 * NWS + 1];  // the NWS x 4 partial maxima of head c16 (read as float4s) and m
    {
      const f32x4* mp = reinterpret_cast<const f32x4*>(&mex[cc & 1][c16][0][0]);
#pragma unroll
      for (int w = 0; w < NWS; ++w) {
        const f32x4 q = mp[w];
#pragma unroll
        for (int i = 0; i < 4; ++i) mv[4 * w + i] = q[i];
      }
      mv[4 * NWS] = m_run;
    }
    const float m_new = max_of(mv) + 0.0f;  // + 0: a zero max is +0 whatever the order
    const float alpha = exp_shifted(m_run, m_new);
    if (sw) {
      float bs[KBW];  // per block: the lane's 4 keys' p_hi + p_lo, summed as a balanced tree
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        uint32_t hw[2], lw[2];  // p_hi and p_lo of keys (0, 1) and (2, 3), packed
        float x[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float p0 = exp_shifted(st[kb][2 * q], m_new), p1 = exp_shifted(st[kb][2 * q + 1], m_new);
          hw[q] = cvt_pk_bf16(p0, p1);
          const float h0 = bf16_lo(hw[q]), h1 = bf16_hi(hw[q]);
          lw[q] = cvt_pk_bf16(p0 - h0, p1 - h1);  // p - p_hi is exact in fp32
          x[2 * q] = h0 + bf16_lo(lw[q]);
          x[2 * q + 1] = h1 + bf16_hi(lw[q]);
        }
        const int blk = sv * KBW + kb;
        reinterpret_cast<u32x2*>(&pexh[cc & 1][blk >> 1][lane])[blk & 1] = u32x2{hw[0], hw[1]};
        reinterpret_cast<u32x2*>(&pexl[cc & 1][blk >> 1][lane])[blk & 1] = u32x2{lw[0], lw[1]};
        bs[kb] = (x[0] + x[1]) + (x[2] + x[3]);
      }
#pragma unroll
      for (int h = 1; h < KBW; h *= 2)  // the wave's adjacent blocks, pairwise
#pragma unroll
        for (int b = 0; b + h < KBW; b += 2 * h) bs[b] = bs[b] + bs[b + h];
      psx[cc & 1][sv][lane] = bs[0];
    }
    m_run = m_new;
    return alpha;
  };
  // all waves: o = o * alpha + P.V over chunk cc for the wave's d blocks;
  // wave 0: l = l * alpha + (the chunk's probability sum)
  auto pv = [&](int64_t cc, float alpha) {
    u32x4 pxh[Cfg::PV], pxl[Cfg::PV];
#pragma unroll
    for (int t = 0; t < Cfg::PV; ++t) {
      pxh[t] = pexh[cc & 1][t][lane];
      pxl[t] = pexl[cc & 1][t][lane];
    }
    float wsum[NWS];
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < NWS; ++w) wsum[w] = psx[cc & 1][w][lane];
    }
    // o is held transposed (d x heads): a lane's column is its own head c16
#pragma unroll
    for (int db = 0; db < DBW; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[db][r] = o[db][r] * alpha;
    const uint8_t* vb = vs[cc & 1];
#pragma unroll
    for (int t = 0; t < Cfg::PV; ++t) {
      // B operand (P^T): head c16, keys {32t + 4 g4 + e} (e < 4) and {32t + 16 + 4 g4 + e - 4}
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pxh[t]);
      const bf16x8 pfl = __builtin_bit_cast(bf16x8, pxl[t]);
      // A operand (V^T): the same keys for d = 16 db + c16, by two transpose reads
      const int k0 = 32 * t + 4 * g4 + tr_m, k1 = k0 + 16;
#pragma unroll
      for (int d = 0; d < DBW; ++d) {
        const int db = wave * DBW + d;
        const int ch = 2 * db + (tr_q >> 1), byte = (tr_q & 1) * 8;
        const s16x4 lo = lds_read_tr16(&vb[k0 * (kD * 2) + vswz(k0, ch) * 16 + byte]);
        const s16x4 hi = lds_read_tr16(&vb[k1 * (kD * 2) + vswz(k1, ch) * 16 + byte]);
        u32x4 vv;
        vv[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1));
        vv[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3));
        vv[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1));
        vv[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, vv);
        o[d] = mfma16(vf, pf, o[d]);   // high parts first,
        o[d] = mfma16(vf, pfl, o[d]);  // then the low parts, in this fixed order
      }
    }
    if (wave == 0) {  // the running sum: the score waves' parts, pairwise, then across lane groups
#pragma unroll
      for (int h = 1; h < NWS; h *= 2)
#pragma unroll
        for (int w = 0; w + h < NWS; w += 2 * h) wsum[w] = wsum[w] + wsum[w + h];
      const float psum = xor_sum_16_32(wsum[0]);
      l_run = l_run * alpha + psum;
    }
  };

  // Software pipeline, one barrier per chunk. Iteration c: the score waves
  // turn chunk c + 1's K into scores and block maxima, then (after the
  // barrier) every wave takes chunk c + 1's max and alpha, the score waves
  // its probabilities, the V waves stage its V, and all waves multiply chunk
  // c's P by its V. The exchange buffers and the V stage alternate by chunk
  // parity; a buffer is rewritten only after the barrier that follows its
  // last reads. Each wave issues the loads of chunk c + 2 as soon as its
  // registers hold nothing of chunk c + 1.
  using T = std::true_type;
  using F = std::false_type;
  float alpha_c = 0.0f;  // alpha of the chunk whose P.V comes next
  if (c0 < c1) {
    load_next(c0);
    if (sw) scores();
    else store_v((int)(c0 & 1));
    if (c0 + 1 < c1) load_next(c0 + 1);
    if (sw) {
      if (c0 + 1 < c1) block_max(c0, F{});
      else block_max(c0, T{});
    }
    __syncthreads();
    alpha_c = softmax(c0);
  }
  auto step = [&](int64_t c, auto has1, auto has2) {
    constexpr bool H1 = decltype(has1)::value, H2 = decltype(has2)::value;
    if constexpr (H1) {
      if (sw) {
        scores();  // chunk c + 1
        if constexpr (H2) load_next(c + 2);
        block_max(c + 1, std::integral_constant<bool, !H2>{});
      }
    }
    __syncthreads();
    if constexpr (H1) {
      if (!sw) {
        store_v((int)((c + 1) & 1));
        if constexpr (H2) load_next(c + 2);
      }
      const float a_next = softmax(c + 1);
      pv(c, alpha_c);
      alpha_c = a_next;
    } else {
      pv(c, alpha_c);
    }
  };
  for (int64_t c = c0; c + 2 < c1; ++c) step(c, T{}, T{});
  if (c0 + 1 < c1) step(c1 - 2, T{}, F{});
  if (c0 < c1) step(c1 - 1, F{}, F{});

  // ---- split state of head c16: o (d = 16 db + 4 g4 + r), m, l
  const int64_t hbase = row * a.Hq + (int64_t)kvh * grp;
  if (c16 < grp) {
    float* st = a.ws + ((hbase + c16) * S + j) * (kD + 2);
#pragma unroll
    for (int d = 0; d < DBW; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(wave * DBW + d) * 16 + 4 * g4 + r] = o[d][r];
    if (wave == 0 && g4 == 0) {
      st[kD] = m_run;
      st[kD + 1] = l_run;
    }
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
  dim3 grid((unsigned)wgs);
  switch (a.kv_chunk) {
    case 32: hipLaunchKernelGGL(attn_split_kernel<32>, grid, dim3(AttnCfg<32>::NW * 64), 0, s, a, scale); break;
    case 64: hipLaunchKernelGGL(attn_split_kernel<64>, grid, dim3(AttnCfg<64>::NW * 64), 0, s, a, scale); break;
    case 128: hipLaunchKernelGGL(attn_split_kernel<128>, grid, dim3(AttnCfg<128>::NW * 64), 0, s, a, scale); break;
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
