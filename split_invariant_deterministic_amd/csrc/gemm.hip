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
// kernels are free to choose tiles by M; padding rows never reach C.
//
// Kernels
//   gemm_ring_kernel    large M: 128 x 128 tile per workgroup of 8 waves,
//                       operands through a deep LDS ring filled by direct
//                       global->LDS loads; the balanced subtree of up to 8
//                       leaves is evaluated in post-order (log2(nl)+1 live
//                       accumulator sets, the last in LDS for 8 leaves).
//   gemm_stream_kernel  small M (<= 64): each wave owns whole leaves of one
//                       16FM x 16 tile and streams its K range straight from
//                       HBM into MFMA fragments; the waves' subtrees are then
//                       combined through LDS with the same balanced tree.
//   tree_combine_kernel fp32 tree over a partial buffer (ranks, leaves).
#include "common.h"
#include "launch.h"

namespace inv {
namespace {

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
  } else if constexpr (NL == 2 && Ctx::kOddLeaves) {
    typename Ctx::Acc right;
    c.leaf_pair(out, right);
    acc_add(out, right);
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
  // logprob-statistics output mode (kOutLP): per row and 16-column block
  float* lp_stats;           // [M, ceil(N/16)] (m, s) pairs
  float* lp_tlogit;          // [M] logit of the row's target column
  const int32_t* lp_target;  // [M]
  // persistent ring launches: tiles blockIdx.x, + gridDim.x, ... below ntiles
  int persist;
  int64_t ntiles;
};

// Output modes of the GEMM kernels: fp32 C, bf16 C, (LM head) no C at all
// but the vocabulary-block statistics of each row and its target's logit, or
// (MoE gate/up, grouped launches) the SwiGLU of each gate column with its up
// column.
constexpr int kOutF32 = 0, kOutBF16 = 1, kOutLP = 2, kOutSwiGLU = 3;

// kOutLP epilogue. A wave's fp32 result block (rows x 16*cols, in the MFMA
// output layout) is transposed through LDS so that lane l holds row l's
// columns; the lane then reduces each 16-column vocabulary block in
// registers (block16_stats) and writes its (m, s), and the target's logit if
// the row's target falls in these columns. t: this wave's LDS scratch of
// rows x STRIDE floats; a row stride of 68 floats (64 columns) or 36 (32
// columns) keeps both the transposing writes and the 16-byte row reads free
// of bank conflicts: 4 * STRIDE / 4 steps through all 16 four-bank groups.
constexpr int kLpStride = 68;

// SWZ: rows of 32 floats whose 16-byte granule g is stored at g ^ (row % 8)
// (the wave's spill slice), so that 8 lanes reading the same granule of 8
// consecutive rows hit distinct banks.
template <int NB, int STRIDE = kLpStride, bool SWZ = false>  // 16-column blocks per row held by the wave; row stride
__device__ __forceinline__ void lp_rows_epilogue(const TileParams& p, const float* t, int64_t row, bool row_ok,
                                                 int64_t col0, int lane) {
  static_assert(!SWZ || STRIDE == 32, "the swizzled layout has 32-float rows");
  const float* mine = t + lane * STRIDE;
  auto at = [&](int col) { return SWZ ? ((((col >> 2) ^ (lane & 7)) << 2) | (col & 3)) : col; };
  const int64_t nb = (p.N + 15) / 16;
  const int32_t tgt = row_ok ? p.lp_target[row] : -1;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t c0 = col0 + 16 * j;
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(mine + at(16 * j + 4 * q));
      v[4 * q] = f.x;
      v[4 * q + 1] = f.y;
      v[4 * q + 2] = f.z;
      v[4 * q + 3] = f.w;
    }
    const int nvalid = (int)min(max(p.N - c0, (int64_t)0), (int64_t)16);
    const MS st = block16_stats(v, nvalid);
    if (row_ok && nvalid > 0) {
      float* d = p.lp_stats + 2 * (row * nb + c0 / 16);
      d[0] = st.m;
      d[1] = st.s;
    }
  }
  if (row_ok && (int64_t)tgt >= col0 && (int64_t)tgt < col0 + 16 * NB && (int64_t)tgt < p.N)
    p.lp_tlogit[row] = mine[at((int)(tgt - col0))];
}

// ---------------------------------------------------------------- ring kernel
//
// Large-M kernel. A workgroup of 8 waves owns a 128 x 128 output tile, each
// wave 64 x 32 (4 x 2 MFMA blocks); at most 256 registers a wave, so a CU
// runs two waves per SIMD and one wave's barrier and LDS waits overlap the
// other's MFMAs. Operands stream through an LDS ring (128 KB; 96 KB for 8
// leaves) of NS stages of BK k (BK = 64; BK = 32 for leaves that are an odd
// multiple of 32), filled by global_load_lds_dwordx4: each wave-wide
// load writes 64 x 16 bytes contiguously at its LDS base, so a stage is laid
// out as rows of BK bf16 with no padding, and the 16-byte chunk c of row r is
// stored at slot c ^ ((r / RPW) % CPR). With that XOR swizzle the 16 lanes
// that read one MFMA operand block (16 rows, same chunk) hit 16 distinct
// 16-byte bank groups. Loads run NS-1 stages ahead of the MFMAs; the only
// waits are an explicit vmcnt/lgkmcnt wait and a plain s_barrier per stage
// (no fence, so prefetches stay in flight across it).
//
// Rows past M and columns past N load a clamped valid row instead of zeros;
// row m of an MFMA result depends only on row m of A (and column n only on
// row n of B), so those rows never touch a stored output.
//
// With 8 leaves (64-k stages) and more tiles than the 256 CUs hold, the
// launch is persistent: workgroup b walks tiles b, b + 256, ...; the next
// tile's addressing is set up before the current tree runs, and the issue
// side of the ring switches to it after the current tile's last stage, so
// the next tile's first stages load while the tree and the epilogue finish.
// The epilogue then transposes through the wave's own spill slice instead
// of the ring. Every output element's chain and tree are the same as in a
// one-tile-per-workgroup launch.

// Waves per ring workgroup: 8 waves, each 64 rows x 32 columns of the
// 128 x 128 tile (4 x 2 MFMA blocks of 16 x 16).
constexpr int kRingWaves = 8;

template <int BK, int RING = 131072, int BM_ = 128>
struct Ring {
  static constexpr int NW = kRingWaves;
  static constexpr int BM = BM_, BN = 128;
  static constexpr int ROWB = BK * 2;          // bytes per staged row
  static constexpr int CPR = BK / 8;           // 16-byte chunks per row
  static constexpr int RPW = 16 / CPR;         // rows per 256-byte bank window
  static constexpr int RPL = 1024 / ROWB;      // rows per wave-wide 1 KB load
  static constexpr int ABYTES = BM * ROWB, BBYTES = BN * ROWB, STAGE = ABYTES + BBYTES;
  static constexpr int LA = ABYTES / (1024 * NW);  // 1 KB loads per wave per stage
  static constexpr int LB = BBYTES / (1024 * NW);
  static constexpr int LOADS = LA + LB;
  static constexpr int NS = RING / STAGE;      // stages in the ring
  static_assert(LA * 1024 * NW == ABYTES && LB * 1024 * NW == BBYTES, "whole 1 KB loads per wave");
  static __device__ __forceinline__ int slot(int r, int c) { return c ^ ((r / RPW) % CPR); }
  static __device__ __forceinline__ int off(int r, int c) { return r * ROWB + (slot(r, c) << 4); }
};

// s_waitcnt vmcnt(n) for n = PER * rem, rem <= R (an immediate operand, hence the recursion)
template <int PER, int R>
__device__ __forceinline__ void wait_vm_only(int rem) {
  if constexpr (R < 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (rem >= R) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER * R) : "memory");
    } else {
      wait_vm_only<PER, R - 1>(rem);
    }
  }
}

// lgkmcnt(0), then vmcnt(PER * rem). The LDS wait goes through the builtin
// on every path, so the compiler knows that every fragment read issued so
// far has landed; with the wait hidden in inline asm it waited again for
// all LDS reads after the barrier, including the next stage's prefetch,
// before the first MFMA of the second k substep. The empty asm keeps
// earlier memory operations from sinking below the wait.
template <int PER, int R>
__device__ __forceinline__ void wait_vm_rem(int rem) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt(63) and expcnt(7) wait for nothing
  wait_vm_only<PER, R>(rem);
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int BK, int RING, bool ODD = false, int BM_ = 128>
struct RingCtx {
  using R = Ring<BK, RING, BM_>;
  static constexpr int NW = R::NW;
  static constexpr int WCOLS = NW / (R::BM / 64);  // waves across the tile's columns
  static constexpr int WN = R::BN / WCOLS;         // wave tile: 64 rows x WN columns
  static constexpr int FN = WN / 16;
  using Acc = AccT<4, FN>;
  static constexpr int USED = R::NS * R::STAGE;  // ring bytes in use
  uint8_t* lds;
  // DMA sources: wave-uniform bases advanced along K, plus per-lane byte
  // offsets fixed for the whole kernel (row * K + 16-byte chunk), so an issue
  // costs scalar adds and the loads take the saddr + voffset form.
  const uint8_t* abase;
  const uint8_t* bbase;
  uint32_t aoff[R::LA];
  uint32_t boff[R::LB];
  int64_t iss_k;  // first k of the next stage to issue
  int iss_off;    // its ring slot (byte offset)
  int issued;     // stages issued so far (over every tile of the workgroup)
  int iss_end;    // issued count at which the issuing tile's stages end
  int limit;      // stages that may be issued: those of the tiles set up so far
  // The next tile's operands (persistent launches): the issue side switches
  // to them at iss_end, so the ring runs on from one tile into the next.
  bool has_next;
  const uint8_t* nabase;
  const uint8_t* nbbase;
  uint32_t naoff[R::LA];
  uint32_t nboff[R::LB];
  int64_t nk0;
  int nstages;
  // Fragment reads: per-lane byte offsets of operand block 0 for k substeps
  // 0 and 1 (block i adds 16 * i rows, an immediate: the swizzle depends on
  // the row only through (row / RPW) % CPR, which 16 rows leave unchanged).
  uint32_t rd_a[BK / 32], rd_b[BK / 32];
  int rd_off;     // ring slot of stage g
  int g;          // next stage to compute (over every tile of the workgroup)
  int spl;        // stages per leaf (ODD: 32-wide substeps per leaf)
  int wave;       // wave-uniform

  // The direct-to-LDS builtin is compiled in the device pass only: seen by the
  // host pass it silently suppresses the host launch stubs of the kernel
  // template's instantiations.
  // Stage issue split in two: the loads are interleaved with the MFMAs of the
  // second k substep (one load per two MFMAs) instead of leaving the barrier
  // as one burst, so the wave never sits in the load queue while its MFMA
  // pipe drains.
  __device__ __forceinline__ void issue_one(int u) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint8_t* dst = lds + iss_off;
    if (u < R::LA)
      __builtin_amdgcn_global_load_lds(abase + iss_k * 2 + aoff[u], &dst[(wave + NW * u) * 1024], 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(bbase + iss_k * 2 + boff[u - R::LA],
                                       &dst[R::ABYTES + (wave + NW * (u - R::LA)) * 1024], 16, 0, 0);
#endif
  }
  // The stage's loads spread evenly over the 4 * F MFMAs of a k substep:
  // before MFMA q go the loads u with ceil(q L / T) <= u < ceil((q+1) L / T)
  // (T = 4F MFMAs, L loads), so the first MFMA always has one before it.
  template <int F>
  __device__ __forceinline__ void issue_before(int q) {
    constexpr int T = 4 * F, L = R::LOADS;
#pragma unroll
    for (int u = (q * L + T - 1) / T; u < ((q + 1) * L + T - 1) / T; ++u) issue_one(u);
  }
  __device__ __forceinline__ void issue_done() {
    iss_k += BK;
    iss_off += R::STAGE;
    if (iss_off == USED) iss_off = 0;
    ++issued;
    if (issued == iss_end && has_next) take_next();  // wave-uniform
  }
  // The issue side moves on to the next tile's operands. Called when the
  // current tile's last stage has been issued and the next tile is set up,
  // whichever of the two comes last: with fewer stages per tile than the
  // ring holds, every stage of a tile can be issued before that tile's own
  // turn in the loop sets up its successor (issued never passes limit,
  // which ends at iss_end until then).
  __device__ __forceinline__ void take_next() {
    abase = nabase;
    bbase = nbbase;
#pragma unroll
    for (int u = 0; u < R::LA; ++u) aoff[u] = naoff[u];
#pragma unroll
    for (int u = 0; u < R::LB; ++u) boff[u] = nboff[u];
    iss_k = nk0;
    iss_end += nstages;
    has_next = false;
  }
  __device__ __forceinline__ void issue_next() {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint8_t* a = abase + iss_k * 2;
    const uint8_t* b = bbase + iss_k * 2;
    uint8_t* dst = lds + iss_off;
#pragma unroll
    for (int u = 0; u < R::LA; ++u)
      __builtin_amdgcn_global_load_lds(a + aoff[u], &dst[(wave + NW * u) * 1024], 16, 0, 0);
#pragma unroll
    for (int u = 0; u < R::LB; ++u)
      __builtin_amdgcn_global_load_lds(b + boff[u], &dst[R::ABYTES + (wave + NW * u) * 1024], 16, 0, 0);
#endif
    issue_done();
  }
  static __device__ __forceinline__ int next_slot(int off) {
    off += R::STAGE;
    return off == USED ? 0 : off;
  }
  __device__ __forceinline__ void read_frags(int slot, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[FN]) {
    const uint8_t* pa = lds + slot + rd_a[ks];
    const uint8_t* pb = lds + slot + rd_b[ks];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(pa + 16 * i * R::ROWB);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(pb + 16 * j * R::ROWB);
  }
  static __device__ __forceinline__ void mma(const bf16x8 (&fa)[4], const bf16x8 (&fb)[FN], Acc& acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc.v[i][j] = mfma16(fa[i], fb[j], acc.v[i][j]);
  }
  // The first MFMA of a leaf: C is the +0 literal rather than a zeroed
  // register set, so no zero set enters the accumulator's loop phi (which
  // made the register allocator rotate accumulators every iteration).
  static __device__ __forceinline__ void mma_first(const bf16x8 (&fa)[4], const bf16x8 (&fb)[FN], Acc& acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc.v[i][j] = mfma16(fa[i], fb[j], f32x4{0.f, 0.f, 0.f, 0.f});
  }

  // BK = 64 keeps the next k-substep's operand fragments in flight while the
  // current substep's 16 MFMAs run: the ks = 0 fragments of a stage are read
  // right after the barrier that publishes it, in the middle of the previous
  // stage, so NS stages are in flight and no LDS read latency is exposed.
  bf16x8 fa0[4], fb0[FN];

  __device__ __forceinline__ void prologue() {
    if constexpr (BK == 64) {
      for (int st = 0; st < R::NS; ++st)
        if (issued < limit) issue_next();
      wait_vm_rem<R::LOADS, R::NS - 1>(issued - 1);
      block_barrier();
      read_frags(rd_off, 0, fa0, fb0);
    } else {
      for (int st = 0; st < R::NS - 1; ++st)
        if (issued < limit) issue_next();
    }
  }

  // One stage of a leaf (BK = 64): ks = 0 from fa0/fb0, ks = 1 read here; in
  // the middle, publish stage g+1 and prefetch its ks = 0 fragments.
  template <bool FIRST>
  __device__ __forceinline__ void stage64(Acc& acc) {
    bf16x8 fa1[4], fb1[FN];
    read_frags(rd_off, 1, fa1, fb1);
    if constexpr (FIRST) mma_first(fa0, fb0, acc);
    else mma(fa0, fb0, acc);
    // Stage g+1 is complete once at most the later stages are outstanding
    // (after the last stage this waits for nothing and the read below
    // fetches a stale slot that is never used: keeping this section
    // unconditional leaves no control-flow merge that would make the
    // compiler drain these reads before the MFMAs that follow).
    wait_vm_rem<R::LOADS, R::NS - 2>(issued - 2 - g);
    block_barrier();  // stage g+1 visible; every wave's reads of stage g are done
    rd_off = next_slot(rd_off);
    read_frags(rd_off, 0, fa0, fb0);
    // MFMAs of substep 1 with the loads of stage g+NS (into stage g's slot)
    // spread between them
    const bool more = issued < limit;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (more) issue_before<FN>(i * FN + j);
        acc.v[i][j] = mfma16(fa1[i], fb1[j], acc.v[i][j]);
      }
    if (more) issue_done();
    ++g;
  }
  // The stages of a tile for a wave whose 64 rows are all padding (the last
  // row tile of a grouped expert): the same waits, barriers and share of the
  // loads as stage64, no fragment reads and no MFMAs, then the ks = 0
  // fragments of the stage that follows (the next tile's first stage64
  // expects them).
  __device__ __forceinline__ void idle_stages(int n) {
    static_assert(BK == 64, "64-k stages");
    for (int st = 0; st < n; ++st) {
      wait_vm_rem<R::LOADS, R::NS - 2>(issued - 2 - g);
      block_barrier();  // stage g+1 visible; every wave's reads of stage g are done
      rd_off = next_slot(rd_off);
      if (issued < limit) issue_next();
      ++g;
    }
    read_frags(rd_off, 0, fa0, fb0);
  }
  template <bool FIRST>
  __device__ __forceinline__ void stage32(Acc& acc) {
    // this thread's loads of stage g are done once at most the loads of
    // the (up to NS-2) later stages already issued are outstanding
    wait_vm_rem<R::LOADS, R::NS - 2>(issued - 1 - g);
    block_barrier();  // every wave's stage g is in LDS; stage g-1 reads are done
    if (issued < limit) issue_next();  // stage g+NS-1, into stage g-1's slot
    bf16x8 fa[4], fb[FN];
    read_frags(rd_off, 0, fa, fb);
    rd_off = next_slot(rd_off);
    if constexpr (FIRST) mma_first(fa, fb, acc);
    else mma(fa, fb, acc);
    ++g;
  }

  // Leaves of an odd number 2m+1 of 32-wide k substeps (kl = 64 m + 32) on
  // 64-k stages. Post-order always runs leaves in pairs (2l, 2l+1), and a pair
  // spans exactly 2m+1 stages: m whole stages of the first leaf, one stage
  // whose k substep 0 ends the first leaf and whose substep 1 starts the
  // second, then m whole stages of the second. The split stage is stage64
  // with the two substeps' MFMAs on different accumulators.
  static constexpr bool kOddLeaves = ODD;
  template <bool AFIRST>
  __device__ __forceinline__ void split_stage(Acc& a, Acc& b) {
    bf16x8 fa1[4], fb1[FN];
    read_frags(rd_off, 1, fa1, fb1);
    if constexpr (AFIRST) mma_first(fa0, fb0, a);
    else mma(fa0, fb0, a);
    wait_vm_rem<R::LOADS, R::NS - 2>(issued - 2 - g);
    block_barrier();  // stage g+1 visible; every wave's reads of stage g are done
    rd_off = next_slot(rd_off);
    read_frags(rd_off, 0, fa0, fb0);
    const bool more = issued < limit;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (more) issue_before<FN>(i * FN + j);
        b.v[i][j] = mfma16(fa1[i], fb1[j], f32x4{0.f, 0.f, 0.f, 0.f});  // the second leaf starts at +0
      }
    if (more) issue_done();
    ++g;
  }
  // Two consecutive leaves (spl = 2m+1 substeps each, m >= 1: leaves of 96,
  // 160, ... k; leaves of exactly 32 run on 32-k stages, see ring_dispatch)
  // into a and b.
  __device__ __forceinline__ void leaf_pair(Acc& a, Acc& b) {
    static_assert(ODD && BK == 64, "odd leaves on 64-k stages");
    const int m = (spl - 1) / 2;
    stage64<true>(a);
#pragma clang loop unroll(disable)
    for (int s = 1; s < m; ++s) stage64<false>(a);
    split_stage<false>(a, b);
#pragma clang loop unroll(disable)
    for (int s = 0; s < m; ++s) stage64<false>(b);
  }

  // One leaf: the chain starts at +0 and takes the leaf's stages in
  // ascending k, each stage as its 32-wide k substeps in ascending order.
  __device__ __forceinline__ void leaf(Acc& acc) {
    static_assert(!ODD, "odd leaves run in pairs (leaf_pair)");
    if constexpr (BK == 64) {
      stage64<true>(acc);
#pragma clang loop unroll(disable)
      for (int s = 1; s < spl; ++s) stage64<false>(acc);
    } else {
      stage32<true>(acc);
#pragma clang loop unroll(disable)
      for (int s = 1; s < spl; ++s) stage32<false>(acc);
    }
  }
};

// With 8 leaves the post-order tree needs four live 64 x 32 accumulator sets
// per wave, more than 256 registers hold next to double-buffered operands;
// the finished left half (leaves 0-3) then waits in LDS (64 KB for the 8
// waves, each lane its own values) while the right half runs in registers,
// and the ring shrinks to 96 KB. The arithmetic is the same tree.
//
// Tiles of 64 rows (M <= 64, 64-k stages): 8 waves side by side, each 64 x 16
// (4 x 1 MFMA blocks). A stage is then 8 KB of A and 16 KB of weights
// instead of 16 + 16 KB, so the same LDS holds twice the weight bytes in
// flight, and no MFMA runs on padding rows. Four 16-register sets hold the
// 8-leaf tree, so there is no spill; the ring takes 5 stages (120 KB) and
// each wave transposes its result through a 5 KB slice of its own, which
// lets every 64-row launch run persistent.
template <int NL, int BM>
constexpr int ring_bytes() { return BM == 64 ? 122880 : NL == 8 ? 98304 : 131072; }

// Position and operand addressing of one output tile of the ring kernel.
template <int LA, int LB>
struct TileAddr {
  int64_t m0, m_end, n0;
  int64_t k0;  // first k of the tile's leaves (64-row tiles)
  int z;       // leaf group, the partial plane of C (64-row tiles)
  const uint8_t* abase;
  const uint8_t* bbase;
  uint32_t aoff[LA];
  uint32_t boff[LB];
};

// ODD: leaves that are an odd multiple of 32 on 64-k stages (NL even, so the
// range is whole stages).
// BM: tile rows, 128 or 64. A 64-row launch folds the leaf groups into the
// tile index (tile = group * tiles + position), so that it can run
// persistent over all of them.
template <int NL, int BK, int OUTM, bool GROUPED, bool ODD = false, int BM = 128>
__global__ __launch_bounds__(64 * kRingWaves, 1) void gemm_ring_kernel(TileParams p) {
  static_assert(BM == 128 || (BM == 64 && BK == 64 && !ODD && !GROUPED), "64-row tiles: plain launches, 64-k stages");
  constexpr int RING = ring_bytes<NL, BM>();
  constexpr int SPILL = BM == 128 && NL == 8 ? 65536 : 0;
  using R = Ring<BK, RING, BM>;
  using Ctx = RingCtx<BK, RING, ODD, BM>;
  static_assert(!ODD || (BK == 64 && NL % 2 == 0), "odd leaves pair up into 64-k stages");
  constexpr int NW = Ctx::NW, WN = Ctx::WN, FN = Ctx::FN;
  constexpr int LPS = WN + 4;  // row stride of the transposed tile (floats)
  // 64-row tiles: each wave's own transpose slice after the ring
  constexpr int EPI = BM == 64 ? NW * 64 * LPS * 4 : 0;
  constexpr int LP_BYTES = OUTM == kOutLP ? NW * 64 * LPS * 4 : 0;
  constexpr int LDS_USED = R::NS * R::STAGE + SPILL + EPI;
  constexpr int LDS_BYTES = LDS_USED > LP_BYTES ? LDS_USED : LP_BYTES;
  static_assert(LDS_BYTES <= 163840, "160 KB of LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
  // Persistent launches take several tiles per workgroup and let the ring
  // run on into the next tile's stages (8 leaves on 64-k stages, odd
  // multiples of 32 included; every 64-row launch).
  constexpr bool PERSIST_OK = (NL == 8 && BK == 64) || BM == 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // Fused SwiGLU: B holds [gate; up] rows (N = 2F). A tile's 128 B rows
  // alternate 16 gate rows and the 16 matching up rows, so each tile covers
  // 64 output columns of A [M, F] and every wave's two 16-column blocks are
  // a gate block and its up block: the SwiGLU needs no exchange.
  constexpr bool SWI = OUTM == kOutSwiGLU;
  static_assert(!SWI || GROUPED, "the fused SwiGLU runs on grouped launches");
  constexpr int TN = SWI ? R::BN / 2 : R::BN;  // output columns per tile
  const int64_t NC = SWI ? p.N / 2 : p.N;      // output columns
  const int tiles_n = (int)((NC + TN - 1) / TN);
  // Tile position and operand addressing: blockIdx.x for a plain launch,
  // tiles blockIdx.x, + gridDim.x, ... for a persistent one. False for a
  // grouped slot past the last tile.
  const uint8_t* A8 = reinterpret_cast<const uint8_t*>(p.A);
  const int cw = __builtin_amdgcn_readfirstlane(wave);
  auto setup = [&](int64_t tile, TileAddr<R::LA, R::LB>& T) -> bool {
    // An opaque copy of the lane id: without it the compiler hoists every
    // lane-only term of the set-up and the epilogue out of the tile loop and
    // keeps them live through the tree (30-60 registers; the grouped fp32
    // kernel spilled).
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    int64_t m0, m_end, n0;
    int z = blockIdx.z;
    const uint16_t* B = p.B;
    if constexpr (GROUPED) {
     if (p.E <= 128) {
      // XCD-aware order over the real tiles: items are (expert, column tile,
      // row tile) in that order (column-major inside an expert), and XCD x
      // (workgroups are dealt round-robin to the 8 XCDs) takes the contiguous
      // eighth [x I / 8, (x+1) I / 8) of the I items, its workgroups walking it
      // in order. Workgroups resident on one XCD at a time then share an
      // expert's weight panels and its gathered row tiles in their L2.
      // The experts' row-tile counts are prefix-summed across the wave (lane
      // l holds experts l and l + 64; temporaries of the set-up only: kept
      // across the tile loop they cost the main loop 30 registers).
      int gt_incl[2], running = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ee = 64 * h + lane;
        int nt = 0;
        if (ee < p.E) {  // offsets come from device memory: clamped into [0, M]
          const int a0 = (int)min(max((int64_t)p.offsets[ee], (int64_t)0), p.M);
          const int a1 = (int)min(max((int64_t)p.offsets[ee + 1], (int64_t)a0), p.M);
          nt = (a1 - a0 + R::BM - 1) / R::BM;
        }
        int incl = nt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_up(incl, off, 64);
          if (lane >= off) incl += v;
        }
        incl += running;
        running = __shfl(incl, 63, 64);
        gt_incl[h] = incl;
      }
      const int64_t I = (int64_t)__builtin_amdgcn_readfirstlane(running) * tiles_n;
      const int x = (int)(tile % 8);
      const int64_t item = x * I / 8 + tile / 8;
      if (item >= (x + 1) * I / 8) return false;  // past this XCD's range (uniform)
      // item < incl * tiles_n <=> item / tiles_n < incl (incl * tiles_n is a multiple of tiles_n)
      const int iq = (int)(item / tiles_n);
      int e = -1, incl = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (e >= 0) continue;  // uniform
        const uint64_t hit = __ballot(64 * h + lane < p.E && iq < gt_incl[h]);
        if (hit) {
          const int f = __ffsll((unsigned long long)hit) - 1;
          e = 64 * h + f;
          incl = __shfl(gt_incl[h], f, 64);
        }
      }
      if (e < 0) return false;
      e = __builtin_amdgcn_readfirstlane(e);
      // the expert's rows, clamped as when the counts were taken
      const int r0 = (int)min(max((int64_t)p.offsets[e], (int64_t)0), p.M);
      const int r1 = (int)min(max((int64_t)p.offsets[e + 1], (int64_t)r0), p.M);
      const int nt = (r1 - r0 + R::BM - 1) / R::BM;
      const int excl = __builtin_amdgcn_readfirstlane(incl) - nt;
      const int64_t local = item - (int64_t)excl * tiles_n;
      n0 = (local / nt) * TN;
      m0 = r0 + (local % nt) * R::BM;
      m_end = r1;
      B += (int64_t)e * p.b_expert_stride;
     } else {
      // more than 128 experts: slot -> (expert, rows), experts owning
      // consecutive runs of ceil(count_e / BM) row tiles in expert order,
      // every row tile spanning all column tiles
      const int t = (int)(tile / tiles_n);
      n0 = (int64_t)(tile % tiles_n) * TN;
      // The tile counts are prefix-summed 64 experts at a time across the
      // wave (two loads per lane, integer shuffles) and the owner found by a
      // ballot, instead of a serial walk over every expert's offsets.
      // Offsets come from device memory: clamp so a malformed table can never
      // address rows outside [0, M).
      int e = -1, tstart = 0, r0 = 0, r1 = 0, running = 0;
      for (int cbase = 0; cbase < p.E && e < 0; cbase += 64) {
        const int ee = cbase + lane;
        int a0 = 0, a1 = 0, nt = 0;
        if (ee < p.E) {
          a0 = (int)min(max((int64_t)p.offsets[ee], (int64_t)0), p.M);
          a1 = (int)min(max((int64_t)p.offsets[ee + 1], (int64_t)a0), p.M);
          nt = (a1 - a0 + R::BM - 1) / R::BM;
        }
        int incl = nt;
  #pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_up(incl, off, 64);
          if (lane >= off) incl += v;
        }
        incl += running;
        const uint64_t hit = __ballot(ee < p.E && t < incl);
        if (hit) {  // wave-uniform
          const int f = __ffsll((unsigned long long)hit) - 1;
          e = cbase + f;
          tstart = __shfl(incl - nt, f, 64);
          r0 = __shfl(a0, f, 64);
          r1 = __shfl(a1, f, 64);
        } else {
          running = __shfl(incl, 63, 64);
        }
      }
      if (e < 0) return false;  // slot past the last tile (uniform)
      m0 = r0 + (int64_t)(t - tstart) * R::BM;
      m_end = r1;
      B += (int64_t)e * p.b_expert_stride;
     }
    } else {
      // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
      // give XCD x a contiguous run of tile ids, and walk tile ids in bands
      // of 4 row tiles so that the workgroups resident on one XCD share A and
      // B panels in its L2.
      const int tiles_m = (int)((p.M + R::BM - 1) / R::BM);
      const int nb = tiles_m * tiles_n;
      if constexpr (BM == 64) {
        z = (int)(tile / nb);
        tile -= (int64_t)z * nb;
      }
      int t = (int)tile;
      if (nb % 8 == 0) t = (t % 8) * (nb / 8) + t / 8;
      constexpr int GM = 4;
      const int band = t / (GM * tiles_n);
      const int rows_in_band = min(GM, tiles_m - band * GM);
      const int within = t - band * GM * tiles_n;
      const int tm = band * GM + within % rows_in_band;
      const int tn = within / rows_in_band;
      m0 = (int64_t)tm * R::BM;
      n0 = (int64_t)tn * R::BN;
      m_end = p.M;
    }
    // A rows: contiguous from m0, or gathered (offsets then from A itself)
    T.abase = (GROUPED && p.rows) ? A8 : A8 + m0 * p.K * 2;
    T.bbase = reinterpret_cast<const uint8_t*>(SWI ? B : B + n0 * p.K);
  #pragma unroll
    for (int u = 0; u < R::LA; ++u) {
      const int r = (cw + NW * u) * R::RPL + lane / R::CPR;
      const int chunk = R::slot(r, lane % R::CPR);  // the slot map is its own inverse
      int64_t row = min(m0 + r, m_end - 1);
      int64_t rel = row - m0;
      if constexpr (GROUPED) {
        if (p.rows) {
          const int64_t gr = p.rows[row];
          rel = (gr >= 0 && gr < p.a_rows) ? gr : 0;
        }
      }
      T.aoff[u] = (uint32_t)((rel * p.K + chunk * 8) * 2);
    }
  #pragma unroll
    for (int u = 0; u < R::LB; ++u) {
      const int r = (cw + NW * u) * R::RPL + lane / R::CPR;
      const int chunk = R::slot(r, lane % R::CPR);
      int64_t brow;  // B row relative to bbase
      if constexpr (SWI) brow = ((r >> 4) & 1) * NC + min(n0 + 16 * (r >> 5) + (r & 15), NC - 1);
      else brow = min(n0 + r, p.N - 1) - n0;
      T.boff[u] = (uint32_t)((brow * p.K + chunk * 8) * 2);
    }
    T.m0 = m0;
    T.m_end = m_end;
    T.n0 = n0;
    T.z = z;
    T.k0 = (int64_t)(p.leaf_lo + z * NL) * p.kl;
    return true;
  };
  TileAddr<R::LA, R::LB> cur;
  int64_t tile = blockIdx.x;
  if (!setup(tile, cur)) return;  // uniform exit before any barrier
  // 128-row tiles: one leaf group per launch row (blockIdx.z), the same for
  // every tile of the workgroup
  const int zg = blockIdx.z;
  const int64_t kg = (int64_t)(p.leaf_lo + zg * NL) * p.kl;

  Ctx c;
  c.lds = lds;
  c.wave = __builtin_amdgcn_readfirstlane(wave);
  c.iss_off = 0;
  c.issued = 0;
  c.rd_off = 0;
  c.spl = ODD ? p.kl / 32 : p.kl / BK;
  c.g = 0;
  const int wm = c.wave / Ctx::WCOLS, wn = c.wave % Ctx::WCOLS;  // wave tile (row, column) in the tile
  {
    const int g4 = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      c.rd_a[ks] = R::off(wm * 64 + r16, 4 * ks + g4);
      c.rd_b[ks] = R::ABYTES + R::off(wn * WN + r16, 4 * ks + g4);
    }
  }
  const int stages = ODD ? NL * p.kl / 64 : c.spl * NL;  // per tile
  c.abase = cur.abase;
  c.bbase = cur.bbase;
#pragma unroll
  for (int u = 0; u < R::LA; ++u) c.aoff[u] = cur.aoff[u];
#pragma unroll
  for (int u = 0; u < R::LB; ++u) c.boff[u] = cur.boff[u];
  c.iss_k = BM == 64 ? cur.k0 : kg;
  c.iss_end = stages;
  c.limit = stages;
  c.has_next = false;
  c.prologue();

  // Epilogue: lane holds rows 4*(lane/16)+r of each 16x16 block, column lane%16.
  auto finish = [&](const TileAddr<R::LA, R::LB>& T, typename Ctx::Acc& acc) {
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    const int z = BM == 64 ? T.z : zg;
    const int64_t rbase = T.m0 + wm * 64 + 4 * (lane >> 4);
    const int64_t cbase = T.n0 + wn * WN + (lane & 15);
    if constexpr (SWI) {
      // Block 0 of the wave is gate, block 1 the matching up columns: both are
      // rounded to bf16 as the unfused GEMM would store them, then the
      // wave stores bf16(silu_mul(g, u)). A malformed gather row is NaN in both
      // halves, as in the unfused path.
      static_assert(FN == 2, "one gate and one up block per wave");
      uint16_t* Ao = reinterpret_cast<uint16_t*>(p.C);
      const int64_t col0 = T.n0 + 16 * wn;  // the wave's 16 output columns
      if constexpr (SPILL > 0) {
        // Whole 16-byte row pieces (8 columns) when the strip is inside A and
        // rows are 16-byte aligned: the 64 x 16 results go through the wave's
        // own spill slice (free once the tree is summed, touched by no other
        // wave), then each lane stores 8 consecutive columns of one row.
        if (col0 + 16 <= NC && NC % 8 == 0 && (reinterpret_cast<uintptr_t>(Ao) & 15u) == 0) {
          uint16_t* t = reinterpret_cast<uint16_t*>(&lds[R::NS * R::STAGE]) + wave * 64 * WN * 2;
  #pragma unroll
          for (int i = 0; i < 4; ++i)
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float g = bf16_bits_to_f32(f32_to_bf16_bits(acc.v[i][0][r]));
              const float u = bf16_bits_to_f32(f32_to_bf16_bits(acc.v[i][1][r]));
              t[(16 * i + 4 * (lane >> 4) + r) * 16 + (lane & 15)] = f32_to_bf16_bits(silu_mul(g, u));
            }
          // the row value of a malformed gather row, computed at run time on
          // the same inputs as the unfused path (not folded by the compiler)
          float qg = __builtin_nanf(""), qu = __builtin_nanf("");
          asm volatile("" : "+v"(qg), "+v"(qu));
          qg = bf16_bits_to_f32(f32_to_bf16_bits(qg));
          qu = bf16_bits_to_f32(f32_to_bf16_bits(qu));
          const uint16_t nanv = f32_to_bf16_bits(silu_mul(qg, qu));
          const uint32_t nan2 = (uint32_t)nanv | ((uint32_t)nanv << 16);
  #pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int rl = 32 * q + (lane >> 1), cs = 8 * (lane & 1);
            const int64_t row = T.m0 + wm * 64 + rl;
            if (row >= T.m_end) continue;
            bool bad = false;
            if (p.rows) {
              const int64_t gr = p.rows[row];
              bad = gr < 0 || gr >= p.a_rows;
            }
            const u32x4 v = bad ? u32x4{nan2, nan2, nan2, nan2} : *reinterpret_cast<const u32x4*>(&t[rl * 16 + cs]);
            *reinterpret_cast<u32x4*>(Ao + row * NC + col0 + cs) = v;
          }
          return;
        }
      }
      const int64_t col = col0 + (lane & 15);
  #pragma unroll
      for (int i = 0; i < 4; ++i)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = rbase + 16 * i + r;
          if (row >= T.m_end || col >= NC) continue;
          bool bad = false;
          if (p.rows) {
            const int64_t gr = p.rows[row];
            bad = gr < 0 || gr >= p.a_rows;
          }
          const float g = bf16_bits_to_f32(f32_to_bf16_bits(bad ? __builtin_nanf("") : acc.v[i][0][r]));
          const float u = bf16_bits_to_f32(f32_to_bf16_bits(bad ? __builtin_nanf("") : acc.v[i][1][r]));
          Ao[row * NC + col] = f32_to_bf16_bits(silu_mul(g, u));
        }
      return;
    }
    if constexpr (OUTM == kOutLP) {
      const int64_t row = T.m0 + wm * 64 + lane;
      if constexpr (SPILL > 0) {
        // the wave's own spill slice, 64 rows of 32 floats, granules swizzled
        // by the row (free once the tree is summed; no barrier)
        static_assert(WN == 32, "32-float rows");
        float* t = reinterpret_cast<float*>(&lds[R::NS * R::STAGE]) + wave * 64 * WN;
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int j = 0; j < FN; ++j)
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int rr = 16 * i + 4 * (lane >> 4) + r, col = 16 * j + (lane & 15);
              t[rr * 32 + ((((col >> 2) ^ (rr & 7)) << 2) | (col & 3))] = acc.v[i][j][r];
            }
        lp_rows_epilogue<FN, 32, true>(p, t, row, row < T.m_end, T.n0 + wn * WN, lane);
      } else {
        // 64-row tiles: the wave's own slice after the ring; else the ring,
        // once every wave has consumed its last stage
        if constexpr (EPI == 0) block_barrier();
        float* t = reinterpret_cast<float*>(lds + (EPI > 0 ? R::NS * R::STAGE : 0)) + wave * 64 * LPS;
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int j = 0; j < FN; ++j)
  #pragma unroll
            for (int r = 0; r < 4; ++r) t[(16 * i + 4 * (lane >> 4) + r) * LPS + 16 * j + (lane & 15)] = acc.v[i][j][r];
        // the wave reads back only what it wrote; its LDS accesses complete in order
        lp_rows_epilogue<FN, LPS>(p, t, row, row < T.m_end, T.n0 + wn * WN, lane);
      }
      return;
    }
    if constexpr (OUTM == kOutBF16 || OUTM == kOutF32) {
      // Whole 16-byte row segments when the wave's column strip is inside C and
      // rows are 16-byte aligned: the block is transposed through LDS (the
      // layout of the statistics epilogue above), then each lane stores 8 bf16
      // or 4 fp32 consecutive columns of one row at once; a wave writes 64- or
      // 128-byte row pieces instead of single elements. fp32 output (LM-head
      // logits, the MoE down projection's rows: read once, by a later pass) is
      // streamed. A malformed gather row is NaN, as below.
      constexpr int EB = OUTM == kOutBF16 ? 2 : 4;  // bytes per element
      constexpr int EPS = 16 / EB;                  // elements per 16-byte segment
      const bool whole = T.n0 + wn * WN + WN <= p.N && p.N % EPS == 0 &&
                         ((reinterpret_cast<uintptr_t>(p.C) | (uintptr_t)(z * p.c_group_stride * EB)) & 15u) == 0;
      // Transpose space: with 8 leaves the wave's own spill slice (64 x WN
      // floats, free once the tree is summed, touched by no other wave; in a
      // persistent launch the ring already holds the next tile's stages), else
      // the ring once every wave has left it.
      // (64-row tiles: the wave's own slice after the ring)
      constexpr int LPX = SPILL > 0 ? WN : LPS;
      if constexpr (SPILL == 0 && EPI == 0) block_barrier();  // every wave has consumed its last ring stage
      if (whole) {
        float* t = SPILL > 0 ? reinterpret_cast<float*>(&lds[R::NS * R::STAGE]) + wave * 64 * WN
                             : reinterpret_cast<float*>(lds + (EPI > 0 ? R::NS * R::STAGE : 0)) + wave * 64 * LPS;
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int j = 0; j < FN; ++j)
  #pragma unroll
            for (int r = 0; r < 4; ++r) t[(16 * i + 4 * (lane >> 4) + r) * LPX + 16 * j + (lane & 15)] = acc.v[i][j][r];
        // the wave reads back only what it wrote; its LDS accesses complete in order
        constexpr int SEG = WN / EPS;    // segments per row
        constexpr int RPI = 64 / SEG;    // rows per pass of the wave
  #pragma unroll
        for (int q = 0; q < 64 / RPI; ++q) {
          const int rl = q * RPI + lane / SEG, cs = EPS * (lane % SEG);
          const int64_t row = T.m0 + wm * 64 + rl;
          const int64_t off = z * p.c_group_stride + row * p.N + T.n0 + wn * WN + cs;
          bool bad = false;
          if constexpr (GROUPED) {
            if (row < T.m_end && p.rows) {
              const int64_t gr = p.rows[row];
              bad = gr < 0 || gr >= p.a_rows;
            }
          }
          const f32x4 nan4 = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
          const f32x4 a0 = bad ? nan4 : *reinterpret_cast<const f32x4*>(&t[rl * LPX + cs]);
          if constexpr (OUTM == kOutBF16) {
            const f32x4 a1 = bad ? nan4 : *reinterpret_cast<const f32x4*>(&t[rl * LPX + cs + 4]);
            const u32x4 o = u32x4{pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]), pack_bf16x2(a1[0], a1[1]),
                                  pack_bf16x2(a1[2], a1[3])};
            if (row < T.m_end) *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.C) + off) = o;
          } else {
            if (row < T.m_end) __builtin_nontemporal_store(a0, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + off));
          }
        }
        return;
      }
    }
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = rbase + 16 * i + r;
        if (row >= T.m_end) continue;
        bool bad = false;
        if constexpr (GROUPED) {
          if (p.rows) {
            const int64_t gr = p.rows[row];
            bad = gr < 0 || gr >= p.a_rows;  // a malformed gather index gives a NaN row
          }
        }
  #pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t col = cbase + 16 * j;
          if (col < p.N) {
            const int64_t off = (int64_t)z * p.c_group_stride + row * p.N + col;
            const float v = bad ? __builtin_nanf("") : acc.v[i][j][r];
            if constexpr (OUTM == kOutBF16)
              reinterpret_cast<uint16_t*>(p.C)[off] = f32_to_bf16_bits(v);
            else
              // streamed: fp32 outputs (LM-head logits, the MoE down projection's
              // rows) are read once, by a later pass
              __builtin_nontemporal_store(v, reinterpret_cast<float*>(p.C) + off);
          }
        }
      }
  };

  for (;;) {
    // the next tile is set up first, so that its stages follow this tile's
    // in the ring
    TileAddr<R::LA, R::LB> nx;
    bool more_tiles = false;
    const int64_t tn = tile + gridDim.x;
    if constexpr (PERSIST_OK) {
      if (p.persist && tn < p.ntiles && setup(tn, nx)) {
        more_tiles = true;
        c.nabase = nx.abase;
        c.nbbase = nx.bbase;
#pragma unroll
        for (int u = 0; u < R::LA; ++u) c.naoff[u] = nx.aoff[u];
#pragma unroll
        for (int u = 0; u < R::LB; ++u) c.nboff[u] = nx.boff[u];
        c.nk0 = BM == 64 ? nx.k0 : kg;
        c.nstages = stages;
        c.has_next = true;
        c.limit += stages;
        if (c.issued == c.iss_end) c.take_next();  // this tile's stages were all issued already
      }
    }
    // All 64 rows of this wave past the expert's last row (grouped launches):
    // the wave keeps the ring's waits, barriers and loads and skips the
    // MFMAs, the tree and the epilogue (which would store nothing). Halves
    // the LDS reads and MFMAs of a tile with 64 valid rows or fewer.
    bool idle = false;
    if constexpr (GROUPED && SPILL > 0 && BK == 64)
      idle = __builtin_amdgcn_readfirstlane((int)(cur.m0 + wm * 64 >= cur.m_end)) != 0;
    if (idle) {
      if constexpr (GROUPED && SPILL > 0 && BK == 64) c.idle_stages(stages);
    } else {
      typename Ctx::Acc acc;
      if constexpr (SPILL > 0) {
        float* spill = reinterpret_cast<float*>(&lds[R::NS * R::STAGE]) + wave * 64 * WN + lane;
        run_tree<4>(c, acc);
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int j = 0; j < FN; ++j)
  #pragma unroll
            for (int r = 0; r < 4; ++r) spill[((i * FN + j) * 4 + r) * 64] = acc.v[i][j][r];
        run_tree<4>(c, acc);
  #pragma unroll
        for (int i = 0; i < 4; ++i)
  #pragma unroll
          for (int j = 0; j < FN; ++j)
  #pragma unroll
            for (int r = 0; r < 4; ++r) acc.v[i][j][r] = spill[((i * FN + j) * 4 + r) * 64] + acc.v[i][j][r];
      } else {
        run_tree<NL>(c, acc);
      }
      finish(cur, acc);
    }
    if (!more_tiles) break;
    cur = nx;
    tile = tn;
  }
}

// -------------------------------------------------------------- stream kernel

template <int FM>
struct StreamCtx {
  using Acc = AccT<FM, 1>;
  // Operands through buffer descriptors: ra covers the tile's valid A rows,
  // rb its valid B rows. A lane's row offset (voa, vob) is fixed; the k
  // position is a wave-uniform byte offset, so a ring slot costs no address
  // registers. Rows past M (columns past N) are clamped to the tile's first
  // row: output element (i, j) depends only on A row i and B row j, and such
  // rows and columns are never stored. No select on loaded data, so loads
  // stay in flight.
  buf_rsrc ra, rb;
  uint32_t voa[FM];
  uint32_t vob;
  uint32_t kb;  // byte offset of this wave's leaf start (wave-uniform)
  int spl;      // 32-k blocks per leaf

  // blocks `base` (uniform, runtime) + d (compile time) of the leaf
  __device__ __forceinline__ void load(uint32_t base, int d, bf16x8 (&a)[FM], bf16x8& b) {
    const uint32_t soff = kb + 64u * base;
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = __builtin_bit_cast(bf16x8, buf_load16(ra, voa[i] + 64u * d, soff));
    b = __builtin_bit_cast(bf16x8, buf_load16(rb, vob + 64u * d, soff));
  }
  __device__ __forceinline__ void mma(const bf16x8 (&a)[FM], const bf16x8& b, Acc& acc) {
#pragma unroll
    for (int i = 0; i < FM; ++i) acc.v[i][0] = mfma16(a[i], b, acc.v[i][0]);
  }
  __device__ __forceinline__ void mma_first(const bf16x8 (&a)[FM], const bf16x8& b, Acc& acc) {
#pragma unroll
    for (int i = 0; i < FM; ++i) acc.v[i][0] = mfma16(a[i], b, f32x4{0.f, 0.f, 0.f, 0.f});
  }
  // One leaf, spl a multiple of DD: a ring of DD blocks in registers, each
  // slot refilled right after its MFMA. Slots are static and the loop body
  // has no branches, so DD blocks stay in flight. The chain is the plain
  // ascending k of the leaf whatever DD is.
  template <int DD>
  __device__ __forceinline__ void leaf_ring(Acc& acc) {
    bf16x8 a[DD][FM], b[DD];
#pragma unroll
    for (int d = 0; d < DD; ++d) load(0, d, a[d], b[d]);
    if (spl == DD) {
      mma_first(a[0], b[0], acc);
#pragma unroll
      for (int d = 1; d < DD; ++d) mma(a[d], b[d], acc);
      return;
    }
    mma_first(a[0], b[0], acc);
    load(DD, 0, a[0], b[0]);
#pragma unroll
    for (int d = 1; d < DD; ++d) {
      mma(a[d], b[d], acc);
      load(DD, d, a[d], b[d]);
    }
#pragma clang loop unroll(disable)
    for (int s = DD; s + DD < spl; s += DD) {
#pragma unroll
      for (int d = 0; d < DD; ++d) {
        mma(a[d], b[d], acc);
        load((uint32_t)(s + DD), d, a[d], b[d]);
      }
    }
#pragma unroll
    for (int d = 0; d < DD; ++d) mma(a[d], b[d], acc);
  }
  // Ring depth: the weight bytes in flight over the grid are
  // N/16 * leaves * depth KiB whatever FM is, so the ring is as deep as the
  // registers allow: up to 8 blocks for 16-32 rows, 4 for 48-64, the largest
  // power of two that divides spl. A single 16-row block with leaves of 32
  // blocks or more (few, long-lived waves) takes 16: the rotated
  // 4096-12288-4096 pair at M = 1 and 7 gains about 2.4 %, while 16 for the
  // 16-block leaves of the first projection (many short waves) or 24 for the
  // second lost occupancy (+23 % and about even).
  static constexpr int D = FM <= 2 ? 8 : 4;
  __device__ __forceinline__ void leaf(Acc& acc) {
    if (FM == 1 && spl >= 32 && spl % 16 == 0) leaf_ring<(FM == 1 ? 16 : 1)>(acc);
    else if (D >= 8 && spl % 8 == 0) leaf_ring<(D >= 8 ? 8 : 1)>(acc);
    else if (D >= 4 && spl % 4 == 0) leaf_ring<(D >= 4 ? 4 : 1)>(acc);
    else if (spl % 2 == 0) leaf_ring<2>(acc);
    else leaf_ring<1>(acc);
  }
};

template <int FM, int NW, int OUTM>
__global__ __launch_bounds__(64 * NW) void gemm_stream_kernel(TileParams p) {
  using Ctx = StreamCtx<FM>;
  __shared__ float xch[NW > 1 ? NW : 1][FM * 4 * 64];
  __shared__ __attribute__((aligned(16))) float lp_buf[OUTM == kOutLP ? 64 * kLpStride : 4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16 * FM;
  const int z = blockIdx.z;
  const int leaf = p.leaf_lo + z * NW + w;  // one leaf per wave

  // Launch guarantees 16 * FM * K * 2 < 2^32, so every byte offset below
  // fits the 32-bit buffer range.
  Ctx c;
  c.spl = p.kl / 32;
  c.kb = (uint32_t)__builtin_amdgcn_readfirstlane(leaf) * (uint32_t)p.kl * 2u;
  const int64_t arows = p.M - m0 < 16 * FM ? p.M - m0 : 16 * FM;
  const int64_t brows = p.N - n0 < 16 ? p.N - n0 : 16;
  c.ra = make_rsrc(p.A + m0 * p.K, (uint32_t)(arows * p.K * 2));
  c.rb = make_rsrc(p.B + n0 * p.K, (uint32_t)(brows * p.K * 2));
  const uint32_t kq = 16u * (uint32_t)(lane >> 4);  // this lane's 8 k values
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = 16 * i + (lane & 15);
    c.voa[i] = (uint32_t)(r < arows ? r : 0) * (uint32_t)p.K * 2u + kq;
  }
  {
    const int r = lane & 15;
    c.vob = (uint32_t)(r < brows ? r : 0) * (uint32_t)p.K * 2u + kq;
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
  if constexpr (OUTM == kOutLP) {
    // wave 0 alone from here on: the 16*FM x 16 block transposed through
    // LDS, lane l < 16*FM owns row l (the other lanes' results are dropped)
    float* t = lp_buf;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) t[(16 * i + 4 * (lane >> 4) + r) * kLpStride + (lane & 15)] = acc.v[i][0][r];
    const int64_t row = m0 + lane;
    lp_rows_epilogue<1>(p, t, row, lane < 16 * FM && row < p.M, n0, lane);
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + 16 * i + 4 * (lane >> 4) + r;
      if (row < p.M && col < p.N) {
        const int64_t off = (int64_t)z * p.c_group_stride + row * p.N + col;
        if constexpr (OUTM == kOutBF16)
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
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < plane; i += (int64_t)gridDim.x * 256) {
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
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y,
                                                        int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = f32_to_bf16_bits(x[i]);
}

// ------------------------------------------------------------------ dispatch

#define INV_RING_CASE(NL_, BK_, ODD_)                                                                        \
  hipLaunchKernelGGL((gemm_ring_kernel<NL_, BK_, OUTM, GROUPED, ODD_>), grid, dim3(64 * kRingWaves), 0, s, p); \
  break;

// Leaves that are a multiple of 64 run on 64-k stages; leaves that are an odd
// multiple of 32 from 96 on run on 64-k stages as 32-wide substeps when the
// leaf count is even; one odd leaf, and leaves of exactly 32, run on 32-k
// stages. The chain of every element is the same in all of them.
template <int OUTM, bool GROUPED>
hipError_t ring_dispatch(const TileParams& p, dim3 grid, int nl, hipStream_t s) {
  const bool bk64 = p.kl % 64 == 0;
  if (p.kl == 32) {
    switch (nl) {
      case 1: INV_RING_CASE(1, 32, false)
      case 2: INV_RING_CASE(2, 32, false)
      case 4: INV_RING_CASE(4, 32, false)
      case 8: INV_RING_CASE(8, 32, false)
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (nl * 2 + (bk64 ? 1 : 0)) {
    case 2: INV_RING_CASE(1, 32, false)
    case 3: INV_RING_CASE(1, 64, false)
    case 4: INV_RING_CASE(2, 64, true)
    case 5: INV_RING_CASE(2, 64, false)
    case 8: INV_RING_CASE(4, 64, true)
    case 9: INV_RING_CASE(4, 64, false)
    case 16: INV_RING_CASE(8, 64, true)
    case 17: INV_RING_CASE(8, 64, false)
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#undef INV_RING_CASE

// 64-row tiles (plain launches, leaves a multiple of 64)
template <int OUTM>
hipError_t ring64_dispatch(const TileParams& p, dim3 grid, int nl, hipStream_t s) {
  switch (nl) {
    case 1: hipLaunchKernelGGL((gemm_ring_kernel<1, 64, OUTM, false, false, 64>), grid, dim3(64 * kRingWaves), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_ring_kernel<2, 64, OUTM, false, false, 64>), grid, dim3(64 * kRingWaves), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_ring_kernel<4, 64, OUTM, false, false, 64>), grid, dim3(64 * kRingWaves), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_ring_kernel<8, 64, OUTM, false, false, 64>), grid, dim3(64 * kRingWaves), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FM, int OUTM>
hipError_t stream_dispatch_nw(const TileParams& p, dim3 grid, int nw, hipStream_t s) {
  switch (nw) {
    case 1: hipLaunchKernelGGL((gemm_stream_kernel<FM, 1, OUTM>), grid, dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_stream_kernel<FM, 2, OUTM>), grid, dim3(128), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_stream_kernel<FM, 4, OUTM>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemm_stream_kernel<FM, 8, OUTM>), grid, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int OUTM>
hipError_t stream_dispatch(const TileParams& p, int fm, dim3 grid, int nw, hipStream_t s) {
  switch (fm) {
    case 1: return stream_dispatch_nw<1, OUTM>(p, grid, nw, s);
    case 2: return stream_dispatch_nw<2, OUTM>(p, grid, nw, s);
    case 3: return stream_dispatch_nw<3, OUTM>(p, grid, nw, s);
    case 4: return stream_dispatch_nw<4, OUTM>(p, grid, nw, s);
    default: return hipErrorInvalidValue;
  }
}

template <int CNT>
hipError_t combine_cnt(const float* P, int64_t plane, void* C, bool out_bf16, bool fold, hipStream_t s) {
  dim3 grid(stride_grid(plane, 256));
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
  p.lp_stats = g.lp_stats;
  p.lp_tlogit = g.lp_tlogit;
  p.lp_target = g.lp_target;
  p.persist = 0;
  p.ntiles = 0;
  const bool lp = g.lp_stats != nullptr;
  // Persistent ring launches (8 leaves on 64-k stages, whole trees, more
  // tiles than the chip holds): one workgroup per CU walks tiles blockIdx.x,
  // + 256, ..., and its ring runs on from each tile into the next, so no tile
  // pays the pipeline's fill or a workgroup launch.
  constexpr int64_t kResident = 256;
  // (8 leaves of 64 k or more: the 64-k stage kernels)
  const bool can_persist = g.nl == 8 && g.kl >= 64 && g.groups == 1;
  if (lp && (g.offsets || g.groups != 1)) return hipErrorInvalidValue;  // statistics need whole trees
  if (g.swiglu && (!g.offsets || g.groups != 1 || g.N % 2 != 0)) return hipErrorInvalidValue;

  if (g.offsets) {  // grouped: row-tile slots = an upper bound on sum_e ceil(count_e / 128)
    const int64_t slots = g.M / 128 + g.E;
    const int64_t tiles_n = g.swiglu ? (g.N / 2 + 63) / 64 : (g.N + 127) / 128;
    // walk positions: with the XCD-aware order (<= 128 experts) every XCD
    // walks at most ceil(items / 8) positions, so round up to a multiple of 8
    const int64_t walk = (slots * tiles_n + 7) / 8 * 8;
    dim3 grid((unsigned)walk, 1u, (unsigned)g.groups);
    if (can_persist && walk > kResident) {
      p.persist = 1;
      p.ntiles = walk;
      grid.x = (unsigned)kResident;
    }
    if (g.swiglu) return ring_dispatch<kOutSwiGLU, true>(p, grid, g.nl, s);
    return g.out_bf16 ? ring_dispatch<kOutBF16, true>(p, grid, g.nl, s)
                      : ring_dispatch<kOutF32, true>(p, grid, g.nl, s);
  }
  // Stream kernel below 8 rows, and up to 16 rows when the ring kernel would
  // run fewer than 256 whole-K tiles; the ring kernel everywhere else. The
  // stream kernel re-reads A per wave, so its time grows with M, while a ring
  // tile costs the same up to 128 rows (measured, 8 leaves, K = 4096:
  // 4096 x 12288 without leaf groups 25.7 / 28.2 / 39.4 / 63.0 us at M = 8 /
  // 16 / 32 / 64 against 33-35 us on the ring; the 4096 x 151936 LM head 271 /
  // 323 / 470 / 787 us against 259-286 us).
  const int64_t ring_tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128) * g.groups;
  if ((g.M < 8 || (g.M <= 16 && g.groups == 1 && ring_tiles < 256)) && g.K < (int64_t{1} << 25)) {
    const int fm = (int)((g.M + 15) / 16);
    // each wave owns one leaf; groups of nl leaves become nl waves per WG
    dim3 grid((unsigned)((g.N + 15) / 16), 1u, (unsigned)g.groups);
    if (lp) return stream_dispatch<kOutLP>(p, fm, grid, g.nl, s);
    return g.out_bf16 ? stream_dispatch<kOutBF16>(p, fm, grid, g.nl, s) : stream_dispatch<kOutF32>(p, fm, grid, g.nl, s);
  }
  if (g.M <= 64 && g.kl % 64 == 0) {
    // 64-row tiles, the leaf groups folded into the tile index; persistent
    // whenever there are more tiles than CUs
    const int64_t items = ((g.N + 127) / 128) * g.groups;
    dim3 grid((unsigned)items);
    if (items > kResident) {
      p.persist = 1;
      p.ntiles = items;
      grid.x = (unsigned)kResident;
    }
    if (lp) return ring64_dispatch<kOutLP>(p, grid, g.nl, s);
    return g.out_bf16 ? ring64_dispatch<kOutBF16>(p, grid, g.nl, s) : ring64_dispatch<kOutF32>(p, grid, g.nl, s);
  }
  const int64_t tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128);
  dim3 grid((unsigned)tiles, 1u, (unsigned)g.groups);
  if (can_persist && tiles > kResident) {
    p.persist = 1;
    p.ntiles = tiles;
    grid.x = (unsigned)kResident;
  }
  if (lp) return ring_dispatch<kOutLP, false>(p, grid, g.nl, s);
  return g.out_bf16 ? ring_dispatch<kOutBF16, false>(p, grid, g.nl, s) : ring_dispatch<kOutF32, false>(p, grid, g.nl, s);
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
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(stride_grid(n, 256)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

}  // namespace inv
