// mfma_dma.hpp -- matrix-core product whose K slices reach LDS by direct
// buffer-to-LDS loads (gfx950 buffer_load_dword[x4] ... lds).
//
// Computes C = alpha * op(A) op(B) + beta * C for one or a strided batch of
// products; the plain C = A x B is alpha = 1, beta = 0, no transposes, one
// product.
//
// The register-staged kernel spends VGPRs on the next slice, then waits for
// those loads and writes them to LDS itself; with one wave per SIMD that
// write-back sits between matrix-core instructions and leaves the matrix
// pipe idle.  Here each wave only issues the loads: the memory system writes
// the bytes of lane l to LDS address M0 + 16 l (or 4 l) of the block, no
// VGPR is involved, and the wave carries on with matrix-core work.  The
// double buffer of the textbook chapter "4. 矩阵乘法性能优化" (section 四)
// becomes: the loads of slice t+2 go out right after the barrier that ends
// slice t, into the stage slice t has just released, and the barrier that
// ends slice t+1 waits for them -- a full slice of latency cover.
//
// Layout.  An operand's slice is BK values of k by D values of m (or n).
// Where k runs along the stored rows (B as given, or A transposed) the LDS
// image is the stored window itself, row-major [BK][D], and the operand
// reads are 32-bit, consecutive lanes on consecutive banks.  Where k runs
// along the stored columns (A as given, or B transposed) the image is
// [D][BK] with k contiguous, read 128 bits (four k) at a time; the rows of a
// 1 KiB load block cannot be padded against bank conflicts as the chapter
// pads its shared tiles (section 三), because a block's LDS image is fixed by
// lane order, so instead each lane fetches the global chunk whose index is
// its LDS chunk index XOR a function of the row (kc_swizzle).  The swizzle
// depends only on row mod 16 and makes the 128-bit reads of 8 (and of 16)
// consecutive rows hit disjoint banks.  The article "硬件加速原理：CUDA核函数
// 优化矩阵乘法的内存访问模式" (section "访问模式对比") makes the same point for
// row- versus column-major operands: keep the loads contiguous and re-lay
// the data out on chip.
//
// Edges.  The buffer descriptor's range check turns a load at an offset
// past num_records into zeros; an element outside op(A) (M x K) or op(B)
// (K x N) is given such an offset, so ragged tiles and the K tail are
// zero-filled by the hardware.  With a ragged K the partial last slice is
// computed first, so its loads, the only ones that need a K test, go out in
// the prologue: an operand whose k runs along its stored rows ends its
// window after the last valid row through num_records, the other one
// compares each load's k index.
//
// Load width.  An operand is fetched in 16-byte chunks (64 lanes x 16 B =
// one 1 KiB block per instruction) or in single floats (256 B per
// instruction).  A 16-byte chunk needs only a dword-aligned address, and it
// fills the same LDS image as four 4-byte loads, so the bits do not depend
// on the width (tested from every row offset mod 16 bytes).  Where
// the chunks run along m or n (A transposed, B as given) the stored width
// must be a multiple of 4, so that no chunk straddles the edge of op(A) or
// op(B); where they run along k, the partial last slice takes 4-byte loads
// when K % 4 != 0.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace sgemm {

typedef __attribute__((address_space(3))) void lds_void_t;

// Chunk swizzle of row `row` of a k-contiguous slice image with BK floats per
// row (SWZ = false keeps the plain layout, for measuring what it buys).  A
// 128-bit LDS read is served 16 lanes at a time over 64 four-byte banks, so
// the 16 rows that 16 consecutive lanes read must land on 16 distinct
// 16-byte bank groups: rows of 64 B share a 256-B bank line four at a time,
// rows of 128 B two at a time, and rows of 256 B or more start on the same
// bank, so their chunk index is XORed with the row mod 16.
template <int BK, bool SWZ>
__device__ __forceinline__ int kc_swizzle(int row) {
  static_assert(BK == 16 || BK == 32 || BK == 64, "swizzle is defined for 4, 8 or 16 chunks");
  if constexpr (!SWZ)
    return 0;
  else if constexpr (BK == 16)
    return ((row >> 1) ^ ((row >> 3) & 1)) & 3;
  else if constexpr (BK == 32)
    return (row ^ ((row >> 3) & 1)) & 7;
  else
    return row & 15;
}

// Word 3 of a raw (untyped, unswizzled) buffer descriptor on CDNA.
constexpr int kRawBufferWord3 = 0x00020000;
// num_records of the descriptors, and the offset given to elements that lie
// outside the matrix: at or past num_records, so they read as zero.
constexpr int kBufferRecords = 0x7ffff000;
constexpr unsigned kOutOfRange = 0x80000000u;

// Barrier that also retires this wave's buffer-to-LDS loads.  The compiler
// does not reliably account for those loads before LDS reads of the stage
// they fill, so the wait is explicit: s_waitcnt vmcnt(0) (expcnt and
// lgkmcnt fields at their "don't wait" maxima: SIMM16 = 0x0f70), then the
// usual workgroup barrier, whose fence adds lgkmcnt(0).
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
}

// The same barrier, but retiring all except this wave's N most recent
// buffer-to-LDS loads (s_waitcnt vmcnt(N); vmcnt is 6 bits, split over bits
// 3:0 and 15:14 of SIMM16).  Loads retire in issue order, so with the loads
// of the later slices as the N most recent, the earlier slices have landed.
template <int N>
__device__ __forceinline__ void dma_barrier_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
  __syncthreads();
}

// One wave-wide buffer-to-LDS load: lane l's 16 (WIDE) or 4 bytes at byte
// offset `off` of the buffer land at LDS address lds + 16 l (or 4 l).
template <bool WIDE>
__device__ __forceinline__ void lds_dma(__amdgpu_buffer_rsrc_t r, float *lds, unsigned off) {
  if constexpr (WIDE)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 4, off, 0, 0, 0);
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<N, I + 1>(f);
  }
}

// Host-side limit of the path: every in-range offset of a slice (relative to
// the slice origin) must stay below kBufferRecords.  rows_a / rows_b: stored
// rows of a slice window (BM, or BK when A is transposed; BK, or BN when B
// is transposed).
inline bool dma_offsets_fit(long rows_a, long lda, long rows_b, long ldb) {
  return rows_a * lda * 4 + 4096 < kBufferRecords && rows_b * ldb * 4 + 4096 < kBufferRecords;
}

// Geometry of one operand's slice: D values of m (or n) by BK values of k.
// KROWS: k runs along the stored rows.  WIDE: 16-byte loads.
template <int D, int BK, bool KROWS, bool WIDE, bool SWZ, int NW>
struct SliceGeom {
  static constexpr int R = KROWS ? BK : D;  // stored rows of the window
  static constexpr int W = KROWS ? D : BK;  // stored columns
  static constexpr int E = WIDE ? 4 : 1;    // floats per lane per load
  static constexpr int FPB = kWave * E;     // floats per wave-wide load
  static constexpr int NB = R * W / FPB;    // loads per slice
  static_assert(R * W % FPB == 0, "a slice is a whole number of wave-wide loads");
  static constexpr int NBW = (NB + NW - 1) / NW;  // loads per wave per slice
  // Where the loads do not split evenly over the waves (the 12-wave 64 x 96
  // tile), the last load of some waves is spare: it reads out of range (no
  // memory traffic) into a dump area of LDS, so that every wave issues the
  // same number of loads and the load counters of the barriers hold.
  static constexpr bool SPARE = NB % NW != 0;
  static constexpr bool KR = KROWS;

  // Stored (row, col) of the window element that lane `lane` fetches in the
  // wave's q-th load: whichever element belongs at that lane's LDS position.
  __device__ __forceinline__ static void elem(int wave, int lane, int q, int &row, int &col) {
    const int f = (wave + q * NW) * FPB + lane * E;
    row = f / W;
    const int pc = f % W;
    if constexpr (KROWS)
      col = pc;
    else
      col = 4 * ((pc / 4) ^ kc_swizzle<BK, SWZ>(row)) + pc % 4;
  }
  __device__ __forceinline__ static int kof(int row, int col) { return KROWS ? row : col; }
  __device__ __forceinline__ static int mnof(int row, int col) { return KROWS ? col : row; }
};

// TA / TB: A / B are stored transposed (op(A) = A^T, op(B) = B^T).
// VA / VB: A / B take 16-byte loads.  KFULL: K % BK == 0 (otherwise the
// partial last slice is computed first).
// KSPLIT: the work-group runs KSPLIT sets of WM x WN waves over the same
// tile; set q takes the k groups g with g % KSPLIT == q of every slice, and
// the sets' partial sums are added in the order 0, 1, .., KSPLIT - 1 through
// LDS at the end, each set adding and storing its share of every block's
// registers.  A small tile then keeps all four SIMDs of its CU busy,
// which is what lets a product with fewer 64 x 64 tiles than CUs spread over
// the whole chip; the order of additions is still fixed for a given call
// shape.
//
// NST: LDS stages.  The loads of slice t+NST go out right after the barrier
// that ends slice t, into the stage slice t has released, and the barrier
// that ends slice t+1 waits only for slice t+1 -- NST-1 slices of latency
// cover.  When K fits NST slices, every slice is in flight from the start.
//
// SCHED: 1 interleaves each group's loads and LDS reads with its
// matrix-core instructions (the product kernel).  2 is the race-triage form:
// no interleaving, and every slice is computed with no load in flight and
// all waves in step -- a barrier that retires every buffer-to-LDS load after
// each slice's loads are issued, after the prologue, and before each k group's
// LDS reads.  Its matrix-core sequence is the product kernel's, so it gives
// the same bits; a result that changes with SCHED points to a missing wait or
// barrier (a race), one that does not to the arithmetic.
//
// PHASES (a diagnostic instantiation): thread 0 of each work-group writes
// the reference-clock time (s_memrealtime) at five points of its run to
// p.phases[8 w + i] -- 0 start, 1 first slice landed, 2 last slice
// computed, 3 k-set sums reduced, 4 stores of C complete -- the shader
// clock (s_memtime) at start and end to entries 5 and 6, and the tile (BM,
// BN, BK, KSPLIT in 16-bit fields) to entry 7.  The only other change is a
// wait for the stores before the last timestamp, which the product kernel
// leaves to the end of the dispatch.
template <int BM, int BN, int BK, int WM, int WN, bool SWZ, bool KFULL, int SCHED, bool VA,
          bool VB, bool TA, bool TB, int KSPLIT = 1, int NST = 2, bool PHASES = false>
__global__ void __launch_bounds__(WM *WN *KSPLIT *kWave)
mfma_gemm_dma_kernel(GemmArgs p, TileMap tmap) {
  auto phase = [&](int i) {
    if constexpr (PHASES) {
      if (threadIdx.x == 0) p.phases[(long)blockIdx.x * 8 + i] = __builtin_amdgcn_s_memrealtime();
    }
  };
  phase(0);
  if constexpr (PHASES) {
    if (threadIdx.x == 0) {
      p.phases[(long)blockIdx.x * 8 + 5] = __builtin_amdgcn_s_memtime();
      p.phases[(long)blockIdx.x * 8 + 7] = (unsigned long long)BM | (unsigned long long)BN << 16 |
                                           (unsigned long long)BK << 32 |
                                           (unsigned long long)KSPLIT << 48;
    }
  }
  constexpr int NWT = WM * WN;       // waves of one k set
  constexpr int NW = NWT * KSPLIT;   // waves of the work-group
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KH = BK / 2, G = KH / 4;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(G >= 2, "BK must be 16, 32 or 64");
  static_assert(G % KSPLIT == 0, "k groups must split evenly over the k sets");
  constexpr int GW = G / KSPLIT;  // k groups per slice of one wave
  // A as given has k along its columns; transposed, along its rows.  B the
  // other way round.
  using GA = SliceGeom<BM, BK, TA, VA, SWZ, NW>;
  using GB = SliceGeom<BN, BK, !TB, VB, SWZ, NW>;

  // One LDS array per stage and operand: with distinct objects the compiler
  // sees that the loads into one stage do not touch the stage being read,
  // and adds no wait for them before the operand reads (with the stages in
  // one array it waits for every load in flight, serialising the pipeline).
  static_assert(NST >= 2 && NST <= 4, "2 to 4 LDS stages");
  constexpr int SA = BM * BK, SB = BK * BN;
  __shared__ __attribute__((aligned(1024))) float As0[SA];
  __shared__ __attribute__((aligned(1024))) float As1[SA];
  __shared__ __attribute__((aligned(1024))) float As2[NST > 2 ? SA : 1];
  __shared__ __attribute__((aligned(1024))) float As3[NST > 3 ? SA : 1];
  __shared__ __attribute__((aligned(1024))) float Bs0[SB];
  __shared__ __attribute__((aligned(1024))) float Bs1[SB];
  __shared__ __attribute__((aligned(1024))) float Bs2[NST > 2 ? SB : 1];
  __shared__ __attribute__((aligned(1024))) float Bs3[NST > 3 ? SB : 1];
  auto stage_a = [&](auto S) -> float * {
    constexpr int i = decltype(S)::value;
    if constexpr (i == 0) return As0;
    else if constexpr (i == 1) return As1;
    else if constexpr (i == 2) return As2;
    else return As3;
  };
  auto stage_b = [&](auto S) -> float * {
    constexpr int i = decltype(S)::value;
    if constexpr (i == 0) return Bs0;
    else if constexpr (i == 1) return Bs1;
    else if constexpr (i == 2) return Bs2;
    else return Bs3;
  };
  // Partial sums that each k set hands to the others for the final
  // reduction (per set, the registers of the other sets).
  constexpr int kRedSlot = NWT * FM * FN * 16 * kWave;
  __shared__ __attribute__((aligned(1024))) float Red[KSPLIT > 1 ? (KSPLIT - 1) * kRedSlot : 1];
  // Landing area of the spare loads (zeros, never read), including those of
  // the 4-byte loads of a ragged K's tail slice.
  constexpr bool kSpare = GA::SPARE || GB::SPARE || SliceGeom<BM, BK, TA, false, SWZ, NW>::SPARE ||
                          SliceGeom<BN, BK, !TB, false, SWZ, NW>::SPARE;
  __shared__ __attribute__((aligned(1024))) float Dump[kSpare ? 4 * kWave : 1];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  // k set and wave within the set (KSPLIT == 1: one set, known at compile time)
  const int kq = KSPLIT > 1 ? wave / NWT : 0;
  const int wl = KSPLIT > 1 ? wave % NWT : wave;
  const int wm = wl / WN, wn = wl % WN;
  const int r32 = lane % 32, half = lane / 32;

  // Launch position -> (product of the batch, tile).
  int bidx, tm, tn;
  tmap.tile(xcd_contiguous_id(blockIdx.x, gridDim.x), bidx, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const float *Ab = p.A + (long)bidx * p.strideA;
  const float *Bb = p.B + (long)bidx * p.strideB;
  float *Cb = p.C + (long)bidx * p.strideC;

  // Per-lane byte offsets relative to the slice origin.  Elements outside
  // op(A)'s rows (M) or op(B)'s columns (N) get the out-of-range offset once
  // and for all; the K tail is handled by the one slice that has it.
  unsigned offA[GA::NBW], offB[GB::NBW];
#pragma unroll
  for (int q = 0; q < GA::NBW; ++q) {
    int row, col;
    GA::elem(wave, lane, q, row, col);
    offA[q] = m0 + GA::mnof(row, col) < p.M ? (unsigned)(row * p.lda + col) * 4u : kOutOfRange;
    if constexpr (GA::SPARE) offA[q] = wave + q * NW < GA::NB ? offA[q] : kOutOfRange;
  }
#pragma unroll
  for (int q = 0; q < GB::NBW; ++q) {
    int row, col;
    GB::elem(wave, lane, q, row, col);
    offB[q] = n0 + GB::mnof(row, col) < p.N ? (unsigned)(row * p.ldb + col) * 4u : kOutOfRange;
    if constexpr (GB::SPARE) offB[q] = wave + q * NW < GB::NB ? offB[q] : kOutOfRange;
  }

  // Slice order.  With a ragged K (not KFULL) the partial last slice is
  // computed first: its loads go out in the prologue, so every slice whose
  // loads the main loop issues is a whole one and needs no K test.  Position
  // u of the order is slice u - 1 for u >= 1 (slice u with KFULL).  A
  // position at or past nk gets descriptors with no records: every lane reads
  // out of range, so nothing is fetched and zeros land in a stage nobody
  // reads again.  This keeps the slice body free of branches, so the
  // scheduler can interleave these loads with matrix-core instructions.
  const int nk = (p.K + BK - 1) / BK;
  auto rsrc = [](const float *base, int records) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, records,
                                             kRawBufferWord3);
  };
  auto origin_a = [&](int k0) { return TA ? Ab + (long)k0 * p.lda + m0 : Ab + (long)m0 * p.lda + k0; };
  auto origin_b = [&](int k0) { return TB ? Bb + (long)n0 * p.ldb + k0 : Bb + (long)k0 * p.ldb + n0; };
  auto dma = [&](auto S, int u) {
    float *as = stage_a(S);
    float *bs = stage_b(S);
    const int t = KFULL ? u : u - 1;
    const int k0 = u < nk ? t * BK : 0;
    const int records = u < nk ? kBufferRecords : 0;
    const float *abase = origin_a(k0);
    const float *bbase = origin_b(k0);
    const __amdgpu_buffer_rsrc_t ra = rsrc(abase, records);
    const __amdgpu_buffer_rsrc_t rb = rsrc(bbase, records);
#pragma unroll
    for (int q = 0; q < GA::NBW; ++q) {
      float *dst = as + (wave + q * NW) * GA::FPB;
      if constexpr (GA::SPARE) dst = wave + q * NW < GA::NB ? dst : Dump;
      lds_dma<VA>(ra, dst, offA[q]);
    }
#pragma unroll
    for (int q = 0; q < GB::NBW; ++q) {
      float *dst = bs + (wave + q * NW) * GB::FPB;
      if constexpr (GB::SPARE) dst = wave + q * NW < GB::NB ? dst : Dump;
      lds_dma<VB>(rb, dst, offB[q]);
    }
  };

  // The partial last slice (K % BK valid k), into stage 0.  An operand whose
  // k runs along its stored rows ends its window after the last valid row,
  // through the descriptor's num_records.  The other one compares each
  // load's k index with the valid count; where K % 4 != 0 its 16-byte chunk
  // at the end of K would hold k past K, so that operand takes 4-byte loads
  // in this slice (they fill the same LDS image, so the bits do not change).
  auto tail_operand = [&](auto geom, auto wide, float *stage, const float *origin, long ld,
                          int mn0, int mn_count, int kl) {
    using Gm = decltype(geom);
    constexpr bool W = decltype(wide)::value;
    const int rec = Gm::KR ? kl * (int)ld * 4 : kBufferRecords;
    const __amdgpu_buffer_rsrc_t r = rsrc(origin, rec);
#pragma unroll
    for (int q = 0; q < Gm::NBW; ++q) {
      int row, col;
      Gm::elem(wave, lane, q, row, col);
      bool in = mn0 + Gm::mnof(row, col) < mn_count && (Gm::KR || Gm::kof(row, col) < kl);
      float *dst = stage + (wave + q * NW) * Gm::FPB;
      if constexpr (Gm::SPARE) {
        in = in && wave + q * NW < Gm::NB;
        dst = wave + q * NW < Gm::NB ? dst : Dump;
      }
      lds_dma<W>(r, dst, in ? (unsigned)(row * ld + col) * 4u : kOutOfRange);
    }
  };
  auto dma_tail = [&](auto S) {
    const int k0 = (nk - 1) * BK;
    const int kl = p.K - k0;
    using GAn = SliceGeom<BM, BK, TA, false, SWZ, NW>;
    using GBn = SliceGeom<BN, BK, !TB, false, SWZ, NW>;
    if (VA && !GA::KR && p.K % 4 != 0)
      tail_operand(GAn(), std::false_type(), stage_a(S), origin_a(k0), p.lda, m0, p.M, kl);
    else
      tail_operand(GA(), std::integral_constant<bool, VA>(), stage_a(S), origin_a(k0), p.lda, m0,
                   p.M, kl);
    if (VB && !GB::KR && p.K % 4 != 0)
      tail_operand(GBn(), std::false_type(), stage_b(S), origin_b(k0), p.ldb, n0, p.N, kl);
    else
      tail_operand(GB(), std::integral_constant<bool, VB>(), stage_b(S), origin_b(k0), p.ldb, n0,
                   p.N, kl);
  };

  // Operand read offsets (floats).  In a k-contiguous image, row
  // base + i*32 + r32 (base a multiple of 32) has swizzle kc_swizzle(r32).
  // Entry i is this wave's i-th k group of a slice, g = kq + KSPLIT * i.
  const int sw = kc_swizzle<BK, SWZ>(r32);
  int a_off[GW], b_off[GW];
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    const int g = kq + KSPLIT * i;
    a_off[i] = TA ? (half * KH + g * 4) * BM + wm * WTM + r32
                  : (wm * WTM + r32) * BK + 4 * ((half * (KH / 4) + g) ^ sw);
    b_off[i] = TB ? (wn * WTN + r32) * BK + 4 * ((half * (KH / 4) + g) ^ sw)
                  : (half * KH + g * 4) * BN + wn * WTN + r32;
  }

  struct Ops {
    f32x4 a[FM];
    f32x4 b[FN];
  };
  auto read_ops = [&](auto S, int g, Ops &o) {
    const float *as = stage_a(S);
    const float *bs = stage_b(S);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (TA) {
#pragma unroll
        for (int t = 0; t < 4; ++t) o.a[i][t] = as[a_off[g] + t * BM + i * 32];
      } else {
        o.a[i] = *reinterpret_cast<const f32x4 *>(as + a_off[g] + i * 32 * BK);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (TB) {
        o.b[j] = *reinterpret_cast<const f32x4 *>(bs + b_off[g] + j * 32 * BK);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) o.b[j][t] = bs[b_off[g] + t * BN + j * 32];
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto mma = [&](const Ops &o) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x2(o.a[i][t], o.b[j][t], acc[i][j]);
  };

  using S0 = std::integral_constant<int, 0>;
  Ops cur, nxt;

  // Instruction interleaving inside one group (SCHED = 1): first one
  // matrix-core instruction per buffer-to-LDS load (last group only), then
  // two per LDS read, so that neither burst leaves the matrix pipe idle.
  // Tiles in two k sets with 32-float slices have four matrix-core
  // instructions per group, too few to cover both: there the last group
  // issues the next slice's LDS reads first, one per matrix-core
  // instruction, and its loads after them (1024^3 1.1 %, 1000 x 1500 x 777
  // 1.3 %, 800 x 1280 x 777 2.2 % faster; the same order cost the four-set
  // and 64-float-slice tiles 2-6 %).
  constexpr int NMFMA = 4 * FM * FN;
  constexpr int NDS = (TA ? 2 * FM : FM) + (TB ? FN : 2 * FN);  // 128-bit or paired 32-bit reads
  auto interleave = [&](auto with_dma) {
    if constexpr (SCHED == 1) {
      constexpr int nv = decltype(with_dma)::value ? GA::NBW + GB::NBW : 0;
      if constexpr (nv > 0 && KSPLIT == 2 && BK == 32) {
#pragma unroll
        for (int q = 0; q < NDS; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix core
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
#pragma unroll
        for (int q = 0; q < nv; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
      } else {
#pragma unroll
        for (int q = 0; q < nv; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < NDS; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        constexpr int left = NMFMA - nv - 2 * NDS;
        if constexpr (left > 0) __builtin_amdgcn_sched_group_barrier(0x008, left, 0);
      }
    }
  };

  // Slice t lives in stage S = t % NST; slices t+1 .. t+NST-1 are already on
  // their way to the other stages.
  constexpr int kLoadsPerSlice = GA::NBW + GB::NBW;  // per wave
  static_assert(SCHED == 1 || SCHED == 2, "schedule 1 (interleaved) or 2 (race triage)");
  auto slice = [&](auto S, int t) {
    constexpr int s = decltype(S)::value;
    using SN = std::integral_constant<int, (s + 1) % NST>;
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      if constexpr (SCHED == 2) dma_barrier();
      if (g + 1 < GW) {
        read_ops(S, g + 1, nxt);
        mma(cur);
        interleave(std::false_type());
      } else {
        // All reads of stage S are done and slice t+1 has landed (only the
        // loads of slices t+2 .. t+NST-1 may still be in flight).
        dma_barrier_keep<(NST - 2) * kLoadsPerSlice>();
        dma(S, t + NST);
        if constexpr (SCHED == 2) dma_barrier();
        read_ops(SN(), 0, nxt);  // harmless if there is no slice t+1
        mma(cur);
        interleave(std::true_type());
      }
      cur = nxt;
    }
  };

  static_for<NST>([&](auto S) {
    if constexpr (!KFULL && decltype(S)::value == 0)
      dma_tail(S);
    else
      dma(S, decltype(S)::value);
  });
  // Slice 0 has landed; slices 1 .. NST-1 may still fly.
  if constexpr (SCHED == 2)
    dma_barrier();
  else
    dma_barrier_keep<(NST - 1) * kLoadsPerSlice>();
  phase(1);
  read_ops(S0(), 0, cur);
  for (int t = 0; t < nk; t += NST) {
    static_for<NST>([&](auto S) {
      if (decltype(S)::value == 0 || t + decltype(S)::value < nk) slice(S, t + decltype(S)::value);
    });
  }
  // The last slices issued loads past K (zero-filling, no memory traffic);
  // let them retire before the work-group gives up its LDS.
  __builtin_amdgcn_s_waitcnt(0x0f70);
  phase(2);

  // Register e of each accumulator block belongs to k set e / EPS: that set
  // adds the block's partial sums for it and stores it.  With one k set
  // everything belongs to set 0.
  static_assert(16 % KSPLIT == 0, "k sets must share the 16 registers of a block evenly");
  constexpr int EPS = 16 / KSPLIT;
  // Register r EPS + ee of block (i, j) for a set number r that is the same
  // in the whole wave but not a compile-time constant: picked by selects
  // (indexed by r, the registers were moved with indexed register moves).
  auto reg = [&](int i, int j, int r, int ee) {
    float v = acc[i][j][ee];
#pragma unroll
    for (int s = 1; s < KSPLIT; ++s) v = r == s ? acc[i][j][s * EPS + ee] : v;
    return v;
  };
  // Slot of writer set w in LDS for the registers of the p-th set other than
  // w (sets in increasing order), block (i, j), register ee of that set's range.
  auto slot = [&](int w, int pos, int i, int j, int ee) {
    return (((((w * (KSPLIT - 1) + pos) * NWT + wl) * FM + i) * FN + j) * EPS + ee) * kWave + lane;
  };
  float res[FM][FN][EPS];  // the reduced sums of set kq's registers
  if constexpr (KSPLIT > 1) {
    // Every set leaves in LDS the registers the other sets own; after the
    // barrier each set adds, for its own registers, the partial sums of sets
    // 0, 1, .., KSPLIT-1 in that order.  The additions and the stores of C
    // are shared by all sets, and each element is the same sum, in the same
    // order, as when one set adds up all of them.
#pragma unroll
    for (int pos = 0; pos < KSPLIT - 1; ++pos) {
      const int r = pos + (pos >= kq ? 1 : 0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int ee = 0; ee < EPS; ++ee) Red[slot(kq, pos, i, j, ee)] = reg(i, j, r, ee);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int ee = 0; ee < EPS; ++ee) {
          const float mine = reg(i, j, kq, ee);
          if constexpr (KSPLIT == 2) {
            // the two-term sum in either order: IEEE addition is commutative
            res[i][j][ee] = mine + Red[slot(1 - kq, 0, i, j, ee)];
          } else {
            // o[pos]: the partial sums of the pos-th other set w, which left
            // set kq's registers at its position kq - (kq > w)
            float o[KSPLIT - 1];
#pragma unroll
            for (int pos = 0; pos < KSPLIT - 1; ++pos) {
              const int w = pos + (pos >= kq ? 1 : 0);
              o[pos] = Red[slot(w, kq - (kq > w ? 1 : 0), i, j, ee)];
            }
            float sum = kq == 0 ? mine : o[0];
#pragma unroll
            for (int r = 1; r < KSPLIT; ++r)
              sum += r < kq ? o[r < KSPLIT - 1 ? r : KSPLIT - 2] : (r == kq ? mine : o[r - 1]);
            res[i][j][ee] = sum;
          }
        }
  }

  phase(3);
  // Epilogue: register e of lane l holds row acc32_row(l, e), column l % 32
  // of its 32x32 block; rows >= M and columns >= N are not stored.  C is read
  // only when beta != 0, and then a block's values per lane are all loaded
  // before any of them is stored (a store could alias a later load, so the
  // compiler would otherwise wait out each load's latency in turn).  Stores
  // that do not follow a read of C are non-temporal: C is not read again by
  // this kernel, and streaming it out instead of leaving it dirty in L2 took
  // 2048^3 from 144.3 to 146.1 TFLOP/s (1024^3: 112.6 to 114.1).  Each k set
  // stores the registers it owns (with k sets, the stores after a read of C
  // are non-temporal as well).
  const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN + r32;
  const bool full = (m0 + BM <= p.M) && (n0 + BN <= p.N);
  const bool plain = p.alpha == 1.f && p.beta == 0.f;
  // The one-set form is written out on its own: folded into the per-set
  // form below, the compiler stops specialising the stores on `full`, and
  // the 128 x 128 kernel grows from about 2500 to 3800 instructions.
  if constexpr (KSPLIT == 1) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 32;
        auto row = [&](int e) { return row0 + i * 32 + acc32_row(lane, e); };
        auto inside = [&](int e) { return full || (row(e) < p.M && col < p.N); };
        auto at = [&](int e) { return Cb + (long)row(e) * p.ldc + col; };
        if (plain) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (inside(e)) __builtin_nontemporal_store(acc[i][j][e], at(e));
        } else if (p.beta == 0.f) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (inside(e)) __builtin_nontemporal_store(p.alpha * acc[i][j][e], at(e));
        } else {
          float c[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) c[e] = inside(e) ? *at(e) : 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (inside(e)) *at(e) = fmaf(p.alpha, acc[i][j][e], p.beta * c[e]);
        }
      }
  } else {
    // Set kq stores its registers kq EPS + ee of each block: rows
    // 2 kq EPS + 8 (ee / 4) + ee % 4 of the block (+ 4 for the upper half of
    // the lanes).  Full tiles store without tests.
    const int rq = row0 + 2 * kq * EPS + 4 * half;
    auto dr = [](int ee) { return 8 * (ee >> 2) + (ee & 3); };
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = col0 + j * 32;
        const int rb = rq + i * 32;
        float *const at0 = Cb + (long)rb * p.ldc + col;
        auto at = [&](int ee) { return at0 + (long)dr(ee) * p.ldc; };
        auto inside = [&](int ee) { return rb + dr(ee) < p.M && col < p.N; };
        if (plain || p.beta == 0.f) {
          float v[EPS];
#pragma unroll
          for (int ee = 0; ee < EPS; ++ee) v[ee] = plain ? res[i][j][ee] : p.alpha * res[i][j][ee];
          if (full) {
#pragma unroll
            for (int ee = 0; ee < EPS; ++ee) __builtin_nontemporal_store(v[ee], at(ee));
          } else {
#pragma unroll
            for (int ee = 0; ee < EPS; ++ee)
              if (inside(ee)) __builtin_nontemporal_store(v[ee], at(ee));
          }
        } else {
          float c[EPS];
#pragma unroll
          for (int ee = 0; ee < EPS; ++ee) c[ee] = full || inside(ee) ? *at(ee) : 0.f;
#pragma unroll
          for (int ee = 0; ee < EPS; ++ee)  // non-temporal as well: the compiler merges the
            if (full || inside(ee))          // last store of each path into one store, which
              __builtin_nontemporal_store(   // keeps the hint only if all of them carry it
                  fmaf(p.alpha, res[i][j][ee], p.beta * c[ee]), at(ee));
        }
      }
  }
  if constexpr (PHASES) {
    __builtin_amdgcn_s_waitcnt(0);
    phase(4);
    if (threadIdx.x == 0) p.phases[(long)blockIdx.x * 8 + 6] = __builtin_amdgcn_s_memtime();
  }
}

template <int BM, int BN, int BK, int WM, int WN, bool SWZ, int SCHED, bool VA, bool VB, bool TA,
          bool TB, int KSPLIT, int NST, bool PHASES = false>
inline void launch_dma_kernel(const GemmArgs &p, hipStream_t stream, int group_m) {
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const dim3 grid((unsigned)((long)tiles_m * tiles_n * p.batch)),
      block(WM * WN * KSPLIT * kWave);
  const TileMap tmap = make_tile_map(tiles_m, tiles_n, group_m);
  if (p.K % BK == 0)
    hipLaunchKernelGGL((mfma_gemm_dma_kernel<BM, BN, BK, WM, WN, SWZ, true, SCHED, VA, VB, TA, TB,
                                             KSPLIT, NST, PHASES>),
                       grid, block, 0, stream, p, tmap);
  else
    hipLaunchKernelGGL((mfma_gemm_dma_kernel<BM, BN, BK, WM, WN, SWZ, false, SCHED, VA, VB, TA,
                                             TB, KSPLIT, NST, PHASES>),
                       grid, block, 0, stream, p, tmap);
}

template <int BM, int BN, int BK, int WM, int WN, bool SWZ, int SCHED, bool TA, bool TB,
          int KSPLIT, int NST, bool PHASES = false>
inline void launch_dma_widths(const GemmArgs &p, bool va, bool vb, hipStream_t stream,
                              int group_m) {
  if (va && vb)
    launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, true, true, TA, TB, KSPLIT, NST, PHASES>(
        p, stream, group_m);
  else if (va)
    launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, true, false, TA, TB, KSPLIT, NST, PHASES>(
        p, stream, group_m);
  else if (vb)
    launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, false, true, TA, TB, KSPLIT, NST, PHASES>(
        p, stream, group_m);
  else
    launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, false, false, TA, TB, KSPLIT, NST, PHASES>(
        p, stream, group_m);
}

}  // namespace sgemm
