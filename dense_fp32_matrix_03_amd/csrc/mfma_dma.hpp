// mfma_dma.hpp -- matrix-core product whose K slices reach LDS by direct
// buffer-to-LDS loads (gfx950 buffer_load_dwordx4 ... lds).
//
// The register-staged kernel spends VGPRs on the next slice, then waits for
// those loads and writes them to LDS itself; with one wave per SIMD that
// write-back sits between matrix-core instructions and leaves the matrix
// pipe idle.  Here each wave only issues the loads: the memory system writes
// the 16 bytes of lane l to LDS address M0 + 16 l of a 1 KiB block, no VGPR
// is involved, and the wave carries on with matrix-core work.  The double
// buffer of the textbook chapter "4. 矩阵乘法性能优化" (section 四) becomes:
// the loads of slice t+2 go out right after the barrier that ends slice t,
// into the stage slice t has just released, and the barrier that ends slice
// t+1 waits for them -- a full slice of latency cover.
//
// Layout.  A slice of A is BM rows x BK floats, rows packed; a 1 KiB block
// holds 64/(BK/4) whole rows.  Because a block's LDS image is fixed by lane
// order, the anti-conflict padding of the chapter (section 三) cannot be
// used; instead lane l of a block fetches the global chunk whose index is
// its LDS chunk index XOR a function of the row (a_swizzle).  The swizzle
// depends only on row mod 16 and makes the 128-bit operand reads of 8 (and
// of 16) consecutive rows hit disjoint banks.  B stays row-major.
//
// Edges.  The buffer descriptor's range check turns a load at an offset
// past num_records into zeros; an element outside the M x K (or K x N)
// matrix is given such an offset, so ragged tiles and the K tail are
// zero-filled by the hardware.  An operand that is 16-byte aligned with a
// leading dimension and width that are multiples of 4 is fetched in 16-byte
// chunks (64 lanes x 16 B = one 1 KiB block per instruction); any other
// operand in single floats (256 B per instruction), which handles any
// alignment and any K.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace sgemm {

typedef __attribute__((address_space(3))) void lds_void_t;

// Chunk swizzle of row `row` of an A slice with BK floats per row (SWZ =
// false keeps the plain layout, for measuring what the swizzle buys).
template <int BK, bool SWZ>
__device__ __forceinline__ int a_swizzle(int row) {
  static_assert(BK == 16 || BK == 32, "A swizzle is defined for 4 or 8 chunks per row");
  if constexpr (!SWZ)
    return 0;
  else if constexpr (BK == 16)
    return ((row >> 1) ^ ((row >> 3) & 1)) & 3;
  else
    return (row ^ ((row >> 3) & 1)) & 7;
}

// Word 3 of a raw (untyped, unswizzled) buffer descriptor on CDNA.
constexpr int kRawBufferWord3 = 0x00020000;
// num_records of the descriptors, and the offset given to chunks that lie
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

// One wave-wide buffer-to-LDS load: lane l's 16 (WIDE) or 4 bytes at byte
// offset `off` of the buffer land at LDS address lds + 16 l (or 4 l).
template <bool WIDE>
__device__ __forceinline__ void lds_dma(__amdgpu_buffer_rsrc_t r, float *lds, unsigned off) {
  if constexpr (WIDE)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 4, off, 0, 0, 0);
}

// Host-side limit of the path: every in-range offset of a slice must stay
// below kBufferRecords.
inline bool dma_offsets_fit(long BM, long BK, long lda, long ldb, long BN) {
  return BM * lda * 4 + 4096 < kBufferRecords && BK * ldb * 4 + BN * 4 + 4096 < kBufferRecords;
}

// VA / VB: A / B are fetched in 16-byte chunks (16-byte aligned, ld % 4 == 0
// and K % 4 == 0 for A, N % 4 == 0 for B), else in single floats.
template <int BM, int BN, int BK, int WM, int WN, bool SWZ, bool KFULL, int SCHED, bool VA,
          bool VB>
__global__ void __launch_bounds__(WM *WN *kWave)
mfma_gemm_dma_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KH = BK / 2, G = KH / 4;
  // Each lane of a load moves EA (EB) floats; a block of one wave-wide load
  // covers 64*EA (64*EB) consecutive floats of the LDS image.
  constexpr int EA = VA ? 4 : 1, EB = VB ? 4 : 1;
  constexpr int FPB_A = kWave * EA, FPB_B = kWave * EB;
  constexpr int DA = BM * BK / FPB_A, DB = BK * BN / FPB_B;  // blocks per slice
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(G >= 2, "BK must be 16 or 32");
  static_assert(DA % NW == 0 && DB % NW == 0, "blocks must split evenly over the waves");
  constexpr int DAW = DA / NW, DBW = DB / NW;

  __shared__ __attribute__((aligned(1024))) float As0[BM * BK];
  __shared__ __attribute__((aligned(1024))) float As1[BM * BK];
  __shared__ __attribute__((aligned(1024))) float Bs0[BK * BN];
  __shared__ __attribute__((aligned(1024))) float Bs1[BK * BN];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane % 32, half = lane / 32;

  int tm, tn;
  grouped_tile(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Slice element fetched by this lane in the wave's q-th block: row and
  // column within the slice (A: row of the m tile, k; B: k, column of the n
  // tile).  The LDS image is A row-major with its 16-byte chunks swizzled,
  // B row-major; a lane's LDS position is fixed, so it fetches whichever
  // element belongs there.
  auto a_elem = [&](int q, int &row, int &k) {
    const int f = (wave + q * NW) * FPB_A + lane * EA;  // LDS position in the slice
    row = f / BK;
    const int pc = f % BK;
    k = 4 * ((pc / 4) ^ a_swizzle<BK, SWZ>(row)) + pc % 4;
  };
  auto b_elem = [&](int q, int &row, int &c) {
    const int f = (wave + q * NW) * FPB_B + lane * EB;
    row = f / BN;
    c = f % BN;
  };

  // Per-lane byte offsets relative to the slice origin (row m0 / column k0
  // of A; row k0 / column n0 of B).  Elements in rows of A past M or columns
  // of B past N get the out-of-range offset once and for all; the K tail is
  // handled per slice.
  unsigned offA[DAW], offB[DBW];
#pragma unroll
  for (int q = 0; q < DAW; ++q) {
    int row, k;
    a_elem(q, row, k);
    offA[q] = m0 + row < p.M ? (unsigned)(row * p.lda + k) * 4u : kOutOfRange;
  }
#pragma unroll
  for (int q = 0; q < DBW; ++q) {
    int row, c;
    b_elem(q, row, c);
    offB[q] = n0 + c < p.N ? (unsigned)(row * p.ldb + c) * 4u : kOutOfRange;
  }

  // Issue the loads of slice t into LDS stage S.  A slice at or past the end
  // of K gets descriptors with no records: every lane reads out of range, so
  // nothing is fetched and zeros land in a stage nobody reads again.  This
  // keeps the slice body free of branches, so the scheduler can interleave
  // these loads with matrix-core instructions.
  const int nk = (p.K + BK - 1) / BK;
  auto dma = [&](auto S, int t) {
    float *as = S.value ? As1 : As0;
    float *bs = S.value ? Bs1 : Bs0;
    const int k0 = t * BK;
    const int records = t < nk ? kBufferRecords : 0;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(p.A + (long)m0 * p.lda + (t < nk ? k0 : 0)), 0, records,
        kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(p.B + (long)(t < nk ? k0 : 0) * p.ldb + n0), 0, records,
        kRawBufferWord3);
#pragma unroll
    for (int q = 0; q < DAW; ++q) {
      unsigned off = offA[q];
      if constexpr (!KFULL) {
        int row, k;
        a_elem(q, row, k);
        off = k0 + k < p.K ? off : kOutOfRange;
      }
      lds_dma<VA>(ra, as + (wave + q * NW) * FPB_A, off);
    }
#pragma unroll
    for (int q = 0; q < DBW; ++q) {
      unsigned off = offB[q];
      if constexpr (!KFULL) {
        int row, c;
        b_elem(q, row, c);
        off = k0 + row < p.K ? off : kOutOfRange;
      }
      lds_dma<VB>(rb, bs + (wave + q * NW) * FPB_B, off);
    }
  };

  // Operand read offsets (floats).  Row wm*WTM + i*32 + r32 of the A slice
  // has swizzle a_swizzle(r32), the same for every i.
  const int sw = a_swizzle<BK, SWZ>(r32);
  int a_off[G];
#pragma unroll
  for (int g = 0; g < G; ++g) a_off[g] = (wm * WTM + r32) * BK + 4 * ((half * (KH / 4) + g) ^ sw);
  const int b_off = half * KH * BN + wn * WTN + r32;

  struct Ops {
    f32x4 a[FM];
    f32x4 b[FN];
  };
  auto read_ops = [&](auto S, int g, Ops &o) {
    const float *as = S.value ? As1 : As0;
    const float *bs = S.value ? Bs1 : Bs0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      o.a[i] = *reinterpret_cast<const f32x4 *>(as + a_off[g] + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) o.b[j][t] = bs[b_off + (g * 4 + t) * BN + j * 32];
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
  using S1 = std::integral_constant<int, 1>;
  Ops cur, nxt;

  // Instruction interleaving inside one group (SCHED = 1): after every two
  // matrix-core instructions, one of the group's LDS reads (and, in the last
  // group, first one buffer-to-LDS load per instruction), so that neither
  // burst leaves the matrix pipe idle.
  constexpr int NMFMA = 4 * FM * FN;
  constexpr int NDS = FM + 2 * FN;  // 128-bit A reads + paired 32-bit B reads
  auto interleave = [&](auto with_dma) {
    if constexpr (SCHED == 1) {
      constexpr int nv = decltype(with_dma)::value ? DAW + DBW : 0;
#pragma unroll
      for (int q = 0; q < nv; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix core
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
#pragma unroll
      for (int q = 0; q < NDS; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      constexpr int left = NMFMA - nv - 2 * NDS;
      if constexpr (left > 0) __builtin_amdgcn_sched_group_barrier(0x008, left, 0);
    }
  };

  auto slice = [&](auto S, int t) {
    constexpr int s = decltype(S)::value;
    using SN = std::integral_constant<int, s ^ 1>;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g + 1 < G) {
        read_ops(S, g + 1, nxt);
        mma(cur);
        interleave(std::false_type());
      } else {
        // All reads of stage S are done and slice t+1 has landed in S^1.
        dma_barrier();
        dma(S, t + 2);
        read_ops(SN(), 0, nxt);  // harmless if there is no slice t+1
        mma(cur);
        interleave(std::true_type());
      }
      cur = nxt;
    }
  };

  dma(S0(), 0);
  dma(S1(), 1);
  dma_barrier();
  read_ops(S0(), 0, cur);
  for (int t = 0; t < nk; t += 2) {
    slice(S0(), t);
    if (t + 1 < nk) slice(S1(), t + 1);
  }
  // The last slices issued loads past K (zero-filling, no memory traffic);
  // let them retire before the work-group gives up its LDS.
  __builtin_amdgcn_s_waitcnt(0x0f70);

  const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN + r32;
  const bool full = (m0 + BM <= p.M) && (n0 + BN <= p.N);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + i * 32 + acc32_row(lane, e);
        const int col = col0 + j * 32;
        if (full || (row < p.M && col < p.N)) p.C[(long)row * p.ldc + col] = acc[i][j][e];
      }
}

template <int BM, int BN, int BK, int WM, int WN, bool SWZ, int SCHED, bool VA, bool VB>
inline void launch_dma_kernel(const GemmArgs &p, hipStream_t stream, int group_m) {
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const dim3 grid((unsigned)((long)tiles_m * tiles_n)), block(WM * WN * kWave);
  if (p.K % BK == 0)
    hipLaunchKernelGGL((mfma_gemm_dma_kernel<BM, BN, BK, WM, WN, SWZ, true, SCHED, VA, VB>), grid,
                       block, 0, stream, p, tiles_m, tiles_n, group_m);
  else
    hipLaunchKernelGGL((mfma_gemm_dma_kernel<BM, BN, BK, WM, WN, SWZ, false, SCHED, VA, VB>),
                       grid, block, 0, stream, p, tiles_m, tiles_n, group_m);
}

// WIDE_ONLY instantiates only the 16-byte-load form; the caller guarantees
// va && vb.
template <int BM, int BN, int BK, int WM, int WN, bool SWZ = true, int SCHED = 1,
          bool WIDE_ONLY = false>
inline hipError_t launch_dma_cfg(const GemmArgs &p, bool va, bool vb, hipStream_t stream,
                                 int group_m = 8) {
  if constexpr (WIDE_ONLY) {
    if (!(va && vb)) return hipErrorInvalidValue;
    launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, true, true>(p, stream, group_m);
  } else {
    if (va && vb)
      launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, true, true>(p, stream, group_m);
    else if (va)
      launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, true, false>(p, stream, group_m);
    else if (vb)
      launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, false, true>(p, stream, group_m);
    else
      launch_dma_kernel<BM, BN, BK, WM, WN, SWZ, SCHED, false, false>(p, stream, group_m);
  }
  return hipGetLastError();
}

}  // namespace sgemm
