// valu_kernels.hip -- the pages' progression on the vector FMA units, kept as
// the ablation ladder beside the matrix-core kernel:
//   rung 0  one thread per output, operands straight from global memory
//           (blog "【infra之路】03_动手写 CUDA Kernel", v1 Naive; article
//           "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问模式", basic kernel);
//   rung 1  32 x 32 blocks through LDS with 64-wide K slices, one output
//           per thread, 16-byte cooperative fetch, zero-filled edges
//           (textbook chapter "4. 矩阵乘法性能优化", section 三);
//   rung 2  128 x 128 x 16 block tiles, 256 threads, 8 x 8 outputs per thread
//           as an outer product of 8 A and 8 B register values (chapter
//           sections 一 and 二);
//   rung 3  rung 2 with two LDS stages: slice t+1 is fetched while slice t is
//           computed (chapter section 四).
// All rungs run every product; none uses packed FMA.
#include "common.hpp"
#include "dispatch.hpp"

namespace sgemm {

// ---------------------------------------------------------------- rung 0
__global__ void __launch_bounds__(256) naive_kernel(GemmArgs p, int tiles_n) {
  const int bx = blockIdx.x % tiles_n, by = blockIdx.x / tiles_n;
  const int col = bx * 16 + (threadIdx.x % 16);
  const int row = by * 16 + (threadIdx.x / 16);
  if (row >= p.M || col >= p.N) return;
  const float *a = p.A + (long)row * p.lda;
  const float *b = p.B + col;
  float sum = 0.f;
  for (int k = 0; k < p.K; ++k) sum = fmaf(a[k], b[(long)k * p.ldb], sum);
  p.C[(long)row * p.ldc + col] = sum;
}

// ---------------------------------------------------------------- rung 1
// Shared-memory tiling (textbook chapter "4. 矩阵乘法性能优化", section 三):
// a work-group computes a 32 x 32 block of C, one output per thread, and
// walks K in 64-wide slices; each slice of A and B is read from global
// memory once per work-group into LDS and then reused by the 32 threads of
// a row or column.  Every thread fetches one 16-byte chunk per slice --
// threads 0-511 of A's 32 x 64 window, 512-1023 of B's 64 x 32 window
// (SliceFetch, zero-filling outside the matrix) -- and A lands k-major, so
// that in the k loop a wave's 64 lanes read one A value per row pair (a
// broadcast) and 32 consecutive B values.
constexpr int kTile = 32, kTileK = 64;

template <bool VA, bool VB>
__global__ void __launch_bounds__(kTile *kTile) lds_tiled_kernel(GemmArgs p, int tiles_n) {
  constexpr int kHalf = kTile * kTile / 2;              // threads per operand
  using FetchA = SliceFetch<kTile, kTileK, kHalf, VA>;  // 32 rows (m) x 64 k
  using FetchB = SliceFetch<kTileK, kTile, kHalf, VB>;  // 64 rows (k) x 32 n
  __shared__ float sAt[kTileK * (kTile + 1)];           // [k][m], rows padded by one
  __shared__ __attribute__((aligned(16))) float sB[kTileK * kTile];  // [k][n]
  const int tid = threadIdx.x;
  const int m0 = (blockIdx.x / tiles_n) * kTile, n0 = (blockIdx.x % tiles_n) * kTile;
  const int r = tid / kTile, c = tid % kTile;  // output row and column within the block
  const bool fetch_a = tid < kHalf;
  const int ft = fetch_a ? tid : tid - kHalf;  // index among the operand's fetch threads
  FetchA fa;
  FetchB fb;
  if (fetch_a)
    fa.init(p.A, p.lda, m0, 0, ft);
  else
    fb.init(p.B, p.ldb, 0, n0, ft);
  float sum = 0.f;
  for (int k0 = 0; k0 < p.K; k0 += kTileK) {
    if (fetch_a) {
      fa.load(p.M, p.K);
      const int wr = FetchA::wrow(ft, 0), wc = FetchA::wcol(ft);
#pragma unroll
      for (int e = 0; e < 4; ++e) sAt[(wc + e) * (kTile + 1) + wr] = fa.v[0][e];
      fa.advance(0, kTileK);
    } else {
      fb.load(p.K, p.N);
      *reinterpret_cast<f32x4 *>(&sB[FetchB::wrow(ft, 0) * kTile + FetchB::wcol(ft)]) = fb.v[0];
      fb.advance(kTileK, 0);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTileK; ++k)
      sum = fmaf(sAt[k * (kTile + 1) + r], sB[k * kTile + c], sum);
    __syncthreads();
  }
  if (m0 + r < p.M && n0 + c < p.N) p.C[(long)(m0 + r) * p.ldc + n0 + c] = sum;
}

// ---------------------------------------------------------------- rungs 2, 3
// Thread (tx, ty) = (tid % 16, tid / 16) owns rows {4ty + i, 64 + 4ty + i}
// and columns {4tx + j, 64 + 4tx + j}, i, j < 4: its 8 x 8 outputs as four
// 4 x 4 quadrants.  A is stored transposed in LDS (k-major), so both operand
// vectors are contiguous 128-bit LDS reads, and the 16 threads of a row of
// the thread grid read 16 consecutive 16-byte chunks of B (no bank
// conflicts, where the chapter pads a k-minor A instead).
constexpr int kRB = 128, kRK = 16, kRT = 256;

template <bool DBUF, bool VA, bool VB>
__global__ void __launch_bounds__(kRT) regtile_kernel(GemmArgs p, int tiles_n) {
  constexpr int NS = DBUF ? 2 : 1;
  constexpr int SAT = kRB + 4;  // LDS row stride of transposed A (k rows)
  using FetchA = SliceFetch<kRB, kRK, kRT, VA>;
  using FetchB = SliceFetch<kRK, kRB, kRT, VB>;
  __shared__ __attribute__((aligned(16))) float sAt[NS][kRK * SAT];
  __shared__ __attribute__((aligned(16))) float sB[NS][kRK * kRB];

  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int bx = blockIdx.x % tiles_n, by = blockIdx.x / tiles_n;
  const int m0 = by * kRB, n0 = bx * kRB;

  FetchA fa;
  FetchB fb;
  fa.init(p.A, p.lda, m0, 0, tid);
  fb.init(p.B, p.ldb, 0, n0, tid);

  auto store_slice = [&](int s) {
#pragma unroll
    for (int i = 0; i < FetchA::CH; ++i) {
      const int r = FetchA::wrow(tid, i), c = FetchA::wcol(tid);
#pragma unroll
      for (int e = 0; e < 4; ++e) sAt[s][(c + e) * SAT + r] = fa.v[i][e];
    }
#pragma unroll
    for (int i = 0; i < FetchB::CH; ++i)
      *reinterpret_cast<f32x4 *>(&sB[s][FetchB::wrow(tid, i) * kRB + FetchB::wcol(tid)]) =
          fb.v[i];
  };

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  // The operand vectors of step k + 1 are read from LDS before the 64 FMAs
  // of step k, so their latency hides behind arithmetic even with one wave
  // per SIMD.
  struct Frag {
    f32x4 a0, a1, b0, b1;
  };
  auto read_frag = [&](int s, int k, Frag &f) {
    f.a0 = *reinterpret_cast<const f32x4 *>(&sAt[s][k * SAT + 4 * ty]);
    f.a1 = *reinterpret_cast<const f32x4 *>(&sAt[s][k * SAT + 64 + 4 * ty]);
    f.b0 = *reinterpret_cast<const f32x4 *>(&sB[s][k * kRB + 4 * tx]);
    f.b1 = *reinterpret_cast<const f32x4 *>(&sB[s][k * kRB + 64 + 4 * tx]);
  };
  auto compute_slice = [&](int s) {
    Frag cur, nxt;
    read_frag(s, 0, cur);
#pragma unroll
    for (int k = 0; k < kRK; ++k) {
      if (k + 1 < kRK) read_frag(s, k + 1, nxt);
      const float a[8] = {cur.a0[0], cur.a0[1], cur.a0[2], cur.a0[3],
                          cur.a1[0], cur.a1[1], cur.a1[2], cur.a1[3]};
      const float b[8] = {cur.b0[0], cur.b0[1], cur.b0[2], cur.b0[3],
                          cur.b1[0], cur.b1[1], cur.b1[2], cur.b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      cur = nxt;
    }
  };

  const int nk = (p.K + kRK - 1) / kRK;
  if constexpr (!DBUF) {
    // load -> barrier -> compute -> barrier, as in the pages' tiled kernels.
    for (int t = 0; t < nk; ++t) {
      fa.load(p.M, p.K);
      fb.load(p.K, p.N);
      store_slice(0);
      __syncthreads();
      compute_slice(0);
      __syncthreads();
      fa.advance(0, kRK);
      fb.advance(kRK, 0);
    }
  } else {
    fa.load(p.M, p.K);
    fb.load(p.K, p.N);
    store_slice(0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      // Slice t + 1 into registers; past K the fetch reads nothing and
      // yields zeros, which land in the stage no one reads again.  Issued
      // before slice t's arithmetic, stored to LDS after it: the sched
      // barrier keeps the compiler from moving the LDS stores (and with
      // them the wait for the loads) above the arithmetic.
      fa.advance(0, kRK);
      fb.advance(kRK, 0);
      fa.load(p.M, p.K);
      fb.load(p.K, p.N);
      compute_slice(t & 1);
      __builtin_amdgcn_sched_barrier(0);
      store_slice((t + 1) & 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = n0 + (j < 4 ? 4 * tx + j : 64 + 4 * tx + j - 4);
      if (row < p.M && col < p.N) p.C[(long)row * p.ldc + col] = acc[i][j];
    }
  }
}

template <bool DBUF>
static void launch_regtile(const GemmArgs &p, bool va, bool vb, hipStream_t stream) {
  const int tiles_n = (p.N + kRB - 1) / kRB, tiles_m = (p.M + kRB - 1) / kRB;
  const dim3 grid((unsigned)((long)tiles_m * tiles_n)), block(kRT);
  if (va && vb)
    hipLaunchKernelGGL((regtile_kernel<DBUF, true, true>), grid, block, 0, stream, p, tiles_n);
  else if (va)
    hipLaunchKernelGGL((regtile_kernel<DBUF, true, false>), grid, block, 0, stream, p, tiles_n);
  else if (vb)
    hipLaunchKernelGGL((regtile_kernel<DBUF, false, true>), grid, block, 0, stream, p, tiles_n);
  else
    hipLaunchKernelGGL((regtile_kernel<DBUF, false, false>), grid, block, 0, stream, p, tiles_n);
}

hipError_t launch_valu(int rung, const GemmArgs &p, bool va, bool vb, hipStream_t stream) {
  switch (rung) {
    case 0: {
      const int tiles_n = (p.N + 15) / 16, tiles_m = (p.M + 15) / 16;
      hipLaunchKernelGGL(naive_kernel, dim3((unsigned)((long)tiles_m * tiles_n)), dim3(256), 0,
                         stream, p, tiles_n);
      break;
    }
    case 1: {
      const int tiles_n = (p.N + kTile - 1) / kTile, tiles_m = (p.M + kTile - 1) / kTile;
      const dim3 grid((unsigned)((long)tiles_m * tiles_n)), block(kTile * kTile);
      if (va && vb)
        hipLaunchKernelGGL((lds_tiled_kernel<true, true>), grid, block, 0, stream, p, tiles_n);
      else if (va)
        hipLaunchKernelGGL((lds_tiled_kernel<true, false>), grid, block, 0, stream, p, tiles_n);
      else if (vb)
        hipLaunchKernelGGL((lds_tiled_kernel<false, true>), grid, block, 0, stream, p, tiles_n);
      else
        hipLaunchKernelGGL((lds_tiled_kernel<false, false>), grid, block, 0, stream, p, tiles_n);
      break;
    }
    case 2: launch_regtile<false>(p, va, vb, stream); break;
    case 3: launch_regtile<true>(p, va, vb, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- C = beta C
// Over p.batch products: C = beta * C, or zeros when beta == 0 (C not read).
// This is the whole product when K == 0 or alpha == 0.
__global__ void __launch_bounds__(256) scale_kernel(GemmArgs p) {
  const long per = (long)p.M * p.N;
  const long total = per * p.batch;
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (long)gridDim.x * blockDim.x) {
    const long b = q / per, r = q % per;
    const long row = r / p.N, col = r % p.N;
    float *c = p.C + b * p.strideC + row * p.ldc + col;
    *c = p.beta == 0.f ? 0.f : p.beta * *c;
  }
}

hipError_t launch_scale(const GemmArgs &p, hipStream_t stream) {
  const long total = (long)p.M * p.N * p.batch;
  long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sgemm
