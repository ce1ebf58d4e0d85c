// bf16 MFMA GEMM for gfx950: C[M, N] = A[M, K] * B[N, K]^T, fp32 accumulation.
//
// Both operands are K-contiguous (row-major with leading dimensions lda, ldb,
// multiples of 8 elements, 16-byte aligned), which is the layout the
// v_mfma_f32_32x32x16_bf16 operands want: each lane supplies 8 consecutive k
// values of one row of A (or of B^T).
//
// Work decomposition:
// * a workgroup of 256 threads (4 waves as 2 x 2) computes a BM x BN tile,
//   each wave a (BM/2) x (BN/2) sub-tile as a grid of 32 x 32 MFMA tiles;
// * K is walked in steps of 64: the next step's A and B tiles are fetched
//   from global memory into registers (128-bit buffer loads, rows beyond M/N
//   read as zero by the buffer resource, k beyond K zeroed) while the MFMAs
//   run on the current step held in LDS, then written to the other half of a
//   double-buffered LDS stage; one barrier per step;
// * LDS rows are padded to 72 elements (144 bytes) so the 16-byte fragment
//   reads of 16 consecutive rows fall in distinct banks;
// * optional split-K: blockIdx enumerates (k-split, tile) pairs and each
//   split covers a contiguous range of K steps;
// * workgroup ids are remapped so that each of the 8 XCDs works on a
//   contiguous range of tiles (tiles that share A or B panels share an L2).
//
// The epilogue is a functor called with the accumulators; see Epi* below and
// in linear_ce.hip.
#pragma once

#include "common.h"

namespace lmx {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kGemmBK = 64;
constexpr int kGemmLdsK = kGemmBK + 8;   // padded LDS row, elements

struct GemmShape {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  int M, N, K;
  int tiles_m, tiles_n;
  int ksplit;            // number of K splits (1 = none)
  int ksteps_per_split;  // K steps of 64 per split
};

template <int BM, int BN>
struct GemmCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int CPR = kGemmBK / 8;                    // 16-byte chunks per row
  static constexpr int A_CH = BM * CPR / kGemmThreads;       // chunks per thread
  static constexpr int B_CH = BN * CPR / kGemmThreads;
  static constexpr int STAGE = (BM + BN) * kGemmLdsK;       // elements per stage
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
};

// Accumulator coordinates: element r of MFMA tile (i, j) of this lane.
struct AccCoord {
  int row0, col0;   // wave sub-tile origin inside the block tile
  int lane;
  __device__ int row(int i, int r) const {
    return row0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  __device__ int col(int j) const { return col0 + j * 32 + (lane & 31); }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t panel_rsrc(const uint16_t* base, int64_t row0,
                                                             int rows_left, int rows, int64_t ld) {
  const int64_t n = rows_left < rows ? rows_left : rows;
  const int64_t bytes = n > 0 ? n * ld * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + row0 * ld), 0,
                                           static_cast<int>(bytes), 0x00020000);
}

// Maps blockIdx.x to (split, tile_m, tile_n): tiles of one XCD are contiguous,
// and within that range the m index runs fastest.
__device__ __forceinline__ void gemm_tile_of_block(const GemmShape& g, int& split, int& tm,
                                                   int& tn) {
  const int nb = gridDim.x;
  int b = blockIdx.x;
  if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
  const int tiles = g.tiles_m * g.tiles_n;
  split = b / tiles;
  const int t = b % tiles;
  tm = t % g.tiles_m;
  tn = t / g.tiles_m;
}

template <int BM, int BN, typename Epi>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_nt_kernel(GemmShape g, Epi epi) {
  using C = GemmCfg<BM, BN>;
  __shared__ __align__(16) uint16_t smem[C::LDS_BYTES / 2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int split, tm, tn;
  gemm_tile_of_block(g, split, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int ksteps = (g.K + kGemmBK - 1) / kGemmBK;
  const int kb = split * g.ksteps_per_split;
  int ke = kb + g.ksteps_per_split;
  if (ke > ksteps) ke = ksteps;

  const __amdgpu_buffer_rsrc_t ra = panel_rsrc(g.A, m0, g.M - m0, BM, g.lda);
  const __amdgpu_buffer_rsrc_t rb = panel_rsrc(g.B, n0, g.N - n0, BN, g.ldb);

  u32x4 ra_regs[C::A_CH], rb_regs[C::B_CH];
  auto fetch = [&](int ks) {
    const int kbase = ks * kGemmBK;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int q = tid + i * kGemmThreads;
      const int r = q / C::CPR, kc = q % C::CPR;
      const int k = kbase + kc * 8;
      const int off = static_cast<int>((static_cast<int64_t>(r) * g.lda + k) * 2);
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      ra_regs[i] = (k < g.K) ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int q = tid + i * kGemmThreads;
      const int r = q / C::CPR, kc = q % C::CPR;
      const int k = kbase + kc * 8;
      const int off = static_cast<int>((static_cast<int64_t>(r) * g.ldb + k) * 2);
      u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
      rb_regs[i] = (k < g.K) ? v : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stash = [&](int stage) {
    uint16_t* sa = smem + stage * C::STAGE;
    uint16_t* sb = sa + BM * kGemmLdsK;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int q = tid + i * kGemmThreads;
      const int r = q / C::CPR, kc = q % C::CPR;
      *reinterpret_cast<u32x4*>(sa + r * kGemmLdsK + kc * 8) = ra_regs[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int q = tid + i * kGemmThreads;
      const int r = q / C::CPR, kc = q % C::CPR;
      *reinterpret_cast<u32x4*>(sb + r * kGemmLdsK + kc * 8) = rb_regs[i];
    }
  };

  f32x16_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (kb < ke) {
    fetch(kb);
    stash(0);
    __syncthreads();
  }
  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  for (int ks = kb; ks < ke; ++ks) {
    const int cur = (ks - kb) & 1;
    const bool more = ks + 1 < ke;
    if (more) fetch(ks + 1);
    const uint16_t* sa = smem + cur * C::STAGE;
    const uint16_t* sb = sa + BM * kGemmLdsK;
#pragma unroll
    for (int kk = 0; kk < kGemmBK / 16; ++kk) {
      bf16x8_t af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm * C::WM + i * 32 + frag_row;
        af[i] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4*>(sa + r * kGemmLdsK + kk * 16 + frag_k));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int r = wn * C::WN + j * 32 + frag_row;
        bfr[j] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4*>(sb + r * kGemmLdsK + kk * 16 + frag_k));
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) stash(cur ^ 1);
    __syncthreads();
  }
  AccCoord ac{wm * C::WM, wn * C::WN, lane};
  epi.template run<BM, BN, C::FM, C::FN>(acc, ac, m0, n0, split, g, smem);
}

}  // namespace lmx
