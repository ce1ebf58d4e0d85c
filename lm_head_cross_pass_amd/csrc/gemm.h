// bf16 / fp16 MFMA GEMM for gfx950: C[M, N] = A[M, K] * B[N, K]^T, fp32
// accumulation.
//
// Both operands are K-contiguous (row-major with leading dimensions lda, ldb,
// multiples of 8 elements, 16-byte aligned), which is the layout the
// v_mfma_f32_32x32x16_bf16 / _f16 operands want: each lane supplies 8
// consecutive k values of one row of A (or of B^T).
//
// Work decomposition:
// * a workgroup computes a BM x BN tile: 512 threads (8 waves as 2 x 4) for
//   256 x 256, 256 threads (4 waves as 2 x 2) for 128 x 128; each wave owns a
//   (BM / 2) x (BN / WAVES_N) sub-tile as a grid of 32 x 32 MFMA tiles
//   (128 x 64 per wave at 256 x 256: 128 fp32 accumulators per lane, which
//   leaves room for two waves per SIMD);
// * K is walked in steps of BK = 64 through a ring of LDS stages (two by
//   default): the tiles of the next step are copied from global memory
//   straight into LDS (buffer_load_dwordx4 ... lds, no staging registers)
//   while the MFMAs run on the current one; one barrier per step. (BK = 32
//   with a deeper ring is supported too; on these shapes it measured slower:
//   its 64-byte row segments halve the size of each memory request.)
// * an LDS tile row of BK bf16 is BK / 8 chunks of 16 bytes, stored without
//   padding with chunk c of row r at slot c ^ f(r) (f(r) = (r ^ (r >> 3)) & 7
//   for 8 chunks, ((r >> 1) ^ (r >> 3)) & 3 for 4), so that the 16-byte
//   fragment reads of 8 or 16 consecutive rows hit distinct banks; each
//   wave-wide copy instruction fills 1 KiB of rows, each lane fetching the
//   global chunk its slot holds;
// * rows beyond M / N lie outside the operand's buffer resource and k beyond
//   K is sent outside it, so both read as zero;
// * optional split-K: blockIdx enumerates (k-split, tile) pairs and each
//   split covers a contiguous range of K steps;
// * workgroup ids are remapped so that each of the 8 XCDs works on a
//   contiguous range of tiles (tiles that share A or B panels share an L2),
//   whatever the grid size.
//
// gemm_nt_bdir_kernel (further down) keeps this structure for A and takes B
// from a fragment-packed copy loaded straight into registers, so that only A
// passes through LDS.
//
// The epilogue is a functor (see linear_ce.hip): init() sets the accumulators
// before the K loop, run() stores them after it, and an epilogue with kRounds
// also rounds them every round_every K steps (round_tile() on each MFMA tile).
#pragma once

#include "common.h"

namespace lmx {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// The MFMA of an element format (Bf16 / F16 of common.h): fragments travel
// as raw 16-byte vectors and are reinterpreted here.
template <typename E> struct Mfma;
template <> struct Mfma<Bf16> {
  __device__ static f32x16_t run(const u32x4& a, const u32x4& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<F16> {
  __device__ static f32x16_t run(const u32x4& a, const u32x4& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};
typedef __attribute__((address_space(3))) void* lds_ptr_t;

#ifndef LMX_GEMM_BK
#define LMX_GEMM_BK 64
#endif
#ifndef LMX_GEMM_STAGES
#define LMX_GEMM_STAGES 2
#endif
constexpr int kGemmBK = LMX_GEMM_BK;          // K per step
constexpr int kGemmStages = LMX_GEMM_STAGES;  // LDS ring depth
constexpr int kRawBufFlags = 0x00020000;
constexpr int kOutOfRange = static_cast<int>(0x80000000u);   // a buffer offset that reads zero

struct GemmShape {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  int M, N, K;
  int a_rows;            // rows of A that exist (M may extend past them into zeros)
  int b_rows;            // rows of B that exist (N may extend past them into zeros)
  int tiles_m, tiles_n;
  int ksplit;            // number of K splits (1 = none)
  int ksteps_per_split;  // K steps per split
  // Optional (at_out != nullptr; gemm_nt_bdir_kernel with an epilogue that has
  // kTransposes): every A tile also written out transposed,
  // at_out[k * ld_at + m] = A[m][k] for k < K, by one of the tiles_n
  // workgroups that load it (the one whose tile_n is the K step modulo
  // tiles_n); columns m >= at_cols are left alone. Rows of A past M read as
  // zero, so columns M .. at_cols - 1 receive zeros.
  uint16_t* at_out;
  int64_t ld_at;
  int at_cols;
  // at_pk_ks > 0 (gemm_nt_bdir_kernel only): at_out is instead the packed copy
  // (layout below) of A^T, whose rows are A's K and whose K runs over A's rows,
  // with at_pk_ks K steps per block; ld_at is then unused.
  int at_pk_ks;
  // K steps between two roundings of the accumulators by the epilogue (its
  // round_tile(); only epilogues with kRounds), 0 for none: the weight-dtype
  // accumulation of grad_weight, one rounding per chunk of the K range.
  int round_every;
  // Optional (Bp != nullptr): B given as its fragment-packed copy (layout
  // below) with bp_ks K steps per 32-row block; the product then runs
  // gemm_nt_bdir_kernel, which loads B straight into registers. Blocks past
  // the ones holding rows < b_rows read as zero.
  const uint16_t* Bp;
  int bp_ks;
};

// Block tile BM x BN: 2 x 2 waves for 128 x 128, 2 x 4 waves for 256 x 256;
// every wave owns a (BM / WAVES_M) x (BN / WAVES_N) sub-tile.
template <int BM, int BN>
struct GemmCfg {
  static constexpr int WAVES_M = 2;
  static constexpr int WAVES_N = BN >= 256 ? 4 : 2;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ROWB = kGemmBK * 2;                  // bytes per LDS tile row
  static constexpr int CPR = kGemmBK / 8;                   // 16-byte chunks per row
  static constexpr int ROWS_PER_COPY = 1024 / ROWB;         // rows one copy instruction fills
  static_assert(kGemmStages >= 2, "at least two LDS stages");
  // LDS: A stages 0..3, then B stages 0..3
  static constexpr int A_STAGE = BM * ROWB;
  static constexpr int B_STAGE = BN * ROWB;
  static constexpr int B_BASE = kGemmStages * A_STAGE;
  static constexpr int LDS_BYTES = kGemmStages * (A_STAGE + B_STAGE);
  static constexpr int A_LOADS = BM / ROWS_PER_COPY / NWAVES;   // copy instructions per wave
  static constexpr int B_LOADS = BN / ROWS_PER_COPY / NWAVES;
  static constexpr int LOADS = A_LOADS + B_LOADS;
};

// Accumulators set to zero (the init() of most epilogues).
template <int FM, int FN>
__device__ __forceinline__ void acc_zero(f32x16_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Slot swizzle of an LDS row of CPR 16-byte chunks (CPR = 4 or 8): 8 or 16
// consecutive rows reading the same logical chunk hit distinct bank groups.
template <int CPR>
__device__ __forceinline__ int lds_swz(int r) {
  if constexpr (CPR == 8) return (r ^ (r >> 3)) & 7;
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

// Accumulator coordinates: element r of MFMA tile (i, j) of this lane.
struct AccCoord {
  int row0, col0;   // wave sub-tile origin inside the block tile
  int lane;
  __device__ int row(int i, int r) const {
    return row0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  __device__ int col(int j) const { return col0 + j * 32 + (lane & 31); }
};

// Buffer resource over up to `rows` rows of a row-major matrix starting at
// row0; rows past the matrix end are left out, so they read as zero and
// writes to them are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t row0,
                                                            int64_t rows_left, int rows,
                                                            int64_t ld_bytes) {
  const int64_t n = rows_left < rows ? rows_left : rows;
  const int64_t bytes = n > 0 ? n * ld_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(base) + row0 * ld_bytes), 0,
      static_cast<int>(bytes), kRawBufFlags);
}

// Maps blockIdx.x to (split, tile_m, tile_n): tiles of one XCD are contiguous,
// and within that range the m index runs fastest. The hardware hands workgroup
// b to XCD b % 8, so XCD x receives workgroups x, x + 8, ...: nb / 8 of them,
// one more for the first nb % 8 XCDs; they take the consecutive work items
// from x (nb / 8) + min(x, nb % 8) on, for any grid size.
__device__ __forceinline__ void gemm_tile_of_block(const GemmShape& g, int& split, int& tm,
                                                   int& tn) {
  const int nb = gridDim.x;
  const int x = static_cast<int>(blockIdx.x) % 8, k = static_cast<int>(blockIdx.x) / 8;
  const int q = nb / 8, r = nb % 8;
  const int b = x * q + (x < r ? x : r) + k;
  const int tiles = g.tiles_m * g.tiles_n;
  split = b / tiles;
  const int t = b % tiles;
  // tiles in groups of kGroupM tile rows, tile row fastest within a group: the
  // 32 workgroups an XCD runs at once share 4 A bands and 8 B bands instead of
  // one B band and 32 A bands of a tall grid (4 measured faster than 2, 3, 6, 8 and
  // 16 on the 126976-row grad_weight product). The rows past the last whole
  // group are a group of their own (all of them when tiles_m < kGroupM).
  constexpr int kGroupM = 4;
  const int full = g.tiles_m / kGroupM * kGroupM;
  if (t < full * g.tiles_n) {
    const int per_group = kGroupM * g.tiles_n;
    const int w = t % per_group;
    tm = t / per_group * kGroupM + w % kGroupM;
    tn = w / kGroupM;
  } else {
    const int w = t - full * g.tiles_n, rem = g.tiles_m - full;
    tm = full + w % rem;
    tn = w / rem;
  }
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone): at most N of this
// wave's vector memory operations, i.e. of its copies into LDS, are still in
// flight. Copies complete in issue order, so this waits for all but the last
// N. The barrier that follows makes every wave's copies visible.
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int V> struct IntC { static constexpr int value = V; };

// Threads of the workgroup for a tile size (a plain function, so the launch
// bounds below read it without template commas).
template <int AREA>
constexpr int gemm_threads() { return AREA >= 256 * 256 ? 512 : 256; }

// The pieces of the main loop are device functions rather than lambdas: a
// lambda is compiled for the host too, where the buffer-resource type and the
// amdgcn builtins do not exist.

// Copies one K step of A and B into LDS stage `stage`. Lane l of a copy
// instruction fills LDS slot (l & 3) of row (l >> 2) of a 16-row block, i.e.
// it fetches global chunk (l & 3) ^ f(row); per lane only the row / chunk part
// of the offset is kept, the K step's byte offset goes in the scalar offset.
template <typename C, bool FULLK>
__device__ __forceinline__ void gemm_copy_stage(char* smem, __amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rb, const int* a_voff,
                                                const int* b_voff, const int* a_kc,
                                                const int* b_kc, int kbase, int stage, int wave,
                                                int K) {
  char* sa = smem + stage * C::A_STAGE + wave * C::A_LOADS * 1024;
  char* sb = smem + C::B_BASE + stage * C::B_STAGE + wave * C::B_LOADS * 1024;
  if (FULLK || kbase + kGemmBK <= K) {   // no chunk of this step lies past K
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(sa + i * 1024), 16,
                                               a_voff[i], kbase * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(sb + i * 1024), 16,
                                               b_voff[i], kbase * 2, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(sa + i * 1024), 16,
                                               kbase + a_kc[i] < K ? a_voff[i] : kOutOfRange,
                                               kbase * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(sb + i * 1024), 16,
                                               kbase + b_kc[i] < K ? b_voff[i] : kOutOfRange,
                                               kbase * 2, 0, 0);
  }
}

// Reads the fragments of k slice KK from LDS. A stage is a power-of-two byte
// size and every offset lies inside stage 0, so switching stage and slice is
// one XOR with a uniform value.
template <typename C, int KK>
__device__ __forceinline__ void gemm_load_frags(const char* smem, const int* a_off,
                                                const int* b_off, int stage_bytes,
                                                u32x4* af, u32x4* bfr) {
  const int flip = stage_bytes | (KK << 5);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    af[i] = *reinterpret_cast<const u32x4*>(smem + (a_off[i] ^ flip));
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    bfr[j] = *reinterpret_cast<const u32x4*>(smem + (b_off[j] ^ flip));
}

// Writes the operand tile of one K step (R rows x kGemmBK in the LDS stage at
// `st`, 16-byte pieces of a row XOR-swizzled) transposed to
// out[(kbase + kk) * ld + r0 + r] for kbase + kk < K and r0 + r < cols. A
// thread takes an 8 x 8 block (8 rows, one 16-byte piece of each), transposes
// it in registers with byte permutes and stores 8 pieces of 8 rows each.
template <typename C, int R>
__device__ __forceinline__ void gemm_store_tile_transposed(const char* st, uint16_t* out,
                                                           int64_t ld, int r0, int cols,
                                                           int kbase, int K) {
  constexpr int RB = R / 8;                   // 8-row blocks
  constexpr int BLOCKS = RB * (kGemmBK / 8);
  for (int t = static_cast<int>(threadIdx.x); t < BLOCKS; t += C::THREADS) {
    const int b = t % RB, c = t / RB;         // rows 8b .. 8b + 7, k piece c
    // cols and K are multiples of 8: a block is wholly inside or outside
    if (r0 + 8 * b + 8 > cols || kbase + 8 * c >= K) continue;
    u32x4 in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * b + i;
      in[i] = *reinterpret_cast<const u32x4*>(st + r * C::ROWB + ((c ^ lds_swz<C::CPR>(r)) << 4));
    }
    // out piece j (k = 8c + j) holds element j of every row: word q of it is
    // (row 2q, row 2q + 1) at k; element j of a row is half (j & 1) of word j / 2
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = in[2 * q][j >> 1], hi = in[2 * q + 1][j >> 1];
        // selector bytes: low half of `lo`-source then low half of `hi`-source
        // (j even), or the high halves (j odd); v_perm_b32 indexes bytes of
        // {src0, src1} as 7..4 = src0, 3..0 = src1
        o[q] = (j & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                       : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
      *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(kbase + 8 * c + j) * ld + r0 + 8 * b) =
          o;
    }
  }
}

template <typename C, typename E>
__device__ __forceinline__ void gemm_mfma_slice(f32x16_t (&acc)[C::FM][C::FN], const u32x4* af,
                                                const u32x4* bfr) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = Mfma<E>::run(af[i], bfr[j], acc[i][j]);
}

// Schedule hints for one k slice (FM + FN fragment reads of slice k + 1, FM x FN
// MFMAs of slice k). SCHED 0: one LDS read, then a few MFMAs, repeated.
// SCHED 1: MFMA and LDS read alternate until the reads are issued, then the
// remaining MFMAs (the reads start earlier; measured 3% faster over a whole
// linear-CE call on 256 x 256 tiles).
template <typename C, int SCHED>
__device__ __forceinline__ void gemm_interleave_hint() {
  constexpr int R = C::FM + C::FN, M = C::FM * C::FN;
  if constexpr (SCHED == 0) {
    constexpr int PER = (M + R - 1) / R;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
    }
  } else {
    static_assert(M >= R, "more MFMAs than fragment reads per slice");
#pragma unroll
    for (int q = 0; q < R; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M - R, 0);
  }
}

// E: the operands' 16-bit element format (Bf16 or F16 of common.h).
// FULLK: K is a multiple of the K step (no step reaches past K), so the
// copies need no per-chunk range test.
template <int BM, int BN, typename Epi, int SCHED, typename E, bool FULLK>
__global__ __launch_bounds__(gemm_threads<BM * BN>(), 1) void gemm_nt_kernel(GemmShape g,
                                                                            Epi epi) {
  using C = GemmCfg<BM, BN>;
  static_assert(C::THREADS == gemm_threads<BM * BN>(), "thread count");
  static_assert((C::A_STAGE & (C::A_STAGE - 1)) == 0 && C::A_STAGE == C::B_STAGE,
                "stage sizes must be equal powers of two");
  __shared__ __align__(16) char smem[C::LDS_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps LDS bases scalar
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  int split, tm, tn;
  gemm_tile_of_block(g, split, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int ksteps = (g.K + kGemmBK - 1) / kGemmBK;
  const int kb = split * g.ksteps_per_split;
  int ke = kb + g.ksteps_per_split;
  if (ke > ksteps) ke = ksteps;

  const __amdgpu_buffer_rsrc_t ra = rows_rsrc(g.A, m0, g.a_rows - m0, BM, g.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = rows_rsrc(g.B, n0, g.b_rows - n0, BN, g.ldb * 2);

  const int lrow = lane / C::CPR;
  const int lslot = lane % C::CPR;
  int a_voff[C::A_LOADS], b_voff[C::B_LOADS], a_kc[C::A_LOADS], b_kc[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int r = (wave * C::A_LOADS + i) * C::ROWS_PER_COPY + lrow;
    a_kc[i] = (lslot ^ lds_swz<C::CPR>(r)) * 8;
    a_voff[i] = static_cast<int>((static_cast<int64_t>(r) * g.lda + a_kc[i]) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int r = (wave * C::B_LOADS + i) * C::ROWS_PER_COPY + lrow;
    b_kc[i] = (lslot ^ lds_swz<C::CPR>(r)) * 8;
    b_voff[i] = static_cast<int>((static_cast<int64_t>(r) * g.ldb + b_kc[i]) * 2);
  }

  // accumulators: zero, or a starting value the epilogue loads
  const AccCoord ac{wm * C::WM, wn * C::WN, lane};
  f32x16_t acc[C::FM][C::FN];
  epi.template init<BM, BN, C::FM, C::FN>(acc, ac, m0, n0, g);

  // Fragment reads: lane l reads 16 bytes of row (l & 31) of each 32-row MFMA
  // tile, k chunk 2 kk + (l >> 5); the byte offset of slice kk is the slice-0
  // offset XOR (kk << 5).
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  int a_off[C::FM], b_off[C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int r = wm * C::WM + i * 32 + frag_row;
    a_off[i] = r * C::ROWB + ((frag_half ^ lds_swz<C::CPR>(r)) << 4);
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int r = wn * C::WN + j * 32 + frag_row;
    b_off[j] = C::B_BASE + r * C::ROWB + ((frag_half ^ lds_swz<C::CPR>(r)) << 4);
  }
  u32x4 fa0[C::FM], fb0[C::FN], fa1[C::FM], fb1[C::FN];
  static_assert(kGemmBK == 32 || kGemmBK == 64, "two or four 16-wide k slices per step");
  constexpr int AHEAD = kGemmStages - 1;   // steps in flight ahead of the one computed

  // Prologue: steps kb .. kb + AHEAD - 1 in flight, then step kb landed.
#pragma unroll
  for (int s = 0; s < AHEAD; ++s) {
    if (kb + s < ke) {
      gemm_copy_stage<C, FULLK>(smem, ra, rb, a_voff, b_voff, a_kc, b_kc,
                         __builtin_amdgcn_readfirstlane((kb + s) * kGemmBK), s, wave, g.K);
    }
  }
  if (kb < ke) {
    if (kb + AHEAD <= ke) wait_copies<(AHEAD - 1) * C::LOADS>(); else wait_copies<0>();
    __syncthreads();
    gemm_load_frags<C, 0>(smem, a_off, b_off, 0, fa0, fb0);
  }
  // (ks + 1) % round_every, kept as a counter (the modulo of a runtime divisor
  // costs some twenty scalar instructions a step)
  [[maybe_unused]] int phase = 1;
  if constexpr (Epi::kRounds)
    if (g.round_every > 0) phase = __builtin_amdgcn_readfirstlane((kb + 1) % g.round_every);
  for (int ks = kb; ks < ke; ++ks) {
    const int t = ks - kb;
    const int cur_bytes = __builtin_amdgcn_readfirstlane((t % kGemmStages) * C::A_STAGE);
    const int nxt_bytes = __builtin_amdgcn_readfirstlane(((t + 1) % kGemmStages) * C::A_STAGE);
    // the stage that step ks - 1 used is free (everyone passed the barrier
    // after reading it): refill it with step ks + AHEAD
    if (ks + AHEAD < ke) {
      gemm_copy_stage<C, FULLK>(smem, ra, rb, a_voff, b_voff, a_kc, b_kc,
                         __builtin_amdgcn_readfirstlane((ks + AHEAD) * kGemmBK),
                         __builtin_amdgcn_readfirstlane((t + AHEAD) % kGemmStages), wave, g.K);
    }
    gemm_load_frags<C, 1>(smem, a_off, b_off, cur_bytes, fa1, fb1);
    gemm_mfma_slice<C, E>(acc, fa0, fb0);
    gemm_interleave_hint<C, SCHED>();
    if constexpr (kGemmBK == 64) {
      gemm_load_frags<C, 2>(smem, a_off, b_off, cur_bytes, fa0, fb0);
      gemm_mfma_slice<C, E>(acc, fa1, fb1);
      gemm_interleave_hint<C, SCHED>();
      gemm_load_frags<C, 3>(smem, a_off, b_off, cur_bytes, fa1, fb1);
      gemm_mfma_slice<C, E>(acc, fa0, fb0);
      gemm_interleave_hint<C, SCHED>();
    }
    gemm_mfma_slice<C, E>(acc, fa1, fb1);
    if constexpr (Epi::kRounds) {
      // a chunk boundary inside the K range: the epilogue rounds the running
      // sums (the last boundary is the epilogue's own rounding)
      if (g.round_every > 0 && phase == 0 && ks + 1 < ke) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) epi.round_tile(acc[i][j]);
      }
      if (++phase == g.round_every) phase = 0;
    }
    if (ks + 1 < ke) {
      // step ks + 1 landed: the copies issued after it (up to AHEAD - 1 steps)
      // may still be in flight
      if (ks + AHEAD < ke) wait_copies<(AHEAD - 1) * C::LOADS>(); else wait_copies<0>();
      __syncthreads();
      gemm_load_frags<C, 0>(smem, a_off, b_off, nxt_bytes, fa0, fb0);
    }
  }
  epi.template run<BM, BN, C::FM, C::FN>(acc, ac, m0, n0, split, g,
                                         reinterpret_cast<uint16_t*>(smem));
}

// ---------------------------------------------------------------- packed B
//
// Fragment-packed copy of a K-contiguous operand M [R, K]: 32-row blocks, each
// a run of K steps of 64, each step four 1 KiB fragments (one per 16-wide k
// slice) laid out the way the 32 x 32 x 16 MFMA takes its B operand. Element
// e of lane l of slice q of step s of block b is M[32 b + (l & 31)][64 s +
// 16 q + 8 (l >> 5) + e] (zero past R or K), stored at
//   packed[((b * KS + s) * 4 + q) * 512 + 8 l + e].
// A wave loads each B fragment as one fully coalesced 1 KiB read straight
// into registers, so B takes no LDS traffic: with B staged in LDS, its
// direct-to-LDS writes and the fragment reads of both operands are what the
// K loop waits on; packed, a step moves 160 KiB through LDS instead of 256.
constexpr int kPackedRows = 32;          // rows per block
constexpr int kPackedStepBytes = 4096;   // one K step of one block

template <typename C, bool FULLK>
__device__ __forceinline__ void gemm_copy_a(char* smem, __amdgpu_buffer_rsrc_t ra,
                                            const int* a_voff, const int* a_kc, int kbase,
                                            int stage, int wave, int K) {
  char* sa = smem + stage * C::A_STAGE + wave * C::A_LOADS * 1024;
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ra, (lds_ptr_t)(sa + i * 1024), 16,
        (FULLK || kbase + a_kc[i] < K) ? a_voff[i] : kOutOfRange, kbase * 2, 0, 0);
}

// This wave's B fragments of slice KK of the K step at byte offset soff.
template <typename C, int KK>
__device__ __forceinline__ void gemm_load_b_slice(u32x4 (&b)[C::FN][4],
                                                  __amdgpu_buffer_rsrc_t rb, const int* b_voff,
                                                  int soff) {
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    b[j][KK] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_voff[j] + KK * 1024, soff, 0));
}

template <typename C, int KK>
__device__ __forceinline__ void gemm_load_a_frags(const char* smem, const int* a_off,
                                                  int stage_bytes, u32x4* af) {
  const int flip = stage_bytes | (KK << 5);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    af[i] = *reinterpret_cast<const u32x4*>(smem + (a_off[i] ^ flip));
}

template <typename C, typename E, int KK>
__device__ __forceinline__ void gemm_mfma_slice_b(f32x16_t (&acc)[C::FM][C::FN], const u32x4* af,
                                                  const u32x4 (&b)[C::FN][4]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = Mfma<E>::run(af[i], b[j][KK], acc[i][j]);
}

// Writes the A tile of one K step (R rows x 64 k in the LDS stage at `st`,
// row pieces swizzled as the copies left them) into the packed copy of A^T
// (rows = k, K = A's rows, ks K steps per block), for tile rows r0 + r <
// cols and k below K rounded up to a whole block (the k past K read as zero).
// As in gemm_store_tile_transposed, a thread transposes an 8 x 8 block in
// registers; piece j of it (k = kbase + 8c + j, rows r0 + 8b .. + 7) is
// lane (k % 32) + 32 ((r0 + 8b) / 8 % 2) of slice (r0 + 8b) / 16 % 4 of step
// (r0 + 8b) / 64 of block k / 32, so the 8 pieces fill 128 contiguous bytes.
template <typename C, int R>
__device__ __forceinline__ void gemm_store_tile_packed_t(const char* st, uint16_t* out, int ks,
                                                        int r0, int cols, int kbase, int K) {
  constexpr int RB = R / 8;
  constexpr int BLOCKS = RB * (kGemmBK / 8);
  const int k_end = (K + kPackedRows - 1) / kPackedRows * kPackedRows;
  for (int t = static_cast<int>(threadIdx.x); t < BLOCKS; t += C::THREADS) {
    const int b = t % RB, c = t / RB;
    if (r0 + 8 * b + 8 > cols || kbase + 8 * c >= k_end) continue;
    u32x4 in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * b + i;
      in[i] = *reinterpret_cast<const u32x4*>(st + r * C::ROWB + ((c ^ lds_swz<C::CPR>(r)) << 4));
    }
    const int v0 = r0 + 8 * b, k0 = kbase + 8 * c;
    uint16_t* dst = out + ((static_cast<int64_t>(k0 / kPackedRows) * ks + v0 / kGemmBK) * 4 +
                           (v0 / 16) % 4) * 512 +
                    ((k0 % kPackedRows) + 32 * ((v0 / 8) % 2)) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = in[2 * q][j >> 1], hi = in[2 * q + 1][j >> 1];
        o[q] = (j & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                       : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
      *reinterpret_cast<u32x4*>(dst + j * 8) = o;
    }
  }
}

// One k slice: MFMA and A fragment read alternate until the FM reads of the
// next slice are issued, then the remaining MFMAs.
template <typename C>
__device__ __forceinline__ void gemm_hint_a_slice() {
  constexpr int R = C::FM, M = C::FM * C::FN;
#pragma unroll
  for (int q = 0; q < R; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, M - R, 0);
}

// C[M, N] = A[M, K] B[N, K]^T with A staged in LDS as in gemm_nt_kernel and
// B read from its packed copy g.Bp. Each k slice's B fragments are reloaded
// for the next K step as soon as that slice's MFMAs are issued, so every load
// has a whole step to land and B needs one set of registers. Every step
// issues the same copies (past the last step, a copy of the last step into
// the stage that is free), which keeps the compiler's wait counts exact. The
// operand formats and the order of the MFMAs over k are those of
// gemm_nt_kernel, so both kernels give the same bits.
template <int BM, int BN, typename Epi, typename E, bool FULLK>
__global__ __launch_bounds__(gemm_threads<BM * BN>(), 1) void gemm_nt_bdir_kernel(GemmShape g,
                                                                                 Epi epi) {
  using C = GemmCfg<BM, BN>;
  static_assert(C::THREADS == gemm_threads<BM * BN>(), "thread count");
  static_assert(kGemmBK == 64 && kGemmStages == 2, "packed steps are 64 wide; two A stages");
  static_assert((C::A_STAGE & (C::A_STAGE - 1)) == 0, "stage size must be a power of two");
  static_assert(C::WN % kPackedRows == 0, "a wave's columns are whole packed blocks");
  __shared__ __align__(16) char smem[C::LDS_BYTES];   // A stages; the epilogue may stage all of it
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  int split, tm, tn;
  gemm_tile_of_block(g, split, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int ksteps = (g.K + kGemmBK - 1) / kGemmBK;
  const int kb = split * g.ksteps_per_split;
  int ke = kb + g.ksteps_per_split;
  if (ke > ksteps) ke = ksteps;

  const __amdgpu_buffer_rsrc_t ra = rows_rsrc(g.A, m0, g.a_rows - m0, BM, g.lda * 2);
  // this wave's FN packed blocks of B (blocks past the existing rows read zero)
  const int nb0 = __builtin_amdgcn_readfirstlane((n0 + wn * C::WN) / kPackedRows);
  int nbl = (g.b_rows + kPackedRows - 1) / kPackedRows - nb0;
  if (nbl > C::FN) nbl = C::FN;
  if (nbl < 0) nbl = 0;
  const int nrec = __builtin_amdgcn_readfirstlane(nbl * g.bp_ks * kPackedStepBytes);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(g.Bp) + static_cast<int64_t>(nb0) * g.bp_ks * (kPackedStepBytes / 2),
      0, nrec, kRawBufFlags);

  const int lrow = lane / C::CPR;
  const int lslot = lane % C::CPR;
  int a_voff[C::A_LOADS], a_kc[C::A_LOADS], b_voff[C::FN];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int r = (wave * C::A_LOADS + i) * C::ROWS_PER_COPY + lrow;
    a_kc[i] = (lslot ^ lds_swz<C::CPR>(r)) * 8;
    a_voff[i] = static_cast<int>((static_cast<int64_t>(r) * g.lda + a_kc[i]) * 2);
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) b_voff[j] = lane * 16 + j * g.bp_ks * kPackedStepBytes;

  const AccCoord ac{wm * C::WM, wn * C::WN, lane};
  f32x16_t acc[C::FM][C::FN];
  epi.template init<BM, BN, C::FM, C::FN>(acc, ac, m0, n0, g);

  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  int a_off[C::FM];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int r = wm * C::WM + i * 32 + frag_row;
    a_off[i] = r * C::ROWB + ((frag_half ^ lds_swz<C::CPR>(r)) << 4);
  }
  u32x4 fa0[C::FM], fa1[C::FM];
  u32x4 bc[C::FN][4];
  constexpr int BLOADS = C::FN * 4;   // B loads per step

  if (kb < ke) {
    const int s0 = __builtin_amdgcn_readfirstlane(kb * kPackedStepBytes);
    gemm_load_b_slice<C, 0>(bc, rb, b_voff, s0);
    gemm_load_b_slice<C, 1>(bc, rb, b_voff, s0);
    gemm_load_b_slice<C, 2>(bc, rb, b_voff, s0);
    gemm_load_b_slice<C, 3>(bc, rb, b_voff, s0);
    gemm_copy_a<C, FULLK>(smem, ra, a_voff, a_kc, __builtin_amdgcn_readfirstlane(kb * kGemmBK), 0,
                          wave, g.K);
    wait_copies<0>();
    __syncthreads();
    gemm_load_a_frags<C, 0>(smem, a_off, 0, fa0);
  }
  // (ks + 1) % round_every, kept as a counter (the modulo of a runtime divisor
  // costs some twenty scalar instructions a step)
  [[maybe_unused]] int phase = 1;
  if constexpr (Epi::kRounds)
    if (g.round_every > 0) phase = __builtin_amdgcn_readfirstlane((kb + 1) % g.round_every);
  for (int ks = kb; ks < ke; ++ks) {
    const int t = ks - kb;
    const int cur = __builtin_amdgcn_readfirstlane((t & 1) * C::A_STAGE);
    const int nxt = __builtin_amdgcn_readfirstlane(((t + 1) & 1) * C::A_STAGE);
    // A of step ks + 1 into the stage step ks - 1 used
    gemm_copy_a<C, FULLK>(smem, ra, a_voff, a_kc,
                          __builtin_amdgcn_readfirstlane((ks + 1 < ke ? ks + 1 : ks) * kGemmBK),
                          (t + 1) & 1, wave, g.K);
    __builtin_amdgcn_sched_barrier(0);
    // this step's A tile written out transposed, when this workgroup's turn:
    // at the start of the step, so the stores are older than the step's B
    // loads (the waits for those never wait for the stores) and the other
    // wave on each SIMD keeps the matrix core busy meanwhile
    if constexpr (Epi::kTransposes) {
      if (g.at_out != nullptr && ks % g.tiles_n == tn) {
        if (g.at_pk_ks > 0)
          gemm_store_tile_packed_t<C, BM>(smem + cur, g.at_out, g.at_pk_ks, m0, g.at_cols,
                                          ks * kGemmBK, g.K);
        else
          gemm_store_tile_transposed<C, BM>(smem + cur, g.at_out, g.ld_at, m0, g.at_cols,
                                            ks * kGemmBK, g.K);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // B of step ks + 1, slice by slice as each slice's registers free up (the
    // last step reloads its own: in bounds and unused)
    const int sn = __builtin_amdgcn_readfirstlane((ks + 1 < ke ? ks + 1 : ks) * kPackedStepBytes);
    gemm_load_a_frags<C, 1>(smem, a_off, cur, fa1);
    gemm_mfma_slice_b<C, E, 0>(acc, fa0, bc);
    gemm_hint_a_slice<C>();
    gemm_load_b_slice<C, 0>(bc, rb, b_voff, sn);
    __builtin_amdgcn_sched_barrier(0);
    gemm_load_a_frags<C, 2>(smem, a_off, cur, fa0);
    gemm_mfma_slice_b<C, E, 1>(acc, fa1, bc);
    gemm_hint_a_slice<C>();
    gemm_load_b_slice<C, 1>(bc, rb, b_voff, sn);
    __builtin_amdgcn_sched_barrier(0);
    gemm_load_a_frags<C, 3>(smem, a_off, cur, fa1);
    gemm_mfma_slice_b<C, E, 2>(acc, fa0, bc);
    gemm_hint_a_slice<C>();
    gemm_load_b_slice<C, 2>(bc, rb, b_voff, sn);
    __builtin_amdgcn_sched_barrier(0);
    gemm_mfma_slice_b<C, E, 3>(acc, fa1, bc);
    gemm_load_b_slice<C, 3>(bc, rb, b_voff, sn);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (Epi::kRounds) {
      if (g.round_every > 0 && phase == 0 && ks + 1 < ke) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) epi.round_tile(acc[i][j]);
      }
      if (++phase == g.round_every) phase = 0;
    }
    if (ks + 1 < ke) {
      // A of step ks + 1 landed (this step's B loads, issued after it, may
      // still be in flight)
      wait_copies<BLOADS>();
      __syncthreads();
      gemm_load_a_frags<C, 0>(smem, a_off, nxt, fa0);
    }
  }
  // the last step's copy and B loads done, every wave past its last LDS read
  wait_copies<0>();
  __syncthreads();
  epi.template run<BM, BN, C::FM, C::FN>(acc, ac, m0, n0, split, g,
                                         reinterpret_cast<uint16_t*>(smem));
}

}  // namespace lmx
