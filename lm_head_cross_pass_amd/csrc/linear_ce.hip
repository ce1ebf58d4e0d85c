// Chunked linear cross-entropy: logits = inputs @ weight^T in row chunks, the
// cross-entropy loss and logits gradient per chunk, grad_inputs written per
// chunk and grad_weight accumulated across chunks (greyhound functional API
// page, "chunked_linear_loss" and "chunked_linear_cross_entropy").
//
// Per call:   count valid targets (global N, needed before any gradient is
//             scaled).
// Per chunk of C rows (r0 .. r0 + C'):
//   1. X_c packed (gemm.h) as step 2's B operand, and    pack, one launch for
//      X_c^T into its K steps of the packed X^T [D, ldk]  every chunk of a
//                                                      grad_weight group
//   2. Z = X_c W^T, bf16, [C', ldv] (padding columns 0) MFMA GEMM, taken as
//      Z^T = W X_c^T (W through LDS); chunk 0's also writes the packed
//      W^T [D, ldv] (zero-padded), step 5's B operand
//   3. the cross-entropy row kernel on Z, in place: loss terms and the
//      gradient of the summed loss, G = (1 + 2 z lse) softmax - onehot
//                                                      same kernel as ce_fwd_bwd
//   4. G^T into its columns of G^T [ldv, ldk]          written by step 5's GEMM
//                                                      (a transpose for a ragged
//                                                      last chunk)
//   5. grad_inputs[r0:] = s G W                        MFMA GEMM (split-K if the
//                                                      tile count cannot fill the chip)
//   6. dW (+)= s G^T X_c                               MFMA GEMM, accumulate epilogue
// where s is 1/N for the mean and 1 for the sum, applied to the fp32
// accumulators in the epilogues rather than to G: G is held in the 16-bit
// input format, and for fp16 the mean's scaled probabilities p/N would fall
// below its smallest subnormal (2^-24) at the batch sizes of the workload.
// Finally the fixed-order loss reduction. In 'fp32' accumulation step 6 runs
// once per group of chunks, on the group's columns of G^T and X^T together
// (K = group ldc, ldk = group ldc; a last, partial group runs on the chunks it
// has): as many chunks as the caller's budget of G^T holds (by default 2 GiB:
// four at a vocabulary of 128256 and chunks of 2048), with dW in an fp32
// workspace that the last product's epilogue rounds to 16 bits, or, when one
// group takes every chunk, one product that writes the 16-bit result directly
// with no fp32 accumulator. The budget bounds the G^T the workspace holds (the
// default keeps it well below the whole batch's logits gradient). In
// 'weight' accumulation the gradient is rounded to the 16-bit format after
// every chunk, as the accumulation mode prescribes: a group's product rounds
// its running sums at each chunk boundary of its K range, and the next group
// starts from the 16-bit result.
//
// The logits and G are kept in the inputs' 16-bit format (bf16 or fp16)
// between steps, as the matmuls produce and consume them; the cross-entropy of
// a chunk is computed in fp32 from the rounded logits, so G is the
// cross-entropy gradient of the rounded logits.
#include "gemm.h"
#include "internal.h"

namespace lmx {

namespace {

constexpr int kTileS = 128;       // small GEMM tile (BM = BN), two workgroups per CU
constexpr int kTileL = 256;       // large GEMM tile, one workgroup per CU
constexpr int kLdvAlign = 256;    // vocabulary padding of the chunk buffers
constexpr int kLdcAlign = 64;     // chunk-row padding of the transposed buffers
constexpr int64_t kGtGroupBytes = int64_t{1} << 31;   // G^T budget of one grad_weight group
constexpr size_t kWsAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up64(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------------ epilogues

// Steps 2 and 5: a 16-bit output tile in the element format E (logits,
// grad_inputs rows), or fp32 split-K partials.
// 1 / n for a positive count, else 1 (no count, or no valid rows: G is zero).
__device__ __forceinline__ float count_scale(const int64_t* n) {
  if (n == nullptr) return 1.0f;
  const int64_t v = *n;
  return v > 0 ? 1.0f / static_cast<float>(v) : 1.0f;
}

// Whether a 16-bit output [*, n] with row stride ld can take the staged
// epilogue (whole, aligned 16-byte pieces).
inline int staged_ok(const void* out, int64_t ld, int64_t n) {
  return reinterpret_cast<uintptr_t>(out) % 16 == 0 && ld % 8 == 0 && n % 8 == 0 ? 1 : 0;
}

// Output modes of EpiOut fixed at compile time: any (chosen per call from the
// split and the staged flag), staged 16-bit stores only (an unsplit product
// with staged set), fp32 split-K partials only (a split product).
constexpr int kOutAny = 0, kOutStaged = 1, kOutPartial = 2;

// TR: the product may also store one of its operands transposed (GemmShape's
// at_out); products that never do, or whose output mode is fixed,
// are compiled without the code they do not use.
template <typename E, bool TR = false, int MODE = kOutAny>
struct EpiOut {
  static constexpr bool kRounds = false;
  static constexpr bool kTransposes = TR;
  uint16_t* out;
  int64_t ldo;
  float* partial;        // [ksplit][M][ldp]
  int64_t ldp;
  const int64_t* mean_count;   // non-null: scale the products by 1 / *mean_count
  // Direct stores staged through LDS as whole 16-byte row pieces (one store
  // instruction per 8 outputs instead of one per output; about 2% faster on
  // the logits product). Needs N, ldo and the output address in multiples of
  // 8 elements / 16 bytes, so that no piece straddles N.
  int staged;

  // Whether a fixed output mode suits the product (host check).
  bool mode_fits(const GemmShape& g) const {
    if (MODE == kOutStaged) return g.ksplit == 1 && staged;
    if (MODE == kOutPartial) return g.ksplit > 1;
    return true;
  }

  // The same epilogue for the sub-matrix starting at (rows, cols) (direct stores).
  EpiOut shifted(int64_t rows, int64_t cols) const {
    EpiOut e = *this;
    e.out = out + rows * ldo + cols;
    return e;
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void init(f32x16_t (&acc)[FM][FN], const AccCoord&, int, int, const GemmShape&) {
    acc_zero(acc);
  }

  // Staged path: the tile in LDS as [BM][BN] 16-bit values, the 16-byte pieces
  // of a row XOR-swizzled by bit 2 of (row >> 2), which sends the two halves of
  // a wave (rows 4 apart) to different banks; then each thread stores whole
  // pieces. The K loop's last fragment reads must be over before the LDS is
  // reused, hence the first barrier.
  template <int BM, int BN, int FM, int FN>
  __device__ void run_staged(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0,
                             const GemmShape& g, uint16_t* smem, float s) {
    static_assert(BM * BN * 2 <= GemmCfg<BM, BN>::LDS_BYTES, "the tile must fit the LDS");
    constexpr int CPR = BN / 8;   // 16-byte pieces per tile row
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = ac.col(j);
      const int piece = col >> 3, within = col & 7;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = ac.row(i, r);
          const int sw = piece ^ (((row >> 2) & 1) << 2);
          smem[row * BN + sw * 8 + within] = E::narrow(s * acc[i][j][r]);
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t ro = rows_rsrc(out, m0, g.M - m0, BM, ldo * 2);
    for (int idx = static_cast<int>(threadIdx.x); idx < BM * CPR; idx += static_cast<int>(blockDim.x)) {
      const int row = idx / CPR, piece = idx % CPR;
      if (n0 + piece * 8 >= g.N) continue;
      const int sw = piece ^ (((row >> 2) & 1) << 2);
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + row * BN + sw * 8);
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, (row * static_cast<int>(ldo) + n0 + piece * 8) * 2,
                                             0, 0);
    }
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void run(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0, int split,
                      const GemmShape& g, uint16_t* smem) {
    const float s = count_scale(mean_count);
    if constexpr (MODE == kOutStaged) {
      run_staged<BM, BN, FM, FN>(acc, ac, m0, n0, g, smem, s);
      return;
    }
    const bool direct = MODE == kOutPartial ? false : g.ksplit == 1;
    if constexpr (MODE == kOutAny) {
      if (direct && staged) {
        run_staged<BM, BN, FM, FN>(acc, ac, m0, n0, g, smem, s);
        return;
      }
    }
    const __amdgpu_buffer_rsrc_t ro =
        direct ? rows_rsrc(out, m0, g.M - m0, BM, ldo * 2)
               : rows_rsrc(partial + static_cast<int64_t>(split) * g.M * ldp, m0, g.M - m0, BM,
                           ldp * 4);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + ac.col(j);
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = ac.row(i, r);   // tile-local; rows >= M fall outside the resource
          if (direct) {
            __builtin_amdgcn_raw_buffer_store_b16(E::narrow(s * acc[i][j][r]), ro,
                                                  (row * static_cast<int>(ldo) + col) * 2, 0, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s * acc[i][j][r]), ro,
                                                  (row * static_cast<int>(ldp) + col) * 4, 0, 0);
          }
        }
    }
  }
};

// Step 2 with its operands swapped: the product runs over (vocabulary row m,
// token n), W as A (through LDS) and the chunk's packed X_c as B, and this
// epilogue writes the tile transposed, out[n][m] = E(acc), for m < m_out (rows
// of A past M are zeros: the padding columns) and n < N. Through LDS: the tile
// staged as [BN][BM] 16-bit values, each lane writing its four consecutive m
// of a column as one 8-byte unit, the units of row n XOR-swizzled by an even
// value from n (so the 32 rows a half-wave writes land in distinct banks, and
// a 16-byte piece of a row stays two adjacent units in order); then whole
// 16-byte pieces of out's rows stored. TR: chunk 0's product also writes the
// packed W^T from its A tiles (GemmShape's at_out with at_pk_ks).
template <typename E, bool TR>
struct EpiOutT {
  static constexpr bool kRounds = false;
  static constexpr bool kTransposes = TR;
  uint16_t* out;
  int64_t ldo;
  int m_out;

  bool mode_fits(const GemmShape& g) const { return g.ksplit == 1; }

  // The same epilogue for the product's sub-matrix starting at (rows, cols).
  EpiOutT shifted(int64_t rows, int64_t cols) const {
    EpiOutT e = *this;
    e.out = out + cols * ldo + rows;
    e.m_out = m_out - static_cast<int>(rows);
    return e;
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void init(f32x16_t (&acc)[FM][FN], const AccCoord&, int, int, const GemmShape&) {
    acc_zero(acc);
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void run(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0, int,
                      const GemmShape& g, uint16_t* smem) {
    static_assert(BM * BN * 2 <= GemmCfg<BM, BN>::LDS_BYTES, "the tile must fit the LDS");
    constexpr int UNITS = BM / 4;                 // 8-byte units per staged row
    constexpr int SWM = (UNITS / 2 - 1) << 1;     // even swizzle values below UNITS
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = ac.col(j);
      const int sw = (n << 1) & SWM;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int u = ac.row(i, 4 * r4) >> 2;   // rows 4 r4 .. 4 r4 + 3 of the lane: one unit
          uint2 v;
          v.x = static_cast<uint32_t>(E::narrow(acc[i][j][4 * r4])) |
                (static_cast<uint32_t>(E::narrow(acc[i][j][4 * r4 + 1])) << 16);
          v.y = static_cast<uint32_t>(E::narrow(acc[i][j][4 * r4 + 2])) |
                (static_cast<uint32_t>(E::narrow(acc[i][j][4 * r4 + 3])) << 16);
          *reinterpret_cast<uint2*>(smem + n * BM + ((u ^ sw) << 2)) = v;
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t ro = rows_rsrc(out, n0, g.N - n0, BN, ldo * 2);
    constexpr int PPR = BM / 8;   // 16-byte pieces per staged row
    for (int idx = static_cast<int>(threadIdx.x); idx < BN * PPR; idx += static_cast<int>(blockDim.x)) {
      const int n = idx / PPR, piece = idx % PPR;
      if (m0 + piece * 8 >= m_out) continue;
      const int sw = (n << 1) & SWM;
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + n * BM + (((2 * piece) ^ sw) << 2));
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, (n * static_cast<int>(ldo) + m0 + piece * 8) * 2,
                                             0, 0);
    }
  }
};

// grad_weight epilogue modes; "W16" is the weight's 16-bit format (bf16 / fp16).
// ('weight' accumulation has its own epilogue, EpiDwW16.)
enum DwMode { kDwStoreF32 = 0, kDwAddF32 = 1, kDwAddF32ToW16 = 2, kDwStoreW16 = 3 };

// Step 6: grad_weight accumulation. Read-modify-write epilogues issue all the
// reads of an accumulator column before any add, so the memory latency is paid
// once per column (this measured faster than fire-and-forget buffer atomics).
template <typename E>
struct EpiDw {
  static constexpr bool kRounds = false;
  static constexpr bool kTransposes = false;
  bool mode_fits(const GemmShape&) const { return true; }
  float* acc32;     // [V][ld] fp32 accumulator ('fp32' mode)
  uint16_t* out16;  // [V][ld] grad_weight in the weight's format E
  int64_t ld;
  int mode;
  const int64_t* mean_count;   // non-null: scale the products by 1 / *mean_count

  // The same epilogue for the sub-matrix starting at (rows, cols).
  EpiDw shifted(int64_t rows, int64_t cols) const {
    EpiDw e = *this;
    if (acc32 != nullptr) e.acc32 = acc32 + rows * ld + cols;
    if (out16 != nullptr) e.out16 = out16 + rows * ld + cols;
    return e;
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void init(f32x16_t (&acc)[FM][FN], const AccCoord&, int, int, const GemmShape&) {
    acc_zero(acc);
  }

  template <int MODE, int FM, int FN>
  __device__ void apply(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int n0, const GemmShape& g,
                        __amdgpu_buffer_rsrc_t r32, __amdgpu_buffer_rsrc_t r16, float s) {
    const int ldi = static_cast<int>(ld);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + ac.col(j);
      if (col >= g.N) continue;
      if constexpr (MODE == kDwAddF32 || MODE == kDwAddF32ToW16) {
        // read-modify-write: all FM x 16 reads of this column first, so their
        // latency is paid once per column instead of once per element
        float old[FM * 16];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = ac.row(i, r) * ldi + col;
            old[i * 16 + r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r32, e * 4, 0, 0));
          }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = ac.row(i, r) * ldi + col;
            const float v = old[i * 16 + r] + s * acc[i][j][r];
            if constexpr (MODE == kDwAddF32) {
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r32, e * 4, 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b16(E::narrow(v), r16, e * 2, 0, 0);
            }
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = ac.row(i, r) * ldi + col;   // tile-local row; rows >= M are dropped
            const float v = s * acc[i][j][r];
            if constexpr (MODE == kDwStoreF32) {
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r32, e * 4, 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b16(E::narrow(v), r16, e * 2, 0, 0);
            }
          }
      }
    }
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void run(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0, int,
                      const GemmShape& g, uint16_t*) {
    const __amdgpu_buffer_rsrc_t r32 = rows_rsrc(acc32, m0, g.M - m0, BM, ld * 4);
    const __amdgpu_buffer_rsrc_t r16 = rows_rsrc(out16, m0, g.M - m0, BM, ld * 2);
    const float s = count_scale(mean_count);
    switch (mode) {
      case kDwStoreF32: apply<kDwStoreF32>(acc, ac, n0, g, r32, r16, s); break;
      case kDwAddF32: apply<kDwAddF32>(acc, ac, n0, g, r32, r16, s); break;
      case kDwAddF32ToW16: apply<kDwAddF32ToW16>(acc, ac, n0, g, r32, r16, s); break;
      default: apply<kDwStoreW16>(acc, ac, n0, g, r32, r16, s); break;
    }
  }
};

// Step 6 in 'weight' accumulation: grad_weight in the weight's 16-bit format E,
// rounded after every chunk, for a product over a group of chunks (K = the
// group's chunk columns of G^T / X^T, round_every K steps per chunk). The
// accumulators hold dW_prev / s + P (s = 1 / N for the mean, 1 for the sum;
// P the fp32 product of the chunks so far in the group), so that at each chunk
// boundary dW = E(s acc) is the running gradient rounded to E, and acc restarts
// from dW / s: the product is the chunk-by-chunk RNE(dW + s P_c), with one
// product per group instead of one per chunk. The first group starts from
// zero; a later group loads the running gradient from grad_weight (preload).
// 1 / s = N is exact in fp32 for N < 2^24, and dW N is exact whenever E's
// significand and N fit 24 bits together (bf16 and N < 2^16).
template <typename E>
struct EpiDwW16 {
  static constexpr bool kRounds = true;
  static constexpr bool kTransposes = false;
  bool mode_fits(const GemmShape&) const { return true; }
  uint16_t* out16;  // [V][ld] grad_weight in E
  int64_t ld;
  const int64_t* mean_count;   // non-null: the mean's N
  int preload;                 // start from the gradient in out16 (a later group)
  // the mean's 1 / N and N for round_tile(), read once by init(): a load inside
  // the K loop would wait for every copy in flight
  float rs = 1.f, rn = 1.f;

  EpiDwW16 shifted(int64_t rows, int64_t cols) const {
    EpiDwW16 e = *this;
    e.out16 = out16 + rows * ld + cols;
    return e;
  }

  __device__ static float count_f(const int64_t* n) {
    if (n == nullptr) return 1.0f;
    const int64_t v = *n;
    return v > 0 ? static_cast<float>(v) : 1.0f;
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void init(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0,
                       const GemmShape& g) {
    rs = count_scale(mean_count);
    rn = count_f(mean_count);
    if (!preload) {
      acc_zero(acc);
      return;
    }
    const float nf = rn;
    const __amdgpu_buffer_rsrc_t r16 = rows_rsrc(out16, m0, g.M - m0, BM, ld * 2);
    const int ldi = static_cast<int>(ld);
    // every load is issued before any value is used (the raw 16 bits go into
    // the accumulator registers), so the tile pays the memory latency once;
    // rows past M lie outside the resource and read zero, and the columns past
    // N (whose offsets may reach into the next row) are zeroed below
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + ac.col(j);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = ac.row(i, r) * ldi + col;
          acc[i][j][r] = __uint_as_float(static_cast<uint32_t>(
              __builtin_amdgcn_raw_buffer_load_b16(r16, e * 2, 0, 0)));
        }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float keep = n0 + ac.col(j) < g.N ? nf : 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint16_t bits = static_cast<uint16_t>(__float_as_uint(acc[i][j][r]));
          acc[i][j][r] = E::widen(bits) * keep;
        }
    }
  }

  // a = N * E(a / N) for one MFMA tile's accumulators, rounded exactly as
  // run() rounds E(s acc), two values per word (the empty asm keeps the
  // compiler from splitting a pair conversion into two single ones)
  __device__ void round_tile(f32x16_t& a) const {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      uint32_t w = E::scaled_pack2(rs, a[r], a[r + 1]);
      asm volatile("" : "+v"(w));
      a[r] = E::lo(w) * rn;
      a[r + 1] = E::hi(w) * rn;
    }
  }

  template <int BM, int BN, int FM, int FN>
  __device__ void run(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0, int,
                      const GemmShape& g, uint16_t*) {
    const __amdgpu_buffer_rsrc_t r16 = rows_rsrc(out16, m0, g.M - m0, BM, ld * 2);
    const float s = count_scale(mean_count);
    const int ldi = static_cast<int>(ld);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + ac.col(j);
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = ac.row(i, r) * ldi + col;   // rows >= M are dropped
          __builtin_amdgcn_raw_buffer_store_b16(E::narrow(s * acc[i][j][r]), r16, e * 2, 0, 0);
        }
    }
  }
};

// ------------------------------------------------------------------ small kernels

// dst[c][r] = src[r][c] for r < R, c < Cs, zero for R <= r < Rp. 64 x 64 tiles.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src,
                                                            int64_t ld_src, int R, int Cs,
                                                            uint16_t* __restrict__ dst,
                                                            int64_t ld_dst) {
  __shared__ uint16_t t[64][64 + 2];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  {
    const int rr = tid / 4, cc = (tid % 4) * 16;
    const int r = r0 + rr;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = c0 + cc + q * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < R && c < Cs) v = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(r) * ld_src + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[rr][cc + q * 8 + 2 * e] = static_cast<uint16_t>(v[e] & 0xffffu);
        t[rr][cc + q * 8 + 2 * e + 1] = static_cast<uint16_t>(v[e] >> 16);
      }
    }
  }
  __syncthreads();
  {
    const int cc = tid / 4, rr = (tid % 4) * 16;
    const int c = c0 + cc;
    if (c < Cs) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = static_cast<uint32_t>(t[rr + q * 8 + 2 * e][cc]) |
                 (static_cast<uint32_t>(t[rr + q * 8 + 2 * e + 1][cc]) << 16);
        }
        *reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(c) * ld_dst + r0 + rr + q * 8) = v;
      }
    }
  }
}

// The packed copies (the fragment-packed B layout of gemm.h) of S [R, Cs]
// (row stride ld, Cs a multiple of 8) from one read of each 64 x 64 tile of S:
// rows_out, when given, gets S itself (blocks of 32 rows, K steps of 64
// columns, KS_r steps per block, rows of the first nb_rows blocks), t_out,
// when given, gets S^T (blocks of 32 columns of S, K running over the rows of
// S: step s_off + y of a buffer with KS_t steps per block, blocks below
// nb_cols). Elements past R or Cs are zeros. Block (y, c) takes rows 64 y .. +
// 63 and columns 64 c .. + 63 (the row steps on grid x, the wider range).
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ src, int64_t ld,
                                                   int R, int Cs, uint16_t* __restrict__ rows_out,
                                                   int KS_r, uint16_t* __restrict__ t_out,
                                                   int KS_t, int s_off, int nb_cols, int zrows,
                                                   int64_t rows_out_z, int s_z) {
  // rows padded by one 16-byte piece: the column gathers of the half-waves
  // (rows 8 apart) land in different banks
  __shared__ __align__(16) uint16_t t[64][64 + 8];
  const int y = blockIdx.x, c = blockIdx.y;
  const int tid = threadIdx.x;
  // slice z of the launch: rows z zrows .. of S, as a source of its own (rows
  // past its zrows read as zero), packed rows_out_z elements further on and
  // s_z K steps further on in the transposed copy
  {
    const int z = blockIdx.z;
    const int64_t zr0 = static_cast<int64_t>(z) * zrows;
    src += zr0 * ld;
    R = R - static_cast<int>(zr0) < zrows ? R - static_cast<int>(zr0) : zrows;
    if (rows_out != nullptr) rows_out += z * rows_out_z;
    s_off += z * s_z;
  }
  const int nb_rows = (R + kPackedRows - 1) / kPackedRows;
  {
    const int rr = tid >> 2, cc = (tid & 3) * 16;
    const int r = y * 64 + rr;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = c * 64 + cc + 8 * h;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < R && col < Cs)
        v = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(r) * ld + col);
      *reinterpret_cast<u32x4*>(&t[rr][cc + 8 * h]) = v;
    }
  }
  __syncthreads();
  // two output pieces per thread for each copy: w = (block half b, slice q, lane l)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int w = tid + 256 * i;                // 0 .. 511
    const int b = w >> 8, q = (w >> 6) & 3, l = w & 63;
    const int lr = l & 31, k0 = 16 * q + 8 * (l >> 5);
    if (rows_out != nullptr && 2 * y + b < nb_rows) {
      // row 32 b + lr of the tile, columns k0 .. k0 + 7
      const u32x4 v = *reinterpret_cast<const u32x4*>(&t[32 * b + lr][k0]);
      *reinterpret_cast<u32x4*>(
          rows_out + ((static_cast<int64_t>(2 * y + b) * KS_r + c) * 4 + q) * 512 + l * 8) = v;
    }
    if (t_out != nullptr && 2 * c + b < nb_cols) {
      // column 32 b + lr of the tile, rows k0 .. k0 + 7
      const int cl = 32 * b + lr;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = static_cast<uint32_t>(t[k0 + 2 * e][cl]) |
               (static_cast<uint32_t>(t[k0 + 2 * e + 1][cl]) << 16);
      *reinterpret_cast<u32x4*>(
          t_out + ((static_cast<int64_t>(2 * c + b) * KS_t + s_off + y) * 4 + q) * 512 + l * 8) = v;
    }
  }
}

// grad_inputs rows = E(sum over splits of the fp32 partials), fixed order.
template <typename E>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int ksplit, int M, int N,
                                                            int64_t ldp,
                                                            uint16_t* __restrict__ out,
                                                            int64_t ldo) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t total = static_cast<int64_t>(M) * N;
  if (i >= total) return;
  const int row = static_cast<int>(i / N), col = static_cast<int>(i % N);
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ksplit; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(
        partial + (static_cast<int64_t>(s) * M + row) * ldp + col);
    a[0] += v.x; a[1] += v.y; a[2] += v.z; a[3] += v.w;
  }
  uint2 o = make_uint2(E::pack2(a[0], a[1]), E::pack2(a[2], a[3]));
  *reinterpret_cast<uint2*>(out + static_cast<int64_t>(row) * ldo + col) = o;
}

// grad_weight rows [rows0, V) from the K-split partials of their large-tile
// launch (already scaled by 1 / N when the mean asks for it): the sum over the
// splits in a fixed order, then the store or accumulation of `mode`, as the
// grad_weight epilogue does it for the other rows. acc32 / out16 point at the
// first of these rows.
template <typename E>
__global__ __launch_bounds__(256) void dw_tail_reduce_kernel(const float* __restrict__ partial,
                                                             int ksplit, int M, int N,
                                                             float* acc32, uint16_t* out16,
                                                             int64_t ld, int mode) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(M) * N) return;
  const int row = static_cast<int>(i / N), col = static_cast<int>(i % N);
  float v = 0.f;
  for (int s = 0; s < ksplit; ++s) v += partial[(static_cast<int64_t>(s) * M + row) * N + col];
  const int64_t e = static_cast<int64_t>(row) * ld + col;
  switch (mode) {
    case kDwStoreF32: acc32[e] = v; break;
    case kDwAddF32: acc32[e] = acc32[e] + v; break;
    case kDwAddF32ToW16: out16[e] = E::narrow(acc32[e] + v); break;
    default: out16[e] = E::narrow(v); break;
  }
}

__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    p[i] = 0;
}

// ------------------------------------------------------------------ host helpers

// SCHED selects the main loop's schedule hints for the large tile (see
// gemm_interleave_hint); the small tile always uses schedule 0.
template <int SCHED, typename E, typename Epi>
int launch_gemm(const GemmShape& g, int tile, const Epi& epi, hipStream_t stream) {
  // an epilogue compiled without the transposed stores must not be given one
  // to do (no caller does; this keeps a future one from dropping them)
  if (!Epi::kTransposes && g.at_out != nullptr) return LMX_ERR_UNSUPPORTED;
  if (!epi.mode_fits(g)) return LMX_ERR_UNSUPPORTED;
  // the transposed A tiles are written by the packed-B kernel only
  if (g.Bp == nullptr && g.at_out != nullptr) return LMX_ERR_UNSUPPORTED;
  const int blocks = g.tiles_m * g.tiles_n * g.ksplit;
  if (blocks == 0) return LMX_OK;
  const bool fullk = g.K % kGemmBK == 0;
  if (g.Bp != nullptr) {
    if (tile == kTileL) {
      constexpr int threads = GemmCfg<kTileL, kTileL>::THREADS;
      if (fullk)
        hipLaunchKernelGGL((gemm_nt_bdir_kernel<kTileL, kTileL, Epi, E, true>), dim3(blocks),
                           dim3(threads), 0, stream, g, epi);
      else
        hipLaunchKernelGGL((gemm_nt_bdir_kernel<kTileL, kTileL, Epi, E, false>), dim3(blocks),
                           dim3(threads), 0, stream, g, epi);
    } else {
      constexpr int threads = GemmCfg<kTileS, kTileS>::THREADS;
      if (fullk)
        hipLaunchKernelGGL((gemm_nt_bdir_kernel<kTileS, kTileS, Epi, E, true>), dim3(blocks),
                           dim3(threads), 0, stream, g, epi);
      else
        hipLaunchKernelGGL((gemm_nt_bdir_kernel<kTileS, kTileS, Epi, E, false>), dim3(blocks),
                           dim3(threads), 0, stream, g, epi);
    }
    return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
  }
  if (tile == kTileL) {
    constexpr int threads = GemmCfg<kTileL, kTileL>::THREADS;
    if (fullk)
      hipLaunchKernelGGL((gemm_nt_kernel<kTileL, kTileL, Epi, SCHED, E, true>), dim3(blocks),
                         dim3(threads), 0, stream, g, epi);
    else
      hipLaunchKernelGGL((gemm_nt_kernel<kTileL, kTileL, Epi, SCHED, E, false>), dim3(blocks),
                         dim3(threads), 0, stream, g, epi);
  } else {
    constexpr int threads = GemmCfg<kTileS, kTileS>::THREADS;
    if (fullk)
      hipLaunchKernelGGL((gemm_nt_kernel<kTileS, kTileS, Epi, 0, E, true>), dim3(blocks),
                         dim3(threads), 0, stream, g, epi);
    else
      hipLaunchKernelGGL((gemm_nt_kernel<kTileS, kTileS, Epi, 0, E, false>), dim3(blocks),
                         dim3(threads), 0, stream, g, epi);
  }
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

// A GEMM on large tiles whose last wave of workgroups would leave most CUs
// idle: the rows (or columns) that make up that wave go to a second launch on
// small tiles, whose work items are a quarter the size, so the tail is spread
// over the chip. Applies to unsplit GEMMs with a direct-store epilogue.
template <int SCHED, typename E, typename Epi>
int launch_gemm_split_tail(const GemmShape& g, const Epi& epi, hipStream_t stream) {
  const int64_t tiles = static_cast<int64_t>(g.tiles_m) * g.tiles_n;
  const int64_t full = (tiles / 256) * 256;
  const int64_t rem = tiles - full;
  if (g.ksplit != 1 || full == 0 || rem == 0 || rem * 3 > 256) {
    return launch_gemm<SCHED, E>(g, kTileL, epi, stream);
  }
  // split along the dimension with more tiles, keeping whole large tiles in
  // the first launch
  GemmShape a = g, b = g;
  if (g.tiles_n >= g.tiles_m) {
    const int n1 = static_cast<int>(full / g.tiles_m);   // large-tile columns kept
    const int cols = n1 * kTileL;
    if (n1 <= 0 || cols >= g.N) return launch_gemm<SCHED, E>(g, kTileL, epi, stream);
    a.N = cols;
    a.b_rows = g.b_rows < cols ? g.b_rows : cols;
    a.tiles_n = n1;
    if (g.B != nullptr) b.B = g.B + static_cast<int64_t>(cols) * g.ldb;
    if (g.Bp != nullptr)
      b.Bp = g.Bp + static_cast<int64_t>(cols / kPackedRows) * g.bp_ks * (kPackedStepBytes / 2);
    b.N = g.N - cols;
    b.b_rows = g.b_rows > cols ? g.b_rows - cols : 0;
    b.tiles_m = (g.M + kTileS - 1) / kTileS;
    b.tiles_n = (b.N + kTileS - 1) / kTileS;
    // transposed A: A's whole tile rows are in both launches (the first writes them)
    b.at_out = nullptr;
    int st = launch_gemm<SCHED, E>(a, kTileL, epi, stream);
    if (st != LMX_OK) return st;
    return launch_gemm<SCHED, E>(b, kTileS, epi.shifted(0, cols), stream);
  }
  const int m1 = static_cast<int>(full / g.tiles_n);       // large-tile rows kept
  const int rows = m1 * kTileL;
  if (m1 <= 0 || rows >= g.M) return launch_gemm<SCHED, E>(g, kTileL, epi, stream);
  a.M = rows;
  a.a_rows = g.a_rows < rows ? g.a_rows : rows;
  a.tiles_m = m1;
  b.A = g.A + static_cast<int64_t>(rows) * g.lda;
  b.M = g.M - rows;
  b.a_rows = g.a_rows > rows ? g.a_rows - rows : 0;
  b.tiles_m = (b.M + kTileS - 1) / kTileS;
  b.tiles_n = (g.N + kTileS - 1) / kTileS;
  a.at_cols = g.at_cols < rows ? g.at_cols : rows;
  // (packed: rows is a whole number of K steps of the packed A^T)
  if (g.at_out != nullptr)
    b.at_out = g.at_out + (g.at_pk_ks > 0 ? static_cast<int64_t>(rows / kGemmBK) * (kPackedStepBytes / 2)
                                          : static_cast<int64_t>(rows));
  b.at_cols = g.at_cols > rows ? g.at_cols - rows : 0;
  int st = launch_gemm<SCHED, E>(a, kTileL, epi, stream);
  if (st != LMX_OK) return st;
  return launch_gemm<SCHED, E>(b, kTileS, epi.shifted(rows, 0), stream);
}

// The large tile when it yields at least one workgroup per CU of the chip
// (256 CUs), possibly with up to `max_split` K splits, else the small one.
int pick_tile(int64_t M, int64_t N, int max_split = 1) {
  const int64_t big = ((M + kTileL - 1) / kTileL) * ((N + kTileL - 1) / kTileL);
  return big * max_split >= 256 ? kTileL : kTileS;
}

// C[M, N] = A[M, K] B[N, K]^T where only the first b_rows rows of B exist
// (the rest of N reads as zeros).
GemmShape make_shape(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N,
                     int b_rows, int K, int ksplit, int tile) {
  const int kTile = tile;
  GemmShape g;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.a_rows = M;
  g.b_rows = b_rows;
  g.K = K;
  g.tiles_m = (M + kTile - 1) / kTile;
  g.tiles_n = (N + kTile - 1) / kTile;
  const int ksteps = (K + kGemmBK - 1) / kGemmBK;
  if (ksplit < 1) ksplit = 1;
  if (ksplit > ksteps) ksplit = ksteps > 0 ? ksteps : 1;
  g.ksteps_per_split = (ksteps + ksplit - 1) / ksplit;
  g.ksplit = ksteps > 0 ? (ksteps + g.ksteps_per_split - 1) / g.ksteps_per_split : 1;
  g.at_out = nullptr;
  g.ld_at = 0;
  g.at_cols = 0;
  g.at_pk_ks = 0;
  g.round_every = 0;
  g.Bp = nullptr;
  g.bp_ks = 0;
  return g;
}

int transpose_pad(const uint16_t* src, int64_t ld_src, int R, int Cs, uint16_t* dst,
                  int64_t ld_dst, int Rp, hipStream_t stream) {
  if (Rp == 0 || Cs == 0) return LMX_OK;
  dim3 grid(Rp / 64, (Cs + 63) / 64);
  hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, stream, src, ld_src, R, Cs, dst,
                     ld_dst);
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

// Steps and bytes of a packed copy of an operand with `rows` rows and K = k.
int64_t packed_steps(int64_t k) { return (k + kGemmBK - 1) / kGemmBK; }
size_t packed_bytes(int64_t rows, int64_t k) {
  return static_cast<size_t>((rows + kPackedRows - 1) / kPackedRows) * packed_steps(k) *
         kPackedStepBytes;
}

// Packed copies of S [R, Cs] (row stride ld): rows_out (when given) gets S
// with KS_r = ceil(Cs / 64) steps per block, the blocks of its first R rows;
// t_out (when given) gets S^T at K steps s_off .. s_off + Rp / 64 - 1 of a
// buffer with KS_t steps per block (rows R .. Rp - 1 of S read as zero; Rp a
// multiple of 64).
// With nz > 1, one launch packs nz consecutive slices of zrows rows each (the
// chunks of a grad_weight group; the last may be shorter, R counting the rows
// of all of them) as nz such calls would: slice z's rows at rows_out + z
// rows_out_z and its transpose at K steps s_off + z s_z .., each slice's rows
// past zrows reading as zero up to Rp.
int pack(const uint16_t* src, int64_t ld, int R, int Cs, int Rp, uint16_t* rows_out,
         uint16_t* t_out, int KS_t, int s_off, hipStream_t stream, int nz = 1, int zrows = 0,
         int64_t rows_out_z = 0, int s_z = 0) {
  if (Rp == 0 || Cs == 0 || nz < 1) return LMX_OK;
  if (nz == 1) zrows = R;
  if (zrows < 1 || static_cast<int64_t>(nz - 1) * zrows >= R) return LMX_ERR_SIZE;
  const int ks_r = static_cast<int>(packed_steps(Cs));
  dim3 grid(Rp / kGemmBK, ks_r, nz);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, stream, src, ld, R, Cs, rows_out, ks_r,
                     t_out, KS_t, s_off, (Cs + kPackedRows - 1) / kPackedRows, zrows,
                     rows_out_z, s_z);
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

// Tile and K splits of a chunk's grad_inputs product (C x D outputs, K = ldv):
// the large tile whenever K splits of at least 8 steps each let its tiles
// occupy most of the chip's 256 CUs in one wave (a small hidden size gives few
// tiles but a long K; a work item more than 256 would start a second wave of
// workgroups, measured 45% slower at D = 768), else the small tile, also split
// to fill the chip.
struct DxPlan {
  int tile;
  int ksplit;
};
DxPlan dx_plan(int64_t C, int64_t D, int64_t ldv) {
  const int64_t ksteps = ldv / kGemmBK;
  const int64_t tl = ((C + kTileL - 1) / kTileL) * ((D + kTileL - 1) / kTileL);
  int64_t sl = 256 / tl;
  if (sl > ksteps / 8) sl = ksteps / 8;
  if (sl < 1) sl = 1;
  if (tl * sl >= 192) return {kTileL, static_cast<int>(sl)};
  const int64_t ts = ((C + kTileS - 1) / kTileS) * ((D + kTileS - 1) / kTileS);
  int64_t ss = (512 + ts - 1) / ts;
  if (ss > ksteps / 4) ss = ksteps / 4;
  if (ss < 1) ss = 1;
  return {kTileS, static_cast<int>(ss)};
}

// grad_inputs rows of one chunk: G [rows, lda_g] times W, with W^T [D, ldv] in
// its packed copy wtp (ldv / 64 K steps a block) as the B operand over K =
// k_len vocabulary columns, scaled by
// 1 / *mean_count when that is given; split-K partials in dxp when the layout
// chose splits. With gt_out, the product also writes G^T (gt_out[v * ld_gt +
// r] for r < gt_cols, zeros for r >= rows) from the G tiles it loads, in place
// of a separate transpose; the caller passes it only when the chunk's tiles
// cover all gt_cols columns (a full chunk).
template <typename E>
int chunk_grad_inputs(const uint16_t* g, int64_t lda_g, int k_len, const uint16_t* wtp,
                      int64_t ldv, int rows, int D, int64_t chunk, int ksplit, float* dxp,
                      uint16_t* gx, int64_t ldx, const int64_t* mean_count, uint16_t* gt_out,
                      int64_t ld_gt, int gt_cols, hipStream_t stream) {
  const int tile = dx_plan(chunk, D, ldv).tile;   // the plan the workspace was sized for
  GemmShape gs = make_shape(g, lda_g, nullptr, 0, rows, D, D, k_len, ksplit, tile);
  gs.Bp = wtp;
  gs.bp_ks = static_cast<int>(packed_steps(ldv));
  gs.at_out = gt_out;   // optional: G^T written by the product that reads G
  gs.ld_at = ld_gt;
  gs.at_cols = gt_cols;
  int st;
  if (gs.ksplit > 1) {
    EpiOut<E, true, kOutPartial> e{gx, ldx, dxp, D, mean_count, 0};
    st = launch_gemm<1, E>(gs, tile, e, stream);
  } else {
    EpiOut<E, true> e{gx, ldx, dxp, D, mean_count, staged_ok(gx, ldx, D)};
    st = launch_gemm<1, E>(gs, tile, e, stream);
  }
  if (st != LMX_OK) return st;
  if (gs.ksplit > 1) {
    const int64_t total = static_cast<int64_t>(rows) * D / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel<E>, dim3(static_cast<unsigned>((total + 255) / 256)),
                       dim3(256), 0, stream, dxp, gs.ksplit, rows, D, static_cast<int64_t>(D),
                       gx, ldx);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
  }
  return LMX_OK;
}

// The grad_weight product's last rows on large tiles with K split, in place of
// the small-tile second launch: when its large tiles leave a last wave under a
// third full and the split goes along the rows (launch_gemm_split_tail's
// case), rows0 .. V - 1 take ksplit large-tile workgroups per tile (one wave
// in all, at least 8 K steps each), and a reduction sums the splits.
struct DwTail {
  int rows0;
  int ksplit;   // 1: no K-split tail
};

DwTail dw_tail_plan(int64_t V, int64_t D, int64_t K) {
  DwTail t{0, 1};
  const int64_t tm = (V + kTileL - 1) / kTileL, tn = (D + kTileL - 1) / kTileL;
  const int64_t tiles = tm * tn, full = tiles / 256 * 256, rem = tiles - full;
  if (full == 0 || rem == 0 || rem * 3 > 256 || tn >= tm) return t;
  const int64_t m1 = full / tn;
  if (m1 <= 0 || m1 * kTileL >= V) return t;
  int64_t ks = 256 / ((tm - m1) * tn);
  const int64_t ksteps = (K + kGemmBK - 1) / kGemmBK;
  if (ks > ksteps / 8) ks = ksteps / 8;
  if (ks < 2) return t;
  t.rows0 = static_cast<int>(m1 * kTileL);
  t.ksplit = static_cast<int>(ks);
  return t;
}

size_t dw_tail_bytes(int64_t V, int64_t D, int64_t K) {
  const DwTail t = dw_tail_plan(V, D, K);
  return t.ksplit > 1 ? static_cast<size_t>(t.ksplit) * (V - t.rows0) * D * 4 : 0;
}

// grad_weight product G^T X over K columns of G^T [V, ldk] and X^T [D, ldk]
// (the packed copy xtp, ldk / 64 K steps a block), scaled by 1 / *mean_count
// when that is given, stored or accumulated
// according to `mode`. tailp (tail_bytes of workspace) holds the K-split
// partials of the last rows when dw_tail_plan splits them.
template <typename E>
int grad_weight_product(const uint16_t* gt, const uint16_t* xtp, int64_t ldk, int K, int V, int D,
                        float* dw, uint16_t* gw, int64_t ldw, int mode,
                        const int64_t* mean_count, float* tailp, size_t tail_bytes,
                        hipStream_t stream) {
  const int tile = pick_tile(V, D);
  GemmShape gs = make_shape(gt, ldk, nullptr, 0, V, D, D, K, 1, tile);
  gs.Bp = xtp;
  gs.bp_ks = static_cast<int>(packed_steps(ldk));
  EpiDw<E> e{dw, gw, ldw, mode, mean_count};
  if (tile == kTileL && tailp != nullptr && dw_tail_bytes(V, D, K) <= tail_bytes) {
    const DwTail tp = dw_tail_plan(V, D, K);
    if (tp.ksplit > 1) {
      GemmShape a = gs;
      a.M = tp.rows0;
      a.a_rows = tp.rows0;
      a.tiles_m = tp.rows0 / kTileL;
      int st = launch_gemm<1, E>(a, kTileL, e, stream);
      if (st != LMX_OK) return st;
      const int rows = V - tp.rows0;
      GemmShape b = make_shape(gt + static_cast<int64_t>(tp.rows0) * ldk, ldk, nullptr, 0, rows,
                               D, D, K, tp.ksplit, kTileL);
      b.Bp = gs.Bp;
      b.bp_ks = gs.bp_ks;
      EpiOut<E, false, kOutPartial> eo{nullptr, 0, tailp, D, mean_count, 0};   // fp32 partials per split
      st = launch_gemm<1, E>(b, kTileL, eo, stream);
      if (st != LMX_OK) return st;
      const EpiDw<E> et = e.shifted(tp.rows0, 0);
      const int64_t total = static_cast<int64_t>(rows) * D;
      hipLaunchKernelGGL(dw_tail_reduce_kernel<E>, dim3(static_cast<unsigned>((total + 255) / 256)),
                         dim3(256), 0, stream, tailp, b.ksplit, rows, D, et.acc32, et.out16, ldw,
                         mode);
      return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
    }
  }
  return tile == kTileL ? launch_gemm_split_tail<1, E>(gs, e, stream)
                        : launch_gemm<1, E>(gs, tile, e, stream);
}

// grad_weight product in 'weight' accumulation over the K = ngroup_chunks *
// ldc columns of a group: rounded to E after every chunk (round_every K steps
// per chunk), starting from zero (the first group) or from the running
// gradient in gw (preload, a later group). No K-split tail: the rounding
// needs the chunks in order within one workgroup, so a ragged last wave goes
// to small tiles instead.
template <typename E>
int grad_weight_product_w16(const uint16_t* gt, const uint16_t* xtp, int64_t ldk, int K, int V,
                            int D, uint16_t* gw, int64_t ldw, const int64_t* mean_count,
                            int round_every, bool preload, hipStream_t stream) {
  const int tile = pick_tile(V, D);
  GemmShape gs = make_shape(gt, ldk, nullptr, 0, V, D, D, K, 1, tile);
  gs.Bp = xtp;
  gs.bp_ks = static_cast<int>(packed_steps(ldk));
  gs.round_every = round_every;
  EpiDwW16<E> e{gw, ldw, mean_count, preload ? 1 : 0};
  return tile == kTileL ? launch_gemm_split_tail<1, E>(gs, e, stream)
                        : launch_gemm<1, E>(gs, tile, e, stream);
}

// The grad_weight product of group gi (of ngroups) over its chunk columns:
// fp32 accumulation (store / read-modify-write of the fp32 workspace, the
// last group rounding to E; one group writes E directly) or the weight
// dtype's per-chunk rounding.
template <typename E>
int grad_weight_group(int accum, int64_t gi, int64_t ngroups, const uint16_t* gt,
                      const uint16_t* xtp, int64_t ldk, int K, int64_t ldc, int V, int D,
                      float* dw, uint16_t* gw, int64_t ldw, const int64_t* mean_count,
                      float* tailp, size_t tail_bytes, hipStream_t stream) {
  if (accum == LMX_ACC_WEIGHT) {
    return grad_weight_product_w16<E>(gt, xtp, ldk, K, V, D, gw, ldw, mean_count,
                                      static_cast<int>(ldc / kGemmBK), gi > 0, stream);
  }
  const bool first = gi == 0, last = gi == ngroups - 1;
  const int mode = ngroups == 1 ? kDwStoreW16
                   : first      ? kDwStoreF32
                   : last       ? kDwAddF32ToW16
                                : kDwAddF32;
  return grad_weight_product<E>(gt, xtp, ldk, K, V, D, dw, gw, ldw, mode, mean_count, tailp,
                                tail_bytes, stream);
}

}  // namespace

int64_t linear_ce_resolve_chunk(int64_t BT, int64_t V, int64_t chunk_size) {
  if (BT <= 0) return 1;
  if (chunk_size > 0) return chunk_size < BT ? chunk_size : BT;
  // Default: the largest power of two whose chunk buffers (logits / G and G^T,
  // 4 bytes per row and padded vocabulary entry) fit in 1 GiB, at least 128.
  const int64_t ldv = round_up64(V, kLdvAlign);
  int64_t c = 1;
  while (c * 2 * ldv * 4 <= (int64_t{1} << 30)) c *= 2;
  if (c < 128) c = 128;
  return c < BT ? c : BT;
}

LinearCeWorkspace linear_ce_workspace_layout(int64_t BT, int64_t D, int64_t V, int64_t chunk,
                                             int accum, bool generic, int64_t group_bytes) {
  LinearCeWorkspace w{};
  const int64_t C = chunk > 0 ? chunk : 1;
  w.ldv = round_up64(V, kLdvAlign);
  w.ldc = round_up64(C, kLdcAlign);
  w.ksplit = dx_plan(C, D, w.ldv).ksplit;
  const int64_t nchunks = BT > 0 ? (BT + C - 1) / C : 0;
  // grad_weight is taken once per group of chunks (K = the group's chunk
  // columns of G^T and X^T): as many chunks as group_bytes of G^T hold, at
  // least one. In fp32 mode a group's product reads and writes the fp32
  // accumulator once instead of once per chunk (none is kept when one group
  // takes every chunk); in weight-dtype mode the product rounds after each of
  // its chunks. The budget bounds the workspace whatever BT is.
  const int64_t budget = group_bytes > 0 ? group_bytes : kGtGroupBytes;
  w.dw_group = 1;
  if (nchunks > 1) {
    const int64_t per_chunk = w.ldv * w.ldc * 2;
    int64_t gsz = budget / per_chunk;
    if (gsz > nchunks) gsz = nchunks;
    // the GEMM addresses 256 rows of G^T / X^T with 32-bit byte offsets
    const int64_t gmax = ((int64_t{1} << 31) - 1) / (256 * 2 * w.ldc);
    if (gsz > gmax) gsz = gmax;
    if (gsz > 1) w.dw_group = gsz;
  }
  w.ldk = w.dw_group * w.ldc;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + (bytes > 0 ? bytes : 1), kWsAlign);
    return o;
  };
  w.n_valid_off = take(8);
  w.row_loss_off = take(static_cast<size_t>(BT) * 4);
  w.z_off = take(generic ? 0 : static_cast<size_t>(C) * w.ldv * 2);
  w.gt_off = take(static_cast<size_t>(w.ldv) * w.ldk * 2);
  // packed copies (gemm.h) of the products' B operands: X^T [D, ldk], W^T
  // [D, ldv] and, for the fused path's logits, the X_c [C, D] of each chunk of a
  // group (packed together at the group's first chunk)
  w.xt_off = take(packed_bytes(D, w.ldk));
  w.wt_off = take(packed_bytes(D, w.ldv));
  w.xp_off = take(generic ? 0 : w.dw_group * packed_bytes(C, D));
  w.dxp_off = take(w.ksplit > 1 ? static_cast<size_t>(w.ksplit) * C * D * 4 : 0);
  w.dw_off = take(accum == LMX_ACC_F32 && nchunks > w.dw_group ? static_cast<size_t>(V) * D * 4
                                                                 : 0);
  // K-split partials of grad_weight's last rows (the largest K any product
  // has; fp32 mode only)
  w.dwp_bytes = accum == LMX_ACC_F32 ? dw_tail_bytes(V, D, w.ldk) : 0;
  w.dwp_off = take(w.dwp_bytes);
  w.total = off;
  return w;
}

template <typename E>
int linear_ce_run(const LinearCeParams& p, void* ws_base, hipStream_t stream) {
  const LinearCeWorkspace wl =
      linear_ce_workspace_layout(p.BT, p.D, p.V, p.chunk, p.accum, false, p.group_bytes);
  char* ws = static_cast<char*>(ws_base);
  int64_t* n_ws = reinterpret_cast<int64_t*>(ws + wl.n_valid_off);
  float* row_loss = reinterpret_cast<float*>(ws + wl.row_loss_off);
  uint16_t* z = reinterpret_cast<uint16_t*>(ws + wl.z_off);
  uint16_t* gt = reinterpret_cast<uint16_t*>(ws + wl.gt_off);
  uint16_t* xtp = reinterpret_cast<uint16_t*>(ws + wl.xt_off);
  uint16_t* wtp = reinterpret_cast<uint16_t*>(ws + wl.wt_off);
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws + wl.xp_off);
  float* dxp = reinterpret_cast<float*>(ws + wl.dxp_off);
  float* dw = reinterpret_cast<float*>(ws + wl.dw_off);
  float* dwp = reinterpret_cast<float*>(ws + wl.dwp_off);
  const int D = static_cast<int>(p.D), V = static_cast<int>(p.V);
  const int64_t ldv = wl.ldv, ldc = wl.ldc, ldk = wl.ldk, grp = wl.dw_group;
  const int64_t* mean_count = p.reduction == LMX_MEAN ? n_ws : nullptr;
  const int ks_d = static_cast<int>(packed_steps(D)), ks_v = static_cast<int>(packed_steps(ldv));
  const int ks_k = static_cast<int>(packed_steps(ldk));
  const int64_t xp_chunk = static_cast<int64_t>(packed_bytes(p.chunk, p.D) / 2);   // elements

  int st = count_enqueue(p.target, p.BT, p.V, p.ignore_index, n_ws, p.n_valid_user, p.bad_user,
                         stream);
  if (st != LMX_OK) return st;
  if (p.BT == 0) {
    const int64_t n = p.V * p.D;
    hipLaunchKernelGGL(zero_u16_kernel, dim3(1024), dim3(256), 0, stream, p.grad_w, n);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
    return finish_enqueue(row_loss, 0, n_ws, p.reduction, p.loss, stream);
  }
  // the packed W^T [D, ldv] (the grad_inputs products' B) is written by chunk
  // 0's logits product, which loads every tile of W (rows of W past V read as
  // zero and give the padding columns)
  const int64_t nchunks = (p.BT + p.chunk - 1) / p.chunk;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t r0 = c * p.chunk;
    const int rows = static_cast<int>(p.BT - r0 < p.chunk ? p.BT - r0 : p.chunk);
    const uint16_t* xc = p.x + r0 * p.D;
    const int64_t* tc = p.target + r0;
    const int64_t slot = c % grp;   // this chunk's columns in G^T and X^T
    // 1. at the group's first chunk, one launch for all its chunks: X_c packed
    // (the logits product's B, one copy per chunk) and X_c^T packed, as the
    // chunk's K steps of the group's X^T
    if (slot == 0) {
      const int64_t nz = grp < nchunks - c ? grp : nchunks - c;
      const int64_t grows = p.BT - r0 < nz * p.chunk ? p.BT - r0 : nz * p.chunk;
      st = pack(xc, p.D, static_cast<int>(grows), D, static_cast<int>(ldc), xp, xtp, ks_k, 0,
                stream, static_cast<int>(nz), static_cast<int>(p.chunk), xp_chunk,
                static_cast<int>(ldc / kGemmBK));
      if (st != LMX_OK) return st;
    }
    // 2. logits Z = X_c W^T over all ldv columns, taken as Z^T = W X_c^T (tiles
    // of W rows through LDS, written out transposed; rows of W past V read as
    // zero and give the padding columns)
    {
      const int tile = pick_tile(ldv, rows);
      GemmShape g = make_shape(p.w, p.D, nullptr, 0, static_cast<int>(ldv), rows, rows, D, 1, tile);
      g.a_rows = V;
      g.Bp = xp + slot * xp_chunk;
      g.bp_ks = ks_d;
      if (c == 0) {
        g.at_out = wtp;
        g.at_pk_ks = ks_v;
        g.at_cols = static_cast<int>(ldv);
        EpiOutT<E, true> e{z, ldv, static_cast<int>(ldv)};
        st = tile == kTileL ? launch_gemm_split_tail<1, E>(g, e, stream)
                            : launch_gemm<1, E>(g, tile, e, stream);
      } else {
        EpiOutT<E, false> e{z, ldv, static_cast<int>(ldv)};
        st = tile == kTileL ? launch_gemm_split_tail<1, E>(g, e, stream)
                            : launch_gemm<1, E>(g, tile, e, stream);
      }
      if (st != LMX_OK) return st;
    }
    // 3. cross-entropy of the chunk rows, G written over Z, loss terms
    {
      CeParams cp{};
      cp.logits = z;
      cp.grad = z;
      cp.target = tc;
      cp.B = rows;
      cp.V = p.V;
      cp.ld = ldv;
      cp.ignore_index = p.ignore_index;
      cp.z = p.z;
      cp.reduction = LMX_SUM;   // the mean's 1/N enters in steps 5 and 6
      cp.n_valid_ws = n_ws;
      cp.row_loss = row_loss + r0;
      cp.few_rows = 1;
      st = ce_rows_enqueue(cp, p.dtype, stream);
      if (st != LMX_OK) return st;
    }
    // 4. G^T for the grad_weight product: written by step 5's product, which
    // loads every tile of G anyway, except for a ragged last chunk
    const bool fuse_gt = rows == p.chunk;
    if (!fuse_gt) {
      st = transpose_pad(z, ldv, rows, V, gt + slot * ldc, ldk, static_cast<int>(ldc), stream);
      if (st != LMX_OK) return st;
    }
    // 5. grad_inputs rows
    st = chunk_grad_inputs<E>(z, ldv, static_cast<int>(ldv), wtp, ldv, rows, D, p.chunk,
                              static_cast<int>(wl.ksplit), dxp, p.grad_x + r0 * p.D, p.D,
                              mean_count, fuse_gt ? gt + slot * ldc : nullptr, ldk,
                              static_cast<int>(ldc), stream);
    if (st != LMX_OK) return st;
    // 6. grad_weight, once per group of chunks
    if (slot == grp - 1 || c == nchunks - 1) {
      st = grad_weight_group<E>(p.accum, c / grp, (nchunks + grp - 1) / grp, gt, xtp, ldk,
                                static_cast<int>((slot + 1) * ldc), ldc, V, D, dw, p.grad_w, p.D,
                                mean_count, dwp, wl.dwp_bytes, stream);
      if (st != LMX_OK) return st;
    }
  }
  return finish_enqueue(row_loss, p.BT, n_ws, p.reduction, p.loss, stream);
}

size_t linear_loss_logits_workspace(int64_t rows, int64_t D) {
  const size_t b = packed_bytes(rows, D);
  return b > kWsAlign ? align_up(b, kWsAlign) : kWsAlign;
}

// The logits of one chunk of the generic loss into the caller's buffer. When
// its rows take whole 16-byte pieces, as the fused path's logits: Z^T = W X_c^T
// with W's tiles through LDS and the chunk's packed X_c (in ws) as the B
// operand, each tile written out transposed (columns >= V untouched); else
// X_c W^T with W through LDS too and element stores.
template <typename E>
int linear_loss_logits_run(const uint16_t* xc, const uint16_t* w, int rows, int D, int V,
                           uint16_t* logits, int64_t ld_logits, void* ws, hipStream_t stream) {
  if (rows == 0) return LMX_OK;
  if (staged_ok(logits, ld_logits, V)) {
    uint16_t* xp = static_cast<uint16_t*>(ws);
    int st = pack(xc, D, rows, D, static_cast<int>(round_up64(rows, kGemmBK)), xp, nullptr, 0, 0,
                  stream);
    if (st != LMX_OK) return st;
    const int tile = pick_tile(V, rows);
    GemmShape g = make_shape(w, D, nullptr, 0, V, rows, rows, D, 1, tile);
    g.Bp = xp;
    g.bp_ks = static_cast<int>(packed_steps(D));
    EpiOutT<E, false> e{logits, ld_logits, V};
    return tile == kTileL ? launch_gemm_split_tail<1, E>(g, e, stream)
                          : launch_gemm<1, E>(g, tile, e, stream);
  }
  const int tile = pick_tile(rows, V);
  GemmShape g = make_shape(xc, D, w, D, rows, V, V, D, 1, tile);
  EpiOut<E> e{logits, ld_logits, nullptr, 0, nullptr, staged_ok(logits, ld_logits, V)};
  return tile == kTileL ? launch_gemm_split_tail<1, E>(g, e, stream)
                        : launch_gemm<1, E>(g, tile, e, stream);
}

template <typename E>
int linear_loss_grads_run(const LinearLossChunk& p, void* ws_base, hipStream_t stream) {
  const LinearCeWorkspace wl = linear_ce_workspace_layout(p.BT, p.D, p.V, p.chunk, p.accum, true, 0);
  char* ws = static_cast<char*>(ws_base);
  uint16_t* gt = reinterpret_cast<uint16_t*>(ws + wl.gt_off);
  uint16_t* xtp = reinterpret_cast<uint16_t*>(ws + wl.xt_off);
  uint16_t* wtp = reinterpret_cast<uint16_t*>(ws + wl.wt_off);
  float* dxp = reinterpret_cast<float*>(ws + wl.dxp_off);
  float* dw = reinterpret_cast<float*>(ws + wl.dw_off);
  float* dwp = reinterpret_cast<float*>(ws + wl.dwp_off);
  const int D = static_cast<int>(p.D), V = static_cast<int>(p.V);
  const int64_t ldv = wl.ldv, ldc = wl.ldc, ldk = wl.ldk, grp = wl.dw_group;
  const int64_t nchunks = (p.BT + p.chunk - 1) / p.chunk;
  const int64_t slot = p.index % grp;   // this chunk's columns in G^T and X^T
  int st;
  if (p.index == 0) {   // packed W^T for every chunk of the pass
    st = pack(p.w, p.D, V, D, static_cast<int>(ldv), nullptr, wtp,
              static_cast<int>(packed_steps(ldv)), 0, stream);
    if (st != LMX_OK) return st;
  }
  st = pack(p.xc, p.D, p.rows, D, static_cast<int>(ldc), nullptr, xtp,
            static_cast<int>(packed_steps(ldk)), static_cast<int>(slot * ldc / kGemmBK), stream);
  if (st != LMX_OK) return st;
  const bool fuse_gt = p.rows == p.chunk;   // G^T from the grad_inputs product
  if (!fuse_gt) {
    st = transpose_pad(p.g, p.ld_g, p.rows, V, gt + slot * ldc, ldk, static_cast<int>(ldc),
                       stream);
    if (st != LMX_OK) return st;
  }
  st = chunk_grad_inputs<E>(p.g, p.ld_g, V, wtp, ldv, p.rows, D, p.chunk,
                            static_cast<int>(wl.ksplit), dxp, p.grad_xc, p.D, nullptr,
                            fuse_gt ? gt + slot * ldc : nullptr, ldk, static_cast<int>(ldc),
                            stream);
  if (st != LMX_OK) return st;
  // grad_weight, once per group of chunks (the group's G^T and X^T columns
  // stay in the workspace between the calls)
  if (slot != grp - 1 && p.index != nchunks - 1) return LMX_OK;
  return grad_weight_group<E>(p.accum, p.index / grp, (nchunks + grp - 1) / grp, gt, xtp, ldk,
                              static_cast<int>((slot + 1) * ldc), ldc, V, D, dw, p.grad_w, p.D,
                              nullptr, dwp, wl.dwp_bytes, stream);
}

int linear_ce_enqueue(const LinearCeParams& p, void* ws, hipStream_t stream) {
  return p.dtype == LMX_F16 ? linear_ce_run<F16>(p, ws, stream)
                            : linear_ce_run<Bf16>(p, ws, stream);
}

int linear_loss_logits_enqueue(int dtype, const uint16_t* xc, const uint16_t* w, int rows, int D,
                               int V, uint16_t* logits, int64_t ld_logits, void* ws,
                               hipStream_t stream) {
  return dtype == LMX_F16
             ? linear_loss_logits_run<F16>(xc, w, rows, D, V, logits, ld_logits, ws, stream)
             : linear_loss_logits_run<Bf16>(xc, w, rows, D, V, logits, ld_logits, ws, stream);
}

int linear_loss_grads_enqueue(const LinearLossChunk& p, void* ws, hipStream_t stream) {
  return p.dtype == LMX_F16 ? linear_loss_grads_run<F16>(p, ws, stream)
                            : linear_loss_grads_run<Bf16>(p, ws, stream);
}

}  // namespace lmx
