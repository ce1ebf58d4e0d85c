// Chunked linear cross-entropy: logits = inputs @ weight^T in row chunks, the
// cross-entropy loss and logits gradient per chunk, grad_inputs written per
// chunk and grad_weight accumulated across chunks (greyhound functional API
// page, "chunked_linear_loss" and "chunked_linear_cross_entropy").
//
// Per call:   count valid targets (global N, needed before any gradient is
//             scaled); W^T [D, ldv] (zero-padded) for the grad_inputs GEMM.
// Per chunk of C rows (r0 .. r0 + C'):
//   1. X_c^T [D, ldc]                                  transpose
//   2. Z = X_c W^T (bf16) and per (row, 128-column tile) (max, sum exp)
//                                                      MFMA GEMM, CE-stats epilogue
//   3. lse per row, row loss terms                     one wave per row
//   4. G = scale ((1 + 2 z lse) softmax - onehot) over Z, in place, and G^T
//                                                      64 x 64 tiles through LDS
//   5. grad_inputs[r0:] = G W                          MFMA GEMM (split-K if the
//                                                      tile count cannot fill the chip)
//   6. dW (+)= G^T X_c                                 MFMA GEMM, read-modify-write epilogue
// Finally the fixed-order loss reduction. In 'fp32' accumulation dW lives in
// an fp32 workspace and the last chunk's epilogue writes the rounded bf16
// result; in 'weight' accumulation the bf16 grad_weight itself is updated per
// chunk (rounded to nearest even after each chunk).
//
// The logits and G are kept in bf16 between steps, as bf16 matmuls produce
// them; the (max, sum exp) statistics are taken from the rounded logits, so G
// is exactly the cross-entropy gradient of the bf16 logits up to fp32 rounding.
#include "gemm.h"
#include "internal.h"

namespace lmx {

namespace {

constexpr int kTile = 128;        // GEMM tile (BM = BN) of all three products
constexpr int kLdvAlign = 256;    // vocabulary padding of the chunk buffers
constexpr int kLdcAlign = 64;     // chunk-row padding of the transposed buffers
constexpr size_t kWsAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up64(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------------ epilogues

// Step 2: logits tile -> bf16 chunk buffer, plus per-row (max, sum exp) of the
// tile's valid columns.
struct EpiLogits {
  uint16_t* z;
  int64_t ldz;
  float2* part;     // [tiles_n][ldp]
  int64_t ldp;
  int V;

  template <int BM, int BN, int FM, int FN>
  __device__ void run(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0, int,
                      const GemmShape& g, uint16_t* smem) {
    constexpr int LD = BN + 8;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          smem[ac.row(i, r) * LD + ac.col(j)] = f32_to_bf16_bits(acc[i][j][r]);
    __syncthreads();
    constexpr int TPR = kGemmThreads / BM;   // threads per row
    constexpr int CPT = BN / TPR;            // columns per thread
    const int tid = threadIdx.x;
    const int row = tid / TPR, h = tid % TPR;
    const int c0 = h * CPT;
    const bool row_ok = m0 + row < g.M;
    float m = -kInf;
    u32x4 v[CPT / 8];
#pragma unroll
    for (int q = 0; q < CPT / 8; ++q) {
      v[q] = *reinterpret_cast<const u32x4*>(smem + row * LD + c0 + q * 8);
      if (row_ok) {
        *reinterpret_cast<u32x4*>(z + static_cast<int64_t>(m0 + row) * ldz + n0 + c0 + q * 8) =
            v[q];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? bf16_hi(v[q][e >> 1]) : bf16_lo(v[q][e >> 1]);
        if (n0 + c0 + q * 8 + e < V) m = fmaxf(m, x);
      }
    }
    float s = 0.f;
    if (m != -kInf) {
#pragma unroll
      for (int q = 0; q < CPT / 8; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (e & 1) ? bf16_hi(v[q][e >> 1]) : bf16_lo(v[q][e >> 1]);
          if (n0 + c0 + q * 8 + e < V) s += exp2_fast((x - m) * kLog2e);
        }
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) {
      const float m2 = __shfl_xor(m, off, 64);
      const float s2 = __shfl_xor(s, off, 64);
      lse_combine(m, s, m2, s2);
    }
    if (h == 0 && row_ok) part[static_cast<int64_t>(n0 / BN) * ldp + m0 + row] = make_float2(m, s);
  }
};

// Step 5: grad_inputs rows (bf16), or fp32 split-K partials.
struct EpiDx {
  uint16_t* out;
  int64_t ldo;
  float* partial;   // [ksplit][M][ldp]
  int64_t ldp;

  template <int BM, int BN, int FM, int FN>
  __device__ void run(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0, int split,
                      const GemmShape& g, uint16_t*) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + ac.row(i, r), col = n0 + ac.col(j);
          if (row < g.M && col < g.N) {
            if (g.ksplit == 1) {
              out[static_cast<int64_t>(row) * ldo + col] = f32_to_bf16_bits(acc[i][j][r]);
            } else {
              partial[(static_cast<int64_t>(split) * g.M + row) * ldp + col] = acc[i][j][r];
            }
          }
        }
  }
};

enum DwMode { kDwStoreF32 = 0, kDwAddF32 = 1, kDwAddF32ToBf16 = 2, kDwStoreBf16 = 3, kDwAddBf16 = 4 };

// Step 6: grad_weight accumulation.
struct EpiDw {
  float* acc32;     // [V][ld] fp32 accumulator ('fp32' mode)
  uint16_t* out16;  // [V][ld] bf16 grad_weight
  int64_t ld;
  int mode;

  template <int BM, int BN, int FM, int FN>
  __device__ void run(f32x16_t (&acc)[FM][FN], const AccCoord& ac, int m0, int n0, int,
                      const GemmShape& g, uint16_t*) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + ac.row(i, r), col = n0 + ac.col(j);
          if (row < g.M && col < g.N) {
            const int64_t idx = static_cast<int64_t>(row) * ld + col;
            const float v = acc[i][j][r];
            switch (mode) {
              case kDwStoreF32: acc32[idx] = v; break;
              case kDwAddF32: acc32[idx] += v; break;
              case kDwAddF32ToBf16: out16[idx] = f32_to_bf16_bits(acc32[idx] + v); break;
              case kDwStoreBf16: out16[idx] = f32_to_bf16_bits(v); break;
              default: out16[idx] = f32_to_bf16_bits(bf16_bits_to_f32(out16[idx]) + v); break;
            }
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

// Step 3: lse of each chunk row from the per-tile statistics, and its loss term.
__global__ __launch_bounds__(256) void chunk_lse_kernel(const float2* __restrict__ part,
                                                        int tiles_n, int64_t ldp,
                                                        const uint16_t* __restrict__ z,
                                                        int64_t ldz,
                                                        const int64_t* __restrict__ target,
                                                        int rows, int V, int64_t ignore_index,
                                                        float zl, float* __restrict__ lse_out,
                                                        float* __restrict__ row_loss) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float m = -kInf, s = 0.f;
  for (int tn = lane; tn < tiles_n; tn += 64) {
    const float2 ps = part[static_cast<int64_t>(tn) * ldp + row];
    lse_combine(m, s, ps.x, ps.y);
  }
  wave_lse_combine(m, s);
  if (lane == 0) {
    const int64_t t = target[row];
    const bool valid = t != ignore_index && t >= 0 && t < V;
    const float log_s = log2_fast(s) * kLn2;
    const float lse = m + log_s;
    lse_out[row] = lse;
    float l = 0.f;
    if (valid) {
      const float zt = bf16_bits_to_f32(z[static_cast<int64_t>(row) * ldz + t]);
      l = (m - zt) + log_s + zl * lse * lse;
    }
    row_loss[row] = l;
  }
}

// Step 4: G over the chunk logits (in place) and G^T, 64 x 64 tiles.
__global__ __launch_bounds__(256) void chunk_grad_kernel(uint16_t* __restrict__ zg, int64_t ldz,
                                                         uint16_t* __restrict__ gt, int64_t ldt,
                                                         const float* __restrict__ lse,
                                                         const int64_t* __restrict__ target,
                                                         const int64_t* __restrict__ n_ws,
                                                         int reduction, float zl, int rows,
                                                         int V, int64_t ignore_index) {
  __shared__ uint16_t t[64][64 + 2];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const float scale = reduction == LMX_MEAN ? 1.0f / static_cast<float>(*n_ws) : 1.0f;
  {
    const int rr = tid / 4, cc = (tid % 4) * 16;
    const int r = r0 + rr;
    bool valid = false;
    int64_t tg = -1;
    float lr = 0.f;
    if (r < rows) {
      tg = target[r];
      valid = tg != ignore_index && tg >= 0 && tg < V;
      lr = lse[r];
    }
    const float c = scale * (1.f + 2.f * zl * lr);
    const float comb = lr * kLog2e;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int col = c0 + cc + q * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < rows) v = *reinterpret_cast<const u32x4*>(zg + static_cast<int64_t>(r) * ldz + col);
      float gv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
        float gval = 0.f;
        if (valid && col + e < V) {
          gval = c * exp2_fast(__builtin_fmaf(x, kLog2e, -comb));
          if (col + e == tg) gval -= scale;
        }
        gv[e] = gval;
      }
      u32x4 o = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]),
                 pack_bf16x2(gv[4], gv[5]), pack_bf16x2(gv[6], gv[7])};
      if (r < rows) *reinterpret_cast<u32x4*>(zg + static_cast<int64_t>(r) * ldz + col) = o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[rr][cc + q * 8 + 2 * e] = static_cast<uint16_t>(o[e] & 0xffffu);
        t[rr][cc + q * 8 + 2 * e + 1] = static_cast<uint16_t>(o[e] >> 16);
      }
    }
  }
  __syncthreads();
  {
    const int cc = tid / 4, rr = (tid % 4) * 16;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = static_cast<uint32_t>(t[rr + q * 8 + 2 * e][cc]) |
               (static_cast<uint32_t>(t[rr + q * 8 + 2 * e + 1][cc]) << 16);
      }
      *reinterpret_cast<u32x4*>(gt + static_cast<int64_t>(c0 + cc) * ldt + r0 + rr + q * 8) = v;
    }
  }
}

// grad_inputs rows = bf16(sum over splits of the fp32 partials), fixed order.
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
  uint2 o = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
  *reinterpret_cast<uint2*>(out + static_cast<int64_t>(row) * ldo + col) = o;
}

__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    p[i] = 0;
}

// ------------------------------------------------------------------ host helpers

template <typename Epi>
int launch_gemm(const GemmShape& g, const Epi& epi, hipStream_t stream) {
  const int blocks = g.tiles_m * g.tiles_n * g.ksplit;
  if (blocks == 0) return LMX_OK;
  hipLaunchKernelGGL((gemm_nt_kernel<kTile, kTile, Epi>), dim3(blocks), dim3(kGemmThreads), 0,
                     stream, g, epi);
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

GemmShape make_shape(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int M, int N,
                     int K, int ksplit) {
  GemmShape g;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_m = (M + kTile - 1) / kTile;
  g.tiles_n = (N + kTile - 1) / kTile;
  const int ksteps = (K + kGemmBK - 1) / kGemmBK;
  if (ksplit < 1) ksplit = 1;
  if (ksplit > ksteps) ksplit = ksteps > 0 ? ksteps : 1;
  g.ksteps_per_split = (ksteps + ksplit - 1) / ksplit;
  g.ksplit = ksteps > 0 ? (ksteps + g.ksteps_per_split - 1) / g.ksteps_per_split : 1;
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

// K splits of the grad_inputs product: enough (split, tile) pairs to give every
// CU two workgroups, but at least 4 K steps per split.
int dx_ksplit(int64_t C, int64_t D, int64_t ldv) {
  const int64_t tiles = ((C + kTile - 1) / kTile) * ((D + kTile - 1) / kTile);
  const int64_t ksteps = ldv / kGemmBK;
  int64_t s = (512 + tiles - 1) / tiles;
  if (s > ksteps / 4) s = ksteps / 4;
  if (s < 1) s = 1;
  return static_cast<int>(s);
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
                                             int accum) {
  LinearCeWorkspace w{};
  const int64_t C = chunk > 0 ? chunk : 1;
  w.ldv = round_up64(V, kLdvAlign);
  w.ldc = round_up64(C, kLdcAlign);
  w.ntn = w.ldv / kTile;
  w.ksplit = dx_ksplit(C, D, w.ldv);
  const int64_t nchunks = BT > 0 ? (BT + C - 1) / C : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + (bytes > 0 ? bytes : 1), kWsAlign);
    return o;
  };
  w.n_valid_off = take(8);
  w.row_loss_off = take(static_cast<size_t>(BT) * 4);
  w.lse_off = take(static_cast<size_t>(C) * 4);
  w.part_off = take(static_cast<size_t>(w.ntn) * C * 8);
  w.z_off = take(static_cast<size_t>(C) * w.ldv * 2);
  w.gt_off = take(static_cast<size_t>(w.ldv) * w.ldc * 2);
  w.xt_off = take(static_cast<size_t>(D) * w.ldc * 2);
  w.wt_off = take(static_cast<size_t>(D) * w.ldv * 2);
  w.dxp_off = take(w.ksplit > 1 ? static_cast<size_t>(w.ksplit) * C * D * 4 : 0);
  w.dw_off = take(accum == LMX_ACC_F32 && nchunks > 1 ? static_cast<size_t>(V) * D * 4 : 0);
  w.total = off;
  return w;
}

int linear_ce_enqueue(const LinearCeParams& p, void* ws_base, hipStream_t stream) {
  const LinearCeWorkspace wl = linear_ce_workspace_layout(p.BT, p.D, p.V, p.chunk, p.accum);
  char* ws = static_cast<char*>(ws_base);
  int64_t* n_ws = reinterpret_cast<int64_t*>(ws + wl.n_valid_off);
  float* row_loss = reinterpret_cast<float*>(ws + wl.row_loss_off);
  float* lse = reinterpret_cast<float*>(ws + wl.lse_off);
  float2* part = reinterpret_cast<float2*>(ws + wl.part_off);
  uint16_t* z = reinterpret_cast<uint16_t*>(ws + wl.z_off);
  uint16_t* gt = reinterpret_cast<uint16_t*>(ws + wl.gt_off);
  uint16_t* xt = reinterpret_cast<uint16_t*>(ws + wl.xt_off);
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + wl.wt_off);
  float* dxp = reinterpret_cast<float*>(ws + wl.dxp_off);
  float* dw = reinterpret_cast<float*>(ws + wl.dw_off);
  const int D = static_cast<int>(p.D), V = static_cast<int>(p.V);
  const int64_t ldv = wl.ldv, ldc = wl.ldc;

  int st = count_enqueue(p.target, p.BT, p.V, p.ignore_index, n_ws, p.n_valid_user, p.bad_user,
                         stream);
  if (st != LMX_OK) return st;
  if (p.BT == 0) {
    const int64_t n = p.V * p.D;
    hipLaunchKernelGGL(zero_u16_kernel, dim3(1024), dim3(256), 0, stream, p.grad_w, n);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
    return finish_enqueue(row_loss, 0, n_ws, p.reduction, p.loss, stream);
  }
  st = transpose_pad(p.w, p.D, V, D, wt, ldv, static_cast<int>(ldv), stream);
  if (st != LMX_OK) return st;
  const int64_t nchunks = (p.BT + p.chunk - 1) / p.chunk;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t r0 = c * p.chunk;
    const int rows = static_cast<int>(p.BT - r0 < p.chunk ? p.BT - r0 : p.chunk);
    const uint16_t* xc = p.x + r0 * p.D;
    const int64_t* tc = p.target + r0;
    // 1. X_c^T
    st = transpose_pad(xc, p.D, rows, D, xt, ldc, static_cast<int>(ldc), stream);
    if (st != LMX_OK) return st;
    // 2. logits and per-tile statistics
    {
      GemmShape g = make_shape(xc, p.D, p.w, p.D, rows, V, D, 1);
      EpiLogits e{z, ldv, part, p.chunk, V};
      st = launch_gemm(g, e, stream);
      if (st != LMX_OK) return st;
    }
    // 3. lse and loss terms
    hipLaunchKernelGGL(chunk_lse_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, part,
                       static_cast<int>((V + kTile - 1) / kTile), p.chunk, z, ldv, tc, rows, V,
                       p.ignore_index, p.z, lse, row_loss + r0);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
    // 4. G in place, and G^T
    hipLaunchKernelGGL(chunk_grad_kernel, dim3(ldv / 64, ldc / 64), dim3(256), 0, stream, z, ldv,
                       gt, ldc, lse, tc, n_ws, p.reduction, p.z, rows, V, p.ignore_index);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
    // 5. grad_inputs rows
    {
      GemmShape g = make_shape(z, ldv, wt, ldv, rows, D, static_cast<int>(ldv),
                               static_cast<int>(wl.ksplit));
      EpiDx e{p.grad_x + r0 * p.D, p.D, dxp, p.D};
      st = launch_gemm(g, e, stream);
      if (st != LMX_OK) return st;
      if (g.ksplit > 1) {
        const int64_t total = static_cast<int64_t>(rows) * D / 4;
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                           dim3(256), 0, stream, dxp, g.ksplit, rows, D, p.D, p.grad_x + r0 * p.D,
                           p.D);
        if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
      }
    }
    // 6. grad_weight
    {
      int mode;
      const bool first = c == 0, last = c == nchunks - 1;
      if (p.accum == LMX_ACC_F32) {
        mode = nchunks == 1 ? kDwStoreBf16 : first ? kDwStoreF32 : last ? kDwAddF32ToBf16 : kDwAddF32;
      } else {
        mode = first ? kDwStoreBf16 : kDwAddBf16;
      }
      GemmShape g = make_shape(gt, ldc, xt, ldc, V, D, static_cast<int>(ldc), 1);
      EpiDw e{dw, p.grad_w, p.D, mode};
      st = launch_gemm(g, e, stream);
      if (st != LMX_OK) return st;
    }
  }
  return finish_enqueue(row_loss, p.BT, n_ws, p.reduction, p.loss, stream);
}

}  // namespace lmx
