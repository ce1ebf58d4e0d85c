// Cross-entropy loss and logits gradient over materialized logits [B, V].
//
// Method (greyhound functional API page, "cross_entropy"; online log-sum-exp as
// on the same page's "selective_log_softmax" entry): per valid row, one read
// sweep finds the row max and the sum of exp(x - max), giving
// lse = max + log(sum); the row loss is lse - x[t] + z lse^2; a second sweep
// writes scale * ((1 + 2 z lse) exp(x - lse) - onehot(t)). Ignored rows are
// only written (zeros).
//
// MI355X layout of the work:
// * one workgroup owns one row at a time and keeps the whole row in VGPRs
//   between the two sweeps, so the logits are read from HBM exactly once and
//   the gradient is written exactly once (a 128256-wide bf16 row is 250.5 KiB:
//   1024 threads x 16 chunks x 16 B);
// * rows are streamed in 16-byte chunks aligned to the buffer, so rows whose
//   byte length is not a multiple of 16 (V = 50257 in bf16) still use 128-bit
//   loads and stores; the partial chunk at each end of a row is masked with
//   -inf on load and written element by element;
// * the workgroup count is the number resident on the chip, and each
//   workgroup walks rows blockIdx, blockIdx + gridDim, ...;
// * rows too wide for the register file fall back to a streaming kernel that
//   reads the row twice (the second read usually hits L2 / MALL).
#include <type_traits>

#include "internal.h"

namespace lmx {

namespace {

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  static constexpr uint32_t kNegInfBits = 0xff800000u;
  __device__ static void unpack(const u32x4& c, float* x) {
    x[0] = __uint_as_float(c.x); x[1] = __uint_as_float(c.y);
    x[2] = __uint_as_float(c.z); x[3] = __uint_as_float(c.w);
  }
  __device__ static u32x4 pack(const float* g) {
    return u32x4{__float_as_uint(g[0]), __float_as_uint(g[1]),
                 __float_as_uint(g[2]), __float_as_uint(g[3])};
  }
  __device__ static float load_one(uintptr_t addr) {
    return *reinterpret_cast<const float*>(addr);
  }
  __device__ static float from_bits(uint32_t b) { return __uint_as_float(b); }
  __device__ static void store_one(__amdgpu_buffer_rsrc_t r, int off, float g) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g), r, off, 0, 0);
  }
  // Element e of a chunk set to -inf.
  __device__ static void set_neg_inf(u32x4& c, int e) { c[e] = kNegInfBits; }
};

template <> struct Elem<uint16_t> {  // bf16 stored as raw 16-bit patterns
  static constexpr int kPerChunk = 8;
  __device__ static void unpack(const u32x4& c, float* x) {
    x[0] = bf16_lo(c.x); x[1] = bf16_hi(c.x); x[2] = bf16_lo(c.y); x[3] = bf16_hi(c.y);
    x[4] = bf16_lo(c.z); x[5] = bf16_hi(c.z); x[6] = bf16_lo(c.w); x[7] = bf16_hi(c.w);
  }
  __device__ static u32x4 pack(const float* g) {
    return u32x4{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]),
                 pack_bf16x2(g[4], g[5]), pack_bf16x2(g[6], g[7])};
  }
  __device__ static float load_one(uintptr_t addr) {
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(addr));
  }
  __device__ static float from_bits(uint32_t b) { return bf16_bits_to_f32(static_cast<uint16_t>(b)); }
  __device__ static void store_one(__amdgpu_buffer_rsrc_t r, int off, float g) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(g), r, off, 0, 0);
  }
  __device__ static void set_neg_inf(u32x4& c, int e) {
    const uint32_t w = c[e >> 1];
    c[e >> 1] = (e & 1) ? ((w & 0x0000ffffu) | 0xff800000u) : ((w & 0xffff0000u) | 0x0000ff80u);
  }
};

// fp16 logits: raw 16-bit patterns, tagged by a distinct 2-byte type.
struct Half {
  uint16_t bits;
};
template <> struct Elem<Half> {
  static constexpr int kPerChunk = 8;
  __device__ static void unpack(const u32x4& c, float* x) {
    x[0] = f16_lo(c.x); x[1] = f16_hi(c.x); x[2] = f16_lo(c.y); x[3] = f16_hi(c.y);
    x[4] = f16_lo(c.z); x[5] = f16_hi(c.z); x[6] = f16_lo(c.w); x[7] = f16_hi(c.w);
  }
  __device__ static u32x4 pack(const float* g) {
    return u32x4{pack_f16x2(g[0], g[1]), pack_f16x2(g[2], g[3]),
                 pack_f16x2(g[4], g[5]), pack_f16x2(g[6], g[7])};
  }
  __device__ static float load_one(uintptr_t addr) {
    return f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(addr));
  }
  __device__ static float from_bits(uint32_t b) { return f16_bits_to_f32(static_cast<uint16_t>(b)); }
  __device__ static void store_one(__amdgpu_buffer_rsrc_t r, int off, float g) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_f16_bits(g), r, off, 0, 0);
  }
  __device__ static void set_neg_inf(u32x4& c, int e) {
    const uint32_t w = c[e >> 1];
    c[e >> 1] = (e & 1) ? ((w & 0x0000ffffu) | 0xfc000000u) : ((w & 0xffff0000u) | 0x0000fc00u);
  }
};

// Makes the compiler forget what it knows about a register-resident chunk, so
// each sweep re-widens the packed data instead of keeping a widened copy of the
// whole row alive (which would not fit the register file).
__device__ __forceinline__ void launder(u32x4& c) { asm volatile("" : "+v"(c)); }

// Whether exponentials fold the shift into one fma (bf16 only). fp32 and fp16
// logits take the difference x - m first: it is exact when x is near the max,
// where the probabilities are large, so the result stays within a few fp32
// ulps whatever the logits' offset. The folded form rounds m log2(e) once, an
// error of up to half an fp32 ulp of |m| log2(e) in every exponent: far below
// a bf16 output's rounding, but visible in fp16 outputs and fp32 losses once
// |m| reaches the thousands.
template <typename T>
constexpr bool kFoldShift = std::is_same<T, uint16_t>::value;

// exp(x - m) * 2^-extra, evaluated as a base-2 exponential (comb = m log2(e)
// + extra, used by the folded form).
template <typename T>
__device__ __forceinline__ float shifted_exp2(float x, float m, float extra, float comb) {
  if constexpr (!kFoldShift<T>) {
    return exp2_fast(__builtin_fmaf(x - m, kLog2e, -extra));
  } else {
    return exp2_fast(__builtin_fmaf(x, kLog2e, -comb));   // comb = m * log2(e) + extra
  }
}

// Buffer descriptor word 3 for untyped (raw) buffer access on CDNA.
constexpr int kRawBufferFlags = 0x00020000;
// Cache policy of the streaming loads and stores: non-temporal.
constexpr int kStreamAux = 2;

// One row as a buffer resource over the 16-byte chunks it touches. Loads past
// the end return zeros and stores past the end are dropped by the hardware, so
// per-chunk offsets are 32-bit and need no range checks.
struct RowView {
  __amdgpu_buffer_rsrc_t in, out;
  uintptr_t first;   // address of the chunk holding the row's first element
  int lead;          // elements of that chunk that precede the row
  int nch;           // chunks touched by the row
};

template <typename T>
__device__ __forceinline__ RowView row_view(uintptr_t base, uintptr_t gbase, int64_t row,
                                            int64_t V, int64_t ld) {
  constexpr int EPC = Elem<T>::kPerChunk;
  RowView r;
  const uintptr_t a0 = base + static_cast<uintptr_t>(row) * static_cast<uintptr_t>(ld) * sizeof(T);
  r.first = a0 & ~static_cast<uintptr_t>(15);
  r.lead = static_cast<int>((a0 - r.first) / sizeof(T));
  r.nch = static_cast<int>((r.lead + V + EPC - 1) / EPC);
  r.in = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(r.first), 0, r.nch * 16,
                                           kRawBufferFlags);
  r.out = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(gbase + (r.first - base)), 0,
                                            r.nch * 16, kRawBufferFlags);
  return r;
}

__device__ __forceinline__ u32x4 load_chunk(const RowView& r, int ci) {
  return __builtin_amdgcn_raw_buffer_load_b128(r.in, ci * 16, 0, kStreamAux);
}

// Sets the elements of chunk ci that are not part of the row to -inf (the
// partial chunks at both ends, and chunks past the end). Column arithmetic is
// 32-bit: the host rejects V >= 2^30.
template <typename T>
__device__ __forceinline__ void mask_edges(u32x4& c, int ci, const RowView& r, int V) {
  constexpr int EPC = Elem<T>::kPerChunk;
  if (ci == 0 || ci >= r.nch - 1) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int j = ci * EPC + e - r.lead;
      if (j < 0 || j >= V) Elem<T>::set_neg_inf(c, e);
    }
  }
}

// Stores gradient chunk ci: one 128-bit store for an interior chunk, element
// stores for the partial chunks at the row's ends. Chunks past the end fall
// outside the buffer resource and are dropped.
template <typename T>
__device__ __forceinline__ bool chunk_is_partial(const RowView& r, int ci, int V) {
  constexpr int EPC = Elem<T>::kPerChunk;
  return (ci == 0 && r.lead != 0) || (ci == r.nch - 1 && (r.lead + V) % EPC != 0);
}

template <typename T>
__device__ __forceinline__ void store_chunk(const RowView& r, int ci, int V, const float* vals) {
  constexpr int EPC = Elem<T>::kPerChunk;
  if (!chunk_is_partial<T>(r, ci, V)) {
    __builtin_amdgcn_raw_buffer_store_b128(Elem<T>::pack(vals), r.out, ci * 16, 0, kStreamAux);
  } else {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int j = ci * EPC + e - r.lead;
      if (j >= 0 && j < V) Elem<T>::store_one(r.out, ci * 16 + e * static_cast<int>(sizeof(T)), vals[e]);
    }
  }
}

__device__ __forceinline__ float reduction_scale(const CeParams& p) {
  const int64_t n = *p.n_valid_ws;
  return p.reduction == LMX_MEAN ? 1.0f / static_cast<float>(n) : 1.0f;
}

__device__ __forceinline__ bool row_is_valid(int64_t t, const CeParams& p) {
  return t != p.ignore_index && t >= 0 && t < p.V;
}

// Writes a zero gradient row (ignored rows); nothing is read.
template <typename T, int THREADS>
__device__ __forceinline__ void zero_row(const CeParams& p, int64_t row) {
  constexpr int EPC = Elem<T>::kPerChunk;
  const uintptr_t gb = reinterpret_cast<uintptr_t>(p.grad);
  const RowView r = row_view<T>(gb, gb, row, p.V, p.ld);
  float z[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) z[e] = 0.f;
  for (int ci = threadIdx.x; ci < r.nch; ci += THREADS) store_chunk<T>(r, ci, static_cast<int>(p.V), z);
}

// Barrier over LDS reads and writes of the threads only: this wave's LDS
// instructions complete (lgkmcnt), then all waves meet. Vector memory
// operations in flight (the next row's loads, direct-to-LDS copies into this
// thread's own slots, the gradient's stores) stay in flight; __syncthreads, or
// a release fence on LDS, would wait for them (the copies write LDS). The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Block-wide combine of per-thread (max, sum) pairs; every thread gets the result.
template <int THREADS>
__device__ __forceinline__ void block_lse(float& m, float& s, float* sm, float* ss) {
  constexpr int W = THREADS / 64;
  wave_lse_combine(m, s);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[w] = m; ss[w] = s; }
  lds_barrier();
  m = sm[0];
  s = ss[0];
#pragma unroll
  for (int i = 1; i < W; ++i) lse_combine(m, s, sm[i], ss[i]);
}

// ------------------------------------------------------------------ kernels

// N = number of valid rows, and the out-of-range flag. One workgroup, so the
// count needs no atomics and no zeroed memory.
__global__ __launch_bounds__(1024) void ce_count_kernel(const int64_t* target, int64_t B,
                                                        int64_t V, int64_t ignore_index,
                                                        int64_t* n_ws, int64_t* n_user,
                                                        int32_t* bad_user) {
  __shared__ int64_t sn[16];
  __shared__ int sb[16];
  int64_t n = 0;
  int bad = 0;
  for (int64_t i = threadIdx.x; i < B; i += 1024) {
    const int64_t t = target[i];
    if (t != ignore_index) {
      if (t >= 0 && t < V) ++n; else bad = 1;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    n += __shfl_xor(n, off, 64);
    bad |= __shfl_xor(bad, off, 64);
  }
  if ((threadIdx.x & 63) == 0) { sn[threadIdx.x >> 6] = n; sb[threadIdx.x >> 6] = bad; }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t tn = 0;
    int tb = 0;
    for (int i = 0; i < 16; ++i) { tn += sn[i]; tb |= sb[i]; }
    *n_ws = tn;
    if (n_user) *n_user = tn;
    if (bad_user) *bad_user = tb;
  }
}

// Hides a lane-index value from loop-invariant code motion, so the per-chunk
// offsets derived from it are recomputed where they are used instead of being
// held in registers across the row loop.
__device__ __forceinline__ int launder_int(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Target of a row, read through the constant address space: a scalar load
// (the targets are never written while a kernel runs: the entry points reject
// a gradient that overlaps them). A vector load would be waited for with the
// row's chunk loads in flight, and vector memory operations complete in order,
// so that wait would cover all of them.
__device__ __forceinline__ int64_t row_target(const CeParams& p, int64_t row) {
  typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;
  return ((const_i64_ptr)p.target)[row];
}

// First valid row at or after `row` in steps of `stride`; the ignored rows
// passed over get a zero loss term and (with a gradient) a zero gradient row.
template <typename T, int THREADS>
__device__ __forceinline__ int64_t next_valid_row(const CeParams& p, int64_t row, int64_t stride,
                                                  bool want_grad) {
  for (; row < p.B; row += stride) {
    if (row_is_valid(row_target(p, row), p)) break;
    if (threadIdx.x == 0) p.row_loss[row] = 0.f;
    if (want_grad) zero_row<T, THREADS>(p, row);
  }
  return row;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt vmcnt(N) alone: at most N of this wave's vector memory operations
// still in flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Chunks [0, PRE) of each thread of row r copied straight into LDS (no
// registers): chunk k of thread tid lands at lds + (k THREADS + tid) 16, the
// slot that thread reads back, so no other thread depends on it.
template <int PRE, int THREADS>
__device__ __forceinline__ void prefetch_to_lds(char* lds, const RowView& r, int tid) {
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r.in, (lds_ptr_t)(lds + k * THREADS * 16 + wave * 1024), 16, (tid + k * THREADS) * 16, 0,
        0, kStreamAux);
  }
}

// Register-resident rows: THREADS x CPT chunks of 16 B must cover a row.
// Once the gradient of a row is stored, the chunks of the workgroup's next
// valid row are loaded into the same registers, and the next row's online
// sweep consumes them as they arrive. (After the last row the loads go to an
// empty buffer resource: they return zeros and touch no memory.)
// GRAD: a gradient is written (p.grad != nullptr); a separate instantiation
// for the loss-only case keeps each variant's registers to its own sweeps.
// BURST: how the gradient is stored (see sweep 2). PRE > 0 (with GRAD): the
// first PRE chunks of every thread's share of the next row are copied into
// LDS as soon as the current row's sweep has read its own, so that part of
// the next row streams in while this row's gradient is computed and stored;
// the other CPT - PRE chunks are loaded into registers after the stores.
// MINW > 1 bounds the registers so that MINW waves fit on each SIMD (more
// workgroups resident per CU).
template <typename T, int THREADS, int CPT, bool GRAD, bool BURST = (THREADS >= 1024),
          int PRE = 0, int MINW = 1>
__global__ __launch_bounds__(THREADS, MINW) void ce_rows_reg_kernel(CeParams p) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int W = THREADS / 64;
  static_assert(PRE == 0 || (GRAD && BURST && PRE < CPT), "LDS prefetch with burst stores only");
  __shared__ float sm[2][W], ss[2][W];
  __shared__ float sxt[2];
  __shared__ __align__(16) char pre_lds[PRE > 0 ? PRE * THREADS * 16 : 16];
  const int tid = threadIdx.x;
  const float scale = reduction_scale(p);
  const uintptr_t base = reinterpret_cast<uintptr_t>(p.logits);
  constexpr bool want_grad = GRAD;
  const uintptr_t gbase = want_grad ? reinterpret_cast<uintptr_t>(p.grad) : base;
  const int V = static_cast<int>(p.V);
  const int64_t stride = gridDim.x;
  int par = 0;        // LDS slot parity; flips once per valid row (each has one barrier)
  int64_t row = next_valid_row<T, THREADS>(p, blockIdx.x, stride, want_grad);
  u32x4 d[CPT];
  if (row < p.B) {
    const RowView r0 = row_view<T>(base, gbase, row, p.V, p.ld);
    const int lt = launder_int(tid);
    if constexpr (PRE > 0) prefetch_to_lds<PRE, THREADS>(pre_lds, r0, lt);
    // chunks loaded in the order the sweep consumes them (here and at the end
    // of each row), so that the wait for chunk k leaves the later ones in flight
#pragma unroll
    for (int k = PRE; k < CPT; ++k) {
      d[k] = load_chunk(r0, lt + k * THREADS);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  bool first = true;
  while (row < p.B) {
    const int64_t t = row_target(p, row);
    const RowView r = row_view<T>(base, gbase, row, p.V, p.ld);
    // the chunk and element that hold x[t]
    const int tpos = r.lead + static_cast<int>(t);
    const int ct = tpos / EPC;
    const int et = tpos % EPC;
    // the workgroup's next valid row, whose chunks are loaded into the
    // registers once this row's are consumed
    const int64_t nrow = next_valid_row<T, THREADS>(p, row + stride, stride, want_grad);
    RowView rn = r;
    if (nrow < p.B) {
      rn = row_view<T>(base, gbase, nrow, p.V, p.ld);
    } else {
      rn.in = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0, 0,
                                                kRawBufferFlags);
    }
    // one online sweep (running max, sum rescaled when the max grows), each
    // chunk masked and consumed as it arrives, so the exponentials overlap the
    // loads still in flight; the thread holding x[t] passes it on through LDS.
    // Without a gradient the chunk's registers are refilled with the next row
    // at once.
    float m = -kInf, s = 0.f;
    if constexpr (PRE > 0) {
      // this row's LDS chunks have landed: after them this wave issued its
      // register loads (CPT - PRE), and, except for the first row, the
      // previous row's stores (at least CPT whole-chunk stores)
      if (first) wait_vm<CPT - PRE>(); else wait_vm<2 * CPT - PRE>();
      first = false;
#pragma unroll
      for (int k = 0; k < PRE; ++k)
        d[k] = *reinterpret_cast<const u32x4*>(pre_lds + (k * THREADS + tid) * 16);
    }
    {
      const int lp = launder_int(tid);
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int ci = lp + k * THREADS;
        mask_edges<T>(d[k], ci, r, V);
        float x[EPC];
        Elem<T>::unpack(d[k], x);
        if (ci == ct) {
          float v = x[0];
#pragma unroll
          for (int e = 1; e < EPC; ++e) v = e == et ? x[e] : v;
          sxt[par] = v;
        }
        float cm = x[0];
#pragma unroll
        for (int e = 1; e < EPC; ++e) cm = fmaxf(cm, x[e]);
        const float nm = fmaxf(m, cm);
        if (nm != -kInf) {
          s *= exp2_fast((m - nm) * kLog2e);
          const float nmL = nm * kLog2e;
#pragma unroll
          for (int e = 0; e < EPC; ++e) s += shifted_exp2<T>(x[e], nm, 0.f, nmL);
        }
        m = nm;
        if constexpr (!want_grad) {
          d[k] = load_chunk(rn, ci);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (PRE > 0) {
      // the sweep has consumed this thread's LDS chunks: refill its slots
      // with the next row's
      if (nrow < p.B) prefetch_to_lds<PRE, THREADS>(pre_lds, rn, launder_int(tid));
    }
    block_lse<THREADS>(m, s, sm[par], ss[par]);
    const float log2s = log2_fast(s);          // lse = m + ln(s), m the row max
    const float lse = m + log2s * kLn2;
    const float xt = sxt[par];
    par ^= 1;
    if (tid == 0) {
      const float rl = (m - xt) + log2s * kLn2 + p.z * lse * lse;
      p.row_loss[row] = p.negate ? -rl : rl;
    }
    if constexpr (!want_grad) {
      row = nrow;
      continue;
    }
    // sweep 2: gradient from the registers. The whole row is stored before
    // any load of the next row is issued: long runs of one direction per
    // workgroup stream faster than stores and loads alternating chunk by
    // chunk (a copy probe of this row layout: 6.0 against 5.2 TB/s). With
    // BURST the gradient is first packed into the row's registers and then
    // stored in one burst (faster for the 1024-thread rows; smaller rows,
    // two workgroups per CU, store each chunk as it is computed).
    const float c = scale * (1.f + 2.f * p.z * lse);
    const bool fold = c > 0.f && c < kInf;   // c folded into the exponent
    const float extra = fold ? log2s - log2_fast(c) : log2s;
    const float comb = m * kLog2e + extra;
    const float mul = fold ? 1.f : c;
#pragma unroll
    for (int k = 0; k < CPT; ++k) launder(d[k]);
    const int lg = launder_int(tid);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int ci = lg + k * THREADS;
      float x[EPC];
      Elem<T>::unpack(d[k], x);
      float gv[EPC];
      if (fold) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) gv[e] = shifted_exp2<T>(x[e], m, extra, comb);
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) gv[e] = mul * shifted_exp2<T>(x[e], m, extra, comb);
      }
      if (ci == ct) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) if (e == et) gv[e] -= scale;
      }
      if constexpr (BURST) {
        // partial chunks (the row's ends) are stored element by element now,
        // whole chunks in the burst below
        if (chunk_is_partial<T>(r, ci, V)) store_chunk<T>(r, ci, V, gv);
        else d[k] = Elem<T>::pack(gv);
      } else {
        store_chunk<T>(r, ci, V, gv);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (BURST) {
      const int ls = launder_int(tid);
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int ci = ls + k * THREADS;
        // chunks past the row's end fall outside the buffer resource
        if (!chunk_is_partial<T>(r, ci, V))
          __builtin_amdgcn_raw_buffer_store_b128(d[k], r.out, ci * 16, 0, kStreamAux);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const int ln = launder_int(tid);
#pragma unroll
      for (int k = PRE; k < CPT; ++k) {
        d[k] = load_chunk(rn, ln + k * THREADS);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    row = nrow;
  }
  if constexpr (PRE > 0) wait_vm<0>();   // no LDS copy outlives the workgroup
}

// Rows of any width: two read sweeps with an online max / sum per thread.
template <typename T, int THREADS>
__global__ __launch_bounds__(THREADS) void ce_rows_stream_kernel(CeParams p) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int W = THREADS / 64;
  __shared__ float sm[2][W], ss[2][W];
  __shared__ float sxt[2];
  const int tid = threadIdx.x;
  const float scale = reduction_scale(p);
  const uintptr_t base = reinterpret_cast<uintptr_t>(p.logits);
  const bool want_grad = p.grad != nullptr;
  const uintptr_t gbase = want_grad ? reinterpret_cast<uintptr_t>(p.grad) : base;
  const int V = static_cast<int>(p.V);
  int par = 0;
  for (int64_t row = blockIdx.x; row < p.B; row += gridDim.x) {
    const int64_t t = p.target[row];
    if (!row_is_valid(t, p)) {
      if (tid == 0) p.row_loss[row] = 0.f;
      if (want_grad) zero_row<T, THREADS>(p, row);
      continue;
    }
    const RowView r = row_view<T>(base, gbase, row, p.V, p.ld);
    if (tid == 0) {
      sxt[par] = Elem<T>::load_one(base + (static_cast<uintptr_t>(row) * p.ld + t) * sizeof(T));
    }
    float m = -kInf, s = 0.f;
    for (int ci = tid; ci < r.nch; ci += THREADS) {
      u32x4 c = load_chunk(r, ci);
      mask_edges<T>(c, ci, r, V);
      float x[EPC];
      Elem<T>::unpack(c, x);
      float cm = x[0];
#pragma unroll
      for (int e = 1; e < EPC; ++e) cm = fmaxf(cm, x[e]);
      if (cm > m) {
        s = (m == -kInf) ? 0.f : s * exp2_fast((m - cm) * kLog2e);
        m = cm;
      }
      if (m != -kInf) {
        const float mL = m * kLog2e;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s += shifted_exp2<T>(x[e], m, 0.f, mL);
      }
    }
    block_lse<THREADS>(m, s, sm[par], ss[par]);
    const float log2s = log2_fast(s);
    const float lse = m + log2s * kLn2;
    const float xt = sxt[par];
    par ^= 1;
    if (tid == 0) {
      const float rl = (m - xt) + log2s * kLn2 + p.z * lse * lse;
      p.row_loss[row] = p.negate ? -rl : rl;
    }
    if (!want_grad) continue;
    const float c = scale * (1.f + 2.f * p.z * lse);
    const int tpos = r.lead + static_cast<int>(t);
    const int ct = tpos / EPC;
    const int et = tpos % EPC;
    const float comb = m * kLog2e + log2s;
    for (int ci = tid; ci < r.nch; ci += THREADS) {
      u32x4 cch = load_chunk(r, ci);
      float x[EPC];
      Elem<T>::unpack(cch, x);
      float gv[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) gv[e] = c * shifted_exp2<T>(x[e], m, log2s, comb);
      if (ci == ct) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) if (e == et) gv[e] -= scale;
      }
      store_chunk<T>(r, ci, V, gv);
    }
  }
}

// Fixed-order sum of the row losses (fp64 partial sums), then / N for mean.
__global__ __launch_bounds__(1024) void ce_finish_kernel(const float* row_loss, int64_t B,
                                                         const int64_t* n_ws, int reduction,
                                                         float* loss) {
  __shared__ double sd[16];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < B; i += 1024) acc += static_cast<double>(row_loss[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) sd[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < 16; ++i) tot += sd[i];
    const double n = static_cast<double>(*n_ws);
    *loss = static_cast<float>(reduction == LMX_MEAN ? tot / n : tot);
  }
}

// Vector-Jacobian product of the unreduced per-row cross-entropy (nuvec FastOp
// page, "CrossEntropyVjp"): grad[i, j] = g_i (exp(x_ij - lse_i) - [j == t_i]),
// where lse_i is recovered from the forward's per-row loss as loss_i + x[i, t_i],
// so no reduction over the row is needed: one read and one write of the
// logits in all. Ignored rows (and rows with a target outside [0, V)) get
// zeros and are not read.
//
// Persistent workgroups of kVjpThreads threads walk rows blockIdx, blockIdx +
// gridDim, ...; a row is streamed kVjpPerThread 16-byte chunks per thread at a
// time (loads of a step, then its stores: the shape of the fastest plain copy
// measured on the chip; 1024 x 8 measured faster than 1024 x 4, 1024 x 16,
// 512 x 8, 512 x 16 and 256 x 8, and 7% faster than one 256-thread
// workgroup per row). The upstream values of row i + 1 (target, g, loss,
// x[t]) are read by scalar loads while row i streams. In place is safe: every
// wave has read x[i + 1, t] (the barrier takes it as an operand, so the load
// has landed) before any wave passes the barrier that starts row i + 1, and
// only this workgroup writes that row.
constexpr int kVjpThreads = 1024;
constexpr int kVjpPerThread = 8;
constexpr int kVjpChunks = kVjpThreads * kVjpPerThread;

// Raw bits of the element at addr through a scalar (uniform) load of the
// 4-byte word holding it. For a 16-bit element that word may include 2 bytes
// just outside the tensor; like the row kernels' aligned 16-byte chunks, the
// read stays inside the aligned granule that holds a tensor byte, so it never
// reaches another page, and the extra half is discarded.
template <typename T>
__device__ __forceinline__ uint32_t uniform_elem_bits(uintptr_t addr) {
  typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
  const uint32_t w = ((const_u32_ptr)(addr & ~static_cast<uintptr_t>(3)))[0];
  if constexpr (sizeof(T) == 4) return w;
  else return (addr & 2) ? (w >> 16) : (w & 0xffffu);
}

struct VjpRow {
  int64_t t;
  bool valid;
  float g;
  float loss;
  uint32_t xt_bits;   // x[t] as stored
};

template <typename T>
__device__ __forceinline__ VjpRow vjp_row(const VjpParams& p, int64_t row) {
  typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;
  typedef const __attribute__((address_space(4))) float* const_f32_ptr;
  VjpRow v{0, false, 0.f, 0.f, 0u};
  if (row >= p.B) return v;
  v.t = ((const_i64_ptr)p.target)[row];
  v.valid = v.t != p.ignore_index && v.t >= 0 && v.t < p.V;
  if (v.valid) {
    v.g = ((const_f32_ptr)p.g)[row];
    v.loss = ((const_f32_ptr)p.loss)[row];
    v.xt_bits = uniform_elem_bits<T>(reinterpret_cast<uintptr_t>(p.logits) +
                                     (static_cast<uintptr_t>(row) * p.V + v.t) * sizeof(T));
  }
  return v;
}

template <typename T>
__global__ __launch_bounds__(kVjpThreads) void ce_vjp_kernel(VjpParams p) {
  constexpr int EPC = Elem<T>::kPerChunk;
  const int tid = threadIdx.x;
  const uintptr_t base = reinterpret_cast<uintptr_t>(p.logits);
  const uintptr_t gbase = reinterpret_cast<uintptr_t>(p.grad);
  const int V = static_cast<int>(p.V);
  int64_t row = blockIdx.x;
  VjpRow cur = vjp_row<T>(p, row);
  while (row < p.B) {
    const int64_t nrow = row + gridDim.x;
    // x[t] of this row has landed in every wave before any wave stores it
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::"s"(cur.xt_bits) : "memory");
    const VjpRow nxt = vjp_row<T>(p, nrow);
    const RowView r = row_view<T>(base, gbase, row, p.V, p.V);
    if (!cur.valid) {
      float z[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) z[e] = 0.f;
      for (int c0 = tid; c0 < r.nch; c0 += kVjpChunks) {
#pragma unroll
        for (int k = 0; k < kVjpPerThread; ++k) store_chunk<T>(r, c0 + k * kVjpThreads, V, z);
      }
    } else {
      const float g = cur.g;
      const float xt = Elem<T>::from_bits(cur.xt_bits);
      // lse = loss + x[t] without a rounding: fp32 and fp16 logits take
      // x - lse in fp64 (the float loss input then carries the only
      // rounding), bf16 logits one fma
      const double lse_d = static_cast<double>(cur.loss) + static_cast<double>(xt);
      const float lseL = static_cast<float>(lse_d * static_cast<double>(kLog2e));
      const int tpos = r.lead + static_cast<int>(cur.t);
      const int ct = tpos / EPC;
      const int et = tpos % EPC;
      for (int c0 = tid; c0 < r.nch; c0 += kVjpChunks) {
        u32x4 d[kVjpPerThread];
#pragma unroll
        for (int k = 0; k < kVjpPerThread; ++k) d[k] = load_chunk(r, c0 + k * kVjpThreads);
#pragma unroll
        for (int k = 0; k < kVjpPerThread; ++k) {
          const int ci = c0 + k * kVjpThreads;
          float x[EPC], gv[EPC];
          Elem<T>::unpack(d[k], x);
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            if constexpr (!kFoldShift<T>) {
              const float dx = static_cast<float>(static_cast<double>(x[e]) - lse_d);
              gv[e] = g * exp2_fast(dx * kLog2e);
            } else {
              gv[e] = g * exp2_fast(__builtin_fmaf(x[e], kLog2e, -lseL));
            }
          }
          if (ci == ct) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) if (e == et) gv[e] -= g;
          }
          store_chunk<T>(r, ci, V, gv);   // chunks past the row fall outside the resource
        }
      }
    }
    cur = nxt;
    row = nrow;
  }
}

// ------------------------------------------------------------------ dispatch

struct RowKernel {
  const void* fn;
  int threads;
  int64_t capacity;  // chunks per row that fit; 0 = any (streaming)
  // for at most kFewRowsPerCu rows per CU (nullptr: fn): the same rows in
  // fewer registers, more workgroups resident per CU
  const void* few_rows_fn;
};

// With few rows per CU each workgroup walks only one or two rows, so the
// reads of a row are not overlapped with the stores of another within a
// workgroup; three workgroups per CU instead of two put more rows in flight
// at once. Taken only where the caller asks (CeParams::few_rows) and at most
// 4 rows per CU: the 1024-row chunks of the 8192 x 768 x 50257 linear
// cross-entropy, whose logits were just written, run 33 against 40 us; on
// logits read from HBM it depends on the width (768 to 1024 rows of 50256 or
// 50257: 1 to 6% slower; of 40001 to 45001: 7 to 10% faster; [4096, 50257]:
// 2.5% slower), so ce_fwd_bwd keeps two per CU.
constexpr int64_t kFewRowsPerCu = 4;

template <typename T, bool G>
const RowKernel* row_kernels(int* count) {
  static const RowKernel k[] = {
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 256, 1, G>), 256, 256, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 256, 2, G>), 256, 512, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 256, 4, G>), 256, 1024, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 256, 8, G>), 256, 2048, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 256, 16, G>), 256, 4096, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 512, 13, G>), 512, 6656,
       G ? reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 512, 13, G, false, 0, 6>)
         : nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 512, 16, G>), 512, 8192, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 1024, 12, G>), 1024, 12288, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_reg_kernel<T, 1024, 16, G, true, G ? 9 : 0>),
       1024, 16384, nullptr},
      {reinterpret_cast<const void*>(&ce_rows_stream_kernel<T, 1024>), 1024, 0, nullptr},
  };
  *count = static_cast<int>(sizeof(k) / sizeof(k[0]));
  return k;
}

}  // namespace

// Largest number of 16-byte chunks one row of this call touches.
int64_t ce_max_row_chunks(uintptr_t base, int64_t V, int64_t ld, int elem_bytes) {
  const int64_t epc = 16 / elem_bytes;
  const int64_t lead0 = static_cast<int64_t>((base & 15u) / elem_bytes);
  if ((ld * elem_bytes) % 16 == 0) return (lead0 + V + epc - 1) / epc;
  return (epc - 1 + V + epc - 1) / epc;
}

// Compute units of the current device (-1 on error).
static int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  return cus;
}

// Workgroups of a row-kernel launch: as many as are resident on the chip, at
// most one per row (each walks rows blockIdx, blockIdx + grid, ...).
static int occupancy_grid(const void* fn, int threads, int64_t rows) {
  const int cus = device_cus();
  if (cus <= 0) return -1;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess)
    return -1;
  if (per_cu < 1) per_cu = 1;
  const int64_t resident = static_cast<int64_t>(per_cu) * cus;
  return static_cast<int>(rows < resident ? rows : resident);
}

int count_enqueue(const int64_t* target, int64_t B, int64_t V, int64_t ignore_index,
                  int64_t* n_ws, int64_t* n_user, int32_t* bad_user, hipStream_t stream) {
  hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, target, B, V, ignore_index,
                     n_ws, n_user, bad_user);
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

int finish_enqueue(const float* row_loss, int64_t B, const int64_t* n_ws, int reduction,
                   float* loss, hipStream_t stream) {
  hipLaunchKernelGGL(ce_finish_kernel, dim3(1), dim3(1024), 0, stream, row_loss, B, n_ws,
                     reduction, loss);
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

int ce_rows_enqueue(const CeParams& p, int dtype, hipStream_t stream) {
  if (p.B > 0) {
    const int eb = dtype == LMX_F32 ? 4 : 2;
    const int64_t need = ce_max_row_chunks(reinterpret_cast<uintptr_t>(p.logits), p.V, p.ld, eb);
    int n = 0;
    const bool g = p.grad != nullptr;
    const RowKernel* ks =
        dtype == LMX_BF16 ? (g ? row_kernels<uint16_t, true>(&n) : row_kernels<uint16_t, false>(&n))
        : dtype == LMX_F16 ? (g ? row_kernels<Half, true>(&n) : row_kernels<Half, false>(&n))
                           : (g ? row_kernels<float, true>(&n) : row_kernels<float, false>(&n));
    const RowKernel* pick = &ks[n - 1];
    for (int i = 0; i < n; ++i) {
      if (ks[i].capacity == 0 || ks[i].capacity >= need) { pick = &ks[i]; break; }
    }
    const void* fn = pick->fn;
    if (p.few_rows && pick->few_rows_fn != nullptr) {
      const int cus = device_cus();
      if (cus <= 0) return LMX_ERR_HIP;
      if (p.B <= kFewRowsPerCu * cus) fn = pick->few_rows_fn;
    }
    const int grid = occupancy_grid(fn, pick->threads, p.B);
    if (grid <= 0) return LMX_ERR_HIP;
    CeParams pc = p;
    void* args[] = {&pc};
    if (hipLaunchKernel(fn, dim3(grid), dim3(pick->threads), args, 0, stream) != hipSuccess)
      return LMX_ERR_HIP;
  }
  return LMX_OK;
}

int ce_enqueue(const CeParams& p, int dtype, hipStream_t stream) {
  int st = count_enqueue(p.target, p.B, p.V, p.ignore_index, p.n_valid_ws, p.n_valid_user,
                         p.bad_user, stream);
  if (st != LMX_OK) return st;
  st = ce_rows_enqueue(p, dtype, stream);
  if (st != LMX_OK) return st;
  return finish_enqueue(p.row_loss, p.B, p.n_valid_ws, p.reduction, p.loss, stream);
}

int ce_vjp_enqueue(const VjpParams& p, int dtype, hipStream_t stream) {
  if (p.B == 0) return LMX_OK;
  if (p.B > INT32_MAX) return LMX_ERR_SIZE;
  const void* fn = dtype == LMX_BF16  ? reinterpret_cast<const void*>(&ce_vjp_kernel<uint16_t>)
                   : dtype == LMX_F16 ? reinterpret_cast<const void*>(&ce_vjp_kernel<Half>)
                                      : reinterpret_cast<const void*>(&ce_vjp_kernel<float>);
  VjpParams pc = p;
  void* args[] = {&pc};
  const int64_t grid = occupancy_grid(fn, kVjpThreads, p.B);
  if (grid <= 0) return LMX_ERR_HIP;
  if (hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(kVjpThreads), args, 0,
                      stream) != hipSuccess)
    return LMX_ERR_HIP;
  return LMX_OK;
}

}  // namespace lmx
