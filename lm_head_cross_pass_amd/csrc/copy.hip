// Plain streaming copy: the copy kernel of known size used to calibrate
// hardware byte counters and to measure the practical HBM ceiling.
#include "internal.h"

namespace lmx {

namespace {

// Four 16-byte chunks per thread in flight, all loads before the stores.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
  constexpr int U = 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * U;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * 256;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

__global__ void copy_tail_kernel(const uint8_t* src, uint8_t* dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

int copy_enqueue(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 > 0) {
    // a large grid (up to 65536 workgroups) moves the most bytes on MI355X
    int64_t blocks = (n16 + 1023) / 1024;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
  }
  const int64_t tail = static_cast<int64_t>(bytes % 16);
  if (tail > 0) {
    hipLaunchKernelGGL(copy_tail_kernel, dim3(1), dim3(64), 0, stream,
                       static_cast<const uint8_t*>(src) + n16 * 16,
                       static_cast<uint8_t*>(dst) + n16 * 16, tail);
    if (hipGetLastError() != hipSuccess) return LMX_ERR_HIP;
  }
  return LMX_OK;
}


// ------------------------------------------------------------------ stream probes
// Streaming patterns of known size over one buffer, the HBM ceilings the
// cross-entropy row kernels are measured against (lmx_stream_probe). Every
// workgroup covers contiguous spans of 16-byte chunks through a buffer
// resource, so chunks past the end read zero and writes past it are dropped.

namespace {

constexpr int kProbeFlags = 0x00020000;   // raw buffer descriptor word 3
constexpr int kProbeAux = 2;              // non-temporal loads and stores

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(const char* base, size_t off,
                                                             size_t total, size_t span) {
  size_t n = off < total ? total - off : 0;
  if (n > span) n = span;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), 0, static_cast<int>(n),
                                           kProbeFlags);
}

// Read: T x U chunks per workgroup step; the XOR of everything read is kept
// in registers (and written to sink only for one impossible value, so the
// loads cannot be dropped and nothing is written).
template <int T, int U>
__global__ __launch_bounds__(T) void probe_read_kernel(const char* src, size_t bytes,
                                                       u32x4* sink) {
  const size_t span = static_cast<size_t>(T) * U * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t off = static_cast<size_t>(blockIdx.x) * span; off < bytes;
       off += static_cast<size_t>(gridDim.x) * span) {
    const __amdgpu_buffer_rsrc_t r = probe_rsrc(src, off, bytes, span);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (threadIdx.x + u * T) * 16, 0, kProbeAux);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0xf39cc060u &&
      acc.w == 0x5ced2b6fu)
    sink[threadIdx.x] = acc;
}

template <int T, int U>
__global__ __launch_bounds__(T) void probe_write_kernel(char* dst, size_t bytes) {
  const size_t span = static_cast<size_t>(T) * U * 16;
  const u32x4 v = {threadIdx.x, blockIdx.x, 0x3c3c3c3cu, 0x3c3c3c3cu};
  for (size_t off = static_cast<size_t>(blockIdx.x) * span; off < bytes;
       off += static_cast<size_t>(gridDim.x) * span) {
    const __amdgpu_buffer_rsrc_t r = probe_rsrc(dst, off, bytes, span);
#pragma unroll
    for (int u = 0; u < U; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v, r, (threadIdx.x + u * T) * 16, 0, kProbeAux);
  }
}

// Copy: each step loads T x U chunks, then stores them (in place allowed).
template <int T, int U>
__global__ __launch_bounds__(T) void probe_copy_kernel(const char* src, char* dst, size_t bytes) {
  const size_t span = static_cast<size_t>(T) * U * 16;
  for (size_t off = static_cast<size_t>(blockIdx.x) * span; off < bytes;
       off += static_cast<size_t>(gridDim.x) * span) {
    const __amdgpu_buffer_rsrc_t ri = probe_rsrc(src, off, bytes, span);
    const __amdgpu_buffer_rsrc_t ro = probe_rsrc(dst, off, bytes, span);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(ri, (threadIdx.x + u * T) * 16, 0, kProbeAux);
#pragma unroll
    for (int u = 0; u < U; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v[u], ro, (threadIdx.x + u * T) * 16, 0, kProbeAux);
  }
}

// Rows of row_bytes with one 1024-thread workgroup per row at a time, 16
// chunks per thread held in registers (the layout of the widest cross-entropy
// row kernel), a workgroup-wide barrier per row. PHASED: a row is stored
// whole, then the next row is loaded whole; otherwise chunk k of a row is
// stored and chunk k of the next row loaded in turn.
template <bool PHASED>
__global__ __launch_bounds__(1024) void probe_rows_kernel(const char* src, char* dst,
                                                          size_t row_bytes, int64_t rows) {
  constexpr int T = 1024, CPT = 16;
  int64_t row = blockIdx.x;
  const size_t total = static_cast<size_t>(rows) * row_bytes;
  u32x4 d[CPT];
  if (row < rows) {
    const __amdgpu_buffer_rsrc_t r = probe_rsrc(src, static_cast<size_t>(row) * row_bytes,
                                                total, row_bytes);
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      d[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (threadIdx.x + k * T) * 16, 0, kProbeAux);
  }
  while (row < rows) {
    const int64_t nrow = row + gridDim.x;
    const __amdgpu_buffer_rsrc_t ro = probe_rsrc(dst, static_cast<size_t>(row) * row_bytes,
                                                 total, row_bytes);
    const __amdgpu_buffer_rsrc_t rn = probe_rsrc(src, static_cast<size_t>(nrow) * row_bytes,
                                                 total, nrow < rows ? row_bytes : 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (PHASED) {
#pragma unroll
      for (int k = 0; k < CPT; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(d[k], ro, (threadIdx.x + k * T) * 16, 0, kProbeAux);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < CPT; ++k)
        d[k] = __builtin_amdgcn_raw_buffer_load_b128(rn, (threadIdx.x + k * T) * 16, 0,
                                                     kProbeAux);
    } else {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        __builtin_amdgcn_raw_buffer_store_b128(d[k], ro, (threadIdx.x + k * T) * 16, 0, kProbeAux);
        d[k] = __builtin_amdgcn_raw_buffer_load_b128(rn, (threadIdx.x + k * T) * 16, 0,
                                                     kProbeAux);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    row = nrow;
  }
}

int probe_grid(size_t bytes, size_t span, int64_t cap) {
  const int64_t g = static_cast<int64_t>((bytes + span - 1) / span);
  return static_cast<int>(g < cap ? (g > 0 ? g : 1) : cap);
}

}  // namespace

int stream_probe_enqueue(const void* src, void* dst, size_t bytes, size_t row_bytes, int mode,
                         hipStream_t stream) {
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return LMX_ERR_HIP;
  switch (mode) {
    case LMX_PROBE_READ:
      hipLaunchKernelGGL((probe_read_kernel<256, 4>), dim3(probe_grid(bytes, 256 * 4 * 16, INT32_MAX)),
                         dim3(256), 0, stream, s, bytes, reinterpret_cast<u32x4*>(d));
      break;
    case LMX_PROBE_WRITE:
      hipLaunchKernelGGL((probe_write_kernel<1024, 8>), dim3(probe_grid(bytes, 1024 * 8 * 16, 4 * cus)),
                         dim3(1024), 0, stream, d, bytes);
      break;
    case LMX_PROBE_COPY:
      hipLaunchKernelGGL((probe_copy_kernel<256, 4>), dim3(probe_grid(bytes, 256 * 4 * 16, INT32_MAX)),
                         dim3(256), 0, stream, s, d, bytes);
      break;
    case LMX_PROBE_COPY_BATCHED:
      hipLaunchKernelGGL((probe_copy_kernel<1024, 8>), dim3(probe_grid(bytes, 1024 * 8 * 16, 4 * cus)),
                         dim3(1024), 0, stream, s, d, bytes);
      break;
    default: {
      const int64_t rows = static_cast<int64_t>(bytes / row_bytes);
      const int grid = static_cast<int>(rows < cus ? rows : cus);
      if (mode == LMX_PROBE_ROWS_PHASED)
        hipLaunchKernelGGL(probe_rows_kernel<true>, dim3(grid), dim3(1024), 0, stream, s, d,
                           row_bytes, rows);
      else
        hipLaunchKernelGGL(probe_rows_kernel<false>, dim3(grid), dim3(1024), 0, stream, s, d,
                           row_bytes, rows);
      break;
    }
  }
  return hipGetLastError() == hipSuccess ? LMX_OK : LMX_ERR_HIP;
}

}  // namespace lmx
