// The C ABI of liblmx.so: argument checks, workspace carving, then the enqueue
// functions of the kernel files. Every check here runs on the host before any
// HIP call, so an invalid call returns a status without touching the device.
#include <limits.h>

#include "internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

bool dtype_ok(int dtype) { return dtype == LMX_F32 || dtype == LMX_BF16 || dtype == LMX_F16; }

// One logits row must fit a 32-bit byte offset (row buffer resources and the
// kernels' per-row offsets are 32-bit), besides V < 2^30.
bool row_fits(int64_t V, int dtype) {
  const int64_t eb = dtype == LMX_F32 ? 4 : 2;
  return V > 0 && V < (int64_t{1} << 30) && V * eb <= INT32_MAX - 64;
}

// Linear-CE limits from the GEMM's 32-bit buffer offsets over 256-row panels
// (256 rows of the padded vocabulary, of D fp32 values, of the chunk rows).
constexpr int64_t kLinMaxV = 4194048, kLinMaxD = 2097088, kLinMaxChunk = 4194240;

bool mul_fits(int64_t a, int64_t b, int64_t c) {
  if (a < 0 || b < 0 || c < 0) return false;
  if (a == 0 || b == 0 || c == 0) return true;
  return a <= INT64_MAX / b && a * b <= INT64_MAX / c;
}

}  // namespace

namespace lmx {

int ce_args_status(const void* logits, const void* grad_logits, const int64_t* target,
                   int64_t B, int64_t V, int dtype, int reduction, const float* loss) {
  if (loss == nullptr) return LMX_ERR_NULL;
  if (B > 0 && (logits == nullptr || target == nullptr)) return LMX_ERR_NULL;
  if (B < 0 || !row_fits(V, dtype)) return LMX_ERR_SIZE;
  if (!dtype_ok(dtype)) return LMX_ERR_ENUM;
  if (reduction != LMX_MEAN && reduction != LMX_SUM) return LMX_ERR_ENUM;
  const int eb = dtype == LMX_F32 ? 4 : 2;
  if (!mul_fits(B, V, eb)) return LMX_ERR_SIZE;
  const size_t bytes = static_cast<size_t>(B) * static_cast<size_t>(V) * eb;
  const uintptr_t pl = reinterpret_cast<uintptr_t>(logits);
  const uintptr_t pg = reinterpret_cast<uintptr_t>(grad_logits);
  if (pl % eb != 0 || reinterpret_cast<uintptr_t>(target) % 8 != 0) return LMX_ERR_ALIGN;
  if (grad_logits != nullptr && (pg % 16) != (pl % 16)) return LMX_ERR_ALIGN;
  if (grad_logits != nullptr && grad_logits != logits &&
      overlaps(logits, bytes, grad_logits, bytes))
    return LMX_ERR_ALIAS;
  if (grad_logits != nullptr && overlaps(grad_logits, bytes, target, B * 8)) return LMX_ERR_ALIAS;
  return LMX_OK;
}

CeWorkspace ce_workspace_layout(int64_t B) {
  CeWorkspace w;
  w.n_valid_off = 0;
  w.row_loss_off = kAlign;
  w.total = w.row_loss_off + round_up(static_cast<size_t>(B > 0 ? B : 1) * sizeof(float), kAlign);
  return w;
}

}  // namespace lmx

extern "C" {

const char* lmx_status_string(int status) {
  switch (status) {
    case LMX_OK: return "ok";
    case LMX_ERR_NULL: return "a required pointer is NULL";
    case LMX_ERR_SIZE: return "a size is out of range";
    case LMX_ERR_ENUM: return "unknown dtype, reduction or accumulation value";
    case LMX_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case LMX_ERR_ALIAS: return "an output overlaps an input";
    case LMX_ERR_ALIGN: return "a pointer or leading dimension breaks the alignment rule";
    case LMX_ERR_CHUNK: return "chunk_size is negative";
    case LMX_ERR_UNSUPPORTED: return "combination not implemented";
    case LMX_ERR_HIP: return "a HIP runtime call failed";
    case LMX_ERR_SCRATCH:
      return "more rows than the fixed scratch buffer of the allocation-free entry point holds";
    default: return "unknown status";
  }
}

size_t ce_workspace_bytes(int64_t B, int64_t V, int dtype) {
  if (B < 0 || !dtype_ok(dtype) || !row_fits(V, dtype)) return 0;
  return lmx::ce_workspace_layout(B).total;
}

int ce_fwd_bwd(const void* logits, void* grad_logits, const int64_t* target, int64_t B,
               int64_t V, int dtype, int64_t ignore_index, int reduction,
               float z_loss_multiplier, float* loss, int64_t* n_valid, int32_t* bad_target,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return LMX_ERR_NULL;
  const int st = lmx::ce_args_status(logits, grad_logits, target, B, V, dtype, reduction, loss);
  if (st != LMX_OK) return st;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return LMX_ERR_WORKSPACE;
  const lmx::CeWorkspace wl = lmx::ce_workspace_layout(B);
  if (workspace_bytes < wl.total) return LMX_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  lmx::CeParams p{};
  p.logits = logits;
  p.grad = grad_logits;
  p.target = target;
  p.B = B;
  p.V = V;
  p.ld = V;
  p.ignore_index = ignore_index;
  p.z = z_loss_multiplier;
  p.reduction = reduction;
  p.n_valid_ws = reinterpret_cast<int64_t*>(ws + wl.n_valid_off);
  p.row_loss = reinterpret_cast<float*>(ws + wl.row_loss_off);
  p.loss = loss;
  p.n_valid_user = n_valid;
  p.bad_user = bad_target;
  return lmx::ce_enqueue(p, dtype, static_cast<hipStream_t>(stream));
}

// Shared checks and launch of the per-row forward entry points: the count
// kernel (N, the out-of-range flag), then the row kernel without a gradient,
// writing its per-row value straight into `out`.
static int rows_forward(const void* logits, const int64_t* target, int64_t B, int64_t V,
                        int dtype, int64_t ignore_index, int negate, float* out,
                        int64_t* n_valid, int32_t* bad, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (workspace == nullptr) return LMX_ERR_NULL;
  if (B > 0 && (logits == nullptr || target == nullptr || out == nullptr)) return LMX_ERR_NULL;
  if (B < 0 || !row_fits(V, dtype)) return LMX_ERR_SIZE;
  if (!dtype_ok(dtype)) return LMX_ERR_ENUM;
  const int eb = dtype == LMX_F32 ? 4 : 2;
  if (!mul_fits(B, V, eb)) return LMX_ERR_SIZE;
  const size_t bytes = static_cast<size_t>(B) * static_cast<size_t>(V) * eb;
  if (reinterpret_cast<uintptr_t>(logits) % eb != 0 ||
      reinterpret_cast<uintptr_t>(target) % 8 != 0 || reinterpret_cast<uintptr_t>(out) % 4 != 0)
    return LMX_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return LMX_ERR_WORKSPACE;
  if (overlaps(out, B * 4, logits, bytes) || overlaps(out, B * 4, target, B * 8))
    return LMX_ERR_ALIAS;
  const lmx::CeWorkspace wl = lmx::ce_workspace_layout(B);
  if (workspace_bytes < wl.total) return LMX_ERR_WORKSPACE;
  if (B == 0) return LMX_OK;
  lmx::CeParams p{};
  p.logits = logits;
  p.grad = nullptr;
  p.target = target;
  p.B = B;
  p.V = V;
  p.ld = V;
  p.ignore_index = ignore_index;
  p.z = 0.f;
  p.reduction = LMX_SUM;
  p.n_valid_ws = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + wl.n_valid_off);
  p.row_loss = out;
  p.n_valid_user = n_valid;
  p.bad_user = bad;
  p.negate = negate;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int r = lmx::count_enqueue(target, B, V, ignore_index, p.n_valid_ws, n_valid, bad, st);
  if (r != LMX_OK) return r;
  return lmx::ce_rows_enqueue(p, dtype, st);
}

int selective_log_softmax(const void* logits, const int64_t* index, int64_t B, int64_t V,
                          int dtype, float* out, int32_t* bad_index, void* workspace,
                          size_t workspace_bytes, void* stream) {
  // no index is ignored: INT64_MIN is never a valid index
  return rows_forward(logits, index, B, V, dtype, INT64_MIN, 1, out, nullptr, bad_index,
                      workspace, workspace_bytes, stream);
}

int ce_loss_rows(const void* logits, const int64_t* target, int64_t B, int64_t V, int dtype,
                 int64_t ignore_index, float* loss_rows, int64_t* n_valid, int32_t* bad_target,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return rows_forward(logits, target, B, V, dtype, ignore_index, 0, loss_rows, n_valid,
                      bad_target, workspace, workspace_bytes, stream);
}

int ce_loss_rows_vjp(const void* logits, const int64_t* target, const float* loss_rows,
                     const float* g, void* grad_logits, int64_t B, int64_t V, int dtype,
                     int64_t ignore_index, void* stream) {
  if (B > 0 && (logits == nullptr || target == nullptr || loss_rows == nullptr ||
                g == nullptr || grad_logits == nullptr))
    return LMX_ERR_NULL;
  if (B < 0 || !row_fits(V, dtype)) return LMX_ERR_SIZE;
  if (!dtype_ok(dtype)) return LMX_ERR_ENUM;
  const int eb = dtype == LMX_F32 ? 4 : 2;
  if (!mul_fits(B, V, eb)) return LMX_ERR_SIZE;
  const size_t bytes = static_cast<size_t>(B) * static_cast<size_t>(V) * eb;
  const uintptr_t pl = reinterpret_cast<uintptr_t>(logits);
  const uintptr_t pg = reinterpret_cast<uintptr_t>(grad_logits);
  if (pl % eb != 0 || reinterpret_cast<uintptr_t>(target) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(loss_rows) % 4 != 0 || reinterpret_cast<uintptr_t>(g) % 4 != 0)
    return LMX_ERR_ALIGN;
  if (pg % 16 != pl % 16) return LMX_ERR_ALIGN;
  if (grad_logits != logits && overlaps(logits, bytes, grad_logits, bytes)) return LMX_ERR_ALIAS;
  if (overlaps(grad_logits, bytes, target, B * 8) || overlaps(grad_logits, bytes, loss_rows, B * 4) ||
      overlaps(grad_logits, bytes, g, B * 4))
    return LMX_ERR_ALIAS;
  if (B == 0) return LMX_OK;
  lmx::VjpParams p{};
  p.logits = logits;
  p.grad = grad_logits;
  p.target = target;
  p.loss = loss_rows;
  p.g = g;
  p.B = B;
  p.V = V;
  p.ignore_index = ignore_index;
  return lmx::ce_vjp_enqueue(p, dtype, static_cast<hipStream_t>(stream));
}

size_t linear_loss_workspace_bytes(int64_t BT, int64_t D, int64_t V, int dtype,
                                   int64_t chunk_size, int accum) {
  if (BT < 0 || D <= 0 || V <= 0 || chunk_size < 0) return 0;
  if (dtype != LMX_BF16 && dtype != LMX_F16) return 0;
  if (accum != LMX_ACC_F32 && accum != LMX_ACC_WEIGHT) return 0;
  if (V > kLinMaxV || D > kLinMaxD) return 0;
  const int64_t c = lmx::linear_ce_resolve_chunk(BT, V, chunk_size);
  if (c > kLinMaxChunk) return 0;
  return lmx::linear_ce_workspace_layout(BT, D, V, c, accum, true, 0).total;
}

size_t linear_loss_logits_workspace_bytes(int64_t rows, int64_t D, int dtype) {
  if (rows < 0 || D <= 0 || D > kLinMaxD || rows > kLinMaxChunk) return 0;
  if (dtype != LMX_BF16 && dtype != LMX_F16) return 0;
  return lmx::linear_loss_logits_workspace(rows, D);
}

int linear_loss_logits(const void* inputs_c, const void* weight, int64_t rows, int64_t D,
                       int64_t V, int dtype, void* logits, int64_t ld_logits, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (weight == nullptr || (rows > 0 && (inputs_c == nullptr || logits == nullptr)))
    return LMX_ERR_NULL;
  // the output's row stride is bounded like V: the GEMM epilogue addresses 256
  // rows of it with 32-bit byte offsets
  if (rows < 0 || D <= 0 || V <= 0 || V > kLinMaxV || D > kLinMaxD || rows > kLinMaxChunk ||
      ld_logits < V || ld_logits > kLinMaxV)
    return LMX_ERR_SIZE;
  if (!dtype_ok(dtype)) return LMX_ERR_ENUM;
  if (dtype == LMX_F32) return LMX_ERR_UNSUPPORTED;
  if (D % 8 != 0 || reinterpret_cast<uintptr_t>(inputs_c) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(weight) % 16 != 0 || reinterpret_cast<uintptr_t>(logits) % 2 != 0)
    return LMX_ERR_ALIGN;
  const size_t lb = static_cast<size_t>(rows > 0 ? rows - 1 : 0) * ld_logits * 2 + V * 2;
  if (rows > 0 && (overlaps(logits, lb, inputs_c, static_cast<size_t>(rows) * D * 2) ||
                   overlaps(logits, lb, weight, static_cast<size_t>(V) * D * 2)))
    return LMX_ERR_ALIAS;
  if (rows == 0) return LMX_OK;
  if (workspace == nullptr) return LMX_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0 ||
      workspace_bytes < lmx::linear_loss_logits_workspace(rows, D))
    return LMX_ERR_WORKSPACE;
  return lmx::linear_loss_logits_enqueue(dtype, static_cast<const uint16_t*>(inputs_c),
                                         static_cast<const uint16_t*>(weight),
                                         static_cast<int>(rows), static_cast<int>(D),
                                         static_cast<int>(V), static_cast<uint16_t*>(logits),
                                         ld_logits, workspace, static_cast<hipStream_t>(stream));
}

int linear_loss_grads(const void* inputs_c, const void* weight, const void* grad_logits,
                      int64_t ld_grad, int64_t rows, int64_t BT, int64_t D, int64_t V, int dtype,
                      int64_t chunk_size, int accum, int64_t chunk_index, void* grad_inputs_c,
                      void* grad_weight, void* workspace, size_t workspace_bytes, void* stream) {
  if (weight == nullptr || grad_weight == nullptr || workspace == nullptr) return LMX_ERR_NULL;
  if (rows > 0 && (inputs_c == nullptr || grad_logits == nullptr || grad_inputs_c == nullptr))
    return LMX_ERR_NULL;
  // the gradient's row stride is bounded like V (256-row operand panels are
  // addressed with 32-bit byte offsets)
  if (BT <= 0 || D <= 0 || V <= 0 || V > kLinMaxV || D > kLinMaxD || ld_grad < V ||
      ld_grad > kLinMaxV)
    return LMX_ERR_SIZE;
  if (chunk_size < 0) return LMX_ERR_CHUNK;
  if (!dtype_ok(dtype)) return LMX_ERR_ENUM;
  if (accum != LMX_ACC_F32 && accum != LMX_ACC_WEIGHT) return LMX_ERR_ENUM;
  if (dtype == LMX_F32) return LMX_ERR_UNSUPPORTED;
  const int64_t c = lmx::linear_ce_resolve_chunk(BT, V, chunk_size);
  if (c > kLinMaxChunk) return LMX_ERR_SIZE;
  const int64_t nchunks = (BT + c - 1) / c;
  if (chunk_index < 0 || chunk_index >= nchunks) return LMX_ERR_CHUNK;
  const int64_t expect = BT - chunk_index * c < c ? BT - chunk_index * c : c;
  if (rows != expect) return LMX_ERR_SIZE;
  if (D % 8 != 0 || V % 8 != 0 || ld_grad % 8 != 0) return LMX_ERR_ALIGN;
  for (const void* q : {inputs_c, weight, grad_logits, static_cast<const void*>(grad_inputs_c),
                        static_cast<const void*>(grad_weight)}) {
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return LMX_ERR_ALIGN;
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return LMX_ERR_WORKSPACE;
  const size_t xb = static_cast<size_t>(rows) * D * 2, wb = static_cast<size_t>(V) * D * 2;
  const size_t gb = static_cast<size_t>(rows) * ld_grad * 2;
  if (overlaps(grad_inputs_c, xb, inputs_c, xb) || overlaps(grad_inputs_c, xb, weight, wb) ||
      overlaps(grad_inputs_c, xb, grad_logits, gb) || overlaps(grad_weight, wb, inputs_c, xb) ||
      overlaps(grad_weight, wb, weight, wb) || overlaps(grad_weight, wb, grad_logits, gb) ||
      overlaps(grad_inputs_c, xb, grad_weight, wb))
    return LMX_ERR_ALIAS;
  const lmx::LinearCeWorkspace wl = lmx::linear_ce_workspace_layout(BT, D, V, c, accum, true, 0);
  if (workspace_bytes < wl.total) return LMX_ERR_WORKSPACE;
  lmx::LinearLossChunk p{};
  p.dtype = dtype;
  p.xc = static_cast<const uint16_t*>(inputs_c);
  p.w = static_cast<const uint16_t*>(weight);
  p.g = static_cast<const uint16_t*>(grad_logits);
  p.ld_g = ld_grad;
  p.rows = static_cast<int>(rows);
  p.BT = BT;
  p.D = D;
  p.V = V;
  p.chunk = c;
  p.accum = accum;
  p.index = chunk_index;
  p.grad_xc = static_cast<uint16_t*>(grad_inputs_c);
  p.grad_w = static_cast<uint16_t*>(grad_weight);
  return lmx::linear_loss_grads_enqueue(p, workspace, static_cast<hipStream_t>(stream));
}

int64_t linear_ce_chunk_rows(int64_t BT, int64_t V, int64_t chunk_size) {
  if (BT < 0 || V <= 0 || chunk_size < 0) return 0;
  return lmx::linear_ce_resolve_chunk(BT, V, chunk_size);
}

size_t linear_ce_workspace_bytes(int64_t BT, int64_t D, int64_t V, int dtype,
                                 int64_t chunk_size, int accum, int64_t group_bytes) {
  if (BT < 0 || D <= 0 || V <= 0 || chunk_size < 0 || group_bytes < 0) return 0;
  if (dtype != LMX_BF16 && dtype != LMX_F16) return 0;
  if (accum != LMX_ACC_F32 && accum != LMX_ACC_WEIGHT) return 0;
  if (V > kLinMaxV || D > kLinMaxD) return 0;
  const int64_t c = lmx::linear_ce_resolve_chunk(BT, V, chunk_size);
  if (c > kLinMaxChunk) return 0;
  return lmx::linear_ce_workspace_layout(BT, D, V, c, accum, false, group_bytes).total;
}

int linear_ce(const void* inputs, const void* weight, const int64_t* target, int64_t BT,
              int64_t D, int64_t V, int dtype, int64_t ignore_index, int reduction,
              float z_loss_multiplier, int64_t chunk_size, int accum, int64_t group_bytes,
              float* loss, void* grad_inputs, void* grad_weight, int64_t* n_valid,
              int32_t* bad_target, void* workspace, size_t workspace_bytes, void* stream) {
  if (weight == nullptr || loss == nullptr || grad_weight == nullptr || workspace == nullptr)
    return LMX_ERR_NULL;
  if (BT > 0 && (inputs == nullptr || target == nullptr || grad_inputs == nullptr))
    return LMX_ERR_NULL;
  if (BT < 0 || D <= 0 || V <= 0 || V > kLinMaxV || D > kLinMaxD || group_bytes < 0)
    return LMX_ERR_SIZE;
  if (chunk_size < 0) return LMX_ERR_CHUNK;
  if (!dtype_ok(dtype)) return LMX_ERR_ENUM;
  if (reduction != LMX_MEAN && reduction != LMX_SUM) return LMX_ERR_ENUM;
  if (accum != LMX_ACC_F32 && accum != LMX_ACC_WEIGHT) return LMX_ERR_ENUM;
  if (dtype == LMX_F32) return LMX_ERR_UNSUPPORTED;
  if (!mul_fits(BT, D, 2) || !mul_fits(V, D, 4) || !mul_fits(BT, V, 2)) return LMX_ERR_SIZE;
  if (D % 8 != 0) return LMX_ERR_ALIGN;
  for (const void* q : {inputs, weight, static_cast<const void*>(grad_inputs),
                        static_cast<const void*>(grad_weight)}) {
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return LMX_ERR_ALIGN;
  }
  if (reinterpret_cast<uintptr_t>(target) % 8 != 0) return LMX_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return LMX_ERR_WORKSPACE;
  const size_t xb = static_cast<size_t>(BT) * D * 2, wb = static_cast<size_t>(V) * D * 2;
  if (overlaps(grad_inputs, xb, inputs, xb) || overlaps(grad_inputs, xb, weight, wb) ||
      overlaps(grad_weight, wb, inputs, xb) || overlaps(grad_weight, wb, weight, wb) ||
      overlaps(grad_inputs, xb, grad_weight, wb) || overlaps(grad_inputs, xb, target, BT * 8) ||
      overlaps(grad_weight, wb, target, BT * 8))
    return LMX_ERR_ALIAS;
  const int64_t c = lmx::linear_ce_resolve_chunk(BT, V, chunk_size);
  if (c > kLinMaxChunk) return LMX_ERR_SIZE;
  const lmx::LinearCeWorkspace wl =
      lmx::linear_ce_workspace_layout(BT, D, V, c, accum, false, group_bytes);
  if (workspace_bytes < wl.total) return LMX_ERR_WORKSPACE;
  lmx::LinearCeParams p{};
  p.dtype = dtype;
  p.x = static_cast<const uint16_t*>(inputs);
  p.w = static_cast<const uint16_t*>(weight);
  p.target = target;
  p.BT = BT;
  p.D = D;
  p.V = V;
  p.ignore_index = ignore_index;
  p.z = z_loss_multiplier;
  p.reduction = reduction;
  p.chunk = c;
  p.accum = accum;
  p.group_bytes = group_bytes;
  p.loss = loss;
  p.grad_x = static_cast<uint16_t*>(grad_inputs);
  p.grad_w = static_cast<uint16_t*>(grad_weight);
  p.n_valid_user = n_valid;
  p.bad_user = bad_target;
  return lmx::linear_ce_enqueue(p, workspace, static_cast<hipStream_t>(stream));
}

int lmx_scale(const void* src, void* dst, int64_t n, int dtype, const float* scale,
              void* stream) {
  if (!dtype_ok(dtype)) return LMX_ERR_ENUM;
  if (n < 0) return LMX_ERR_SIZE;
  if (n == 0) return LMX_OK;
  if (src == nullptr || dst == nullptr || scale == nullptr) return LMX_ERR_NULL;
  const size_t es = dtype == LMX_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(src) % es != 0 || reinterpret_cast<uintptr_t>(dst) % es != 0 ||
      reinterpret_cast<uintptr_t>(scale) % 4 != 0)
    return LMX_ERR_ALIGN;
  if (static_cast<uint64_t>(n) > (UINT64_MAX / 2) / es) return LMX_ERR_SIZE;
  const size_t bytes = static_cast<size_t>(n) * es;
  if (src != dst && overlaps(src, bytes, dst, bytes)) return LMX_ERR_ALIAS;
  if (overlaps(scale, 4, dst, bytes)) return LMX_ERR_ALIAS;
  return lmx::scale_enqueue(src, dst, n, dtype, scale, static_cast<hipStream_t>(stream));
}

int lmx_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return LMX_OK;
  if (src == nullptr || dst == nullptr) return LMX_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return LMX_ERR_ALIGN;
  if (overlaps(src, bytes, dst, bytes)) return LMX_ERR_ALIAS;
  return lmx::copy_enqueue(src, dst, bytes, static_cast<hipStream_t>(stream));
}

int lmx_stream_probe(const void* src, void* dst, size_t bytes, size_t row_bytes, int mode,
                     void* stream) {
  if (mode < LMX_PROBE_READ || mode > LMX_PROBE_ROWS_PHASED) return LMX_ERR_ENUM;
  if (bytes == 0) return LMX_OK;
  if (dst == nullptr || (mode != LMX_PROBE_WRITE && src == nullptr)) return LMX_ERR_NULL;
  if (bytes % 16 != 0) return LMX_ERR_SIZE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return LMX_ERR_ALIGN;
  const bool rows = mode == LMX_PROBE_ROWS_INTERLEAVED || mode == LMX_PROBE_ROWS_PHASED;
  if (rows && (row_bytes == 0 || row_bytes % 16 != 0 || row_bytes > 262144 ||
               bytes % row_bytes != 0))
    return LMX_ERR_SIZE;
  // copies and rows: in place, or two separate buffers; read: dst is a 16 KiB sink
  if (mode == LMX_PROBE_READ) {
    if (overlaps(src, bytes, dst, 16384)) return LMX_ERR_ALIAS;
  } else if (mode != LMX_PROBE_WRITE && src != dst && overlaps(src, bytes, dst, bytes)) {
    return LMX_ERR_ALIAS;
  }
  return lmx::stream_probe_enqueue(src, dst, bytes, row_bytes, mode,
                                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
