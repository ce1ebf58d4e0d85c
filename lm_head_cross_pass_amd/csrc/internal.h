// Host-side interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.h"

namespace lmx {

// Arguments of one cross-entropy call, as the kernels see them.
struct CeParams {
  const void* logits;       // [B, V]
  void* grad;               // [B, V] or nullptr (loss only); may equal logits
  const int64_t* target;    // [B]
  int64_t B, V;
  int64_t ld;               // row stride of logits and grad, in elements (>= V)
  int64_t ignore_index;
  float z;                  // z_loss_multiplier
  int reduction;            // LMX_MEAN / LMX_SUM
  int64_t* n_valid_ws;      // workspace: N (written by the count kernel)
  float* row_loss;          // workspace: [B] row loss terms
  float* loss;              // output scalar
  int64_t* n_valid_user;    // optional output
  int32_t* bad_user;        // optional output
  int negate;               // row outputs x[t] - lse instead of lse - x[t] (z must be 0)
  int few_rows;             // 1: with few rows per CU, the row kernel may take its instance
                            // with more workgroups per CU (the linear-CE chunk rows)
};

// N and the out-of-range flag over `target` (one workgroup, no zeroed memory needed).
int count_enqueue(const int64_t* target, int64_t B, int64_t V, int64_t ignore_index,
                  int64_t* n_ws, int64_t* n_user, int32_t* bad_user, hipStream_t stream);
// Fixed-order sum of B row losses, divided by N for mean, into *loss.
int finish_enqueue(const float* row_loss, int64_t B, const int64_t* n_ws, int reduction,
                   float* loss, hipStream_t stream);

// Enqueues only the row kernel (loss terms into row_loss, gradient), with N
// already in *n_valid_ws.
int ce_rows_enqueue(const CeParams& p, int dtype, hipStream_t stream);

// Enqueues count -> rows -> finish for one cross-entropy call.
int ce_enqueue(const CeParams& p, int dtype, hipStream_t stream);

// Largest number of 16-byte chunks any row touches (for kernel selection).
int64_t ce_max_row_chunks(uintptr_t base, int64_t V, int64_t ld, int elem_bytes);

// Per-row vector-Jacobian product of the unreduced cross-entropy:
// grad[i, :] = g[i] (softmax(x_i) - onehot(t_i)) with lse_i = loss[i] + x[i, t_i].
struct VjpParams {
  const void* logits;       // [B, V]
  void* grad;               // [B, V]; may equal logits
  const int64_t* target;    // [B]
  const float* loss;        // [B] forward per-row losses
  const float* g;           // [B] upstream gradient per row
  int64_t B, V;
  int64_t ignore_index;
};
int ce_vjp_enqueue(const VjpParams& p, int dtype, hipStream_t stream);

// Host checks of ce_fwd_bwd's arguments other than the workspace (LMX_OK when
// the call may proceed); no HIP call.
int ce_args_status(const void* logits, const void* grad_logits, const int64_t* target,
                   int64_t B, int64_t V, int dtype, int reduction, const float* loss);

// Workspace layout of ce_fwd_bwd.
struct CeWorkspace {
  size_t n_valid_off, row_loss_off, total;
};
CeWorkspace ce_workspace_layout(int64_t B);

// Linear cross-entropy.
struct LinearCeParams {
  int dtype;                // LMX_BF16 or LMX_F16 (inputs, weight and the gradients)
  const uint16_t* x;        // [BT, D]
  const uint16_t* w;        // [V, D]
  const int64_t* target;    // [BT]
  int64_t BT, D, V;
  int64_t ignore_index;
  float z;
  int reduction;
  int64_t chunk;            // rows per chunk (resolved, > 0)
  int accum;                // LMX_ACC_F32 / LMX_ACC_WEIGHT
  int64_t group_bytes;      // G^T budget of one grad_weight product (0: the default)
  float* loss;
  uint16_t* grad_x;         // [BT, D]
  uint16_t* grad_w;         // [V, D]
  int64_t* n_valid_user;
  int32_t* bad_user;
};

struct LinearCeWorkspace {
  int64_t ldv;              // padded vocabulary stride of the chunk buffers
  int64_t ldc;              // padded chunk-row stride of the transposed buffers
  int64_t ksplit;           // K splits of the grad_inputs GEMM
  int64_t dw_group;         // chunks per grad_weight product (as many as the G^T budget holds)
  int64_t ldk;              // K of a group: G^T's row stride, the packed X^T's K extent (dw_group * ldc)
  size_t n_valid_off, row_loss_off, z_off, gt_off, xt_off, wt_off, xp_off, dxp_off, dw_off,
      dwp_off, total;
  size_t dwp_bytes;         // K-split partials of grad_weight's last rows (0: none)
};
// generic = true: the layout of the generic chunked loss (no chunk logits
// buffer: the caller holds them). group_bytes: the G^T budget of one
// grad_weight product (0: the default, 2 GiB).
LinearCeWorkspace linear_ce_workspace_layout(int64_t BT, int64_t D, int64_t V, int64_t chunk,
                                             int accum, bool generic, int64_t group_bytes);
int64_t linear_ce_resolve_chunk(int64_t BT, int64_t V, int64_t chunk_size);
int linear_ce_enqueue(const LinearCeParams& p, void* ws, hipStream_t stream);

// Generic chunked linear loss (the caller's loss and logits gradient per chunk):
// logits of one chunk, then its gradients.
int linear_loss_logits_enqueue(int dtype, const uint16_t* xc, const uint16_t* w, int rows, int D,
                               int V, uint16_t* logits, int64_t ld_logits, void* ws,
                               hipStream_t stream);
// Workspace bytes of linear_loss_logits: the packed copy of the chunk's inputs.
size_t linear_loss_logits_workspace(int64_t rows, int64_t D);
struct LinearLossChunk {
  int dtype;                // LMX_BF16 or LMX_F16
  const uint16_t* xc;       // [rows, D]
  const uint16_t* w;        // [V, D]
  const uint16_t* g;        // [rows, ld_g]: d(loss)/d(logits) of the chunk
  int64_t ld_g;
  int rows;
  int64_t BT, D, V, chunk;  // chunk: rows per chunk of the whole pass (resolved)
  int accum;
  int64_t index;            // chunk number within the pass
  uint16_t* grad_xc;        // [rows, D]
  uint16_t* grad_w;         // [V, D]
};
int linear_loss_grads_enqueue(const LinearLossChunk& p, void* ws, hipStream_t stream);

int copy_enqueue(const void* src, void* dst, size_t bytes, hipStream_t stream);
int stream_probe_enqueue(const void* src, void* dst, size_t bytes, size_t row_bytes, int mode,
                         hipStream_t stream);

// dst[i] = RNE(src[i] * (*scale)) in fp32 arithmetic, for n elements of dtype.
int scale_enqueue(const void* src, void* dst, int64_t n, int dtype, const float* scale,
                  hipStream_t stream);

}  // namespace lmx
