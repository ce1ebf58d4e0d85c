/*
 * lmx.h -- C ABI of liblmx.so, large-vocabulary cross-entropy on MI355X (gfx950).
 *
 * Two operations following the greyhound functional API page:
 *
 *   ce_fwd_bwd  -- cross-entropy over materialized logits [B, V]: the reduced
 *                  loss and the logits gradient in one streaming pass
 *                  (page entry "cross_entropy": signature, Parameters, Returns).
 *   linear_ce   -- chunked linear cross-entropy: logits = inputs @ weight.T in
 *                  row chunks, the same loss and logits gradient per chunk, and
 *                  grad_inputs / grad_weight accumulated chunk by chunk without
 *                  materializing the full logits (page entries
 *                  "chunked_linear_loss" and "chunked_linear_cross_entropy").
 *
 * the building blocks of the generic chunked linear loss, whose per-chunk loss
 * and logits gradient come from the caller (page entries "chunked_linear_loss"
 * and "autograd_loss_and_logits_grad"):
 *
 *   linear_loss_logits -- the logits of one row chunk, inputs_c @ weight.T;
 *   linear_loss_grads  -- given the chunk's logits gradient, its grad_inputs
 *                  rows and the chunk's share of grad_weight;
 *
 * and three per-row operations on materialized logits:
 *
 *   selective_log_softmax -- log_softmax(x_i)[index_i] per row (greyhound
 *                  functional API page, entry "selective_log_softmax").
 *   ce_loss_rows   -- the unreduced per-row cross-entropy lse_i - x[i, t_i]
 *                  (nuvec FastOp page, variant "CrossEntropy").
 *   ce_loss_rows_vjp -- its gradient for the logits given a per-row upstream
 *                  gradient and the forward's per-row losses (nuvec FastOp
 *                  page, variant "CrossEntropyVjp").
 *
 * Common conventions
 * ------------------
 * - Every pointer argument, except the host-side `workspace_bytes` values, is a
 *   DEVICE pointer on the current HIP device. Tensors are dense row-major.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *   call only enqueues work on that stream: it never allocates, frees or
 *   synchronizes, and its outputs are valid once the stream reaches that point.
 * - The caller owns every buffer, including `workspace`, which must hold at
 *   least the byte count returned by the matching *_workspace_bytes query and
 *   be 256-byte aligned. Its contents on entry do not matter; calls that
 *   overlap in time must not share a workspace.
 * - Return value: LMX_OK (0) when the work was enqueued, or a negative status
 *   for an error found on the host; on such an error nothing is enqueued.
 *   lmx_status_string() names a status.
 * - Rows whose target equals ignore_index contribute neither loss nor
 *   gradient (their gradient rows are written as zeros). A valid target
 *   outside [0, V) breaks the page's precondition; the device sets
 *   *bad_target = 1 and treats that row as ignored (not counted in N).
 * - reduction LMX_MEAN divides by N, the number of valid rows of the whole
 *   call (N = 0 gives a NaN loss and zero gradients); LMX_SUM does not divide.
 * - The z-loss adds z_loss_multiplier * lse^2 per valid row inside the
 *   reduction, lse being the natural-log log-sum-exp of the row's logits.
 * - Arithmetic: fp32 accumulation everywhere; gradients are stored in the
 *   dtype of the tensor they belong to, rounded to nearest even; the loss is
 *   an fp32 scalar. The loss is reduced in a fixed order, so repeated calls on
 *   the same inputs give bitwise-identical results.
 */
#ifndef LMX_H_
#define LMX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the ABI are the only ones the library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define LMX_API __attribute__((visibility("default")))
#else
#define LMX_API
#endif

/* Element type of logits / inputs / weight and of their gradients (LMX_F16 is
 * IEEE binary16). */
typedef enum { LMX_F32 = 0, LMX_BF16 = 1, LMX_F16 = 2 } lmx_dtype;

/* The page's reduction literal: 'mean' or 'sum' (no 'none'). */
typedef enum { LMX_MEAN = 0, LMX_SUM = 1 } lmx_reduction;

/* The page's grad_weight_accum_dtype: 'fp32' (fp32 accumulator, cast once at
 * the end) or 'weight' (accumulate in the weight dtype, rounding between
 * chunks). */
typedef enum { LMX_ACC_F32 = 0, LMX_ACC_WEIGHT = 1 } lmx_accum;

/* Status codes. */
enum {
  LMX_OK = 0,
  LMX_ERR_NULL = -1,        /* a required pointer is NULL */
  LMX_ERR_SIZE = -2,        /* a size is negative or zero where it must be positive */
  LMX_ERR_ENUM = -3,        /* unknown dtype / reduction / accumulation value */
  LMX_ERR_WORKSPACE = -4,   /* workspace too small or not 256-byte aligned */
  LMX_ERR_ALIAS = -5,       /* an output partially overlaps an input */
  LMX_ERR_ALIGN = -6,       /* a pointer or leading dimension breaks the alignment rule */
  LMX_ERR_CHUNK = -7,       /* chunk_size < 0 */
  LMX_ERR_UNSUPPORTED = -8, /* a valid combination this library does not implement */
  LMX_ERR_HIP = -9,         /* a HIP runtime call failed while enqueuing */
  LMX_ERR_SCRATCH = -10     /* more rows than ce_fwd_bwd_noalloc's fixed scratch holds */
};

/*
 * ce_fwd_bwd -- cross-entropy loss and logits gradient from materialized logits.
 *
 * Defined by the greyhound functional API page, entry "cross_entropy": logits
 * [B, V], targets [B] in [0, V), ignore_index, reduction 'mean' | 'sum', and
 * z_loss_multiplier; it returns the cross-entropy plus the z-loss scaled by z.
 * Per valid row i:  loss_i = lse_i - x[i, t_i] + z * lse_i^2;
 * gradient row i:   scale * ((1 + 2 z lse_i) * softmax(x_i) - onehot(t_i)),
 * scale = 1/N (mean) or 1 (sum). This is the gradient for an upstream
 * gradient of 1; autograd wrappers multiply it by the upstream scalar.
 *
 *   logits        [B, V] of `dtype`, row-major, element-aligned.
 *   grad_logits   [B, V] of `dtype`, or NULL for the loss alone. It may be
 *                 exactly `logits` (the raw helper that overwrites the logits
 *                 with their gradient); any other overlap is LMX_ERR_ALIAS.
 *                 Its address must equal that of `logits` modulo 16
 *                 (LMX_ERR_ALIGN otherwise; any two 16-byte aligned buffers do).
 *   target        [B] int64, 8-byte aligned.
 *   B             rows, >= 0 (B = 0 writes loss = NaN for mean, 0 for sum).
 *   V             vocabulary size, 1 <= V < 2^30, and one row of `dtype` must
 *                 stay under 2^31 - 64 bytes (fp32: V < 536870896); the kernels
 *                 address a row with 32-bit byte offsets (LMX_ERR_SIZE otherwise).
 *   loss          one fp32 on the device (required).
 *   n_valid       one int64 on the device: N; may be NULL.
 *   bad_target    one int32 on the device, set to 1 if a valid target lies
 *                 outside [0, V), else 0; may be NULL.
 *   workspace     >= ce_workspace_bytes(B, V, dtype) bytes.
 */
LMX_API int ce_fwd_bwd(const void* logits, void* grad_logits, const int64_t* target,
               int64_t B, int64_t V, int dtype, int64_t ignore_index,
               int reduction, float z_loss_multiplier,
               float* loss, int64_t* n_valid, int32_t* bad_target,
               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes ce_fwd_bwd needs for these sizes (0 for invalid sizes). */
LMX_API size_t ce_workspace_bytes(int64_t B, int64_t V, int dtype);

/*
 * ce_fwd_bwd_noalloc -- ce_fwd_bwd without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.
 *
 * Same arguments, results and errors as ce_fwd_bwd, minus workspace /
 * workspace_bytes. The workspace is a fixed array inside the library, one per
 * GPU, held until the process ends (256 bytes + 4 MiB): it takes at most
 * 1048576 rows; a larger B returns LMX_ERR_SCRATCH before anything is
 * enqueued. The call allocates nothing. The first call on a device looks up
 * the array's device address there (a HIP runtime query, not an allocation).
 * Every call on one GPU uses that GPU's array, so calls that overlap in time
 * on one GPU (other streams, other threads) race: serialize them.
 */
LMX_API int ce_fwd_bwd_noalloc(const void* logits, void* grad_logits, const int64_t* target,
                               int64_t B, int64_t V, int dtype, int64_t ignore_index,
                               int reduction, float z_loss_multiplier,
                               float* loss, int64_t* n_valid, int32_t* bad_target,
                               void* stream);

/*
 * linear_ce -- chunked linear cross-entropy, loss plus grad_inputs and grad_weight.
 *
 * Defined by the greyhound functional API page, entries "chunked_linear_loss"
 * (row chunks of inputs @ weight.T, a loss and logits gradient per chunk,
 * gradients accumulated chunk by chunk, chunk_size rows per chunk) and
 * "chunked_linear_cross_entropy" (the cross-entropy specialization with
 * ignore_index, reduction, z_loss_multiplier and grad_weight_accum_dtype; bf16
 * or fp16 matmuls with fp32 accumulator state). 'mean' divides by the number
 * of valid tokens of the whole call, not of each chunk; that 1/N multiplies the
 * fp32 products, and the 16-bit logits gradient between the matmuls is that of
 * the summed loss (in fp16, p/N would underflow at large N).
 * "16-bit" below is the format `dtype` names, for every 16-bit buffer alike.
 *
 *   inputs        [BT, D] 16-bit, row-major, 16-byte aligned; D % 8 == 0.
 *   Size limits (LMX_ERR_SIZE beyond them; the GEMMs address 256-row panels
 *   with 32-bit byte offsets): V <= 4194048, D <= 2097088, and at most
 *   4194240 rows per chunk.
 *   weight        [V, D]  16-bit, row-major, 16-byte aligned.
 *   target        [BT] int64.
 *   dtype         LMX_BF16 or LMX_F16 (LMX_F32 gives LMX_ERR_UNSUPPORTED:
 *                 the matmuls take 16-bit operands).
 *   chunk_size    rows per chunk; 0 picks a size from a 1 GiB budget for the
 *                 chunk's logits; < 0 is LMX_ERR_CHUNK.
 *   accum         LMX_ACC_F32: grad_weight is accumulated in fp32 (within a
 *                 product over a group of chunks, and across groups in an fp32
 *                 workspace) and rounded once; LMX_ACC_WEIGHT: it is
 *                 accumulated in the weight's 16-bit format, rounding after
 *                 each chunk (within a group's product, and from one group to
 *                 the next through grad_weight itself).
 *   group_bytes   the most workspace bytes that the transposed logits
 *                 gradient of one grad_weight product may take: that product
 *                 covers as many chunks as that holds (at least one), and one
 *                 group's transposed gradient is all the workspace keeps of
 *                 it, whatever BT. 0 selects the default, 2 GiB. A larger
 *                 budget means fewer grad_weight passes (in fp32 mode, none
 *                 over an fp32 accumulator once one group takes every chunk)
 *                 for more workspace; < 0 is LMX_ERR_SIZE.
 *   loss          one fp32 on the device.
 *   grad_inputs   [BT, D] 16-bit output, 16-byte aligned.
 *   grad_weight   [V, D]  16-bit output, 16-byte aligned.
 *   n_valid, bad_target as for ce_fwd_bwd (may be NULL).
 *   workspace     >= linear_ce_workspace_bytes(BT, D, V, dtype, chunk_size, accum,
 *                 group_bytes);
 *                 its contents on entry do not matter.
 * Outputs must not overlap the inputs (LMX_ERR_ALIAS).
 */
LMX_API int linear_ce(const void* inputs, const void* weight, const int64_t* target,
              int64_t BT, int64_t D, int64_t V, int dtype,
              int64_t ignore_index, int reduction, float z_loss_multiplier,
              int64_t chunk_size, int accum, int64_t group_bytes,
              float* loss, void* grad_inputs, void* grad_weight,
              int64_t* n_valid, int32_t* bad_target,
              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes linear_ce needs (0 for invalid arguments). */
LMX_API size_t linear_ce_workspace_bytes(int64_t BT, int64_t D, int64_t V, int dtype,
                                 int64_t chunk_size, int accum, int64_t group_bytes);

/*
 * linear_loss_logits -- logits of one row chunk for the generic chunked loss.
 *
 * Greyhound functional API page, entry "chunked_linear_loss": inputs @ weight.T
 * evaluated in row chunks; this is one chunk, with 16-bit operands (`dtype`
 * LMX_BF16 or LMX_F16, the page's bf16/fp16 matmuls) and fp32 accumulation,
 * rounded to nearest even into the same format.
 *
 *   inputs_c    [rows, D] 16-bit, 16-byte aligned, D % 8 == 0.
 *   weight      [V, D] 16-bit, 16-byte aligned.
 *   logits      [rows, ld_logits] 16-bit output (ld_logits >= V; columns >= V
 *               are not written), not overlapping the inputs; ld_logits is
 *               bounded like V (<= 4194048, LMX_ERR_SIZE beyond).
 *   workspace   >= linear_loss_logits_workspace_bytes(rows, D, dtype) bytes,
 *               256-byte aligned (LMX_ERR_WORKSPACE otherwise; may be NULL
 *               when rows is 0): the packed copy of inputs_c that the matmul
 *               reads. Its contents on entry do not matter.
 * Limits as for linear_ce (LMX_ERR_SIZE); LMX_F32 is LMX_ERR_UNSUPPORTED.
 */
LMX_API int linear_loss_logits(const void* inputs_c, const void* weight, int64_t rows,
                               int64_t D, int64_t V, int dtype, void* logits,
                               int64_t ld_logits, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Workspace bytes linear_loss_logits needs (0 for invalid arguments). */
LMX_API size_t linear_loss_logits_workspace_bytes(int64_t rows, int64_t D, int dtype);

/*
 * linear_loss_grads -- gradients of one chunk of the generic chunked loss.
 *
 * Greyhound functional API page, entry "chunked_linear_loss": with the chunk's
 * logits gradient G_c (returned by the caller's loss-and-gradient function),
 *   grad_inputs[chunk rows] = G_c @ weight,
 *   grad_weight            (+)= G_c^T @ inputs_c,
 * accumulated over the chunks in fp32 (LMX_ACC_F32: a workspace accumulator,
 * rounded to the 16-bit format once, by the last chunk's call; the product is
 * taken once per group of chunks whose G_c^T the workspace holds together,
 * so some calls only store their chunk's operands) or in grad_weight itself
 * (LMX_ACC_WEIGHT: rounded after every chunk), the page's
 * grad_weight_accum_dtype.
 *
 * One pass over BT rows is nchunks = ceil(BT / c) calls, c =
 * linear_ce_chunk_rows(BT, V, chunk_size), with chunk_index 0, 1, ..., in
 * order, on one stream, sharing one workspace of
 * linear_loss_workspace_bytes(BT, D, V, dtype, chunk_size, accum) bytes that
 * must not be touched in between (chunk 0 stores weight.T there for the later
 * chunks). grad_weight is complete after the call for the last chunk.
 *
 *   inputs_c      [rows, D] 16-bit rows of this chunk (`dtype` LMX_BF16 or
 *                 LMX_F16 for every 16-bit buffer); rows must be the chunk's
 *                 size (c, or what is left of BT for the last one).
 *   grad_logits   [rows, ld_grad] 16-bit, 16-byte aligned; ld_grad >= V and
 *                 V % 8 == 0 and ld_grad % 8 == 0 (LMX_ERR_ALIGN otherwise);
 *                 ld_grad <= 4194048 like V (LMX_ERR_SIZE beyond).
 *                 Used as given: any reduction scale is the caller's.
 *   grad_inputs_c [rows, D] 16-bit output for this chunk's rows.
 *   grad_weight   [V, D] 16-bit output / accumulator.
 * Outputs must not overlap the inputs (LMX_ERR_ALIAS); a chunk_index outside
 * [0, nchunks) is LMX_ERR_CHUNK.
 */
LMX_API int linear_loss_grads(const void* inputs_c, const void* weight, const void* grad_logits,
                              int64_t ld_grad, int64_t rows, int64_t BT, int64_t D, int64_t V,
                              int dtype, int64_t chunk_size, int accum, int64_t chunk_index,
                              void* grad_inputs_c, void* grad_weight, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Workspace bytes linear_loss_grads needs for one pass (0 for invalid arguments). */
LMX_API size_t linear_loss_workspace_bytes(int64_t BT, int64_t D, int64_t V, int dtype,
                                           int64_t chunk_size, int accum);

/* Rows per chunk that linear_ce uses for this chunk_size argument (resolves 0). */
LMX_API int64_t linear_ce_chunk_rows(int64_t BT, int64_t V, int64_t chunk_size);

/*
 * selective_log_softmax -- one log-probability per row, without materializing
 * the log-softmax.
 *
 * Defined by the greyhound functional API page, entry "selective_log_softmax":
 * the equivalent of gather(log_softmax(logits, -1), -1, index), i.e. per row
 * out_i = x[i, index_i] - lse_i, computed with fp32 accumulation.
 *
 *   logits      [B, V] of `dtype`, row-major, element-aligned; V as for
 *               ce_fwd_bwd.
 *   index       [B] int64 in [0, V), 8-byte aligned.
 *   out         [B] fp32 output, 4-byte aligned, not overlapping the inputs.
 *   bad_index   one int32 on the device, set to 1 if an index lies outside
 *               [0, V) (that row's output is 0), else 0; may be NULL.
 *   workspace   >= ce_workspace_bytes(B, V, dtype) bytes.
 * B = 0 enqueues nothing but is valid.
 */
LMX_API int selective_log_softmax(const void* logits, const int64_t* index, int64_t B,
                                  int64_t V, int dtype, float* out, int32_t* bad_index,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * ce_loss_rows -- the unreduced per-row cross-entropy.
 *
 * Defined by the nuvec FastOp page, variant "CrossEntropy": per row
 * logsumexp(x_i) - x[i, t_i] in fp32. As everywhere in this library, a row
 * whose target equals ignore_index gets 0 (the page has no ignore index: pass
 * a value no target takes, e.g. -100, to reproduce it exactly); a valid target
 * outside [0, V) sets *bad_target = 1 and gets 0.
 *
 *   logits      [B, V] of `dtype`, row-major, element-aligned; V as for
 *               ce_fwd_bwd.
 *   target      [B] int64, 8-byte aligned.
 *   loss_rows   [B] fp32 output, 4-byte aligned, not overlapping the inputs.
 *   n_valid, bad_target as for ce_fwd_bwd (may be NULL).
 *   workspace   >= ce_workspace_bytes(B, V, dtype) bytes.
 */
LMX_API int ce_loss_rows(const void* logits, const int64_t* target, int64_t B, int64_t V,
                         int dtype, int64_t ignore_index, float* loss_rows, int64_t* n_valid,
                         int32_t* bad_target, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * ce_loss_rows_vjp -- gradient of sum_i g_i * ce_loss_rows_i for the logits.
 *
 * Defined by the nuvec FastOp page, variant "CrossEntropyVjp" (inputs logits,
 * targets, the forward's loss and the upstream gradient g): per valid row
 *   grad[i, :] = g_i * (softmax(x_i) - onehot(t_i)),
 * with the row's lse taken from the forward as loss_rows_i + x[i, t_i], so the
 * call is a single read of the logits and a single write of the gradient.
 * Ignored rows, and rows whose target lies outside [0, V), get zero rows.
 *
 *   logits      [B, V] of `dtype`, row-major, element-aligned; V as for
 *               ce_fwd_bwd.
 *   target      [B] int64, 8-byte aligned.
 *   loss_rows   [B] fp32: ce_loss_rows of the same logits and targets.
 *   g           [B] fp32 upstream gradient per row.
 *   grad_logits [B, V] of `dtype`; may be exactly `logits` (in place), any
 *               other overlap with an input is LMX_ERR_ALIAS; its address must
 *               equal that of `logits` modulo 16.
 * No workspace.
 */
LMX_API int ce_loss_rows_vjp(const void* logits, const int64_t* target, const float* loss_rows,
                             const float* g, void* grad_logits, int64_t B, int64_t V, int dtype,
                             int64_t ignore_index, void* stream);

/*
 * lmx_scale -- dst[i] = src[i] * (*scale), in fp32 arithmetic, rounded to
 * nearest even into `dtype` (LMX_F32, LMX_BF16 or LMX_F16).
 *
 * The upstream-gradient step of the reduced losses (greyhound functional API
 * page, "cross_entropy", "chunked_linear_cross_entropy" and
 * "chunked_linear_loss": normal autograd behaviour): the entry points above
 * return the gradients for an upstream gradient of 1, and an autograd backward
 * multiplies them by the upstream scalar. Taking the product in fp32 keeps a
 * large fp16 loss scale (2^16 and more) from overflowing and a scale such as
 * 1/3 from being rounded to 16 bits first.
 *
 *   src, dst   n elements of `dtype`, element-aligned (16-byte alignment of
 *              both takes the vector path); dst may be exactly src (in
 *              place); any other overlap is LMX_ERR_ALIAS.
 *   n          >= 0 (0 launches nothing; < 0 is LMX_ERR_SIZE).
 *   scale      one fp32 on the device, 4-byte aligned, not inside dst.
 */
LMX_API int lmx_scale(const void* src, void* dst, int64_t n, int dtype, const float* scale,
                      void* stream);

/* Human-readable name of a status code (static storage). */
LMX_API const char* lmx_status_string(int status);

/*
 * lmx_copy -- plain streaming copy of `bytes` bytes from src to dst on `stream`
 * (device pointers, 16-byte aligned, non-overlapping). A measurement aid: it is
 * the copy kernel of known size against which hardware byte counters and the
 * practical bandwidth ceiling are calibrated. Not part of either operation.
 */
LMX_API int lmx_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * lmx_stream_probe -- streaming patterns of known size: the practical HBM
 * ceilings that the cross-entropy row kernels (one read of the logits, one
 * write of the gradient) are measured against. A measurement aid like
 * lmx_copy, not part of either operation. Non-temporal 16-byte accesses.
 *
 *   LMX_PROBE_READ             read `bytes` of src (dst: a 16 KiB sink, left
 *                              untouched in practice)
 *   LMX_PROBE_WRITE            write `bytes` of dst (src unused, may be NULL)
 *   LMX_PROBE_COPY             copy src -> dst, 256 threads x 4 chunks per step
 *   LMX_PROBE_COPY_BATCHED     copy, 1024 threads x 8 chunks (128 KiB) loaded
 *                              then stored per step, 4 workgroups per CU
 *   LMX_PROBE_ROWS_INTERLEAVED rows of row_bytes, one 1024-thread workgroup
 *                              per row, 16 chunks a thread in registers:
 *                              chunk k of a row stored, then chunk k of the
 *                              workgroup's next row loaded, in turn
 *   LMX_PROBE_ROWS_PHASED      the same rows: a row stored whole, then the next
 *                              row loaded whole
 *
 * src and dst 16-byte aligned; bytes a multiple of 16 (LMX_ERR_SIZE); the row
 * modes need 16 <= row_bytes <= 262144, a multiple of 16 dividing bytes. Copy
 * and row modes may run in place (dst == src); any other overlap is
 * LMX_ERR_ALIAS. An unknown mode is LMX_ERR_ENUM.
 */
enum {
  LMX_PROBE_READ = 0,
  LMX_PROBE_WRITE = 1,
  LMX_PROBE_COPY = 2,
  LMX_PROBE_COPY_BATCHED = 3,
  LMX_PROBE_ROWS_INTERLEAVED = 4,
  LMX_PROBE_ROWS_PHASED = 5
};
LMX_API int lmx_stream_probe(const void* src, void* dst, size_t bytes, size_t row_bytes,
                             int mode, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LMX_H_ */
