// ce_fwd_bwd_noalloc: ce_fwd_bwd with its workspace in a fixed device array
// of the library, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives for the whole process, one copy per GPU the library runs
// on. Its device address is looked up once per device (hipGetSymbolAddress,
// with that device current) and every call on that device then passes that
// address as the workspace of ce_fwd_bwd's kernels. Nothing in it must start
// at zero: the count kernel writes N, the row kernel writes every row's loss
// term, the finish kernel reads only those. Calls that overlap in time on
// one GPU share the array and race.
#include <mutex>

#include "internal.h"

namespace {

// N (one 256-byte slot) and up to kNoallocMaxRows fp32 row-loss terms: the
// workspace layout of ce_fwd_bwd for B = kNoallocMaxRows.
constexpr int64_t kNoallocMaxRows = int64_t{1} << 20;
constexpr size_t kScratchBytes = 256 + static_cast<size_t>(kNoallocMaxRows) * 4;

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (nullptr on error).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int ce_fwd_bwd_noalloc(const void* logits, void* grad_logits, const int64_t* target, int64_t B,
                       int64_t V, int dtype, int64_t ignore_index, int reduction,
                       float z_loss_multiplier, float* loss, int64_t* n_valid,
                       int32_t* bad_target, void* stream) {
  const int st = lmx::ce_args_status(logits, grad_logits, target, B, V, dtype, reduction, loss);
  if (st != LMX_OK) return st;
  if (B > kNoallocMaxRows) return LMX_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return LMX_ERR_HIP;
  return ce_fwd_bwd(logits, grad_logits, target, B, V, dtype, ignore_index, reduction,
                    z_loss_multiplier, loss, n_valid, bad_target, ws, kScratchBytes, stream);
}

}  // extern "C"
