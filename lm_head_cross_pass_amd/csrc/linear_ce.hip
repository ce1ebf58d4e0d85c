// Chunked linear cross-entropy (placeholder until the MFMA path lands).
#include "internal.h"

namespace lmx {

int64_t linear_ce_resolve_chunk(int64_t BT, int64_t V, int64_t chunk_size) {
  if (BT <= 0) return 1;
  if (chunk_size > 0) return chunk_size < BT ? chunk_size : BT;
  return BT;
}

LinearCeWorkspace linear_ce_workspace_layout(int64_t, int64_t, int64_t, int64_t, int) {
  LinearCeWorkspace w{};
  w.total = 256;
  return w;
}

int linear_ce_enqueue(const LinearCeParams&, void*, hipStream_t) { return LMX_ERR_UNSUPPORTED; }

}  // namespace lmx
