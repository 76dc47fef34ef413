// qk_sparse_attn_indexed without a caller workspace, for callers that cannot
// allocate: the attention's key-split partials live in a file-scope device
// array.  Host code never passes the array's name to a kernel (in host code it
// is a stand-in, not a device address); each device's address comes from
// hipGetSymbolAddress on the first call on that device, with it current.
#include <mutex>

#include "../../include/qk.h"
#include "qk_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

}  // namespace

extern "C" qk_status qk_sparse_attn_indexed_noalloc(const qk_shape* s, const void* q,
                                                    const void* k, const void* v,
                                                    const int32_t* idx, int32_t ld_idx,
                                                    const int32_t* sel_len, void* out,
                                                    float* lse, qk_stream_t stream) {
  if (!s) return QK_ERR_NULL;
  const size_t need = qk_workspace_bytes(s, QK_OP_SPARSE_ATTN);
  if (need > QK_NOALLOC_SCRATCH_BYTES) return QK_ERR_SCRATCH_LIMIT;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QK_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QK_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev] {
    g_lookup[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_lookup[dev] != hipSuccess || !g_scratch[dev]) return QK_ERR_HIP;
  // every entry of the partials that the combine reads is written by the
  // attention kernel first, so the array needs no clearing between calls
  return qk_sparse_attn_indexed(s, q, k, v, idx, ld_idx, sel_len, out, lse,
                                need ? g_scratch[dev] : nullptr, need, stream);
}
