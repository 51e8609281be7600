// dcpmla_rank_attention_static: the per-rank attention and segment merge with
// their workspace (split-KV partials, the split query) in a device array of
// the library instead of caller memory, for callers that cannot allocate.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

using namespace dcpmla;

constexpr int kMaxDevices = 64;
constexpr int kMaxGroups = 1024;

// The array itself.  In host code `scratch` names a host-side stand-in, not
// device memory: only the per-device address from hipGetSymbolAddress below
// is ever handed to a kernel or a copy.  Every GPU the library runs on holds
// its own copy until the process ends.
__device__ __align__(256) uint8_t scratch[DCPMLA_STATIC_SCRATCH_BYTES];

std::mutex g_mu;
void *g_ptr[kMaxDevices];

// Device address of this device's copy of `scratch`, resolved once per device
// with that device current (the caller's current device).
int scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DCPMLA_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DCPMLA_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DCPMLA_E_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return DCPMLA_OK;
}

}  // namespace

extern "C" {

int dcpmla_rank_attention_static(const dcpmla_geom *g, const void *q, const void *kv_pool,
                                 float kv_scale, float softmax_scale, const dcpmla_meta *m,
                                 void *out_rank, float *lse_rank, hipStream_t stream) {
  const int v = dcpmla_validate(g);
  if (v != DCPMLA_OK) return v;
  if (!q || !kv_pool || !out_rank || !lse_rank || !m || !m->work) return DCPMLA_E_INVALID;
  // the workspace the caller would otherwise pass, for the same persistent grid
  int groups = g->groups;
  if (groups == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DCPMLA_E_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return DCPMLA_E_HIP;
    groups = cus < kMaxGroups ? cus : kMaxGroups;
  }
  const int64_t rows = (int64_t)g->batch * g->qlen * g->num_heads;
  const int64_t need = ws_total_bytes(groups, rows);
  if (need > (int64_t)DCPMLA_STATIC_SCRATCH_BYTES) return DCPMLA_E_SCRATCH;
  void *ws = nullptr;
  const int s = scratch_address(&ws);
  if (s != DCPMLA_OK) return s;
  // nothing in the workspace needs to start at zero: the attention launch writes
  // every partial, LSE and split-query byte that the segment merge then reads
  const int a = dcpmla_partial_attention(g, q, kv_pool, kv_scale, softmax_scale, m, ws, need, out_rank,
                                         lse_rank, stream);
  if (a != DCPMLA_OK) return a;
  return dcpmla_merge_segments(g, m, ws, need, out_rank, lse_rank, stream);
}

int64_t dcpmla_static_scratch_bytes(void) { return (int64_t)DCPMLA_STATIC_SCRATCH_BYTES; }

}  // extern "C"
