// igc_sparse_conv_noalloc: igc_sparse_conv for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid it). The kernels'
// temporaries (transposed or packed weights, the mask-sorted tile plan of the gather-GEMM-scatter
// path, per-leaf dispatch flags) live in one file-scope device array of fixed size instead of a
// workspace; every other step is the one igc_sparse_conv runs, on the same kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "igc_host.h"

namespace igc {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;

// One copy per GPU the library runs on, held until the process ends. Every call on a GPU
// shares it, and every call rewrites what it reads (nothing in it must start at zero).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;  // per device: the array's device address

// The device address of `scratch` on the current device (looked up once per device, with that
// device current; in host code the array's name is not a device address).
int scratch_address(void** out, const char* fn) {
  int dev = 0;
  IGC_HIP(hipGetDevice(&dev), fn);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return IGC_OK;
}

}  // namespace
}  // namespace igc

using namespace igc;

extern "C" int igc_sparse_conv_noalloc(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype,
                                       int32_t cin, const void* d_w, int32_t cout, void* d_out, int32_t path,
                                       igc_stream stream) {
  clear_error();
  const char* fn = "igc_sparse_conv_noalloc";
  int32_t p = path;
  int rc = check_conv_args(fn, g, d_map, d_feats, dtype, cin, d_w, cout, d_out, &p);
  if (rc || g->n_voxels == 0) return rc;
  const uint32_t dense_min = p == IGC_PATH_MIXED ? mixed_dense_rows(cin) : 0u;
  size_t need = 0;
  if (p == IGC_PATH_GATHER) need = gather_scratch_bytes(cin, cout);
  if (p == IGC_PATH_LEAF || p == IGC_PATH_MIXED) need = leaf_scratch_bytes(dtype, cin, cout);
  if (p == IGC_PATH_GGS || p == IGC_PATH_MIXED)
    need = std::max(need, ggs_scratch_bytes(g->n_voxels, cin, cout, dense_min != 0));
  if (need > kScratchBytes)
    return set_error(IGC_ERR_CAPACITY, std::string(fn) + ": this layer needs " + std::to_string(need) +
                                           " bytes of scratch memory; the static scratch holds " +
                                           std::to_string(kScratchBytes) + " (use igc_sparse_conv)");
  void* sp = nullptr;
  if (need > 0 && (rc = scratch_address(&sp, fn))) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (p == IGC_PATH_GATHER)
    return launch_conv_gather(g, d_map, g->n_voxels, g->n_voxels, d_feats, dtype, cin, d_w, cout, d_out, s, sp);
  if (p == IGC_PATH_LEAF) return launch_conv_leaf(g, d_feats, dtype, cin, d_w, cout, d_out, s, 0, sp);
  if (p == IGC_PATH_MIXED) {
    // The two launches run in stream order, so the leaf pass may reuse the scratch after the
    // gather-GEMM-scatter pass has read it.
    rc = launch_conv_ggs(g, d_map, d_feats, dtype, cin, d_w, cout, d_out, s, dense_min, -1, sp);
    if (rc) return rc;
    return launch_conv_leaf(g, d_feats, dtype, cin, d_w, cout, d_out, s, dense_min, sp);
  }
  return launch_conv_ggs(g, d_map, d_feats, dtype, cin, d_w, cout, d_out, s, 0, -1, sp);
}
