// extern "C" entry points of libigconv: host-side validation, error reporting, allocation
// and dispatch to the HIP kernels. Every check runs on the host before any launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "igc_host.h"

namespace igc {

namespace {
thread_local std::string g_last_error;
thread_local void* g_staging = nullptr;
thread_local void* g_staging_dev = nullptr;  // the same pinned buffer as the device addresses it
thread_local size_t g_staging_bytes = 0;

// Per device: the library's private stream-ordered memory pool (free blocks kept across calls:
// repeated builds do not return memory to the driver between calls; the device's default pool
// and other users of it are left as they are) and the cached workspace block (see Workspace).
struct DevMem {
  hipMemPool_t pool = nullptr;
  bool pool_tried = false;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  bool ws_busy = false;
  hipEvent_t ws_released = nullptr;  // recorded on the last user's stream at release
};
std::mutex g_mem_mutex;
std::vector<DevMem> g_mem;

DevMem& dev_mem(int dev) {  // g_mem_mutex held
  if ((int)g_mem.size() <= dev) g_mem.resize(dev + 1);
  return g_mem[dev];
}

// The device's private pool, created on first use (nullptr if the runtime refuses one: the
// device's default pool then serves, unchanged).
hipMemPool_t private_pool(int dev) {  // g_mem_mutex held
  DevMem& m = dev_mem(dev);
  if (!m.pool_tried) {
    m.pool_tried = true;
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
      uint64_t threshold = ~0ull;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
      m.pool = pool;
    } else {
      (void)hipGetLastError();
    }
  }
  return m.pool;
}

int pool_alloc(void** p, size_t bytes, int dev, hipStream_t s) {  // g_mem_mutex held
  hipMemPool_t pool = private_pool(dev);
  const hipError_t e = pool ? hipMallocFromPoolAsync(p, bytes, pool, s) : hipMallocAsync(p, bytes, s);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
  }
  return e;
}
}  // namespace

int set_error(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

void clear_error() { g_last_error.clear(); }

int hip_status(hipError_t e, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return set_error(e == hipErrorOutOfMemory ? IGC_ERR_OOM : IGC_ERR_HIP, m);
}

int dev_alloc(void** p, size_t bytes, hipStream_t s, const char* what, const igc_allocator* a) {
  *p = nullptr;
  if (bytes == 0) bytes = 256;
  if (a) {
    *p = a->alloc(a->ctx, bytes, (igc_stream)s);
    if (!*p)
      return set_error(IGC_ERR_OOM, std::string(what) + ": the caller's allocator returned NULL for " +
                                        std::to_string(bytes) + " bytes");
    return IGC_OK;
  }
  int dev = 0;
  IGC_HIP(hipGetDevice(&dev), what);
  hipError_t e;
  {
    std::lock_guard<std::mutex> lock(g_mem_mutex);
    e = (hipError_t)pool_alloc(p, bytes, dev, s);
  }
  if (e != hipSuccess)
    return set_error(e == hipErrorOutOfMemory ? IGC_ERR_OOM : IGC_ERR_HIP,
                     std::string(what) + ": device allocation of " + std::to_string(bytes) +
                         " bytes failed: " + hipGetErrorString(e));
  return IGC_OK;
}

void dev_free(void* p, size_t bytes, hipStream_t s, const igc_allocator* a) {
  if (!p) return;
  if (a) a->release(a->ctx, p, bytes ? bytes : 256, (igc_stream)s);
  else (void)hipFreeAsync(p, s);
}

int ws_acquire(Workspace* w, size_t bytes, hipStream_t s, const char* what, const igc_allocator* a) {
  *w = Workspace{};
  if (bytes == 0) bytes = 256;
  if (a) {
    w->a = a;
    w->bytes = bytes;
    return dev_alloc(&w->p, bytes, s, what, a);
  }
  int dev = 0;
  IGC_HIP(hipGetDevice(&dev), what);
  {
    std::lock_guard<std::mutex> lock(g_mem_mutex);
    DevMem& m = dev_mem(dev);
    if (!m.ws_busy) {
      if (m.ws_released) IGC_HIP(hipStreamWaitEvent(s, m.ws_released, 0), what);
      if (m.ws_bytes < bytes) {
        if (m.ws) (void)hipFreeAsync(m.ws, s);
        m.ws = nullptr;
        m.ws_bytes = 0;
        const size_t want = std::max(bytes, align_up(bytes + bytes / 4, 1 << 20));
        if (pool_alloc(&m.ws, want, dev, s) == hipSuccess) m.ws_bytes = want;
      }
      if (m.ws) {
        m.ws_busy = true;
        w->p = m.ws;
        w->bytes = m.ws_bytes;
        w->dev = dev;
        w->cached = true;
        return IGC_OK;
      }
    }
  }
  w->dev = dev;
  w->bytes = bytes;
  return dev_alloc(&w->p, bytes, s, what);
}

void ws_release(Workspace* w, hipStream_t s) {
  if (!w->p) return;
  if (!w->cached) {
    dev_free(w->p, w->bytes, s, w->a);
  } else {
    std::lock_guard<std::mutex> lock(g_mem_mutex);
    DevMem& m = dev_mem(w->dev);
    if (!m.ws_released) (void)hipEventCreateWithFlags(&m.ws_released, hipEventDisableTiming);
    if (m.ws_released) (void)hipEventRecord(m.ws_released, s);
    m.ws_busy = false;
  }
  *w = Workspace{};
}

void* host_staging(size_t bytes, void** device_view) {
  if (g_staging_bytes < bytes) {
    if (g_staging) (void)hipHostFree(g_staging);
    g_staging = nullptr;
    g_staging_dev = nullptr;
    g_staging_bytes = 0;
    void* p = nullptr;
    void* d = nullptr;
    if (hipHostMalloc(&p, bytes, hipHostMallocDefault) != hipSuccess) return nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess) {
      (void)hipHostFree(p);
      return nullptr;
    }
    g_staging = p;
    g_staging_dev = d;
    g_staging_bytes = bytes;
  }
  if (device_view) *device_view = g_staging_dev;
  return g_staging;
}

static void free_grid(igc_grid* g) {
  if (!g) return;
  dev_free(g->block, g->bytes, g->stream, grid_alloc(g));  // the root table lives in the same allocation
  delete g;
}

static bool allocator_ok(const igc_allocator* a) { return !a || (a->alloc && a->release); }

static bool leaf_occupancy_ok(const igc_grid* g, int32_t cin) {
  // Leaf path pays for 512 positions per leaf; the fVDB notes put its break-even against a
  // general backend at a leaf occupancy of about 20%. With 64 input channels the window holds
  // one leaf per CU and the gather-GEMM-scatter path wins up to a higher occupancy (measured,
  // bf16 64 -> 64: 9.1 against 12.6 ms at 0.23, 1.33 against 1.25 ms at 0.60).
  const double min_occ = cin >= 64 ? 0.5 : 0.2;
  return g->n_leaf > 0 && (double)g->n_voxels >= min_occ * 512.0 * (double)g->n_leaf;
}

// Active voxels from which a leaf takes the leaf window under per-leaf dispatch (the same
// occupancy bars as the whole-grid choice below; IGC_MIXED_MIN overrides it).
static uint32_t mixed_dense_min(int32_t cin) {
  if (const char* e = std::getenv("IGC_MIXED_MIN")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v <= 512) return (uint32_t)v;
  }
  return cin >= 64 ? 256u : 103u;
}

static int choose_path(const igc_grid* g, int32_t dtype, int32_t cin, int32_t cout, int32_t* path) {
  const bool leaf_ok = leaf_conv_supported(dtype, cin, cout);
  const bool ggs_ok = ggs_conv_supported(dtype, cin, cout);
  if (const char* e = std::getenv("IGC_PATH")) {
    if (!std::strcmp(e, "leaf") && leaf_ok) return *path = IGC_PATH_LEAF, IGC_OK;
    if (!std::strcmp(e, "ggs") && ggs_ok) return *path = IGC_PATH_GGS, IGC_OK;
  }
  if (leaf_ok && (leaf_occupancy_ok(g, cin) || !ggs_ok)) return *path = IGC_PATH_LEAF, IGC_OK;
  if (ggs_ok) return *path = IGC_PATH_GGS, IGC_OK;
  if (gather_conv_supported(dtype, cin, cout)) return *path = IGC_PATH_GATHER, IGC_OK;
  return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv: no path supports dtype " + std::to_string(dtype) +
                                            " with cin " + std::to_string(cin) + " and cout " + std::to_string(cout));
}

uint32_t mixed_dense_rows(int32_t cin) { return mixed_dense_min(cin); }

int check_conv_args(const char* fn, const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype,
                    int32_t cin, const void* d_w, int32_t cout, void* d_out, int32_t* path) {
  const std::string f(fn);
  if (!g) return set_error(IGC_ERR_INVALID_ARG, f + ": grid is null");
  if (dtype != IGC_F32 && dtype != IGC_BF16) return set_error(IGC_ERR_INVALID_ARG, f + ": bad dtype");
  if (cin < 1 || cout < 1) return set_error(IGC_ERR_INVALID_ARG, f + ": cin and cout must be positive");
  const int32_t p0 = *path;
  if (p0 != IGC_PATH_AUTO && p0 != IGC_PATH_LEAF && p0 != IGC_PATH_GGS && p0 != IGC_PATH_MIXED &&
      p0 != IGC_PATH_GATHER)
    return set_error(IGC_ERR_INVALID_ARG, f + ": bad path");
  if (!d_w) return set_error(IGC_ERR_INVALID_ARG, f + ": d_w is null");
  if (g->n_voxels > 0 && (!d_feats || !d_out)) return set_error(IGC_ERR_INVALID_ARG, f + ": d_feats or d_out is null");
  if (d_feats && d_feats == d_out) return set_error(IGC_ERR_INVALID_ARG, f + ": d_out aliases d_feats");
  int32_t p = p0;
  if (p == IGC_PATH_AUTO) {
    const int rc = choose_path(g, dtype, cin, cout, &p);
    if (rc) return rc;
  }
  if (p == IGC_PATH_LEAF && !leaf_conv_supported(dtype, cin, cout))
    return set_error(IGC_ERR_UNSUPPORTED, f + ": leaf path does not support this dtype / cin / cout");
  if (p == IGC_PATH_GGS && !ggs_conv_supported(dtype, cin, cout))
    return set_error(IGC_ERR_UNSUPPORTED, f + ": gather-GEMM-scatter path does not support this dtype / cin / cout");
  if (p == IGC_PATH_MIXED &&
      !(dtype == IGC_BF16 && leaf_conv_supported(dtype, cin, cout) && ggs_conv_supported(dtype, cin, cout)))
    return set_error(IGC_ERR_UNSUPPORTED, f + ": per-leaf dispatch needs a shape both paths support");
  if (p == IGC_PATH_GATHER && !gather_conv_supported(dtype, cin, cout))
    return set_error(IGC_ERR_UNSUPPORTED, f + ": general-shape path takes at most " +
                                              std::to_string(kGatherMaxChannels) + " channels");
  if ((p == IGC_PATH_GGS || p == IGC_PATH_MIXED || p == IGC_PATH_GATHER) && !d_map && g->n_voxels > 0)
    return set_error(IGC_ERR_INVALID_ARG, f + ": the gather-GEMM-scatter and general-shape paths need d_map");
  *path = p;
  return IGC_OK;
}

}  // namespace igc

using namespace igc;

extern "C" {

int igc_grid_build(const int32_t* d_ijk, int64_t n_in, const igc_allocator* alloc, igc_stream stream,
                   igc_grid** out) {
  clear_error();
  if (!out) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_build: out is null");
  *out = nullptr;
  if (n_in < 0) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_build: n_in is negative");
  if (n_in > 0 && !d_ijk) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_build: d_ijk is null");
  if (n_in > INT32_MAX) return set_error(IGC_ERR_RANGE, "igc_grid_build: n_in exceeds 2^31-1");
  if (!allocator_ok(alloc))
    return set_error(IGC_ERR_INVALID_ARG, "igc_grid_build: the allocator needs both alloc and release");
  igc_grid* g = new (std::nothrow) igc_grid();
  if (!g) return set_error(IGC_ERR_OOM, "igc_grid_build: host allocation");
  g->stream = (hipStream_t)stream;
  if (alloc) g->alloc = *alloc;
  if (n_in > 0) {  // an empty grid does no device work
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
      delete g;
      return hip_status(e, "igc_grid_build: hipGetDevice");
    }
    g->device = dev;
  }
  const int rc = build_grid(d_ijk, n_in, (hipStream_t)stream, g);
  if (rc != IGC_OK) {
    free_grid(g);
    return rc;
  }
  *out = g;
  return IGC_OK;
}

int igc_grid_destroy(igc_grid* grid) {
  clear_error();
  if (!grid) return IGC_OK;
  free_grid(grid);  // stream-ordered: the memory is released once the build stream reaches this point
  return IGC_OK;
}

int igc_grid_info(const igc_grid* g, igc_grid_info_t* out) {
  clear_error();
  if (!g || !out) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_info: null argument");
  out->n_input = g->n_input;
  out->n_voxels = g->n_voxels;
  out->n_leaf = g->n_leaf;
  out->n_lower = g->n_lower;
  out->n_upper = g->n_upper;
  out->topology_bytes = (int64_t)g->bytes;
  out->sort_passes = g->sort_passes;
  out->root_capacity = (int32_t)g->root_cap;
  out->host_syncs = g->host_syncs;
  out->reserved = 0;
  return IGC_OK;
}

int igc_release_memory(void) {
  clear_error();
  std::lock_guard<std::mutex> lock(g_mem_mutex);
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  int rc = IGC_OK;
  for (int dev = 0; dev < (int)g_mem.size(); ++dev) {
    DevMem& m = g_mem[dev];
    if (!m.ws && !m.pool) continue;
    if (m.ws_busy) {
      rc = set_error(IGC_ERR_INVALID_ARG, "igc_release_memory: a library call is in flight on device " +
                                              std::to_string(dev));
      continue;
    }
    if (hipSetDevice(dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      rc = hip_status(hipGetLastError(), "igc_release_memory: device synchronize");
      continue;
    }
    if (m.ws) {
      (void)hipFreeAsync(m.ws, nullptr);
      (void)hipStreamSynchronize(nullptr);
      m.ws = nullptr;
      m.ws_bytes = 0;
    }
    if (m.pool) (void)hipMemPoolTrimTo(m.pool, 0);
  }
  if (have_cur) (void)hipSetDevice(cur);
  return rc;
}

int igc_grid_active_ijk(const igc_grid* g, int32_t* d_out, igc_stream stream) {
  clear_error();
  if (!g) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_active_ijk: grid is null");
  if (!d_out && g->n_voxels > 0) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_active_ijk: d_out is null");
  return launch_active_ijk(g, d_out, (hipStream_t)stream);
}

int igc_grid_ijk_to_index(const igc_grid* g, const int32_t* d_q, int64_t m, int32_t* d_idx, igc_stream stream) {
  clear_error();
  if (!g) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_ijk_to_index: grid is null");
  if (m < 0) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_ijk_to_index: m is negative");
  if (m > 0 && (!d_q || !d_idx)) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_ijk_to_index: null buffer");
  return launch_ijk_to_index(g, d_q, m, d_idx, (hipStream_t)stream);
}

int igc_grid_export(const igc_grid* g, const igc_topology_host* out) {
  clear_error();
  if (!g || !out) return set_error(IGC_ERR_INVALID_ARG, "igc_grid_export: null argument");
  hipStream_t s = g->stream;
  IGC_HIP(hipStreamSynchronize(s), "igc_grid_export: stream synchronize");
  const int64_t U = g->n_upper, L = g->n_lower, F = g->n_leaf;
  auto copy = [&](void* dst, const void* src, size_t bytes, const char* what) -> int {
    if (!dst || bytes == 0) return IGC_OK;
    IGC_HIP(hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost), what);
    return IGC_OK;
  };
  auto origins = [&](int32_t* dst, const int4* src, int64_t n, const char* what) -> int {
    if (!dst || n == 0) return IGC_OK;
    std::vector<int4> tmp((size_t)n);
    IGC_HIP(hipMemcpy(tmp.data(), src, (size_t)n * sizeof(int4), hipMemcpyDeviceToHost), what);
    for (int64_t r = 0; r < n; ++r) {
      dst[3 * r] = tmp[r].x;
      dst[3 * r + 1] = tmp[r].y;
      dst[3 * r + 2] = tmp[r].z;
    }
    return IGC_OK;
  };
  int rc;
  if ((rc = copy(out->root_key, g->root_list, U * 8, "igc_grid_export: root keys"))) return rc;
  if ((rc = origins(out->upper_origin, g->upper_origin, U, "igc_grid_export: upper origins"))) return rc;
  if ((rc = copy(out->upper_mask, g->upper_mask, U * 512 * 8, "igc_grid_export: upper masks"))) return rc;
  if ((rc = copy(out->upper_first, g->upper_first, U * 4, "igc_grid_export: upper links"))) return rc;
  if ((rc = origins(out->lower_origin, g->lower_origin, L, "igc_grid_export: lower origins"))) return rc;
  if ((rc = copy(out->lower_mask, g->lower_mask, L * 64 * 8, "igc_grid_export: lower masks"))) return rc;
  if ((rc = copy(out->lower_first, g->lower_first, L * 4, "igc_grid_export: lower links"))) return rc;
  if ((rc = origins(out->leaf_origin, g->leaf_origin, F, "igc_grid_export: leaf origins"))) return rc;
  if (F > 0 && (out->leaf_mask || out->leaf_offset || out->leaf_prefix)) {
    std::vector<LeafRec> tmp((size_t)F);
    IGC_HIP(hipMemcpy(tmp.data(), g->leaf, (size_t)F * sizeof(LeafRec), hipMemcpyDeviceToHost),
            "igc_grid_export: leaves");
    for (int64_t f = 0; f < F; ++f) {
      if (out->leaf_mask) std::memcpy(out->leaf_mask + 8 * f, tmp[f].mask, 64);
      if (out->leaf_offset) out->leaf_offset[f] = tmp[f].offset;
      if (out->leaf_prefix) out->leaf_prefix[f] = tmp[f].prefix;
    }
  }
  return IGC_OK;
}

int igc_kernel_map(const igc_grid* g, const int32_t* h_offsets, int32_t K, int32_t* d_map, uint32_t* d_nbmask,
                   igc_stream stream) {
  clear_error();
  if (!g) return set_error(IGC_ERR_INVALID_ARG, "igc_kernel_map: grid is null");
  if (!h_offsets) return set_error(IGC_ERR_INVALID_ARG, "igc_kernel_map: h_offsets is null");
  if (K < 1 || K > 256) return set_error(IGC_ERR_INVALID_ARG, "igc_kernel_map: K must be in [1, 256]");
  for (int32_t a = 0; a < 3 * K; ++a)
    if (h_offsets[a] < -8 || h_offsets[a] > 8)
      return set_error(IGC_ERR_INVALID_ARG, "igc_kernel_map: offset component outside [-8, 8]");
  if (d_nbmask && K > 32) return set_error(IGC_ERR_INVALID_ARG, "igc_kernel_map: d_nbmask needs K <= 32");
  if (!d_map && g->n_voxels > 0) return set_error(IGC_ERR_INVALID_ARG, "igc_kernel_map: d_map is null");
  return launch_kernel_map(g, h_offsets, K, d_map, d_nbmask, (hipStream_t)stream);
}

int igc_select_path(const igc_grid* g, int32_t dtype, int32_t cin, int32_t cout, int32_t* path) {
  clear_error();
  if (!g || !path) return set_error(IGC_ERR_INVALID_ARG, "igc_select_path: null argument");
  if (dtype != IGC_F32 && dtype != IGC_BF16) return set_error(IGC_ERR_INVALID_ARG, "igc_select_path: bad dtype");
  return choose_path(g, dtype, cin, cout, path);
}

int igc_sparse_conv(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                    const void* d_w, int32_t cout, void* d_out, int32_t path, igc_stream stream) {
  clear_error();
  int32_t p = path;
  int rc = check_conv_args("igc_sparse_conv", g, d_map, d_feats, dtype, cin, d_w, cout, d_out, &p);
  if (rc || g->n_voxels == 0) return rc;
  if (p == IGC_PATH_LEAF) return launch_conv_leaf(g, d_feats, dtype, cin, d_w, cout, d_out, (hipStream_t)stream);
  if (p == IGC_PATH_GATHER)
    return launch_conv_gather(g, d_map, g->n_voxels, g->n_voxels, d_feats, dtype, cin, d_w, cout, d_out,
                              (hipStream_t)stream);
  if (p == IGC_PATH_MIXED) {
    // Per-leaf dispatch: leaves with at least dense_min active voxels on the leaf window, the
    // rest on gather-GEMM-scatter (which writes zeros into the dense leaves' rows first).
    const uint32_t dense_min = mixed_dense_min(cin);
    rc = launch_conv_ggs(g, d_map, d_feats, dtype, cin, d_w, cout, d_out, (hipStream_t)stream, dense_min);
    if (rc) return rc;
    return launch_conv_leaf(g, d_feats, dtype, cin, d_w, cout, d_out, (hipStream_t)stream, dense_min);
  }
  return launch_conv_ggs(g, d_map, d_feats, dtype, cin, d_w, cout, d_out, (hipStream_t)stream);
}

int igc_sparse_conv_backward(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype,
                             int32_t cin, const void* d_w, int32_t cout, const void* d_dout, void* d_dfeats,
                             float* d_dw, int32_t path, igc_stream stream) {
  clear_error();
  if (!g) return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_backward: grid is null");
  if (dtype != IGC_F32 && dtype != IGC_BF16)
    return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_backward: bad dtype");
  if (cin < 1 || cout < 1)
    return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_backward: cin and cout must be positive");
  if (path != IGC_PATH_AUTO && path != IGC_PATH_LEAF && path != IGC_PATH_GGS && path != IGC_PATH_GATHER)
    return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_backward: bad path");
  if (!d_w) return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_backward: d_w is null");
  if (g->n_voxels > 0 && (!d_map || !d_dout || (d_dw && !d_feats)))
    return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_backward: d_map, d_dout or d_feats is null");
  if (d_dfeats && (d_dfeats == d_dout || d_dfeats == d_feats))
    return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_backward: d_dfeats aliases an input");
  int32_t p = path;
  if (d_dfeats) {
    if (p == IGC_PATH_AUTO) {
      const int rc = choose_path(g, dtype, cout, cin, &p);
      if (rc) return rc;
    }
    if (p == IGC_PATH_LEAF && !leaf_conv_supported(dtype, cout, cin))
      return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv_backward: leaf path does not support the input-gradient shape");
    if (p == IGC_PATH_GGS && !ggs_conv_supported(dtype, cout, cin))
      return set_error(IGC_ERR_UNSUPPORTED,
                       "igc_sparse_conv_backward: gather-GEMM-scatter path does not support the input-gradient shape");
    if (p == IGC_PATH_GATHER && !gather_conv_supported(dtype, cout, cin))
      return set_error(IGC_ERR_UNSUPPORTED,
                       "igc_sparse_conv_backward: general-shape path does not support the input-gradient shape");
  }
  if (d_dw && !wgrad_supported(dtype, cin, cout))
    return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv_backward: weight gradient does not support this dtype / cin / cout");
  if (g->n_voxels == 0) {
    if (d_dw) return fill_u32((uint32_t*)d_dw, (int64_t)27 * cin * cout, 0u, (hipStream_t)stream);
    return IGC_OK;
  }
  return launch_conv_backward(g, d_map, d_feats, dtype, cin, d_w, cout, d_dout, d_dfeats, d_dw, p, (hipStream_t)stream);
}

int igc_conv_grid(const igc_grid* in, const int32_t* h_stride, int32_t transposed, const igc_allocator* alloc,
                  igc_stream stream, igc_grid** out) {
  clear_error();
  if (!out) return set_error(IGC_ERR_INVALID_ARG, "igc_conv_grid: out is null");
  *out = nullptr;
  if (!in || !h_stride) return set_error(IGC_ERR_INVALID_ARG, "igc_conv_grid: in or h_stride is null");
  if (!allocator_ok(alloc))
    return set_error(IGC_ERR_INVALID_ARG, "igc_conv_grid: the allocator needs both alloc and release");
  int n[3];
  if (!conv_grid_slots(h_stride, transposed, n))
    return set_error(IGC_ERR_UNSUPPORTED, "igc_conv_grid: strides must be 1, 2 or 3");
  igc_grid* g = new (std::nothrow) igc_grid();
  if (!g) return set_error(IGC_ERR_OOM, "igc_conv_grid: host allocation");
  g->stream = (hipStream_t)stream;
  g->device = in->device;
  if (alloc) g->alloc = *alloc;
  const int32_t tr = transposed ? 1 : 0;
  // Built from the input's leaves with the counts on the device (one read-back) where the
  // derived build covers the input; otherwise as the coordinate build of candidate outputs.
  const int rc = in->n_voxels > 0 && derive_supported(in, h_stride, tr)
                     ? derive_chain(in, 1, h_stride, &tr, (hipStream_t)stream, &g)
                     : build_conv_grid(in, h_stride, transposed, (hipStream_t)stream, g);
  if (rc != IGC_OK) {
    free_grid(g);
    return rc;
  }
  *out = g;
  return IGC_OK;
}

int igc_conv_grid_chain(const igc_grid* in, int32_t n_stages, const int32_t* h_strides, const int32_t* h_transposed,
                        const igc_allocator* alloc, igc_stream stream, igc_grid** out) {
  clear_error();
  if (!out) return set_error(IGC_ERR_INVALID_ARG, "igc_conv_grid_chain: out is null");
  if (n_stages < 1 || n_stages > IGC_MAX_CHAIN)
    return set_error(IGC_ERR_INVALID_ARG, "igc_conv_grid_chain: n_stages must be 1 .. 16");
  for (int k = 0; k < n_stages; ++k) out[k] = nullptr;
  if (!in || !h_strides) return set_error(IGC_ERR_INVALID_ARG, "igc_conv_grid_chain: in or h_strides is null");
  if (!allocator_ok(alloc))
    return set_error(IGC_ERR_INVALID_ARG, "igc_conv_grid_chain: the allocator needs both alloc and release");
  int32_t tr[IGC_MAX_CHAIN];
  for (int k = 0; k < n_stages; ++k) {
    int n[3];
    tr[k] = h_transposed && h_transposed[k] ? 1 : 0;
    if (!conv_grid_slots(h_strides + 3 * k, tr[k], n))
      return set_error(IGC_ERR_UNSUPPORTED, "igc_conv_grid_chain: strides must be 1, 2 or 3");
  }
  igc_grid* g[IGC_MAX_CHAIN] = {};
  for (int k = 0; k < n_stages; ++k) {
    g[k] = new (std::nothrow) igc_grid();
    if (!g[k]) {
      for (int q = 0; q < k; ++q) free_grid(g[q]);
      return set_error(IGC_ERR_OOM, "igc_conv_grid_chain: host allocation");
    }
    g[k]->stream = (hipStream_t)stream;
    g[k]->device = in->device;
    if (alloc) g[k]->alloc = *alloc;
  }
  const int rc = derive_chain(in, n_stages, h_strides, tr, (hipStream_t)stream, g);
  if (rc != IGC_OK) {
    for (int k = 0; k < n_stages; ++k) free_grid(g[k]);
    return rc;
  }
  for (int k = 0; k < n_stages; ++k) out[k] = g[k];
  return IGC_OK;
}

int igc_conv_map(const igc_grid* in, const igc_grid* out, const int32_t* h_stride, int32_t transposed,
                 int32_t* d_map, igc_stream stream) {
  clear_error();
  if (!in || !out || !h_stride) return set_error(IGC_ERR_INVALID_ARG, "igc_conv_map: null argument");
  int n[3];
  if (!conv_grid_slots(h_stride, transposed, n))
    return set_error(IGC_ERR_UNSUPPORTED, "igc_conv_map: strides must be 1, 2 or 3");
  if (out->n_voxels > 0 && !d_map) return set_error(IGC_ERR_INVALID_ARG, "igc_conv_map: d_map is null");
  return launch_conv_map(in, out, h_stride, transposed, d_map, (hipStream_t)stream);
}

int igc_sparse_conv_between(const igc_grid* out, const int32_t* d_map, int64_t n_in, const void* d_feats,
                            int32_t dtype, int32_t cin, const void* d_w, int32_t cout, void* d_out,
                            igc_stream stream) {
  clear_error();
  if (!out) return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_between: grid is null");
  if (dtype != IGC_F32 && dtype != IGC_BF16) return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_between: bad dtype");
  if (cin < 1 || cout < 1 || n_in < 0)
    return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_between: cin, cout must be positive and n_in >= 0");
  if (!d_w) return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_between: d_w is null");
  const bool ggs = ggs_conv_supported(dtype, cin, cout);
  if (!ggs && !gather_conv_supported(dtype, cin, cout))
    return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv_between: no path supports this dtype / cin / cout");
  if (out->n_voxels > 0 && (!d_map || !d_out || (n_in > 0 && !d_feats)))
    return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_between: d_map, d_feats or d_out is null");
  if (d_feats && d_feats == d_out) return set_error(IGC_ERR_INVALID_ARG, "igc_sparse_conv_between: d_out aliases d_feats");
  if (out->n_voxels == 0) return IGC_OK;
  if (!ggs)
    return launch_conv_gather(out, d_map, out->n_voxels, n_in, d_feats, dtype, cin, d_w, cout, d_out, (hipStream_t)stream);
  return launch_conv_ggs(out, d_map, d_feats, dtype, cin, d_w, cout, d_out, (hipStream_t)stream, 0, n_in);
}

const char* igc_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
