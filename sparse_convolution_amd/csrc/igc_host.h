// Host-side internals of libigconv: the grid object, error reporting and allocation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/igconv.h"
#include "igc_internal.h"

struct igc_grid {
  int device = 0;
  hipStream_t stream = nullptr;  // stream the grid was built on (destroy waits for it)
  int64_t n_input = 0, n_voxels = 0, n_leaf = 0, n_lower = 0, n_upper = 0;
  int32_t sort_passes = 0;
  int32_t host_syncs = 0;  // host synchronisations the build took
  uint32_t root_cap = 0;
  size_t bytes = 0;
  void* block = nullptr;  // one device allocation holding every array below
  igc_allocator alloc{};  // the caller's memory provider (alloc.alloc == nullptr: the library's pool)

  uint64_t* root_keys = nullptr;   // [root_cap]
  int32_t* root_vals = nullptr;    // [root_cap]
  uint64_t* root_list = nullptr;   // [U] tile keys in upper-node order
  int4* upper_origin = nullptr;    // [U]
  uint64_t* upper_mask = nullptr;  // [U*512]
  uint16_t* upper_pre = nullptr;   // [U*512]
  uint32_t* upper_first = nullptr; // [U]
  int4* lower_origin = nullptr;    // [Lw]
  uint64_t* lower_mask = nullptr;  // [Lw*64]
  uint16_t* lower_pre = nullptr;   // [Lw*64]
  uint32_t* lower_first = nullptr; // [Lw]
  igc::LeafRec* leaf = nullptr;    // [F]
  int4* leaf_origin = nullptr;     // [F]
  int32_t* leaf_nbr = nullptr;     // [F*27] neighbour leaves (the 3x3x3 block around each leaf)

  igc::GridView view() const {
    igc::GridView v;
    v.root_keys = root_keys;
    v.root_vals = root_vals;
    v.root_mask = root_cap ? root_cap - 1u : 0u;
    v.upper_mask = upper_mask;
    v.upper_pre = upper_pre;
    v.upper_first = upper_first;
    v.lower_mask = lower_mask;
    v.lower_pre = lower_pre;
    v.lower_first = lower_first;
    v.leaf = leaf;
    v.leaf_origin = leaf_origin;
    v.leaf_nbr = leaf_nbr;
    v.n_voxels = n_voxels;
    v.n_leaf = n_leaf;
    return v;
  }
};

namespace igc {

// Records the message for igc_last_error and returns the status.
int set_error(int status, const std::string& msg);
void clear_error();

// Status from a HIP call, with the call site named in the message.
int hip_status(hipError_t e, const char* what);

#define IGC_HIP(call, what)                                   \
  do {                                                        \
    hipError_t e_ = (call);                                   \
    if (e_ != hipSuccess) return ::igc::hip_status(e_, what); \
  } while (0)

// The memory provider of a grid, or nullptr for the library's own pool.
inline const igc_allocator* grid_alloc(const igc_grid* g) { return g && g->alloc.alloc ? &g->alloc : nullptr; }

// Stream-ordered device allocation: through `a` when given, else from the library's private
// per-device memory pool (free blocks kept across calls until igc_release_memory).
int dev_alloc(void** p, size_t bytes, hipStream_t s, const char* what, const igc_allocator* a = nullptr);
void dev_free(void* p, size_t bytes, hipStream_t s, const igc_allocator* a = nullptr);

// Pinned host staging buffer (per host thread) of at least `bytes` for small device -> host
// reads; *device_view (if given) receives the address kernels write it through.
void* host_staging(size_t bytes, void** device_view = nullptr);

// Temporary device workspace of one call. With a caller's allocator it is allocated through it
// and returned at release. Otherwise each device keeps one block that is handed to one call at
// a time and grows to the largest request (a call that finds it taken allocates its own): a
// stream-ordered allocation and free cost tens of microseconds of host time per call, and the
// block makes the common case free of both. On release an event is recorded on the caller's
// stream, and the next user's stream waits for it, so work still reading the block finishes
// first.
struct Workspace {
  void* p = nullptr;
  size_t bytes = 0;
  int dev = -1;
  bool cached = false;
  const igc_allocator* a = nullptr;
};
int ws_acquire(Workspace* w, size_t bytes, hipStream_t s, const char* what, const igc_allocator* a = nullptr);
void ws_release(Workspace* w, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Host-side checks shared by igc_sparse_conv and igc_sparse_conv_noalloc (fn names the call in
// messages); *path is the requested path on entry and the one to run on success.
int check_conv_args(const char* fn, const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype,
                    int32_t cin, const void* d_w, int32_t cout, void* d_out, int32_t* path);
// Active voxels from which a leaf takes the leaf window under per-leaf dispatch.
uint32_t mixed_dense_rows(int32_t cin);

// Launchers (defined in the .hip files).
int build_grid(const int32_t* d_ijk, int64_t n_in, hipStream_t s, igc_grid* g);
// Output grids of a chain of strided / transposed 3x3x3 convolutions (stage k reads stage
// k-1's output), built from leaves with the counts on the device and one host synchronisation.
// strides [n][3]; outs[k] are allocated igc_grid objects (device, stream, allocator set) whose
// topology this fills. derive_supported: whether one stage over `in` fits the derived build
// (at most 4096 root tiles, record indices within the sort key).
bool derive_supported(const igc_grid* in, const int32_t* stride, int32_t transposed);
int derive_chain(const igc_grid* in, int n, const int32_t* strides, const int32_t* transposed, hipStream_t s,
                 igc_grid** outs);
int launch_active_ijk(const igc_grid* g, int32_t* d_out, hipStream_t s);
int launch_ijk_to_index(const igc_grid* g, const int32_t* d_q, int64_t m, int32_t* d_idx, hipStream_t s);
int launch_kernel_map(const igc_grid* g, const int32_t* h_offsets, int32_t K, int32_t* d_map, uint32_t* d_nbmask,
                      hipStream_t s);
bool leaf_conv_supported(int32_t dtype, int32_t cin, int32_t cout);
bool ggs_conv_supported(int32_t dtype, int32_t cin, int32_t cout);
// General-shape path (any channel counts up to kGatherMaxChannels, fp32 or bf16).
constexpr int32_t kGatherMaxChannels = 4096;
bool gather_conv_supported(int32_t dtype, int32_t cin, int32_t cout);
// d_map int32[27, N]; entries outside [0, n_in) read as absent. scratch (may be null): at least
// gather_scratch_bytes() of device memory used instead of a workspace from g's allocator.
int launch_conv_gather(const igc_grid* g, const int32_t* d_map, int64_t N, int64_t n_in, const void* d_feats,
                       int32_t dtype, int32_t cin, const void* d_w, int32_t cout, void* d_out, hipStream_t s,
                       void* scratch = nullptr);
size_t gather_scratch_bytes(int32_t cin, int32_t cout);
int launch_wgrad_gather(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                        const void* d_dout, int32_t cout, float* d_dw, hipStream_t s);
// dw[e] = sum over c < chunks of part[c * E + e] in fp64, in a fixed order (weight gradients).
int launch_wgrad_reduce(const float* part, int64_t chunks, int64_t E, float* dw, hipStream_t s);

// Row order of the gather-GEMM-scatter plan for one layer: rows sorted by neighbour mask within
// spans of `span` rows (256, 1024 or 4096), key bit order 0 = natural, 1 = class (corners,
// edges, faces, centre); from the rules igc_tuning_load read (default: 256, natural).
struct GgsTuning {
  int span = 256;
  int order = 0;
  int bn = 0;  // output channels per workgroup tile (0: the widest the shape allows)
  int kc = 0;  // input channels per chunk: 32 forces 32-channel chunks (0: 64 where cin allows)
  int rows = 0;  // output rows per workgroup: 128 takes half of a 256-row plan tile (0: whole)
};
GgsTuning ggs_tuning(int32_t cin, int32_t cout, int64_t n_voxels, int64_t n_leaf);
// min_count > 0 (bf16 only): leaves with fewer active voxels are skipped (their rows untouched).
// scratch (may be null): caller-provided device memory of at least leaf_scratch_bytes() used
// instead of a workspace (nothing is allocated then).
int launch_conv_leaf(const igc_grid* g, const void* d_feats, int32_t dtype, int32_t cin, const void* d_w, int32_t cout,
                     void* d_out, hipStream_t s, uint32_t min_count = 0, void* scratch = nullptr);
size_t leaf_scratch_bytes(int32_t dtype, int32_t cin, int32_t cout);
// dense_min > 0: rows of leaves with at least dense_min active voxels get no pairs (zero output).
// n_in: rows of d_feats (map entries outside [0, n_in) read as absent); -1 = the grid's N.
// scratch (may be null): caller-provided device memory of at least ggs_scratch_bytes() used
// instead of a workspace (nothing is allocated then).
int launch_conv_ggs(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                    const void* d_w, int32_t cout, void* d_out, hipStream_t s, uint32_t dense_min = 0,
                    int64_t n_in = -1, void* scratch = nullptr);
size_t ggs_scratch_bytes(int64_t N, int32_t cin, int32_t cout, bool with_skip);
// Mask-sorted tiles of 256 output rows (row order perm, 16-row blocks with pairs per offset blk);
// rows with skip[row] != 0 (if skip is given) count as having no neighbours.
int launch_ggs_plan(const int32_t* d_map, int64_t N, int32_t* perm, uint16_t* blk, hipStream_t s,
                    const uint8_t* skip = nullptr);
// Leaf-local fp32 weight gradient: `groups` partial dW blocks [groups][27][cin][cout] in `part`.
bool wgrad_leaf_supported(int32_t cin, int32_t cout);
int64_t wgrad_leaf_groups(const igc_grid* g);
int launch_wgrad_leaf(const igc_grid* g, const void* d_feats, int32_t cin, const void* d_dout, int32_t cout,
                      float* part, int64_t groups, hipStream_t s);
// Output grids of strided / transposed 3x3x3 convolutions and the map between two grids.
int conv_grid_slots(const int32_t* stride, int32_t transposed, int* n);
int build_conv_grid(const igc_grid* in, const int32_t* stride, int32_t transposed, hipStream_t s, igc_grid* out);
int launch_conv_map(const igc_grid* in, const igc_grid* out, const int32_t* stride, int32_t transposed,
                    int32_t* d_map, hipStream_t s);
// Fills n 32-bit words with v on stream s (a kernel, so it can sit in captured work).
int fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
bool wgrad_supported(int32_t dtype, int32_t cin, int32_t cout);
bool wgrad_tuned_supported(int32_t dtype, int32_t cin, int32_t cout);
int launch_conv_backward(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                         const void* d_w, int32_t cout, const void* d_dout, void* d_dfeats, float* d_dw,
                         int32_t dgrad_path, hipStream_t s);

}  // namespace igc
