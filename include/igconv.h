/*
 * igconv.h - C ABI of libigconv: a VDB-style IndexGrid built on the GPU from voxel
 * coordinates, its neighbour (kernel) map, and the 3x3x3 submanifold sparse convolution
 * over it, for AMD Instinct MI355X (gfx950).
 *
 * Sources of what each call computes:
 *  - "fVDB: A Deep-Learning Framework for Sparse, Large Scale, and High Performance Spatial
 *    Intelligence", reading notes (woaixuexisr.github.io), sections "core method"
 *    (VDB tree: hashed root, dense child nodes of fanout 32/16/8 per axis), "IndexGrid:
 *    separating topology from values" (the tree returns an index into an external linear
 *    "sidecar" array; only active voxels are indexed; bitmask prefix sums + popcount),
 *    "GPU-accelerated IndexGrid build" (64-bit root keys, radix sort, run-length encoding,
 *    per-tile keys, local radix sort, node counts, top-down registration), and
 *    "accelerated operators for sparse convolution" (leaf-local densification of 8^3 leaves
 *    plus a one-voxel halo; gather-GEMM-scatter over tiles of consecutive outputs for very
 *    sparse inputs with high channel counts; automatic backend choice).
 *  - DriveRT (lucabrembilla.dev/projects/drivert): "Shared neighbour maps" (a map is
 *    defined by coordinate domain, kernel geometry and row order), "Compilation and
 *    deployment" (runtime behind a C ABI; dynamic sizes: buffers start from an estimate
 *    and the invocation repeats with a larger buffer, never a truncated result), "Inspection
 *    and debugging" (errors name the operation; precision is never changed implicitly).
 *
 * Conventions for every call:
 *  - Pointers prefixed d_ are device memory (hipMalloc / torch CUDA tensors) on the current
 *    device; h_ pointers are host memory. The caller owns every buffer it passes in.
 *  - `stream` is a hipStream_t (NULL = the null stream). All device work is enqueued on it;
 *    calls return when the work is enqueued, except where a host synchronisation is stated.
 *  - Layouts are row-major and densely packed. Coordinates are int32 triples (i, j, k).
 *  - Every call returns IGC_OK (0) or an igc_status code; igc_last_error() then returns a
 *    message naming the call and the argument or step that failed (per host thread).
 *    Arguments are validated on the host before anything is launched. On error no grid is
 *    created and output buffers hold unspecified values.
 *  - Linear index: the row of an active voxel in every feature array over the grid; rows are
 *    0-based, -1 means "not an active voxel". The row order is the depth-first tree order:
 *    root tiles by their packed 64-bit key (i field most significant, each field the 32-bit
 *    pattern shifted right logically by 12), then children x-major inside each node (upper
 *    32^3, lower 16^3, leaf 8^3).
 */
#ifndef IGCONV_H
#define IGCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct igc_grid igc_grid; /* opaque, immutable once built */
typedef void* igc_stream;         /* hipStream_t */

typedef enum {
  IGC_OK = 0,
  IGC_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum value, bad offset list */
  IGC_ERR_UNSUPPORTED = 2, /* dtype / channel count / path combination not implemented */
  IGC_ERR_OOM = 3,         /* device or pinned host allocation failed */
  IGC_ERR_HIP = 4,         /* a HIP runtime call failed; the message holds hipGetErrorString */
  IGC_ERR_RANGE = 5,       /* a size beyond the int32 row range (more than 2^31-1 rows) */
  IGC_ERR_CAPACITY = 6,    /* an internal capacity retry was exhausted */
  IGC_ERR_INTERNAL = 7     /* a device-side consistency check failed */
} igc_status;

typedef enum { IGC_F32 = 0, IGC_BF16 = 1 } igc_dtype;

typedef enum {
  IGC_PATH_AUTO = 0, /* choose from measured leaf occupancy, neighbour count and channels */
  IGC_PATH_LEAF = 1, /* leaf-local dense convolution over an LDS window of 10^3 voxels */
  IGC_PATH_GGS = 2,  /* gather-GEMM-scatter over tiles of consecutive output rows */
  IGC_PATH_MIXED = 3, /* per-leaf dispatch: dense leaves on LEAF, the other rows on GGS */
  IGC_PATH_GATHER = 4 /* general shapes: one wave per output row, fp32 accumulation */
} igc_path;

/* Device memory provider. When a grid is created with an allocator (igc_grid_build,
 * igc_conv_grid), every device allocation the library makes for that grid goes through it: the
 * grid's own topology block (returned by igc_grid_destroy) and the temporaries of every later
 * call on the grid (returned at the end of that call). Both are stream-ordered, like
 * hipMallocAsync / hipFreeAsync and a PyTorch caching allocator: `alloc` returns memory usable
 * by work enqueued on `stream` from now on (NULL on failure, which the calling function reports
 * as IGC_ERR_OOM naming itself), and `release` hands back a block whose last use has been
 * enqueued on `stream` (the provider may reuse it for work enqueued later on that stream).
 * Blocks must be at least 256-byte aligned. The struct is copied; `ctx` must stay valid until
 * the grid is destroyed. A NULL allocator selects the library's own per-device memory pool. */
typedef struct igc_allocator {
  void* (*alloc)(void* ctx, size_t bytes, igc_stream stream);
  void (*release)(void* ctx, void* ptr, size_t bytes, igc_stream stream);
  void* ctx;
} igc_allocator;

typedef struct {
  int64_t n_input;        /* coordinates passed to igc_grid_build (duplicates included) */
  int64_t n_voxels;       /* N: distinct active voxels = rows of every feature array */
  int64_t n_leaf;         /* F: 8^3 leaf nodes */
  int64_t n_lower;        /* Lw: 128^3 lower internal nodes */
  int64_t n_upper;        /* U: 4096^3 upper internal nodes = root tiles */
  int64_t topology_bytes; /* device bytes held by the grid */
  int32_t sort_passes;    /* digit passes the build's radix sort ran */
  int32_t root_capacity;  /* slots of the root hash table */
  int32_t host_syncs;     /* host synchronisations the build took (1 unless a capacity was repeated) */
  int32_t reserved;
} igc_grid_info_t;

/* Host buffers for igc_grid_export, sized from igc_grid_info_t (U, Lw, F). A null pointer
 * skips that array. Layouts:
 *   root_key     uint64[U]      packed tile key of each upper node, ascending
 *   upper_origin int32[U,3]     coordinate of the node's first voxel (low 12 bits clear)
 *   upper_mask   uint64[U,512]  child mask, bit c = (x*32+y)*32+z in word c/64
 *   upper_first  uint32[U]      row of the node's first lower node
 *   lower_origin int32[Lw,3]    (low 7 bits clear)
 *   lower_mask   uint64[Lw,64]  child mask, bit c = (x*16+y)*16+z
 *   lower_first  uint32[Lw]     row of the node's first leaf
 *   leaf_origin  int32[F,3]     (low 3 bits clear)
 *   leaf_mask    uint64[F,8]    active mask, word = x, bit = y*8+z
 *   leaf_offset  uint64[F]      linear index of the leaf's first active voxel
 *   leaf_prefix  uint64[F]      for w = 1..7, active voxels in words 0..w-1, 9 bits each at
 *                               bit 9*(w-1)
 * The per-leaf index record (8 mask words, offset, prefix) is 80 bytes, as in the fVDB
 * notes' "IndexGrid" section. */
typedef struct {
  uint64_t* root_key;
  int32_t* upper_origin;
  uint64_t* upper_mask;
  uint32_t* upper_first;
  int32_t* lower_origin;
  uint64_t* lower_mask;
  uint32_t* lower_first;
  int32_t* leaf_origin;
  uint64_t* leaf_mask;
  uint64_t* leaf_offset;
  uint64_t* leaf_prefix;
} igc_topology_host;

/* Builds an IndexGrid from d_ijk int32[n_in,3] (device; any order; duplicates allowed;
 * n_in == 0 gives an empty grid) - fVDB notes, "GPU-accelerated IndexGrid build": root
 * tile keys, radix sort of per-tile 64-bit keys, run-length encoding, upper / lower / leaf
 * counts, allocation, top-down registration of nodes and leaf bit masks.
 * Memory: `alloc` (may be NULL, see igc_allocator) provides the grid's block and the build's
 * temporaries. Host synchronisations (DriveRT, "Counts kept on the GPU"): one, at the end
 * (the counts N, F, Lw, U come back together) for scenes of at most 4096 root tiles. The sort
 * is planned on the device and the node arrays are sized from the previous build's rows per
 * coordinate. If an estimate was too small, the build runs once more with the exact counts (two).
 * A scene with more root tiles falls back to read-backs after the tile pass and after the counts
 * (four), and grows its root hash table if it overflows (DriveRT, "Compilation and deployment":
 * dynamic sizes, never truncated). None for n_in == 0 (no device work is done then);
 * igc_grid_info reports the count. Errors: IGC_ERR_INVALID_ARG (out null, d_ijk null with n_in > 0, n_in < 0, an
 * allocator without both functions), IGC_ERR_RANGE (n_in > 2^31-1), IGC_ERR_OOM (including an
 * allocator returning NULL), IGC_ERR_HIP, IGC_ERR_CAPACITY, IGC_ERR_INTERNAL; every block taken
 * so far is returned on error. On success *out owns one device allocation until
 * igc_grid_destroy. Without an allocator the temporaries come from a workspace block that the
 * library keeps per device and reuses across calls (grown to the largest request, returned by
 * igc_release_memory; a call that finds it in use allocates its own). d_ijk may be freed once
 * the stream reaches the end of the call. */
int igc_grid_build(const int32_t* d_ijk, int64_t n_in, const igc_allocator* alloc, igc_stream stream,
                   igc_grid** out);

/* Frees the grid's device memory in order on the stream the grid was built on (no host
 * synchronisation): work already queued on that stream finishes reading the grid first. Work
 * that reads the grid on other streams must be complete, or ordered before that stream's
 * current point, when this is called. NULL is accepted. */
int igc_grid_destroy(igc_grid* grid);

/* Counts and sizes of the grid (host only, no device work). */
int igc_grid_info(const igc_grid* grid, igc_grid_info_t* out);

/* Returns the library's cached device memory (the per-device workspace blocks and the free
 * blocks of its memory pools) to the driver. Synchronises every device it holds memory on; no
 * other library call may be in flight. Memory of grids built with an allocator is not held by
 * the library and is not affected. */
int igc_release_memory(void);

/* d_out int32[N,3] (device): the active voxels in linear-index order. This is the row order
 * every feature array over the grid uses. */
int igc_grid_active_ijk(const igc_grid* grid, int32_t* d_out, igc_stream stream);

/* d_idx[r] = linear index of d_q[r] (int32[m,3], device), -1 if inactive - fVDB notes,
 * "IndexGrid": root hash, fixed-fanout descent, mask test and popcount of the masked word
 * plus the leaf's prefix count. */
int igc_grid_ijk_to_index(const igc_grid* grid, const int32_t* d_q, int64_t m, int32_t* d_idx,
                          igc_stream stream);

/* Synchronous copy of the topology into caller-owned host buffers (see igc_topology_host). */
int igc_grid_export(const igc_grid* grid, const igc_topology_host* out);

/* Neighbour map (DriveRT, "Shared neighbour maps"): d_map int32[K,N] (device, caller-owned),
 * d_map[o*N + r] = linear index of active voxel r shifted by h_offsets[o] (host int32[K,3]),
 * or -1. Neighbours outside the int32 coordinate range are absent. d_nbmask (uint32[N],
 * device, may be NULL) gets bit o set when d_map[o*N+r] >= 0; it requires K <= 32.
 * Limits: 1 <= K <= 256 and |offset component| <= 8 (IGC_ERR_INVALID_ARG otherwise).
 * The 3x3x3 convolution uses K = 27 in the order o = (di+1)*9 + (dj+1)*3 + (dk+1). */
int igc_kernel_map(const igc_grid* grid, const int32_t* h_offsets, int32_t K, int32_t* d_map,
                   uint32_t* d_nbmask, igc_stream stream);

/* Submanifold 3x3x3 convolution (fVDB notes, "accelerated operators for sparse
 * convolution"): for every active voxel r,
 *     d_out[r, co] = sum_{o, ci : map[o, r] >= 0} d_feats[map[o, r], ci] * d_w[o, ci, co]
 * with the 27 offsets ordered as in igc_kernel_map. d_feats [N,cin], d_w [27,cin,cout] and
 * d_out [N,cout] all have type `dtype`; accumulation is fp32; bf16 outputs are rounded to
 * nearest even. Precision is never changed implicitly: an fp32 call computes in fp32.
 * d_map (int32[27,N] from igc_kernel_map with the standard 27 offsets) is required by
 * IGC_PATH_GGS and ignored by IGC_PATH_LEAF; with IGC_PATH_AUTO it is required whenever the
 * choice (see igc_select_path) is GGS. Supported combinations:
 *     LEAF: dtype F32, (cin, cout) in {(4,8), (4,16), (4,32), (8,8), (8,16), (8,32),
 *           (16,16), (8,4), (16,4), (16,8)};
 *           dtype BF16 (the leaf window of the pages' brick backend: a dense bf16 10^3 halo
 *           per leaf), cin in {16, 32, 64}, cout in {16, 32, 64}
 *     GGS : dtype BF16, cin a multiple of 32 up to 1024, cout a multiple of 64 up to 1024
 *     MIXED (per-leaf dispatch, fVDB notes, "accelerated operators for sparse convolution",
 *           which name picking a kernel per leaf by its local sparsity as future work): dtype
 *           BF16 with a shape both LEAF and GGS support; leaves with at least 256 (cin >= 64)
 *           or 103 active voxels run on the leaf window, all other rows on GGS (d_map
 *           required). Never chosen by IGC_PATH_AUTO: measured slower than both single paths on
 *           the workloads tried (the GGS pass costs nearly as much with the dense leaves' rows
 *           removed).
 *     GATHER (general shapes): dtype F32 or BF16, any cin and cout from 1 to 4096 (d_map
 *           required; map entries outside [0, N) read as absent). One wave per output row with
 *           fp32 accumulation in offset-then-channel order, no matrix cores: IGC_PATH_AUTO takes it
 *           only for shapes neither LEAF nor GGS supports (for example a bf16 first layer with 3 or
 *           4 input channels, bf16 128 -> 32, or fp32 32 -> 32).
 * Anything else returns IGC_ERR_UNSUPPORTED. d_out must not alias d_feats. */
int igc_sparse_conv(const igc_grid* grid, const int32_t* d_map, const void* d_feats, int32_t dtype,
                    int32_t cin, const void* d_w, int32_t cout, void* d_out, int32_t path,
                    igc_stream stream);

/* Loads the per-layer configuration of the gather-GEMM-scatter row order from a text file
 * (DriveRT, "Kernels selected per GPU": tile sizes, bit orders and offset groups are
 * configuration values measured per layer on the target GPU; "Measurement and
 * reproducibility": the selection is stored in a documented file). The plan sorts the output
 * rows by their 27-bit neighbour mask within spans of consecutive rows and cuts them into tiles
 * of 256; each tile computes only its group of offsets (those some of its rows have), so wider
 * spans give smaller offset groups and gather from a wider stretch of rows. One rule per line
 * ('#' starts a comment, first match wins):
 *     ggs <cin|*> <cout|*> <occupancy_lo> <occupancy_hi> <span> <natural|class> [tile]
 * matches a layer by channels and the grid's leaf occupancy N / (512 F) in [lo, hi); span is
 * 256, 1024 or 4096 rows; the key's bit order is natural (offset o at bit o) or class (corner,
 * then edge, face and centre offsets most significant); tile is the output channels per
 * workgroup (auto = the widest the layer allows, or 256, 128, 64; 128k32 and 64k32 take that
 * width with 32-channel chunks, whose smaller LDS stages let two workgroups share a CU; a
 * trailing h on a 128- or 64-channel tile, e.g. 128h or 64k32h, gives each workgroup half of a
 * 256-row tile with only the offsets its own rows have; a width the layer cannot use is
 * ignored). A layer no rule matches sorts within its 256-row tiles in natural order with
 * automatic tiles. The table is process-wide, replaced whole by each load
 * (path NULL clears it), and read by later igc_sparse_conv / _noalloc / _between calls on the
 * gather-GEMM-scatter path. Neither changes an output value: the row order changes which
 * offsets a tile visits (rows only gain exact zero products), and every tile shape accumulates
 * the same 32-channel MFMA steps in the same (offset, channel) order, so the fp32 summation
 * order depends only on cin. Errors: IGC_ERR_INVALID_ARG for an unreadable
 * file or a malformed line (the table is then unchanged). */
int igc_tuning_load(const char* path);

/* igc_sparse_conv for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. Same arguments, paths, results and errors
 * as igc_sparse_conv, on the same kernels, but it calls no allocator (not hipMalloc, not the
 * grid's igc_allocator): the temporaries (transposed weights, the gather-GEMM-scatter tile plan,
 * per-leaf dispatch flags) live in a static device array of 64 MiB that the library holds on each
 * GPU it runs on until the process ends. A layer that needs more (about 27*cin*cout*2 bytes plus
 * 4.5 bytes per output row on the gather-GEMM-scatter path; the fp32 leaf path needs none)
 * returns IGC_ERR_CAPACITY before any launch. Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (different streams or host threads without ordering between them)
 * race and give undefined results. */
int igc_sparse_conv_noalloc(const igc_grid* grid, const int32_t* d_map, const void* d_feats, int32_t dtype,
                            int32_t cin, const void* d_w, int32_t cout, void* d_out, int32_t path, igc_stream stream);

/* Backward pass of igc_sparse_conv (the same operator differentiated; fVDB notes, "accelerated
 * operators for sparse convolution", which list training support for these backends as future
 * work). Given d_dout = dL/dY [N, cout] (type `dtype`):
 *     d_dfeats[s, ci] = sum over (o, r) with map[o, r] = s of sum_co d_dout[r, co] * W[o, ci, co]
 *                       ([N, cin], type `dtype`; NULL skips it)
 *     d_dw[o, ci, co] = sum over r with map[o, r] >= 0 of feats[map[o, r], ci] * d_dout[r, co]
 *                       ([27, cin, cout] float32, summed in fp32 per chunk of rows and over the
 *                       chunks in fp64, in a fixed order; NULL skips it)
 * d_map (int32[27, N], standard offsets) is required. The input gradient is the forward
 * convolution of d_dout with W~[o] = W[26 - o]^T (the map is symmetric under offset negation),
 * so it runs on the path igc_select_path picks for (dtype, cout, cin) unless `path` forces one;
 * that shape must be supported (see igc_sparse_conv; the fp32 leaf path also takes 8 -> 4,
 * 16 -> 4, 16 -> 8; IGC_PATH_GATHER takes any shape up to 4096 channels). The weight gradient
 * runs on matrix-core kernels for BF16 with cin a multiple of 32 and cout a multiple of 64 (up
 * to 1024), on the leaf window for the small F32 shapes the leaf path covers, and on a
 * general-shape kernel (tiles of up to 64 x 64 channels, rows staged in LDS, 4 x 4 register
 * blocks) for every other F32 or BF16 shape up to 4096 channels; all of them sum in fp32 within
 * row chunks and in fp64 across chunks in a fixed order. Anything else returns
 * IGC_ERR_UNSUPPORTED. Outputs must not alias inputs. */
int igc_sparse_conv_backward(const igc_grid* grid, const int32_t* d_map, const void* d_feats, int32_t dtype,
                             int32_t cin, const void* d_w, int32_t cout, const void* d_dout, void* d_dfeats,
                             float* d_dw, int32_t path, igc_stream stream);

/* Output grid of a 3x3x3 convolution with per-axis stride h_stride[0..2] (host, each 1, 2 or 3)
 * over `in` (the grid-to-grid ops ConvGrid and ConvTransposeGrid in the op table of the "ONNX
 * Runtime support for fVDB operations" proposal; the pages name the ops without a formula, so
 * the plain reading is taken), offsets d in {-1, 0, 1}^3:
 *     transposed == 0: y is active iff some active x of `in` has x = stride * y + d
 *                      (stride 1 gives the dilation of `in` by one voxel);
 *     transposed != 0: y is active iff y = stride * x + d for some active x of `in`.
 * The result is a new immutable grid (*out, library-owned, freed with igc_grid_destroy) in the
 * canonical order of igc_grid_build, whose memory comes from `alloc` (may be NULL) as for
 * igc_grid_build. Errors: IGC_ERR_UNSUPPORTED for strides outside 1..3,
 * IGC_ERR_RANGE when an output coordinate leaves the int32 range; *out is then NULL. Built
 * from the input's leaves with one host synchronisation (as igc_conv_grid_chain with one stage)
 * when the output spans at most 4096 root tiles, else as igc_grid_build of the candidate outputs
 * (one synchronisation more than igc_grid_build). */
int igc_conv_grid(const igc_grid* in, const int32_t* h_stride, int32_t transposed, const igc_allocator* alloc,
                  igc_stream stream, igc_grid** out);

/* Output grids of a chain of those convolutions, stage k's input being stage k-1's output
 * (stage 0's: `in`), with the voxel counts kept on the device through the chain (DriveRT,
 * "Counts kept on the GPU"): one host synchronisation for the whole chain instead of one per
 * grid. h_strides int32[n_stages][3] (host, each 1, 2 or 3), h_transposed int32[n_stages]
 * (host; NULL means none transposed), 1 <= n_stages <= 16. out[0 .. n_stages) receives new
 * immutable grids (library-owned, each freed with igc_grid_destroy), identical to those of
 * n_stages igc_conv_grid calls in turn, with memory from `alloc` as for igc_grid_build. Node
 * arrays are sized from estimates; when a stage outgrows one the chain runs again from that
 * stage with the exact counts it reported (DriveRT, "Compilation and deployment": results are
 * never truncated), which adds one synchronisation per repetition. Errors as for
 * igc_conv_grid, plus IGC_ERR_UNSUPPORTED when a stage's output spans more than 4096 root tiles
 * (build such stages with igc_conv_grid); on any error every out[k] is NULL. */
#define IGC_MAX_CHAIN 16
int igc_conv_grid_chain(const igc_grid* in, int32_t n_stages, const int32_t* h_strides, const int32_t* h_transposed,
                        const igc_allocator* alloc, igc_stream stream, igc_grid** out);

/* Neighbour map between two grids for that convolution (DriveRT, "Shared neighbour maps", for
 * two coordinate domains): d_map int32[27, N_out] (device, caller-owned, N_out = voxels of
 * `out`), offsets ordered as in igc_kernel_map:
 *     transposed == 0: d_map[o*N_out + r] = row of `in` at stride * y_r + d_o, or -1;
 *     transposed != 0: d_map[o*N_out + r] = row of `in` at (y_r - d_o) / stride where the
 *                      stride divides y_r - d_o on every axis, else -1.
 * y_r are the coordinates of `out` in row order. Any two grids are accepted (`out` need not come
 * from igc_conv_grid). Strides must be 1, 2 or 3 (IGC_ERR_UNSUPPORTED otherwise). */
int igc_conv_map(const igc_grid* in, const igc_grid* out, const int32_t* h_stride, int32_t transposed,
                 int32_t* d_map, igc_stream stream);

/* Convolution between two grids (strided and transposed sparse convolution): for every active
 * voxel r of `out`,
 *     d_out[r, co] = sum_{o, ci : map[o, r] >= 0} d_feats[map[o, r], ci] * d_w[o, ci, co]
 * with d_map from igc_conv_map (int32[27, N_out], values < n_in), d_feats [n_in, cin] the input
 * grid's features, d_w [27, cin, cout] and d_out [N_out, cout]. Runs on the gather-GEMM-scatter
 * path for the BF16 shapes igc_sparse_conv supports there and on the general-shape path for
 * every other F32 or BF16 shape up to 4096 channels (fp32 accumulation, bf16 outputs rounded to
 * nearest even; map entries outside [0, n_in) read as absent); anything else returns
 * IGC_ERR_UNSUPPORTED. d_out must not alias d_feats. */
int igc_sparse_conv_between(const igc_grid* out, const int32_t* d_map, int64_t n_in, const void* d_feats,
                            int32_t dtype, int32_t cin, const void* d_w, int32_t cout, void* d_out,
                            igc_stream stream);

/* The path IGC_PATH_AUTO takes for this grid and layer shape (host only). LEAF when LEAF
 * supports (dtype, cin, cout) and either GGS does not or the grid's leaf occupancy (active
 * voxels / (512 x leaves)) is at least 0.2 for cin <= 32 or 0.5 for cin >= 64 (the fVDB notes
 * put the leaf backend's break-even near 20%; the higher bar at 64 channels is measured);
 * GGS when GGS supports the shape; GATHER for the other shapes up to 4096 channels;
 * IGC_ERR_UNSUPPORTED beyond. The IGC_PATH environment variable ("leaf" / "ggs") overrides the
 * automatic choice where that path supports the shape. */
int igc_select_path(const igc_grid* grid, int32_t dtype, int32_t cin, int32_t cout, int32_t* path);

/* Message of the last failed call on this host thread ("" if none). */
const char* igc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IGCONV_H */
