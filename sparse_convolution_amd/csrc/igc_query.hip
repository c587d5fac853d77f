// Queries over a built IndexGrid: active coordinates in row order, coordinate -> row, and the
// neighbour (kernel) map.
//
// Kernel map (DriveRT, "Shared neighbour maps"; fVDB notes, sparse-conv operators): for each
// active voxel and each kernel offset, the row of the voxel at coordinate + offset, or -1.
// One wave handles one leaf. It reads the leaf's 3x3x3 block of neighbour leaves from the
// grid's neighbour table, keeps the 27 leaf index records (80 B each) in LDS, compacts the
// leaf's active voxels, and then answers every (voxel, offset) pair with an LDS mask test,
// the prefix count and a popcount - no tree walk per pair. Offsets up to 8 voxels per axis
// stay inside the 3x3x3 block of leaves. For a fixed offset the wave's 64 voxels have
// consecutive rows, so every store of map[o, r] is one contiguous 256-byte run.
#include <hip/hip_runtime.h>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

constexpr int kMaxOffsets = 256;

struct OffsetList {
  int8_t d[kMaxOffsets][3];
  int32_t K;
};

__global__ __launch_bounds__(256) void k_active_ijk(GridView g, int32_t* __restrict__ out) {
  const int lane = lane_id();
  const int64_t f = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (f >= g.n_leaf) return;
  const int4 o = g.leaf_origin[f];
  const LeafRec& L = g.leaf[f];
  uint64_t row = L.offset;
  for (int w = 0; w < 8; ++w) {
    const uint64_t word = L.mask[w];
    if ((word >> lane) & 1ull) {
      const uint64_t r = row + (uint64_t)__popcll(word & ((1ull << lane) - 1ull));
      if (r >= (uint64_t)g.n_voxels) return;
      out[3 * r] = o.x + w;
      out[3 * r + 1] = o.y + (lane >> 3);
      out[3 * r + 2] = o.z + (lane & 7);
    }
    row += (uint64_t)__popcll(word);
  }
}

__global__ __launch_bounds__(256) void k_ijk_to_index(GridView g, const int32_t* __restrict__ q, int64_t m,
                                                      int32_t* __restrict__ idx) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < m; r += (int64_t)gridDim.x * blockDim.x) {
    const int32_t i = q[3 * r], j = q[3 * r + 1], k = q[3 * r + 2];
    int32_t out = -1;
    const int32_t f = find_leaf(g, i, j, k);
    if (f >= 0) {
      const LeafRec& L = g.leaf[f];
      out = leaf_row(L.mask, L.offset, L.prefix, (((uint32_t)i & 7u) << 6) | (((uint32_t)j & 7u) << 3) | ((uint32_t)k & 7u));
    }
    idx[r] = out;
  }
}

__global__ void k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) p[e] = v;
}

__global__ __launch_bounds__(256) void k_kernel_map(GridView g, OffsetList off, int32_t* __restrict__ map,
                                                    uint32_t* __restrict__ nbmask) {
  __shared__ uint64_t s_mask[4][27][8];
  __shared__ uint64_t s_off[4][27];
  __shared__ uint64_t s_pre[4][27];
  __shared__ uint16_t s_pos[4][512];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t f = (int64_t)blockIdx.x * 4 + wave;
  const bool has_leaf = f < g.n_leaf;

  // The 27 leaf records around this one (slot 13 is the leaf itself), from the neighbour table.
  if (has_leaf && lane < 27) {
    const int32_t nl = g.leaf_nbr[f * 27 + lane];
    if (nl >= 0) {
      const LeafRec& L = g.leaf[nl];
      for (int w = 0; w < 8; ++w) s_mask[wave][lane][w] = L.mask[w];
      s_off[wave][lane] = L.offset;
      s_pre[wave][lane] = L.prefix;
    } else {
      for (int w = 0; w < 8; ++w) s_mask[wave][lane][w] = 0;
      s_off[wave][lane] = 0;
      s_pre[wave][lane] = 0;
    }
  }
  __syncthreads();

  // Active voxels of the leaf, compacted in row order.
  uint32_t count = 0;
  if (has_leaf) {
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int w = 0; w < 8; ++w) {
      const uint64_t word = s_mask[wave][13][w];
      if ((word >> lane) & 1ull) s_pos[wave][count + (uint32_t)__popcll(word & lt)] = (uint16_t)(w * 64 + lane);
      count += (uint32_t)__popcll(word);
    }
  }
  __syncthreads();
  if (!has_leaf) return;

  const int64_t N = g.n_voxels;
  const uint64_t base = s_off[wave][13];
  for (uint32_t q = 0; q < count; q += 64) {
    const uint32_t t = q + lane;
    const bool act = t < count && base + t < (uint64_t)g.n_voxels;
    const uint32_t n = act ? s_pos[wave][t] : 0u;
    const int pi = (int)(n >> 6), pj = (int)((n >> 3) & 7u), pk = (int)(n & 7u);
    uint32_t bits = 0;
    for (int o = 0; o < off.K; ++o) {
      const int ni = pi + off.d[o][0], nj = pj + off.d[o][1], nk = pk + off.d[o][2];
      const int slot = ((ni >> 3) + 1) * 9 + ((nj >> 3) + 1) * 3 + ((nk >> 3) + 1);
      const uint32_t w = (uint32_t)(ni & 7);
      const uint32_t b = ((uint32_t)(nj & 7) << 3) | (uint32_t)(nk & 7);
      const uint64_t word = s_mask[wave][slot][w];
      const uint64_t bit = 1ull << b;
      int32_t idx = -1;
      if (word & bit) {
        const uint32_t pre = w ? (uint32_t)(s_pre[wave][slot] >> (9u * (w - 1u))) & 511u : 0u;
        idx = (int32_t)(s_off[wave][slot] + pre + (uint32_t)__popcll(word & (bit - 1ull)));
        if (o < 32) bits |= 1u << o;
      }
      if (act) map[(size_t)o * (size_t)N + base + t] = idx;
    }
    if (nbmask && act) nbmask[base + t] = bits;
  }
}

// Kernel map for offsets inside the 3x3x3 block (|component| <= 1): one wave per leaf builds
// the 10 x 10 x 10 window of row indices around its leaf in LDS (one mask test + prefix +
// popcount per cell), after which each (voxel, offset) pair is a single LDS read at a constant
// cell offset, stored contiguously per offset.
__global__ __launch_bounds__(256) void k_kernel_map_window(GridView g, OffsetList off, int32_t* __restrict__ map,
                                                           uint32_t* __restrict__ nbmask) {
  __shared__ uint64_t s_mask[4][27][8];
  __shared__ uint64_t s_off[4][27];
  __shared__ uint64_t s_pre[4][27];
  __shared__ int32_t s_idx[4][1000];
  __shared__ uint16_t s_pos[4][512];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t f = (int64_t)blockIdx.x * 4 + wave;
  const bool has_leaf = f < g.n_leaf;

  if (has_leaf && lane < 27) {
    const int32_t nl = g.leaf_nbr[f * 27 + lane];
    if (nl >= 0) {
      const LeafRec& L = g.leaf[nl];
      for (int w = 0; w < 8; ++w) s_mask[wave][lane][w] = L.mask[w];
      s_off[wave][lane] = L.offset;
      s_pre[wave][lane] = L.prefix;
    } else {
      for (int w = 0; w < 8; ++w) s_mask[wave][lane][w] = 0;
      s_off[wave][lane] = 0;
      s_pre[wave][lane] = 0;
    }
  }
  __syncthreads();

  uint32_t count = 0;
  if (has_leaf) {
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int w = 0; w < 8; ++w) {
      const uint64_t word = s_mask[wave][13][w];
      if ((word >> lane) & 1ull) s_pos[wave][count + (uint32_t)__popcll(word & lt)] = (uint16_t)(w * 64 + lane);
      count += (uint32_t)__popcll(word);
    }
    for (int c = lane; c < 1000; c += 64) {
      const int x = c / 100 - 1, y = (c / 10) % 10 - 1, z = c % 10 - 1;
      const int slot = ((x >> 3) + 1) * 9 + ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
      const uint32_t q = (uint32_t)(x & 7);
      const uint64_t word = s_mask[wave][slot][q];
      const uint64_t bit = 1ull << ((uint32_t)((y & 7) << 3) | (uint32_t)(z & 7));
      int32_t idx = -1;
      if (word & bit) {
        const uint32_t pre = q ? (uint32_t)(s_pre[wave][slot] >> (9u * (q - 1u))) & 511u : 0u;
        idx = (int32_t)(s_off[wave][slot] + pre + (uint32_t)__popcll(word & (bit - 1ull)));
      }
      s_idx[wave][c] = idx;
    }
  }
  __syncthreads();
  if (!has_leaf) return;

  const int64_t N = g.n_voxels;
  const uint64_t base = s_off[wave][13];
  for (uint32_t q = 0; q < count; q += 64) {
    const uint32_t t = q + lane;
    const bool act = t < count && base + t < (uint64_t)N;
    const uint32_t n = act ? s_pos[wave][t] : 0u;
    const int cell0 = (int)((n >> 6) * 100 + ((n >> 3) & 7u) * 10 + (n & 7u)) + 111;  // cell of offset 0
    int32_t* dst = map + base + t;
    uint32_t bits = 0;
    for (int o = 0; o < off.K; ++o) {
      const int idx = s_idx[wave][cell0 + off.d[o][0] * 100 + off.d[o][1] * 10 + off.d[o][2]];
      if (idx >= 0 && o < 32) bits |= 1u << o;
      if (act) dst[(size_t)o * (size_t)N] = idx;
    }
    if (nbmask && act) nbmask[base + t] = bits;
  }
}

}  // namespace

int launch_active_ijk(const igc_grid* g, int32_t* d_out, hipStream_t s) {
  if (g->n_leaf == 0) return IGC_OK;
  k_active_ijk<<<(unsigned)((g->n_leaf + 3) / 4), 256, 0, s>>>(g->view(), d_out);
  IGC_HIP(hipGetLastError(), "igc_grid_active_ijk: launch");
  return IGC_OK;
}

int launch_ijk_to_index(const igc_grid* g, const int32_t* d_q, int64_t m, int32_t* d_idx, hipStream_t s) {
  if (m == 0) return IGC_OK;
  int64_t blocks = (m + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (g->n_voxels == 0) {
    k_fill_i32<<<(unsigned)blocks, 256, 0, s>>>(d_idx, m, -1);
  } else {
    k_ijk_to_index<<<(unsigned)blocks, 256, 0, s>>>(g->view(), d_q, m, d_idx);
  }
  IGC_HIP(hipGetLastError(), "igc_grid_ijk_to_index: launch");
  return IGC_OK;
}

int launch_kernel_map(const igc_grid* g, const int32_t* h_offsets, int32_t K, int32_t* d_map, uint32_t* d_nbmask,
                      hipStream_t s) {
  if (g->n_voxels == 0) return IGC_OK;
  OffsetList off;
  off.K = K;
  for (int o = 0; o < K; ++o)
    for (int a = 0; a < 3; ++a) off.d[o][a] = (int8_t)h_offsets[3 * o + a];
  bool unit = true;
  for (int a = 0; a < 3 * K; ++a) unit = unit && h_offsets[a] >= -1 && h_offsets[a] <= 1;
  if (unit)
    k_kernel_map_window<<<(unsigned)((g->n_leaf + 3) / 4), 256, 0, s>>>(g->view(), off, d_map, d_nbmask);
  else
    k_kernel_map<<<(unsigned)((g->n_leaf + 3) / 4), 256, 0, s>>>(g->view(), off, d_map, d_nbmask);
  IGC_HIP(hipGetLastError(), "igc_kernel_map: launch");
  return IGC_OK;
}

}  // namespace igc
