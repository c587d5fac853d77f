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

#include <algorithm>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

constexpr int kMaxOffsets = 256;
constexpr int64_t kMapGroups = 1280;  // workgroups of the persistent kernel-map form (5 per CU)
constexpr uint32_t kVoxelMajor = 128;  // leaves with at most this many voxels take the voxel-major stores

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

// Unit-stencil form (every offset within one voxel per axis). Waves are persistent: wave w
// of the grid walks leaves w, w + W, ... (W waves in all), and while it answers one leaf, the
// neighbour-table entries and leaf records of the next one are already on their way into
// registers of lanes 0..26. Each wave owns its LDS slice (no workgroup barriers). Per leaf
// the wave fills a 10^3 window of row indices (cell (x+1, y+1, z+1) for leaf-local x, y, z in
// [-1, 8], -1 where there is no voxel) once from the 27 records, so a pair is one LDS read.
// Offset o's rows of the leaf, map[o, base .. base + count), are written in 16-byte quads
// aligned in memory (the quad grid of a row is shifted by (o N + base) mod 4); only the two
// edge quads of a row, which the neighbouring leaves share, are written element by element.
__global__ __launch_bounds__(256) void k_kernel_map_window(GridView g, OffsetList off, int32_t* __restrict__ map,
                                                           uint32_t* __restrict__ nbmask) {
  __shared__ uint64_t s_mask[4][27][8];
  __shared__ uint64_t s_off[4][27];
  __shared__ uint64_t s_pre[4][27];
  __shared__ int32_t s_idx[4][1000];
  __shared__ uint16_t s_cell[4][512];
  __shared__ int16_t s_delta[kMaxOffsets];  // window-cell offset of each stencil offset
  for (int o = threadIdx.x; o < off.K; o += blockDim.x)
    s_delta[o] = (int16_t)(off.d[o][0] * 100 + off.d[o][1] * 10 + off.d[o][2]);
  __syncthreads();
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t W = (int64_t)gridDim.x * 4;
  const int64_t F = g.n_leaf, N = g.n_voxels;
  int64_t f = (int64_t)blockIdx.x * 4 + wave;

  // Lanes 0..26: the records of the leaf to answer next (m, ro, rp) and the neighbour-table
  // entry of the one after it (nb).
  uint64_t m0 = 0, m1 = 0, m2 = 0, m3 = 0, m4 = 0, m5 = 0, m6 = 0, m7 = 0, ro = 0, rp = 0;
#define IGC_LOAD_REC(nl_)                                                                   \
  {                                                                                         \
    const int32_t nl__ = (nl_);                                                             \
    const bool ok__ = lane < 27 && nl__ >= 0;                                               \
    const LeafRec* L__ = g.leaf + (ok__ ? nl__ : 0);                                        \
    m0 = ok__ ? L__->mask[0] : 0ull; m1 = ok__ ? L__->mask[1] : 0ull;                       \
    m2 = ok__ ? L__->mask[2] : 0ull; m3 = ok__ ? L__->mask[3] : 0ull;                       \
    m4 = ok__ ? L__->mask[4] : 0ull; m5 = ok__ ? L__->mask[5] : 0ull;                       \
    m6 = ok__ ? L__->mask[6] : 0ull; m7 = ok__ ? L__->mask[7] : 0ull;                       \
    ro = ok__ ? L__->offset : 0ull; rp = ok__ ? L__->prefix : 0ull;                         \
  }
  auto load_nb = [&](int64_t leaf) -> int32_t { return lane < 27 && leaf < F ? g.leaf_nbr[leaf * 27 + lane] : -1; };
  IGC_LOAD_REC(load_nb(f));
  int32_t nb = load_nb(f + W);

  for (; f < F; f += W) {
    if (lane < 27) {
      uint64_t* sm = s_mask[wave][lane];
      sm[0] = m0; sm[1] = m1; sm[2] = m2; sm[3] = m3; sm[4] = m4; sm[5] = m5; sm[6] = m6; sm[7] = m7;
      s_off[wave][lane] = ro;
      s_pre[wave][lane] = rp;
    }
    IGC_LOAD_REC(nb);  // the next leaf's records, in flight while this one is answered
    nb = load_nb(f + 2 * W);
    wave_sync();

    // Window cells of the active voxels in row order, and the window of row indices.
    uint32_t count = 0;
    const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint64_t word = s_mask[wave][13][w];
      if ((word >> lane) & 1ull)
        s_cell[wave][count + (uint32_t)__popcll(word & lt)] = (uint16_t)(w * 100 + (lane >> 3) * 10 + (lane & 7) + 111);
      count += (uint32_t)__popcll(word);
    }
    // Lane p < 100 takes the window column (y, z) = (p / 10 - 1, p % 10 - 1) for all ten x.
    for (int p = lane; p < 100; p += 64) {
      const int y = p / 10 - 1, z = p % 10 - 1;
      const int syz = ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
      const uint64_t bit = 1ull << ((uint32_t)((y & 7) << 3) | (uint32_t)(z & 7));
#pragma unroll
      for (int xi = 0; xi < 10; ++xi) {
        const int slot = (xi == 0 ? 0 : xi == 9 ? 18 : 9) + syz;
        const uint32_t q = (uint32_t)((xi + 7) & 7);  // x & 7 for x = xi - 1
        const uint64_t word = s_mask[wave][slot][q];
        int32_t idx = -1;
        if (word & bit) {
          const uint32_t pre = q ? (uint32_t)(s_pre[wave][slot] >> (9u * (q - 1u))) & 511u : 0u;
          idx = (int32_t)(s_off[wave][slot] + pre + (uint32_t)__popcll(word & (bit - 1ull)));
        }
        s_idx[wave][xi * 100 + p] = idx;
      }
    }
    wave_sync();

    const uint64_t base = s_off[wave][13];
    if (base + count > (uint64_t)N) count = base < (uint64_t)N ? (uint32_t)(N - base) : 0u;
    if (count <= kVoxelMajor) {
      // Sparse leaf: lane t takes voxel t (and t + 64) for every offset, 4-byte stores that are
      // contiguous over the lanes - fewer instructions than the quads for a short leaf.
      for (uint32_t t = lane; t < count; t += 64) {
        const int cell = s_cell[wave][t];
        int32_t* dst = map + base + t;
        uint32_t bits = 0;
        for (int o = 0; o < off.K; ++o) {
          const int idx = s_idx[wave][cell + s_delta[o]];
          if (idx >= 0 && o < 32) bits |= 1u << o;
          dst[(size_t)o * (size_t)N] = idx;
        }
        if (nbmask) nbmask[base + t] = bits;
      }
      wave_sync();
      continue;
    }
    // A row of the leaf spans at most (count + 6) / 4 quads; rows shorter than the wave share
    // it: lanes [G r, G r + G) take row ob + r, with G the smallest power of two that holds
    // the row's quads.
    const uint32_t nqm = (count + 6u) >> 2;
    uint32_t G = 1;
    while (G < nqm && G < 64u) G <<= 1;
    const int R = 64 / (int)G;
    const int sub = lane / (int)G;
    const uint32_t k0 = (uint32_t)lane & (G - 1u);
    for (int ob = 0; ob < off.K; ob += R) {
      const int o = ob + sub;
      if (o >= off.K) break;
      const int delta = s_delta[o];
      const uint64_t g0 = (uint64_t)o * (uint64_t)N + base;  // element of (o, base)
      const uint64_t q0 = g0 & ~3ull;                         // first 16-byte aligned quad
      const uint32_t nq = (uint32_t)((g0 + count + 3 - q0) >> 2);
      for (uint32_t k = k0; k < nq; k += G) {
        const uint64_t e0 = q0 + 4ull * k;
        int v[4];
        bool in[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t t = (int64_t)(e0 + e) - (int64_t)g0;  // voxel of this element
          in[e] = t >= 0 && t < (int64_t)count;
          v[e] = in[e] ? s_idx[wave][s_cell[wave][t] + delta] : 0;
        }
        if (in[0] && in[3]) {
          *(int4*)(map + e0) = make_int4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (in[e]) map[e0 + e] = v[e];
        }
      }
    }
    if (nbmask) {
      for (uint32_t t = lane; t < count; t += 64) {
        const int cell = s_cell[wave][t];
        uint32_t bits = 0;
        for (int o = 0; o < off.K && o < 32; ++o)
          if (s_idx[wave][cell + s_delta[o]] >= 0) bits |= 1u << o;
        nbmask[base + t] = bits;
      }
    }
    wave_sync();
  }
}
#undef IGC_LOAD_REC

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
  // The window form stores 16-byte quads: it needs a 16-byte aligned map.
  if (unit && ((uintptr_t)d_map & 15u) == 0)
    k_kernel_map_window<<<(unsigned)std::min<int64_t>((g->n_leaf + 3) / 4, kMapGroups), 256, 0, s>>>(g->view(), off,
                                                                                                   d_map, d_nbmask);
  else
    k_kernel_map<<<(unsigned)((g->n_leaf + 3) / 4), 256, 0, s>>>(g->view(), off, d_map, d_nbmask);
  IGC_HIP(hipGetLastError(), "igc_kernel_map: launch");
  return IGC_OK;
}

}  // namespace igc
