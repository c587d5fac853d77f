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

#include <cstdlib>
#include <cstring>

#include <algorithm>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

constexpr int kMaxOffsets = 256;
constexpr int64_t kMapGroups = 1280;  // workgroups of the persistent kernel-map form (5 per CU)
constexpr int64_t kMapGroupsPc = 512;   // workgroups of the producer / consumer form (2 per CU)
constexpr int64_t kMapPcLeaves = 16384; // grids with at least this many leaves take the producer / consumer form
constexpr uint32_t kVoxelMajor = 128;  // leaves with at most this many voxels take the voxel-major stores
// The quad stores place each row's head and tail elements at voxels c and count - 6 + c: a
// leaf needs at least 3 voxels there, or that index wraps below zero.
static_assert(kVoxelMajor >= 2, "the quad-store path needs leaves of at least 3 voxels");

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

// Standard-stencil form (the 27 offsets in the order o = (dx+1)*9 + (dy+1)*3 + (dz+1)). Waves
// are persistent: wave w of an XCD walks leaves b + w, b + w + W, ... of the XCD's range (W
// waves on the XCD), and while it answers one leaf, the neighbour-table entries and leaf
// records of the next one are already on their way into registers of lanes 0..26. Each wave
// owns its LDS slice (no workgroup barriers). Per leaf the wave fills a 10^3 window of row
// indices (cell (x+1)*100 + (y+1)*10 + (z+1) for leaf-local x, y, z in [-1, 8], -1 where there
// is no voxel) once from the 27 records, so a pair is one LDS read at a constant offset from the
// voxel's cell. The reads of a phase are all issued before their results are used, which keeps
// the per-leaf chain of LDS round trips short, and the per-leaf vector work is kept small
// (32-bit mask arithmetic, offsets folded into the LDS instructions, store addresses as a
// uniform row pointer plus a 32-bit lane offset). Leaves of at most kVoxelMajor voxels are
// written voxel-major (lane = voxel, 4-byte stores contiguous over the lanes). Fuller leaves
// write offset o's row, map[o, base .. base + count), as 16-byte quads aligned in memory
// (lane = quad; the quad grid of a row is shifted by (o N + base) mod 4), and the at most
// three elements before the first and after the last whole quad of each row, shared with the
// neighbouring leaves' rows, 64 (row, element) pairs to a 4-byte store.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRecWords = 20;  // a leaf record in LDS as 32-bit words: masks 0..15, offset 16-17, prefix 18-19

// Window-cell distance of offset o of the standard stencil from cell (0, 0, 0) of the voxel's
// 3x3x3 neighbourhood: the neighbour of the voxel in cell c is cell c - 111 + win_off(o).
__host__ __device__ constexpr int win_off(int o) { return 100 * (o / 9) + 10 * ((o / 3) % 3) + o % 3; }

// Window column (y, z) = (p / 10 - 1, p % 10 - 1) for the ten x = -1 .. 8: row index or -1.
// rec holds the 27 records of the leaf's 3x3x3 block (zero records where a leaf is absent).
// Rows fit in 32 bits, so the records' offsets are used by their low words.
__device__ __forceinline__ void window_column(const uint32_t (*rec)[kRecWords], int p, int32_t* __restrict__ col) {
  const int y = p / 10 - 1, z = p % 10 - 1;
  const int syz = ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
  const uint32_t b = ((uint32_t)(y & 7) << 3) | (uint32_t)(z & 7);  // bit of (y, z) in a mask word
  const uint32_t bit = 1u << (b & 31u), below = bit - 1u;
  const bool high = b >= 32u;
  const uint32_t tlo = high ? 0u : bit, thi = high ? bit : 0u;       // the bit, by half word
  const uint32_t mlo = high ? ~0u : below, mhi = high ? below : 0u;  // the bits below it
  const uint32_t* A = rec[syz];       // x = -1: mask word 7 of the leaf below in x
  const uint32_t* B = rec[9 + syz];   // x = 0 .. 7
  const uint32_t* C = rec[18 + syz];  // x = 8: mask word 0 of the leaf above in x
  const uint32_t a_lo = A[14], a_hi = A[15], a_off = A[16], a_pre = A[19];
  const uint32_t c_lo = C[0], c_hi = C[1], c_off = C[16];
  const uint32_t b_off = B[16], p_lo = B[18], p_hi = B[19];
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = B[i];
  auto cell = [&](uint32_t lo, uint32_t hi, uint32_t first) -> int32_t {
    const bool on = ((lo & tlo) | (hi & thi)) != 0u;
    return on ? (int32_t)(first + (uint32_t)__popc(lo & mlo) + (uint32_t)__popc(hi & mhi)) : -1;
  };
  // Prefix of mask word q (q >= 1): 9-bit field q - 1 of the 64-bit prefix word.
  auto pre = [&](int q) -> uint32_t {
    const int sh = 9 * (q - 1);
    if (sh + 9 <= 32) return (p_lo >> sh) & 511u;
    if (sh >= 32) return (p_hi >> (sh - 32)) & 511u;
    return ((p_lo >> sh) | (p_hi << (32 - sh))) & 511u;
  };
  col[0] = cell(a_lo, a_hi, a_off + ((a_pre >> 22) & 511u));  // field 6 = bits 54..62
  col[100] = cell(w[0], w[1], b_off);
#pragma unroll
  for (int q = 1; q < 8; ++q) col[100 * (1 + q)] = cell(w[2 * q], w[2 * q + 1], b_off + pre(q));
  col[900] = cell(c_lo, c_hi, c_off);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5, 8))) void k_kernel_map_window(
    GridView g, int32_t* __restrict__ map, uint32_t* __restrict__ nbmask) {
  __shared__ __align__(16) uint32_t s_rec[4][27][kRecWords];
  __shared__ int32_t s_idx[4][1000];
  __shared__ uint16_t s_cell[4][512];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t F = g.n_leaf, N = g.n_voxels;
  // Workgroups go to the eight XCDs in turn (workgroup b to XCD b mod 8); each XCD takes one
  // contiguous range of leaves, in proportion to its waves, so the map rows of neighbouring
  // leaves - which share their edge cache lines - are written through the same L2.
  const int64_t G = gridDim.x, x = blockIdx.x & 7, q = G >> 3, rem = G & 7;
  const int64_t before = x * q + (x < rem ? x : rem), mine = q + (x < rem ? 1 : 0);
  const int64_t f_end = F * (before + mine) / G;
  const int64_t W = 4 * mine;  // waves of this XCD
  int64_t f = F * before / G + (int64_t)(blockIdx.x >> 3) * 4 + wave;

  // Lanes 0..26: the record of neighbour slot `lane` of the leaf to answer next, as five
  // 16-byte parts (r0..r4; stored as zeros when the slot has no leaf), and the neighbour-table
  // entry of the leaf after it (nb).
  u32x4 r0 = {0, 0, 0, 0}, r1 = r0, r2 = r0, r3 = r0, r4 = r0;
  bool rok = false;
#define IGC_LOAD_REC(nl_)                                                 \
  {                                                                       \
    const int32_t nl__ = (nl_);                                           \
    rok = nl__ >= 0;                                                      \
    if (lane < 27) {                                                      \
      const u32x4* p__ = (const u32x4*)(g.leaf + (nl__ >= 0 ? nl__ : 0)); \
      r0 = p__[0]; r1 = p__[1]; r2 = p__[2]; r3 = p__[3]; r4 = p__[4];    \
    }                                                                     \
  }
  auto load_nb = [&](int64_t leaf) -> int32_t { return lane < 27 && leaf < f_end ? g.leaf_nbr[leaf * 27 + lane] : -1; };
  IGC_LOAD_REC(load_nb(f));
  int32_t nb = load_nb(f + W);

  for (; f < f_end; f += W) {
    // The lane number through an opaque copy: values derived from it are recomputed per leaf
    // instead of being kept live (or spilled) across the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (ln < 27) {
      u32x4* d = (u32x4*)s_rec[wave][ln];
      const u32x4 z = {0, 0, 0, 0};
      d[0] = rok ? r0 : z; d[1] = rok ? r1 : z; d[2] = rok ? r2 : z; d[3] = rok ? r3 : z; d[4] = rok ? r4 : z;
    }
    IGC_LOAD_REC(nb);  // the next leaf's records, in flight while this one is answered
    nb = load_nb(f + 2 * W);
    wave_sync();

    // Window cells of the active voxels in row order (mbcnt: set bits of the word below the lane).
    const uint32_t* own = s_rec[wave][13];
    uint32_t mw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) mw[i] = own[i];
    const uint32_t base = own[16];
    uint32_t count = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t lo = mw[2 * w], hi = mw[2 * w + 1];
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, count));
      if ((((uint64_t)hi << 32 | lo) >> ln) & 1ull)
        s_cell[wave][rank] = (uint16_t)(w * 100 + (ln >> 3) * 10 + (ln & 7) + 111);
      count += (uint32_t)__popc(lo) + (uint32_t)__popc(hi);
    }
    // The window, one column (ten cells along x) per lane and pass.
#pragma unroll 1
    for (int p = ln; p < 100; p += 64) window_column(s_rec[wave], p, &s_idx[wave][p]);
    wave_sync();

    if ((uint64_t)base + count > (uint64_t)N) count = (uint64_t)base < (uint64_t)N ? (uint32_t)(N - base) : 0u;
    if (count <= kVoxelMajor) {
      // Lane t takes voxel t (and t + 64) for every offset: 27 LDS reads in flight, then 27
      // stores that are contiguous over the lanes.
      for (uint32_t t = ln; t < count; t += 64) {
        const int32_t* nbh = &s_idx[wave][s_cell[wave][t] - 111];
        int32_t v[27];
#pragma unroll
        for (int o = 0; o < 27; ++o) v[o] = nbh[win_off(o)];
#pragma unroll
        for (int o = 0; o < 27; ++o) (map + (size_t)o * (size_t)N + base)[t] = v[o];
        if (nbmask) {
          uint32_t bits = 0;
#pragma unroll
          for (int o = 0; o < 27; ++o) bits |= (v[o] >= 0 ? 1u : 0u) << o;
          nbmask[base + t] = bits;
        }
      }
      wave_sync();
      continue;
    }
    // Rows: map[o, base .. base + count) starts at element g0 = o N + base, s = g0 mod 4; its
    // first hd = (4 - s) mod 4 elements precede a 16-byte boundary, then fq whole quads.
    const uint32_t n4 = (uint32_t)N & 3u, s0 = base & 3u;
#pragma unroll 1
    for (int ox = 0; ox < 3; ++ox) {
#pragma unroll
      for (int r = 0; r < 9; ++r) {
        const int o = 9 * ox + r;
        const uint32_t s = (s0 + (uint32_t)o * n4) & 3u;
        const uint32_t hd = (4u - s) & 3u;
        const uint32_t fq = ((s + count) >> 2) - (s ? 1u : 0u);
        int32_t* rowp = map + (size_t)o * (size_t)N + base + hd;  // 16-byte aligned
        for (uint32_t k = ln; k < fq; k += 64) {
          const uint32_t t0 = hd + 4u * k;
          int32_t v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = s_idx[wave][(int)s_cell[wave][t0 + e] - 111 + 100 * ox + win_off(r)];
          *(i32x4*)(rowp + 4u * k) = i32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
    // The elements outside the whole quads: voxel c (c < 3) of the row's head, voxel
    // count - 6 + c (c >= 3) of its tail; pair p = 6 o + c.
    for (uint32_t p = ln; p < 162u; p += 64) {
      const uint32_t o = p / 6u, c = p - 6u * o;
      const uint32_t s = (s0 + o * n4) & 3u;
      const uint32_t hd = (4u - s) & 3u;
      const uint32_t fq = ((s + count) >> 2) - (s ? 1u : 0u);
      const uint32_t t = c < 3u ? c : count - 6u + c;
      if (c < 3u ? t < hd : t >= hd + 4u * fq)
        (map + (size_t)o * (size_t)N + base)[t] = s_idx[wave][(int)s_cell[wave][t] - 111 + win_off((int)o)];
    }
    if (nbmask) {
      for (uint32_t t = ln; t < count; t += 64) {
        const int32_t* nbh = &s_idx[wave][s_cell[wave][t] - 111];
        uint32_t bits = 0;
#pragma unroll
        for (int o = 0; o < 27; ++o) bits |= (nbh[win_off(o)] >= 0 ? 1u : 0u) << o;
        nbmask[base + t] = bits;
      }
    }
    wave_sync();
  }
}
#undef IGC_LOAD_REC

// Producer / consumer form of the standard-stencil kernel map. Stores and loads share one
// completion counter on this GPU, in issue order, so a wave that loads the next leaf's records
// after storing this leaf's map rows waits for those stores too: the store latency is exposed
// once per leaf. Here the four consumer waves of a workgroup issue no global loads at all; a
// fifth wave loads the 27 records of the next leaf of every consumer into a second LDS buffer
// while they answer the current ones, and one workgroup barrier (ordering LDS only, so it waits
// for no store) separates the steps. The consumers' work per leaf is that of the form above:
// window of row indices, then voxel-major or quad stores.
constexpr int kPcConsumers = 4;
constexpr int kPcThreads = 64 * (kPcConsumers + 1);

__device__ __forceinline__ void lds_step_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ __launch_bounds__(kPcThreads) __attribute__((amdgpu_waves_per_eu(5, 8))) void k_kernel_map_pc(
    GridView g, int32_t* __restrict__ map,
                                                               uint32_t* __restrict__ nbmask) {
  __shared__ __align__(16) uint32_t s_rec[2][kPcConsumers][27][kRecWords];
  __shared__ int32_t s_idx[kPcConsumers][1000];
  __shared__ uint16_t s_cell[kPcConsumers][512];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t F = g.n_leaf, N = g.n_voxels;
  // Workgroup b goes to XCD b mod 8; each XCD takes one contiguous range of leaves [lo, hi),
  // and at step k the consumers of local workgroup j answer leaves lo + (k * mine + j) * 4 + c.
  const int64_t G = gridDim.x, x = blockIdx.x & 7, q = G >> 3, rem = G & 7;
  const int64_t before = x * q + (x < rem ? x : rem), mine = q + (x < rem ? 1 : 0);
  const int64_t lo = F * before / G, hi = F * (before + mine) / G;
  const int64_t j = blockIdx.x >> 3;
  const int64_t span = hi - lo - kPcConsumers * j;
  const int64_t steps = span > 0 ? (span + kPcConsumers * mine - 1) / (kPcConsumers * mine) : 0;
  auto leaf_of = [&](int64_t k, int c) -> int64_t {
    const int64_t f = lo + (k * mine + j) * kPcConsumers + c;
    return f < hi ? f : -1;
  };

  if (wave == kPcConsumers) {
    // Producer. Lane l serves (consumer, slot) pairs l and l + 64 of the 4 * 27 = 108.
    const int p0 = lane, p1 = lane + 64;
    const bool has1 = p1 < kPcConsumers * 27;
    const int c0 = p0 / 27, t0 = p0 % 27, c1 = has1 ? p1 / 27 : 0, t1 = has1 ? p1 % 27 : 0;
    auto nbr_of = [&](int64_t k, int c, int t) -> int32_t {
      const int64_t f = k < steps ? leaf_of(k, c) : -1;
      return f >= 0 ? g.leaf_nbr[f * 27 + t] : -1;
    };
    auto fill = [&](int buf, int c, int t, int32_t nl) {
      const u32x4 z = {0, 0, 0, 0};
      u32x4 r[5] = {z, z, z, z, z};
      if (nl >= 0) {
        const u32x4* src = (const u32x4*)(g.leaf + nl);
#pragma unroll
        for (int i = 0; i < 5; ++i) r[i] = src[i];
      }
      u32x4* d = (u32x4*)s_rec[buf][c][t];
#pragma unroll
      for (int i = 0; i < 5; ++i) d[i] = r[i];
    };
    int32_t n0 = nbr_of(0, c0, t0), n1 = has1 ? nbr_of(0, c1, t1) : -1;
    fill(0, c0, t0, n0);
    if (has1) fill(0, c1, t1, n1);
    n0 = nbr_of(1, c0, t0);
    n1 = has1 ? nbr_of(1, c1, t1) : -1;
    lds_step_barrier();
    for (int64_t k = 0; k < steps; ++k) {
      // Records of step k + 1 into the other buffer; neighbour entries of step k + 2.
      const int buf = (int)((k + 1) & 1);
      const int32_t m0 = nbr_of(k + 2, c0, t0), m1 = has1 ? nbr_of(k + 2, c1, t1) : -1;
      fill(buf, c0, t0, n0);
      if (has1) fill(buf, c1, t1, n1);
      n0 = m0;
      n1 = m1;
      lds_step_barrier();
    }
    return;
  }

  // Consumer `wave`.
  const int c = wave;
  lds_step_barrier();
  for (int64_t k = 0; k < steps; ++k) {
    const int64_t f = leaf_of(k, c);
    if (f >= 0) {
      const uint32_t(*rec)[kRecWords] = s_rec[k & 1][c];
      int ln = lane;
      asm volatile("" : "+v"(ln));
      // Window cells of the active voxels in row order (mbcnt: set bits of the word below the lane).
      const uint32_t* own = rec[13];
      uint32_t mw[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) mw[i] = own[i];
      const uint32_t base = own[16];
      uint32_t count = 0;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const uint32_t lo32 = mw[2 * w], hi32 = mw[2 * w + 1];
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(hi32, __builtin_amdgcn_mbcnt_lo(lo32, count));
        if ((((uint64_t)hi32 << 32 | lo32) >> ln) & 1ull)
          s_cell[c][rank] = (uint16_t)(w * 100 + (ln >> 3) * 10 + (ln & 7) + 111);
        count += (uint32_t)__popc(lo32) + (uint32_t)__popc(hi32);
      }
#pragma unroll 1
      for (int p = ln; p < 100; p += 64) window_column(rec, p, &s_idx[c][p]);
      wave_sync();

      if ((uint64_t)base + count > (uint64_t)N) count = (uint64_t)base < (uint64_t)N ? (uint32_t)(N - base) : 0u;
      if (count <= kVoxelMajor) {
        for (uint32_t t = ln; t < count; t += 64) {
          const int32_t* nbh = &s_idx[c][s_cell[c][t] - 111];
          int32_t v[27];
#pragma unroll
          for (int o = 0; o < 27; ++o) v[o] = nbh[win_off(o)];
#pragma unroll
          for (int o = 0; o < 27; ++o) (map + (size_t)o * (size_t)N + base)[t] = v[o];
          if (nbmask) {
            uint32_t bits = 0;
#pragma unroll
            for (int o = 0; o < 27; ++o) bits |= (v[o] >= 0 ? 1u : 0u) << o;
            nbmask[base + t] = bits;
          }
        }
      } else {
        const uint32_t n4 = (uint32_t)N & 3u, s0 = base & 3u;
#pragma unroll 1
        for (int ox = 0; ox < 3; ++ox) {
#pragma unroll
          for (int r = 0; r < 9; ++r) {
            const int o = 9 * ox + r;
            const uint32_t s = (s0 + (uint32_t)o * n4) & 3u;
            const uint32_t hd = (4u - s) & 3u;
            const uint32_t fq = ((s + count) >> 2) - (s ? 1u : 0u);
            int32_t* rowp = map + (size_t)o * (size_t)N + base + hd;  // 16-byte aligned
            for (uint32_t kq = ln; kq < fq; kq += 64) {
              const uint32_t tq = hd + 4u * kq;
              int32_t v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = s_idx[c][(int)s_cell[c][tq + e] - 111 + 100 * ox + win_off(r)];
              *(i32x4*)(rowp + 4u * kq) = i32x4{v[0], v[1], v[2], v[3]};
            }
          }
        }
        for (uint32_t p = ln; p < 162u; p += 64) {
          const uint32_t o = p / 6u, e = p - 6u * o;
          const uint32_t s = (s0 + o * n4) & 3u;
          const uint32_t hd = (4u - s) & 3u;
          const uint32_t fq = ((s + count) >> 2) - (s ? 1u : 0u);
          const uint32_t t = e < 3u ? e : count - 6u + e;
          if (e < 3u ? t < hd : t >= hd + 4u * fq)
            (map + (size_t)o * (size_t)N + base)[t] = s_idx[c][(int)s_cell[c][t] - 111 + win_off((int)o)];
        }
        if (nbmask) {
          for (uint32_t t = ln; t < count; t += 64) {
            const int32_t* nbh = &s_idx[c][s_cell[c][t] - 111];
            uint32_t bits = 0;
#pragma unroll
            for (int o = 0; o < 27; ++o) bits |= (nbh[win_off(o)] >= 0 ? 1u : 0u) << o;
            nbmask[base + t] = bits;
          }
        }
      }
      wave_sync();
    }
    lds_step_barrier();
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
  bool standard = K == 27;
  for (int o = 0; o < K && standard; ++o)
    standard = h_offsets[3 * o] == o / 9 - 1 && h_offsets[3 * o + 1] == (o / 3) % 3 - 1 && h_offsets[3 * o + 2] == o % 3 - 1;
  // The window form stores 16-byte quads: it needs a 16-byte aligned map.
  if (standard && ((uintptr_t)d_map & 15u) == 0) {
    // Large grids are bound by the map's stores: the producer / consumer form keeps them from
    // being waited on. Small grids are bound by per-leaf latency, where the persistent form with
    // four independent waves and no workgroup barrier is faster. IGC_TEST_KMAP_FORM = "pc" or
    // "window" forces one form (tests).
    bool pc = g->n_leaf >= kMapPcLeaves;
    if (const char* e = std::getenv("IGC_TEST_KMAP_FORM")) {
      if (std::strcmp(e, "pc") == 0) pc = true;
      if (std::strcmp(e, "window") == 0) pc = false;
    }
    if (pc)
      k_kernel_map_pc<<<(unsigned)std::min<int64_t>((g->n_leaf + 3) / 4, kMapGroupsPc), kPcThreads, 0, s>>>(
          g->view(), d_map, d_nbmask);
    else
      k_kernel_map_window<<<(unsigned)std::min<int64_t>((g->n_leaf + 3) / 4, kMapGroups), 256, 0, s>>>(
          g->view(), d_map, d_nbmask);
  } else {
    k_kernel_map<<<(unsigned)((g->n_leaf + 3) / 4), 256, 0, s>>>(g->view(), off, d_map, d_nbmask);
  }
  IGC_HIP(hipGetLastError(), "igc_kernel_map: launch");
  return IGC_OK;
}

}  // namespace igc
