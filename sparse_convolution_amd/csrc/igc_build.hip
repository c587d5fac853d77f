// GPU IndexGrid build (fVDB notes, "GPU-accelerated IndexGrid build").
//
// The pages' build: 64-bit root keys (i, j, k each >> 12, packed 21+21+21 bits), a full radix
// sort and run-length encoding of them, a 64-bit in-tile key per coordinate, a local radix
// sort, upper / lower / leaf counts from the runs and unique keys, allocation from the
// counts, and top-down registration of nodes and voxel bit masks.
//
// What this implementation keeps and changes on gfx950:
//  1. Root tiles are deduplicated in an open-addressing hash table instead of by a full
//     sort + RLE of N keys: a wave first collapses equal tile keys with ballots, the leader
//     reads the slot and only then tries a compare-and-swap, so the few tiles of a scene
//     cost a cached read per wave. The U distinct tiles are then sorted (U is small) and
//     their rank in key order is stored back in the table. This gives the same tile order
//     as the sort + RLE of the pages at a fraction of the traffic. The table is the root of
//     the finished tree.
//  2. Per coordinate, key2 = tile rank << 36 | upper child (15 bits) << 21 | lower child
//     (12 bits) << 9 | leaf voxel (9 bits). The pass that writes key2 also builds the digit
//     histograms of every radix pass, and only the bit span where keys differ is sorted
//     (the OR and AND of all keys, taken in the tile pass, give that span).
//  3. Keys are sorted by their leaf part (key2 >> 9) only: the voxel bits inside a leaf are
//     OR-ed into the leaf's mask, so their order never matters, and the sort needs
//     ceil(varying leaf-key bits / 9) passes instead of ceil(varying key bits / 9). The sort
//     is an LSD radix sort with 8- or 9-bit digits over tiles of 4096 keys. Each pass is
//     reduce-then-scan: per-tile digit counts, a scan of every digit's counts over the tiles,
//     and a scatter that ranks the tile's keys (LDS atomics in the first pass, which needs no
//     stability; 64-lane ballots, a stable multisplit, in later ones), sorts them in LDS and
//     writes them out as runs per digit. A single-pass form with decoupled
//     look-back was measured slower here: with all tiles resident at once, late tiles walk
//     back over hundreds of predecessors that have published only their own counts.
//  4. Leaves, lower and upper nodes are counted in one pass over the sorted keys (a key
//     starts a leaf / lower / upper when its leaf / lower / upper part differs from its
//     predecessor's; the keys stay compacted, and those parts are compared at their compacted
//     bit positions); after the read-back of the counts, a second pass gives every key its
//     leaf / node rows from the scanned block counts and registers the nodes top-down. Leaf
//     mask bits are OR-ed in (duplicates set the same bit), first in LDS per block of keys:
//     leaves that lie inside the block are stored whole, the block's first and last leaf
//     are OR-ed into memory. Unique voxels are then the masks' popcounts: a scan over the
//     leaves gives every leaf its first row and the voxel count N (read back last). At each of
//     the three read-backs the last kernel before it writes the build state into pinned host
//     memory itself.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

constexpr int kThreads = 256;
constexpr int kKeysPerThread = 16;
constexpr int kTileKeys = kThreads * kKeysPerThread;  // 4096 keys per counting / registration block
constexpr int kSortKPT = 16;                           // keys per thread of a radix pass
constexpr int kSortTile = kThreads * kSortKPT;         // keys per onesweep tile
constexpr int kMaxPasses = 8;
constexpr int kMaxDigitBits = 9;                       // digits of 8 or 9 bits (wider ones measured slower)
constexpr int kMaxBins = 1 << kMaxDigitBits;
constexpr int kHistWidth = 4096;                       // passes * bins of the LDS histograms
constexpr int kSmallSort = 4096;             // tile-key sorts up to this size run in one workgroup
constexpr int kTileCache = 64;               // per-workgroup LDS cache of tiles already in the table
constexpr int kRootInLds = 512;              // root tables up to this capacity are copied to LDS

struct BuildState {
  uint32_t overflow;          // root table ran out of probes
  uint32_t n_tiles;           // distinct root tiles inserted
  uint32_t tile_list_count;   // compaction cursor
  uint32_t guard;             // a device-side bounds check failed (the build is rejected)
  uint32_t range;             // a derived grid's coordinate left the int32 range
  uint32_t cap_over;          // node arrays sized from an estimate were too small (the build is repeated)
  uint32_t sort_passes;       // radix passes the counted build's plan chose
  uint32_t sort_span;         // bits those passes cover
  uint64_t off_or, off_and;   // OR / AND over all in-tile offsets
  uint64_t key_or, key_and;   // OR / AND over all tile keys
  uint64_t counts[4];         // N, F, Lw, U from the sorted keys
  uint64_t n_rec;             // a derived grid's records (input leaves x slots); later kernels stop there
};

// The build state as the host reads it at a synchronisation: one thread of the last kernel
// before it copies the state into pinned host memory and makes the copy visible system-wide,
// which saves a device -> host copy (and its dispatch) per read-back.
__device__ __forceinline__ void publish_state(const BuildState* st, BuildState* host) {
  const uint64_t* src = reinterpret_cast<const uint64_t*>(st);
  uint64_t* dst = reinterpret_cast<uint64_t*>(host);
#pragma unroll
  for (int w = 0; w < (int)(sizeof(BuildState) / 8); ++w) dst[w] = src[w];
  __threadfence_system();
}

// ------------------------------------------------------------------------------ utilities

// Zeroes fill[0 .. nfill) and copies src[0 .. ncopy) to dst (one launch for both).
__global__ void k_fill_copy_u64(uint64_t* __restrict__ fill, int64_t nfill, uint64_t* __restrict__ dst,
                                const uint64_t* __restrict__ src, int64_t ncopy) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nfill + ncopy;
       e += (int64_t)gridDim.x * blockDim.x) {
    if (e < nfill) fill[e] = 0ull;
    else dst[e - nfill] = src[e - nfill];
  }
}

__global__ void k_fill_u64(uint64_t* __restrict__ p, int64_t n, uint64_t v) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
    p[e] = v;
}

// Build state reset and root table fill (every slot empty).
__global__ void k_init_root(BuildState* st, uint64_t* __restrict__ keys, int64_t cap) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < cap; e += (int64_t)gridDim.x * blockDim.x)
    keys[e] = kEmptyKey;
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    st->overflow = 0;
    st->n_tiles = 0;
    st->tile_list_count = 0;
    st->guard = 0;
    st->range = 0;
    st->cap_over = 0;
    st->sort_passes = 0;
    st->off_or = 0;
    st->off_and = ~0ull;
    st->key_or = 0;
    st->key_and = ~0ull;
    for (int c = 0; c < 4; ++c) st->counts[c] = 0;
    st->n_rec = 0;
  }
}

int grid_for(int64_t n, int threads, int cap) {
  int64_t b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (int)b;
}

int fill_u64(uint64_t* p, int64_t n, uint64_t v, hipStream_t s) {
  if (n <= 0) return IGC_OK;
  k_fill_u64<<<grid_for(n, 256, 4096), 256, 0, s>>>(p, n, v);
  IGC_HIP(hipGetLastError(), "igc_grid_build: fill kernel launch");
  return IGC_OK;
}

// ------------------------------------------------------------------------------ root tiles

// A key that is new to the table also goes to list[its insertion number] while that number is
// below list_cap, so that up to list_cap distinct tiles need no compaction pass.
__device__ void insert_tile(uint64_t* keys, uint32_t mask, uint32_t limit, uint64_t key, BuildState* st,
                            uint64_t* list, uint32_t list_cap) {
  uint32_t s = hash_tile(key) & mask;
  for (uint32_t p = 0; p < limit; ++p) {
    uint64_t cur = keys[s];  // cached read first; a stale empty slot is settled by the CAS
    if (cur != key && cur == kEmptyKey) cur = __hip_atomic_load(&keys[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (cur == key) return;
    if (cur == kEmptyKey) {
      const unsigned long long prev = atomicCAS((unsigned long long*)&keys[s], (unsigned long long)kEmptyKey,
                                                (unsigned long long)key);
      if (prev == kEmptyKey) {
        const uint32_t idx = atomicAdd(&st->n_tiles, 1u);
        if (idx < list_cap) list[idx] = key;
        return;
      }
      if (prev == key) return;
    }
    s = (s + 1) & mask;
  }
  atomicOr(&st->overflow, 1u);
}

// Tile pass: every workgroup collects the distinct tile keys of its coordinates in an LDS set
// (a wave first collapses equal keys with ballots) and inserts each of them into the global
// table once, at the end. The global table's slots therefore see one access per workgroup and
// distinct tile, not one per wave (same-address device atomics serialise). Keys that do not
// fit the LDS set go to the table directly. Also records OR / AND of keys and in-tile offsets.
__global__ __launch_bounds__(256) void k_tile_insert(const int32_t* __restrict__ ijk, int64_t n,
                                                     uint64_t* __restrict__ keys, uint32_t mask, uint32_t limit,
                                                     uint64_t* __restrict__ partial, BuildState* st,
                                                     uint64_t* __restrict__ list, uint32_t list_cap) {
  __shared__ uint64_t s_red[4][4];
  __shared__ uint64_t s_set[kTileCache];
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x < kTileCache) s_set[threadIdx.x] = kEmptyKey;
  __syncthreads();
  uint64_t off_or = 0, off_and = ~0ull, key_or = 0, key_and = ~0ull;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  constexpr int U4 = 4;  // coordinates in flight per thread
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < n; base += U4 * stride) {
    int32_t ci[U4], cj[U4], ck[U4];
#pragma unroll
    for (int u = 0; u < U4; ++u) {  // clamped, unconditional: all loads in flight before the first use
      const int64_t e = min(base + u * stride + threadIdx.x, n - 1);
      ci[u] = ijk[3 * e];
      cj[u] = ijk[3 * e + 1];
      ck[u] = ijk[3 * e + 2];
    }
#pragma unroll
    for (int u = 0; u < U4; ++u) {
      const int64_t e = base + u * stride + threadIdx.x;
      const bool valid = e < n;
      uint64_t key = kEmptyKey;
      if (valid) {
        key = tile_key(ci[u], cj[u], ck[u]);
        const uint64_t off = tile_offset(ci[u], cj[u], ck[u]);
        off_or |= off;
        off_and &= off;
        key_or |= key;
        key_and &= key;
      }
      // Keys already in the workgroup's cache need nothing more: each lane looks its own up
      // with plain LDS reads, and only the rest go through the per-key leader rounds.
      bool need = valid;
      if (valid) {
        const uint32_t h = hash_tile(key) & (kTileCache - 1);
        for (int p = 0; p < 8; ++p) {
          const uint64_t v = s_set[(h + p) & (kTileCache - 1)];
          if (v == key) {
            need = false;
            break;
          }
          if (v == kEmptyKey) break;
        }
      }
      uint64_t pending = __ballot(need);
      while (pending) {
        const int leader = __ffsll((unsigned long long)pending) - 1;
        const uint64_t lk = shfl64(key, leader);
        const uint64_t same = __ballot(need && key == lk);
        if (lane == leader) {
          const uint32_t h = hash_tile(lk) & (kTileCache - 1);
          bool placed = false;
          for (int p = 0; p < 8; ++p) {
            const unsigned long long prev = atomicCAS((unsigned long long*)&s_set[(h + p) & (kTileCache - 1)],
                                                      (unsigned long long)kEmptyKey, (unsigned long long)lk);
            if (prev == kEmptyKey || prev == lk) {
              placed = true;
              break;
            }
          }
          if (!placed) insert_tile(keys, mask, limit, lk, st, list, list_cap);
        }
        pending &= ~same;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < kTileCache && s_set[threadIdx.x] != kEmptyKey)
    insert_tile(keys, mask, limit, s_set[threadIdx.x], st, list, list_cap);
  off_or = wave_or64(off_or);
  off_and = wave_and64(off_and);
  key_or = wave_or64(key_or);
  key_and = wave_and64(key_and);
  if (lane == 0) {
    s_red[wave][0] = off_or;
    s_red[wave][1] = off_and;
    s_red[wave][2] = key_or;
    s_red[wave][3] = key_and;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) {
      off_or |= s_red[w][0];
      off_and &= s_red[w][1];
      key_or |= s_red[w][2];
      key_and &= s_red[w][3];
    }
    // Per-workgroup partials (same-address atomics from every workgroup would serialise).
    partial[4 * blockIdx.x + 0] = off_or;
    partial[4 * blockIdx.x + 1] = off_and;
    partial[4 * blockIdx.x + 2] = key_or;
    partial[4 * blockIdx.x + 3] = key_and;
  }
}

// OR / AND of the tile pass's per-workgroup partials into the state. One workgroup.
__global__ __launch_bounds__(256) void k_reduce_bits(const uint64_t* __restrict__ partial, int nb, BuildState* st,
                                                     BuildState* host) {
  __shared__ uint64_t s_red[4][4];
  uint64_t off_or = 0, off_and = ~0ull, key_or = 0, key_and = ~0ull;
  constexpr int R = 8;  // partials per thread and round, loaded before any is combined
  for (int b0 = threadIdx.x; b0 < nb; b0 += R * 256) {
    ulonglong2 v[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int b = min(b0 + r * 256, nb - 1);  // a repeated partial changes no OR / AND
      v[r][0] = reinterpret_cast<const ulonglong2*>(partial)[2 * b];
      v[r][1] = reinterpret_cast<const ulonglong2*>(partial)[2 * b + 1];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      off_or |= v[r][0].x;
      off_and &= v[r][0].y;
      key_or |= v[r][1].x;
      key_and &= v[r][1].y;
    }
  }
  off_or = wave_or64(off_or);
  off_and = wave_and64(off_and);
  key_or = wave_or64(key_or);
  key_and = wave_and64(key_and);
  const int wave = threadIdx.x >> 6;
  if (lane_id() == 0) {
    s_red[wave][0] = off_or;
    s_red[wave][1] = off_and;
    s_red[wave][2] = key_or;
    s_red[wave][3] = key_and;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) {
      off_or |= s_red[w][0];
      off_and &= s_red[w][1];
      key_or |= s_red[w][2];
      key_and &= s_red[w][3];
    }
    st->off_or = off_or;
    st->off_and = off_and;
    st->key_or = key_or;
    st->key_and = key_and;
    publish_state(st, host);
  }
}

__global__ void k_tile_compact(const uint64_t* __restrict__ keys, uint32_t cap, uint64_t* __restrict__ list,
                               uint32_t U, BuildState* st) {
  for (uint32_t s = blockIdx.x * blockDim.x + threadIdx.x; s < cap; s += gridDim.x * blockDim.x) {
    const uint64_t k = keys[s];
    if (k != kEmptyKey) {
      const uint32_t pos = atomicAdd(&st->tile_list_count, 1u);
      if (pos < U) list[pos] = k; else atomicOr(&st->guard, 1u);
    }
  }
}

// Bitonic sort of up to kSmallSort keys in LDS by one workgroup of 1024 threads (s holds the
// keys ascending afterwards, padded with kEmptyKey to a power of two).
__device__ __forceinline__ void bitonic_sort_lds(const uint64_t* __restrict__ in, uint64_t* s, int n) {
  int p2 = 2;
  while (p2 < n) p2 <<= 1;
  for (int t = threadIdx.x; t < p2; t += blockDim.x) s[t] = t < n ? in[t] : kEmptyKey;
  __syncthreads();
  for (int size = 2; size <= p2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < p2 / 2; t += blockDim.x) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = s[lo], b = s[hi];
        if ((a > b) == up) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Slot of tile key k (present by construction); flags the guard if it is missing.
__device__ __forceinline__ int64_t probe_slot(const uint64_t* __restrict__ keys, uint32_t mask, uint64_t k,
                                              BuildState* st) {
  uint32_t s = hash_tile(k) & mask;
  for (uint32_t p = 0; p <= mask; ++p) {
    if (keys[s] == k) return s;
    s = (s + 1) & mask;
  }
  atomicOr(&st->guard, 1u);
  return -1;
}

__global__ void k_tile_rank(const uint64_t* __restrict__ sorted, int64_t U, const uint64_t* __restrict__ keys,
                            int32_t* __restrict__ vals, uint32_t mask, BuildState* st) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < U; r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = probe_slot(keys, mask, sorted[r], st);
    if (s >= 0) vals[s] = (int32_t)r;
  }
}

// Up to kSmallSort tile keys: bitonic sort in one workgroup, then each key's rank into the
// table (the sort and the rank pass of larger tile sets in one launch).
// n < 0: the count is the state's tile count. When that exceeds ucap (or kSmallSort), or the
// table overflowed, the table is emptied (every later lookup then misses instead of returning
// a rank beyond the node arrays) and cap_over is set.
__global__ __launch_bounds__(1024) void k_sort_rank_small(const uint64_t* __restrict__ in, uint64_t* __restrict__ out,
                                                          int n, uint64_t* __restrict__ keys,
                                                          int32_t* __restrict__ vals, uint32_t mask, BuildState* st,
                                                          int64_t ucap) {
  __shared__ uint64_t s[kSmallSort];
  if (n < 0) {
    const uint32_t nt = st->n_tiles;
    if ((int64_t)nt > (ucap < kSmallSort ? ucap : kSmallSort) || st->overflow) {
      for (uint32_t t = threadIdx.x; t <= mask; t += blockDim.x) keys[t] = kEmptyKey;
      if (threadIdx.x == 0) atomicOr(&st->cap_over, 1u);
      return;
    }
    n = (int)nt;
  }
  bitonic_sort_lds(in, s, n);
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    const uint64_t k = s[t];
    out[t] = k;
    const int64_t slot = probe_slot(keys, mask, k, st);
    if (slot >= 0) vals[slot] = t;
  }
}

// ------------------------------------------------------------------------------ radix sort

struct PassSpec {
  int lo_bit;  // bit of digit 0
  int passes;  // number of digits
  int bits;    // bits per digit, 8..10 (digit p is bits [lo_bit + bits p, lo_bit + bits (p + 1)))
};

// The varying bits of the keys' leaf part (key2 >> 9) as runs of consecutive bits: the sort
// orders keys compacted to those bits ((leaf part gathered to the low bits) << 9 | voxel bits),
// which keeps their order and takes fewer digits. The sorted keys stay compacted; a key is
// expanded only where it starts a leaf.
struct BitRuns {
  int n;                             // 0: keys are sorted as they are
  uint8_t lo[16], len[16], pos[16];  // run i: bits [lo, lo + len) of the leaf part -> [pos, pos + len)
  uint64_t cbits;                    // bits of the leaf part that are the same in every key
};

// Runs are applied by a recursion over the fixed slot indices with a uniform exit: every
// run's fields sit at constant offsets of the kernel argument and are read as scalars once
// per wave (a loop over r.n leaves a remainder loop that reads them per key).
template <int I>
__device__ __forceinline__ void compress_from(uint64_t x, uint64_t& c, const BitRuns& r) {
  if constexpr (I < 16) {
    if (I < r.n) {
      c |= ((x >> r.lo[I]) & ((1ull << r.len[I]) - 1ull)) << r.pos[I];
      compress_from<I + 1>(x, c, r);
    }
  }
}

template <int I>
__device__ __forceinline__ void expand_from(uint64_t c, uint64_t& x, const BitRuns& r) {
  if constexpr (I < 16) {
    if (I < r.n) {
      x |= ((c >> r.pos[I]) & ((1ull << r.len[I]) - 1ull)) << r.lo[I];
      expand_from<I + 1>(c, x, r);
    }
  }
}

__device__ __forceinline__ uint64_t runs_compress(uint64_t key, const BitRuns& r) {
  uint64_t c = 0;
  compress_from<0>(key >> 9, c, r);
  return (c << 9) | (key & 511u);
}

__device__ __forceinline__ uint64_t runs_expand(uint64_t sk, const BitRuns& r) {
  uint64_t x = r.cbits;
  expand_from<0>(sk >> 9, x, r);
  return (x << 9) | (sk & 511u);
}

// Digits over the varying bits at or above min_bit: as few passes as digits of up to
// kMaxDigitBits allow, each digit as narrow as that pass count allows (at least 8 bits).
__host__ __device__ PassSpec pass_spec(uint64_t varying, int min_bit = 0) {
  PassSpec ps{0, 0, 8};
  if (min_bit > 0) varying &= ~((1ull << min_bit) - 1ull);
  if (!varying) return ps;
  const int lo = __builtin_ctzll(varying);
  const int hi = 63 - __builtin_clzll(varying);
  const int span = hi - lo + 1;
  ps.lo_bit = lo;
  ps.passes = (span + kMaxDigitBits - 1) / kMaxDigitBits;
  ps.bits = (span + ps.passes - 1) / ps.passes;
  if (ps.bits < 8) ps.bits = 8;
  // The key pass keeps passes * bins counters in LDS (at most kHistWidth).
  while ((ps.passes << ps.bits) > kHistWidth) {
    ++ps.passes;
    ps.bits = (span + ps.passes - 1) / ps.passes;
    if (ps.bits < 8) ps.bits = 8;
  }
  return ps;
}

// The shifts that leave a key's leaf / lower / upper part: 9 / 21 / 36 for whole keys, the
// compacted positions of those boundaries for compacted ones.
struct KeyForm {
  int cs_lower, cs_upper;
  BitRuns runs;  // runs.n > 0: keys are compacted
};

// How the keys of one build are sorted, from the OR / AND of the in-tile offsets and the tile
// count U: the leaf part of key2 (rank << 27 | upper child << 12 | lower child) is compacted to
// its varying bits when they form at most 16 runs, and only the digits over those bits are
// sorted. digit_bits > 0: digits of exactly that width (the counted build, whose passes are
// launched before the plan is known and skip themselves past `passes`).
struct SortPlan {
  KeyForm kf;
  PassSpec ps;
  int32_t span;  // sorted key bits (0: nothing to sort)
  int32_t shift[kMaxPasses];  // bit of pass p's digit, -1 past the last pass
};

__host__ __device__ inline SortPlan make_sort_plan(uint64_t off_or, uint64_t off_and, uint64_t U, int digit_bits) {
  SortPlan pl{};
  int rank_bits = 0;
  while (rank_bits < 27 && (1ull << rank_bits) < U) ++rank_bits;
  const uint64_t varying = (off_or ^ off_and) | (rank_bits ? (((1ull << rank_bits) - 1ull) << 36) : 0ull);
  BitRuns runs{};
  const uint64_t leaf_var = varying >> 9;
  if (leaf_var) {
    int pos = 0;
    for (int b = 0; b < 55 && runs.n <= 16;) {
      if (!((leaf_var >> b) & 1ull)) {
        ++b;
        continue;
      }
      int e = b;
      while (e < 55 && ((leaf_var >> e) & 1ull)) ++e;
      if (runs.n == 16) {
        runs.n = 17;
        break;
      }
      runs.lo[runs.n] = (uint8_t)b;
      runs.len[runs.n] = (uint8_t)(e - b);
      runs.pos[runs.n] = (uint8_t)pos;
      ++runs.n;
      pos += e - b;
      b = e;
    }
    if (runs.n > 16 || (runs.n == 1 && runs.lo[0] == 0)) runs.n = 0;  // too fragmented, or already compact
    else runs.cbits = (off_and >> 9) & ~leaf_var;
  }
  const uint64_t sort_var = runs.n ? (((1ull << __builtin_popcountll(leaf_var)) - 1ull) << 9) : varying;
  PassSpec ps = pass_spec(sort_var, 9);
  if (ps.passes > 0) {
    const int lo = ps.lo_bit, hi = 63 - __builtin_clzll(sort_var & ~((1ull << 9) - 1ull));
    pl.span = hi - lo + 1;
    if (digit_bits > 0) {
      ps.bits = digit_bits;
      ps.passes = (pl.span + digit_bits - 1) / digit_bits;
    }
  }
  if (ps.passes == 0) runs.n = 0;
  pl.kf.cs_lower = 21;
  pl.kf.cs_upper = 36;
  pl.kf.runs = runs;
  if (runs.n) {
    pl.kf.cs_lower = 9 + __builtin_popcountll(leaf_var & 0xFFFull);
    pl.kf.cs_upper = 9 + __builtin_popcountll(leaf_var & ((1ull << 27) - 1ull));
  }
  pl.ps = ps;
  for (int p = 0; p < kMaxPasses; ++p) pl.shift[p] = p < ps.passes ? ps.lo_bit + ps.bits * p : -1;
  return pl;
}

// The counted build sorts with digits of 8 or 9 bits, chosen on the host before the key span is
// known (5 passes cover the <= 12 rank and 27 leaf-part bits of up to 4096 tiles either way).
constexpr int kCountedPasses = 5;

// The counted build's plan, from the tile pass's state (one thread).
__global__ void k_make_plan(BuildState* st, SortPlan* plan, int digit_bits) {
  if (threadIdx.x != 0) return;
  const uint64_t U = st->n_tiles <= (uint32_t)kSmallSort ? st->n_tiles : 1u;
  const SortPlan pl = make_sort_plan(st->off_or, st->off_and, U, digit_bits);
  *plan = pl;
  st->sort_passes = (uint32_t)pl.ps.passes;
  st->sort_span = (uint32_t)pl.span;
}

// LDS histograms of every pass digit (one copy per workgroup), merged into the global ones.
__device__ __forceinline__ void hist_add(uint32_t* s_hist, uint64_t key, PassSpec ps) {
  const uint32_t bins = 1u << ps.bits;
  for (int p = 0; p < ps.passes; ++p) {
    const uint32_t d = (uint32_t)(key >> (ps.lo_bit + ps.bits * p)) & (bins - 1u);
    atomicAdd(&s_hist[p * bins + d], 1u);
  }
}

// Writes this workgroup's histograms to its row of `part` ([blocks][passes * bins]).
__device__ __forceinline__ void hist_flush(const uint32_t* s_hist, uint32_t* part, PassSpec ps, int width = 0) {
  __syncthreads();
  if (width <= 0) width = ps.passes << ps.bits;
  uint32_t* row = part + (size_t)blockIdx.x * width;
  for (int x = threadIdx.x; x < width; x += blockDim.x) row[x] = s_hist[x];
}

// hist[x] = sum over workgroups b of part[b][x]. A workgroup owns 16 columns; its 16 row
// slices of 16 threads sum interleaved rows, then combine in LDS.
__global__ __launch_bounds__(256) void k_hist_reduce(const uint32_t* __restrict__ part, int nb, int width,
                                                     uint32_t* __restrict__ hist) {
  __shared__ uint32_t s_sum[16][16];
  const int cl = threadIdx.x & 15, slice = threadIdx.x >> 4;
  const int col = blockIdx.x * 16 + cl;
  constexpr int R = 16;  // rows per thread and round, all loaded before any is added
  uint32_t acc = 0;
  if (col < width) {
    int b = slice;
    for (; b + 16 * (R - 1) < nb; b += 16 * R) {
      uint32_t v[R];
#pragma unroll
      for (int u = 0; u < R; ++u) v[u] = part[(size_t)(b + 16 * u) * width + col];
#pragma unroll
      for (int u = 0; u < R; ++u) acc += v[u];
    }
    for (; b < nb; b += 16) acc += part[(size_t)b * width + col];
  }
  s_sum[slice][cl] = acc;
  __syncthreads();
  if (slice == 0 && col < width) {
    uint32_t t = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += s_sum[k][cl];
    hist[col] = t;
  }
}

// key2 for every coordinate, plus the digit histograms of every sort pass. When there are at
// most kRootInLds tiles, ranks come from a binary search of the sorted tile list in LDS;
// otherwise from the global root table.
__global__ __launch_bounds__(256) void k_key2(const int32_t* __restrict__ ijk, int64_t n,
                                              const uint64_t* __restrict__ root_keys,
                                              const int32_t* __restrict__ root_vals, uint32_t mask,
                                              const uint64_t* __restrict__ tiles, int64_t U,
                                              uint64_t* __restrict__ out, PassSpec ps, BitRuns runs,
                                              uint32_t* __restrict__ hist, BuildState* st,
                                              const SortPlan* plan = nullptr, int hist_width = 0,
                                              uint64_t* __restrict__ out_odd = nullptr) {
  __shared__ uint32_t s_hist[kHistWidth];
  __shared__ uint64_t s_tiles[kRootInLds];
  // Counted build: the plan, the tile count and the output buffer come from the device (keys go
  // where the first radix pass reads them); a build whose tile step failed writes zero keys.
  bool dead = false;
  if (plan) {
    ps = plan->ps;
    runs = plan->kf.runs;
    U = (int64_t)st->n_tiles;
    dead = st->cap_over != 0u || st->overflow != 0u || U > kSmallSort;
    if (dead) U = 0;
    if (ps.passes & 1) out = out_odd;
  }
  const int width = hist_width > 0 ? hist_width : (ps.passes << ps.bits);
  for (int x = threadIdx.x; x < width; x += blockDim.x) s_hist[x] = 0;
  const bool local = U <= kRootInLds;
  if (local)
    for (int x = threadIdx.x; x < U; x += blockDim.x) s_tiles[x] = tiles[x];
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  constexpr int U4 = 4;  // coordinates in flight per thread
  for (int64_t e0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e0 < n; e0 += U4 * stride) {
   int32_t ci[U4], cj[U4], ck[U4];
#pragma unroll
   for (int u = 0; u < U4; ++u) {  // clamped, unconditional: all loads in flight before the first use
     const int64_t e = min(e0 + u * stride, n - 1);
     ci[u] = ijk[3 * e];
     cj[u] = ijk[3 * e + 1];
     ck[u] = ijk[3 * e + 2];
   }
#pragma unroll
   for (int u = 0; u < U4; ++u) {
    const int64_t e = e0 + u * stride;
    if (e >= n) break;
    const int32_t i = ci[u], j = cj[u], k = ck[u];
    const uint64_t tk = tile_key(i, j, k);
    uint64_t rank = 0;
    if (dead) {
      out[e] = 0ull;
      hist_add(s_hist, 0ull, ps);
      continue;
    }
    if (local) {
      int lo = 0, hi = (int)U - 1;  // s_tiles is ascending and holds tk
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_tiles[mid] < tk) lo = mid + 1; else hi = mid;
      }
      rank = (uint64_t)lo;
    } else {
      const int64_t s = probe_slot(root_keys, mask, tk, st);
      rank = s >= 0 ? (uint64_t)(uint32_t)root_vals[s] : 0ull;
    }
    uint64_t key = (rank << 36) | tile_offset(i, j, k);
    if (runs.n) key = runs_compress(key, runs);
    out[e] = key;
    hist_add(s_hist, key, ps);
   }
  }
  hist_flush(s_hist, hist, ps, width);
}

// Digit histograms of an existing key array (used for the tile-key sort when U is large).
__global__ __launch_bounds__(256) void k_hist(const uint64_t* __restrict__ keys, int64_t n, PassSpec ps,
                                              uint32_t* __restrict__ hist) {
  __shared__ uint32_t s_hist[kHistWidth];
  for (int x = threadIdx.x; x < (ps.passes << ps.bits); x += blockDim.x) s_hist[x] = 0;
  __syncthreads();
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
    hist_add(s_hist, keys[e], ps);
  hist_flush(s_hist, hist, ps);
}

// One LSD pass over the BITS-bit digit at `shift` runs as three kernels over tiles of
// kSortTile keys (reduce-then-scan): per-tile digit counts, a scan of every digit's counts
// over the tiles, and a stable scatter that ranks the tile's keys with 64-lane ballots, sorts
// them in LDS and writes them out in per-digit runs.

// Stable rank of every key among the equal digits of its wave (wave w owns the tile's keys
// [w*64*kSortKPT, (w+1)*64*kSortKPT), 64 consecutive keys per round): the lanes holding the
// same digit are found with BITS ballots, and the first of them adds their number to the
// wave's count of that digit, so no two lanes update one counter in the same round.
// STABLE = false (the first pass of a sort): ranks come from one LDS atomic add per key, in
// whatever order the adds land. An LSD sort needs only its later passes to keep the order of
// equal digits; the first pass has no earlier order to keep.
template <int BITS, bool STABLE>
__device__ __forceinline__ void rank_keys(const uint64_t* __restrict__ src, int64_t n, int64_t wbase, int shift,
                                          uint64_t* key, uint32_t* rank, uint32_t* cnt) {
  const int lane = lane_id();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kSortKPT; ++r) key[r] = wbase + r * 64 < n ? src[wbase + r * 64] : 0ull;
  if constexpr (!STABLE) {
#pragma unroll
    for (int r = 0; r < kSortKPT; ++r) {
      const uint32_t d = (uint32_t)(key[r] >> shift) & ((1u << BITS) - 1u);
      rank[r] = wbase + r * 64 < n ? atomicAdd(&cnt[d], 1u) : 0u;
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < kSortKPT; ++r) {
    const bool valid = wbase + r * 64 < n;
    const uint32_t d = (uint32_t)(key[r] >> shift) & ((1u << BITS) - 1u);
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
      const bool set = (d >> b) & 1u;
      const uint64_t bb = __ballot(set);
      m &= set ? bb : ~bb;
    }
    const uint32_t before = (uint32_t)__popcll(m & lt_mask);
    uint32_t old = 0;
    if (valid) old = cnt[d];
    if (valid && before == 0) cnt[d] = old + (uint32_t)__popcll(m);
    rank[r] = old + before;
  }
}

// Step 1: cnt[d * T + tile] = keys of the tile with digit d, counted with LDS atomics into
// one histogram per wave (only the counts are needed here, not the ranks).
template <int BITS>
__global__ __launch_bounds__(kThreads) void k_radix_hist(const uint64_t* __restrict__ src, int64_t n, int shift,
                                                         uint32_t* __restrict__ cnt, int64_t T, const uint64_t* dn,
                                                         const SortPlan* plan, int pass, const uint64_t* alt) {
  if (dn && (int64_t)*dn < n) n = (int64_t)*dn;
  if (plan) {  // counted build: pass `pass` of plan->ps.passes reads buffer (passes - pass) & 1
    if (pass >= plan->ps.passes) return;
    shift = plan->shift[pass];
    if ((plan->ps.passes - pass) & 1) src = alt;
  }
  constexpr int D = 1 << BITS;
  __shared__ uint32_t s_cnt[4][D];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int x = tid; x < 4 * D; x += kThreads) (&s_cnt[0][0])[x] = 0;
  __syncthreads();
  const int64_t tile = blockIdx.x;
  const int64_t wbase = tile * kSortTile + wave * (64 * kSortKPT) + lane_id();
  uint64_t key[kSortKPT];
#pragma unroll
  for (int r = 0; r < kSortKPT; ++r) key[r] = wbase + r * 64 < n ? src[wbase + r * 64] : 0ull;
#pragma unroll
  for (int r = 0; r < kSortKPT; ++r)
    if (wbase + r * 64 < n) atomicAdd(&s_cnt[wave][(uint32_t)(key[r] >> shift) & (D - 1u)], 1u);
  __syncthreads();
  for (int d = tid; d < D; d += kThreads) cnt[(int64_t)d * T + tile] = s_cnt[0][d] + s_cnt[1][d] + s_cnt[2][d] + s_cnt[3][d];
}

// Step 2, one workgroup per digit d: off[d * T + t] = (keys whose digit is below d) +
// (keys with digit d in tiles before t). hist holds the pass's digit counts over all keys.
__global__ __launch_bounds__(kThreads) void k_radix_scan(const uint32_t* __restrict__ cnt, int64_t T,
                                                         const uint32_t* __restrict__ hist, uint32_t* __restrict__ off,
                                                         const SortPlan* plan, int pass) {
  if (plan && pass >= plan->ps.passes) return;
  __shared__ uint64_t s_tmp[kThreads / 64];
  const int d = blockIdx.x, tid = threadIdx.x;
  uint64_t below = 0;
  for (int x = tid; x < d; x += kThreads) below += hist[x];
  uint64_t carry = 0;
  block_excl_scan64<kThreads>(below, s_tmp, &carry);
  for (int64_t b = 0; b < T; b += kThreads) {
    const int64_t t = b + tid;
    const uint64_t c = t < T ? (uint64_t)cnt[(int64_t)d * T + t] : 0ull;
    uint64_t sum = 0;
    const uint64_t ex = block_excl_scan64<kThreads>(c, s_tmp, &sum);
    if (t < T) off[(int64_t)d * T + t] = (uint32_t)(carry + ex);
    carry += sum;
  }
}

// Step 3: stable scatter of one tile to its digits' runs. Thread tid owns the J consecutive
// digits [tid J, tid J + J).
template <int BITS, bool STABLE>
__global__ __launch_bounds__(kThreads) void k_radix_scatter(const uint64_t* __restrict__ src,
                                                            uint64_t* __restrict__ dst, int64_t n, int shift,
                                                            const uint32_t* __restrict__ off, int64_t T,
                                                            uint32_t* guard, const uint64_t* dn,
                                                            const SortPlan* plan, int pass) {
  if (dn && (int64_t)*dn < n) n = (int64_t)*dn;
  if (plan) {
    if (pass >= plan->ps.passes) return;
    shift = plan->shift[pass];
    if ((plan->ps.passes - pass) & 1) {
      uint64_t* t = (uint64_t*)src;
      src = dst;
      dst = t;
    }
  }
  constexpr int D = 1 << BITS, J = D / kThreads;
  __shared__ uint64_t s_keys[kSortTile];
  __shared__ uint32_t s_cnt[4][D];
  __shared__ uint32_t s_tile_start[D];
  __shared__ int64_t s_base[D];
  __shared__ uint64_t s_tmp[kThreads / 64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int64_t tile = blockIdx.x;
  const int64_t tile_base = tile * kSortTile;
  uint32_t goff[J];  // in flight during the ranking
#pragma unroll
  for (int j = 0; j < J; ++j) goff[j] = off[(int64_t)(tid * J + j) * T + tile];
  for (int x = tid; x < 4 * D; x += kThreads) (&s_cnt[0][0])[x] = 0;
  __syncthreads();
  uint64_t key[kSortKPT];
  uint32_t rank[kSortKPT];
  const int64_t wbase = tile_base + wave * (64 * kSortKPT) + lane_id();
  rank_keys<BITS, STABLE>(src, n, wbase, shift, key, rank, s_cnt[wave]);
  __syncthreads();

  // Tile counts of the owned digits, per-wave exclusive offsets and the tile scan.
  uint32_t c[J][4], tot[J], mine = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int d = tid * J + j;
#pragma unroll
    for (int w = 0; w < 4; ++w) c[j][w] = s_cnt[w][d];
    tot[j] = c[j][0] + c[j][1] + c[j][2] + c[j][3];
    mine += tot[j];
  }
  uint32_t tstart = (uint32_t)block_excl_scan64<kThreads>(mine, s_tmp, nullptr);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int d = tid * J + j;
    s_cnt[0][d] = 0;
    s_cnt[1][d] = c[j][0];
    s_cnt[2][d] = c[j][0] + c[j][1];
    s_cnt[3][d] = c[j][0] + c[j][1] + c[j][2];
    s_tile_start[d] = tstart;
    s_base[d] = (int64_t)goff[j] - (int64_t)tstart;
    tstart += tot[j];
  }
  __syncthreads();

  // Digit-sorted order inside the tile, staged in LDS, then written out in per-digit runs.
#pragma unroll
  for (int r = 0; r < kSortKPT; ++r) {
    if (wbase + r * 64 < n) {
      const uint32_t dd = (uint32_t)(key[r] >> shift) & (D - 1u);
      s_keys[s_tile_start[dd] + s_cnt[wave][dd] + rank[r]] = key[r];
    }
  }
  __syncthreads();
  const int64_t valid_count = n - tile_base < kSortTile ? n - tile_base : kSortTile;
#pragma unroll
  for (int q = 0; q < kSortKPT; ++q) {
    const int p = q * kThreads + tid;
    if (p < valid_count) {
      const uint64_t k = s_keys[p];
      const int64_t gp = s_base[(uint32_t)(k >> shift) & (D - 1u)] + p;
      if (gp >= 0 && gp < n) dst[gp] = k; else atomicOr(guard, 1u);
    }
  }
}

template <int BITS>
void radix_pass(const uint64_t* src, uint64_t* dst, int64_t n, int shift, const uint32_t* hist, uint32_t* cnt,
                uint32_t* off, int64_t tiles, uint32_t* guard, bool first, hipStream_t s, const uint64_t* dn,
                const SortPlan* plan = nullptr, int pass = 0) {
  k_radix_hist<BITS><<<(unsigned)tiles, kThreads, 0, s>>>(src, n, shift, cnt, tiles, dn, plan, pass, dst);
  k_radix_scan<<<1u << BITS, kThreads, 0, s>>>(cnt, tiles, hist, off, plan, pass);
  if (first)
    k_radix_scatter<BITS, false><<<(unsigned)tiles, kThreads, 0, s>>>(src, dst, n, shift, off, tiles, guard, dn, plan,
                                                                      pass);
  else
    k_radix_scatter<BITS, true><<<(unsigned)tiles, kThreads, 0, s>>>(src, dst, n, shift, off, tiles, guard, dn, plan,
                                                                     pass);
}

// Sorts keys[0..n) (in a, scratch b) over the digits of ps; returns the buffer holding the
// result. hist holds the digit counts of every pass ([passes][bins]); cnt and off hold
// kMaxBins * cap_tiles words each. Compacted keys stay compacted. dn (device, may be null):
// only keys below *dn are sorted (hist must count exactly those).
int radix_sort(uint64_t* a, uint64_t* b, int64_t n, PassSpec ps, const uint32_t* hist, uint32_t* cnt, uint32_t* off,
               int64_t cap_tiles, uint32_t* guard, hipStream_t s, uint64_t** result, const uint64_t* dn = nullptr) {
  *result = a;
  if (n <= 0 || ps.passes == 0) return IGC_OK;
  const int64_t tiles = (n + kSortTile - 1) / kSortTile;
  if (tiles > cap_tiles || ps.passes > kMaxPasses || ps.bits < 8 || ps.bits > kMaxDigitBits)
    return set_error(IGC_ERR_INTERNAL, "igc_grid_build: radix sort workspace too small");
  uint64_t* src = a;
  uint64_t* dst = b;
  for (int p = 0; p < ps.passes; ++p) {
    const int shift = ps.lo_bit + ps.bits * p;
    const uint32_t* hp = hist + ((size_t)p << ps.bits);
    if (ps.bits == 8) radix_pass<8>(src, dst, n, shift, hp, cnt, off, tiles, guard, p == 0, s, dn);
    else radix_pass<9>(src, dst, n, shift, hp, cnt, off, tiles, guard, p == 0, s, dn);
    IGC_HIP(hipGetLastError(), "igc_grid_build: radix pass launch");
    std::swap(src, dst);
  }
  *result = src;
  return IGC_OK;
}

// ------------------------------------------------------------------------------ counting

// Block b counts, among keys [b*4096, (b+1)*4096), those that start a new voxel, leaf, lower
// node and upper node, packed in the 16-bit fields 0..3 of one 64-bit word (duplicate
// coordinates have equal keys, so voxel starts count the unique voxels).
__device__ __forceinline__ uint64_t start_flags(uint64_t key, uint64_t prev, bool first, int cs_lower, int cs_upper) {
  if (first) return 0x0001000100010001ull;
  return (uint64_t)(key != prev) | ((uint64_t)((key >> 9) != (prev >> 9)) << 16) |
         ((uint64_t)((key >> cs_lower) != (prev >> cs_lower)) << 32) |
         ((uint64_t)((key >> cs_upper) != (prev >> cs_upper)) << 48);
}

// A block's keys sit in LDS with one pad entry after every 16: each thread then reads its 16
// consecutive keys at a lane stride of 17 entries, which spreads a wave over the banks (a
// stride of 16 entries, 128 bytes, puts every lane on the same bank).
constexpr int kPaddedKeys = kTileKeys + kTileKeys / 16;
__device__ __forceinline__ int kpad(int p) { return p + (p >> 4); }

__device__ __forceinline__ void stage_block(const uint64_t* __restrict__ keys, int64_t n, int64_t base,
                                            uint64_t* s_keys, uint64_t* s_prev) {
  uint64_t v[kKeysPerThread];  // every load issued before the first LDS store waits on one
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q) v[q] = keys[min(base + q * kThreads + threadIdx.x, n - 1)];
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q) {
    const int p = q * kThreads + threadIdx.x;
    if (base + p < n) s_keys[kpad(p)] = v[q];
  }
  if (threadIdx.x == 0) *s_prev = base > 0 ? keys[base - 1] : 0ull;
  __syncthreads();
}

__global__ __launch_bounds__(256) void k_count(const uint64_t* __restrict__ keys, int64_t n,
                                               uint64_t* __restrict__ block_counts, int cs_lower, int cs_upper,
                                               const SortPlan* plan = nullptr) {
  __shared__ uint64_t s_keys[kPaddedKeys];
  __shared__ uint64_t s_prev;
  if (plan) {
    cs_lower = plan->kf.cs_lower;
    cs_upper = plan->kf.cs_upper;
  }
  __shared__ uint64_t s_tmp[4];
  const int64_t base = (int64_t)blockIdx.x * kTileKeys;
  stage_block(keys, n, base, s_keys, &s_prev);
  uint64_t c = 0;
  for (int q = 0; q < kKeysPerThread; ++q) {
    const int p = threadIdx.x * kKeysPerThread + q;
    const int64_t e = base + p;
    if (e < n) c += start_flags(s_keys[kpad(p)], p ? s_keys[kpad(p - 1)] : s_prev, e == 0, cs_lower, cs_upper);
  }
  uint64_t total;
  block_excl_scan64<kThreads>(c, s_tmp, &total);
  if (threadIdx.x == 0) block_counts[blockIdx.x] = total;
}

// Exclusive scan of the per-block packed counts into 64-bit prefixes per block, and the totals
// N, F, Lw, U. One workgroup.
__global__ __launch_bounds__(1024) void k_scan_blocks(const uint64_t* __restrict__ block_counts, int64_t nb,
                                                      uint64_t* __restrict__ prefix, BuildState* st,
                                                      BuildState* host) {
  __shared__ uint64_t s_tmp[16];
  const int64_t per = (nb + 1023) / 1024;
  const int64_t b0 = threadIdx.x * per;
  uint64_t run[4] = {0, 0, 0, 0};
  for (int64_t b = b0; b < b0 + per && b < nb; ++b)
    for (int c = 0; c < 4; ++c) run[c] += (block_counts[b] >> (16 * c)) & 0xFFFFull;
  uint64_t excl[4] = {0, 0, 0, 0}, tot[4] = {0, 0, 0, 0};
  for (int c = 0; c < 4; ++c) excl[c] = block_excl_scan64<1024>(run[c], s_tmp, &tot[c]);
  for (int64_t b = b0; b < b0 + per && b < nb; ++b)
    for (int c = 0; c < 4; ++c) {
      prefix[b * 4 + c] = excl[c];
      excl[c] += (block_counts[b] >> (16 * c)) & 0xFFFFull;
    }
  if (threadIdx.x == 0) {
    for (int c = 0; c < 4; ++c) st->counts[c] = tot[c];
    publish_state(st, host);
  }
}

// ------------------------------------------------------------------------------ registration

struct Topo {
  int64_t n_leaf, n_lower, n_upper;  // allocation sizes (bounds checks)
  uint32_t* guard;
  uint32_t* cap_over;  // a row past an allocation size (sizes from an estimate: the build is repeated)
  const uint64_t* tiles;  // [U] tile keys in rank order
  uint64_t* root_list;
  int4* upper_origin;
  uint64_t* upper_mask;
  uint32_t* upper_first;
  int4* lower_origin;
  uint64_t* lower_mask;
  uint32_t* lower_first;
  LeafRec* leaf;
  int4* leaf_origin;
};

__device__ __forceinline__ int4 key_origin(uint64_t key, uint64_t tile, uint32_t clear_bits) {
  const uint32_t up = (uint32_t)(key >> 21) & 0x7FFFu;
  const uint32_t lo = (uint32_t)(key >> 9) & 0xFFFu;
  const uint32_t lf = (uint32_t)key & 511u;
  const uint32_t i = ((uint32_t)(tile >> 42) << 12) | ((up >> 10) << 7) | ((lo >> 8) << 3) | (lf >> 6);
  const uint32_t j = ((uint32_t)((tile >> 21) & 0xFFFFFu) << 12) | (((up >> 5) & 31u) << 7) | (((lo >> 4) & 15u) << 3) |
                     ((lf >> 3) & 7u);
  const uint32_t k = ((uint32_t)(tile & 0xFFFFFu) << 12) | ((up & 31u) << 7) | ((lo & 15u) << 3) | (lf & 7u);
  const uint32_t m = ~((1u << clear_bits) - 1u);
  return make_int4((int32_t)(i & m), (int32_t)(j & m), (int32_t)(k & m), 0);
}

constexpr int kLeafCache = 64;  // leaves of a block whose masks are merged in LDS

__global__ __launch_bounds__(256) void k_register(const uint64_t* __restrict__ keys, int64_t n,
                                                  const uint64_t* __restrict__ prefix, Topo t, KeyForm kf,
                                                  const SortPlan* plan = nullptr) {
  if (plan) kf = plan->kf;
  __shared__ uint64_t s_keys[kPaddedKeys];
  __shared__ uint64_t s_prev;
  __shared__ uint64_t s_tmp[4];
  __shared__ uint64_t s_lmask[kLeafCache][8];
  for (int x = threadIdx.x; x < kLeafCache * 8; x += kThreads) (&s_lmask[0][0])[x] = 0;
  const int64_t base = (int64_t)blockIdx.x * kTileKeys;
  stage_block(keys, n, base, s_keys, &s_prev);
  const int p0 = threadIdx.x * kKeysPerThread;
  uint64_t c = 0;
  for (int q = 0; q < kKeysPerThread; ++q) {
    const int64_t e = base + p0 + q;
    if (e < n)
      c += start_flags(s_keys[kpad(p0 + q)], (p0 + q) ? s_keys[kpad(p0 + q - 1)] : s_prev, e == 0, kf.cs_lower,
                       kf.cs_upper);
  }
  uint64_t total;
  const uint64_t excl = block_excl_scan64<kThreads>(c, s_tmp, &total);
  // Running inclusive counts; ids are count - 1.
  const int64_t pf = (int64_t)prefix[blockIdx.x * 4 + 1];
  int64_t nf = pf + (int64_t)((excl >> 16) & 0xFFFF);
  int64_t nl = (int64_t)prefix[blockIdx.x * 4 + 2] + (int64_t)((excl >> 32) & 0xFFFF);
  int64_t nu = (int64_t)prefix[blockIdx.x * 4 + 3] + (int64_t)((excl >> 48) & 0xFFFF);
  // Leaves of the block's first and last key; the leaves between them lie inside the block.
  const bool first_starts = base == 0 || (s_keys[0] >> 9) != (s_prev >> 9);
  const int64_t lf0 = pf + (first_starts ? 1 : 0) - 1;
  const int64_t lf1 = pf + (int64_t)((total >> 16) & 0xFFFF) - 1;

  int64_t run_word = -1;  // leaf * 8 + word of the pending mask bits (leaves past the LDS cache)
  uint64_t run_bits = 0;
  for (int q = 0; q < kKeysPerThread; ++q) {
    const int64_t e = base + p0 + q;
    if (e >= n) break;
    const uint64_t key = s_keys[kpad(p0 + q)];
    const uint64_t f =
        start_flags(key, (p0 + q) ? s_keys[kpad(p0 + q - 1)] : s_prev, e == 0, kf.cs_lower, kf.cs_upper);
    nf += (int64_t)((f >> 16) & 1);
    nl += (int64_t)((f >> 32) & 1);
    nu += (int64_t)((f >> 48) & 1);
    const int64_t lf = nf - 1, lw = nl - 1, u = nu - 1;
    if (lf < lf0) {
      atomicOr(t.guard, 1u);
      break;
    }
    if (lf >= t.n_leaf || lw >= t.n_lower || u >= t.n_upper) {
      atomicOr(t.cap_over, 1u);
      break;
    }
    if (f & 0x0001000100010000ull) {  // starts a leaf (and maybe its lower / upper node): expanded, tile read, only here
      const uint64_t key = kf.runs.n ? runs_expand(s_keys[kpad(p0 + q)], kf.runs) : s_keys[kpad(p0 + q)];
      if ((int64_t)(key >> 36) >= t.n_upper) {
        atomicOr(t.cap_over, 1u);
        break;
      }
      const uint64_t tile = t.tiles[key >> 36];
      if ((f >> 48) & 1) {
        t.root_list[u] = tile;
        t.upper_origin[u] = key_origin(key, tile, 12);
        t.upper_first[u] = (uint32_t)lw;
      }
      if ((f >> 32) & 1) {
        const uint32_t cu = (uint32_t)(key >> 21) & 0x7FFFu;
        atomicOr((unsigned long long*)&t.upper_mask[u * 512 + (cu >> 6)], 1ull << (cu & 63u));
        t.lower_origin[lw] = key_origin(key, tile, 7);
        t.lower_first[lw] = (uint32_t)lf;
      }
      if ((f >> 16) & 1) {
        const uint32_t cl = (uint32_t)(key >> 9) & 0xFFFu;
        atomicOr((unsigned long long*)&t.lower_mask[lw * 64 + (cl >> 6)], 1ull << (cl & 63u));
        t.leaf_origin[lf] = key_origin(key, tile, 3);
      }
    }
    const uint32_t vox = (uint32_t)key & 511u;
    if (lf - lf0 < kLeafCache) {
      atomicOr((unsigned long long*)&s_lmask[lf - lf0][vox >> 6], 1ull << (vox & 63u));
      continue;
    }
    const int64_t word = lf * 8 + (vox >> 6);
    if (word != run_word) {
      if (run_word >= 0) atomicOr((unsigned long long*)&t.leaf[run_word >> 3].mask[run_word & 7], run_bits);
      run_word = word;
      run_bits = 0;
    }
    run_bits |= 1ull << (vox & 63u);
  }
  if (run_word >= 0) atomicOr((unsigned long long*)&t.leaf[run_word >> 3].mask[run_word & 7], run_bits);
  __syncthreads();
  // The block owns the masks of its inner leaves whole; its first and last leaf may have keys
  // in the neighbouring blocks.
  const int64_t nloc = lf1 - lf0 + 1 < kLeafCache ? lf1 - lf0 + 1 : kLeafCache;
  for (int x = threadIdx.x; x < nloc * 8; x += kThreads) {
    const int slot = x >> 3, w = x & 7;
    const int64_t lf = lf0 + slot;
    if (lf < 0) {
      atomicOr(t.guard, 1u);
      continue;
    }
    if (lf >= t.n_leaf) {
      atomicOr(t.cap_over, 1u);
      continue;
    }
    const uint64_t v = s_lmask[slot][w];
    if (slot == 0 || lf == lf1) {
      if (v) atomicOr((unsigned long long*)&t.leaf[lf].mask[w], v);
    } else {
      t.leaf[lf].mask[w] = v;
    }
  }
}

// Voxel rows of the leaves: per leaf the packed 9-bit prefix counts of its mask words and its
// popcount; the exclusive voxel count of the leaf within its group of kLeafGroup leaves goes
// to offset, the group's total to group_sum (a scan over the groups and k_leaf_offset finish
// the rows).
constexpr int kLeafPer = 4;                       // leaves per thread
constexpr int kLeafGroup = 256 * kLeafPer;        // leaves per workgroup
__global__ __launch_bounds__(256) void k_leaf_count(LeafRec* __restrict__ leaf, int64_t F,
                                                    uint64_t* __restrict__ group_sum, const uint64_t* dcnt) {
  __shared__ uint64_t s_tmp[4];
  if (dcnt && (int64_t)dcnt[1] < F) F = (int64_t)dcnt[1];
  const int64_t f0 = (int64_t)blockIdx.x * kLeafGroup + (int64_t)threadIdx.x * kLeafPer;
  uint32_t cnt[kLeafPer];
  uint64_t tsum = 0;
#pragma unroll
  for (int q = 0; q < kLeafPer; ++q) {
    const int64_t f = f0 + q;
    cnt[q] = 0;
    if (f < F) {
      uint64_t packed = 0, run = 0;
      for (int w = 0; w < 8; ++w) {
        if (w) packed |= run << (9 * (w - 1));
        run += (uint64_t)__popcll(leaf[f].mask[w]);
      }
      leaf[f].prefix = packed;
      cnt[q] = (uint32_t)run;
    }
    tsum += cnt[q];
  }
  uint64_t total;
  uint64_t run = block_excl_scan64<256>(tsum, s_tmp, &total);
#pragma unroll
  for (int q = 0; q < kLeafPer; ++q) {
    const int64_t f = f0 + q;
    if (f < F) leaf[f].offset = run;
    run += cnt[q];
  }
  if (threadIdx.x == 0) group_sum[blockIdx.x] = total;
}

// In-place exclusive scan of v[0..nb); the total is the voxel count N. One workgroup.
__global__ __launch_bounds__(1024) void k_scan_groups(uint64_t* __restrict__ v, int64_t nb, BuildState* st,
                                                      BuildState* host) {
  __shared__ uint64_t s_tmp[16];
  uint64_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += 1024) {
    const int64_t b = b0 + threadIdx.x;
    const uint64_t x = b < nb ? v[b] : 0ull;
    uint64_t tot;
    const uint64_t ex = block_excl_scan64<1024>(x, s_tmp, &tot);
    if (b < nb) v[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    st->counts[0] = carry;
    publish_state(st, host);
  }
}

__global__ __launch_bounds__(256) void k_leaf_offset(LeafRec* __restrict__ leaf, int64_t F,
                                                     const uint64_t* __restrict__ group_pre, const uint64_t* dcnt) {
  if (dcnt && (int64_t)dcnt[1] < F) F = (int64_t)dcnt[1];
  const uint64_t add = group_pre[blockIdx.x];
  const int64_t f0 = (int64_t)blockIdx.x * kLeafGroup + (int64_t)threadIdx.x * kLeafPer;
#pragma unroll
  for (int q = 0; q < kLeafPer; ++q)
    if (f0 + q < F) leaf[f0 + q].offset += add;
}

// Per-word prefix counts of internal-node child masks: one wave per node, lower nodes (64
// words) in the first nbl workgroups and upper nodes (512 words) after them.
__global__ __launch_bounds__(256) void k_node_prefix(const uint64_t* __restrict__ lmask, uint16_t* __restrict__ lpre,
                                                     int64_t nl, int64_t nbl, const uint64_t* __restrict__ umask,
                                                     uint16_t* __restrict__ upre, int64_t nu, const uint64_t* dcnt) {
  const int lane = lane_id();
  if (dcnt) {
    if ((int64_t)dcnt[2] < nl) nl = (int64_t)dcnt[2];
    if ((int64_t)dcnt[3] < nu) nu = (int64_t)dcnt[3];
  }
  const bool lower = (int64_t)blockIdx.x < nbl;
  const int64_t node = (lower ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - nbl) * 4 + (threadIdx.x >> 6);
  const int words = lower ? 64 : 512;
  if (node >= (lower ? nl : nu)) return;
  const uint64_t* mask = lower ? lmask : umask;
  uint16_t* pre = lower ? lpre : upre;
  uint32_t base = 0;
  for (int w0 = 0; w0 < words; w0 += 64) {
    const uint32_t c = (uint32_t)__popcll(mask[node * words + w0 + lane]);
    const uint32_t inc = wave_incl_scan(c);
    pre[node * words + w0 + lane] = (uint16_t)(base + inc - c);
    base += (uint32_t)__shfl((int)inc, 63, 64);
  }
}

// The 3x3x3 block of leaves around every leaf, resolved once through the tree (root hash and
// fixed-fanout descent) for the kernel map and the leaf-local convolution.
__global__ __launch_bounds__(256) void k_leaf_neighbors(GridView g, int32_t* __restrict__ nbr, const uint64_t* dcnt) {
  const int64_t total = (dcnt && (int64_t)dcnt[1] < g.n_leaf ? (int64_t)dcnt[1] : g.n_leaf) * 27;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = e / 27;
    const int slot = (int)(e - f * 27);
    int32_t nl = (int32_t)f;
    if (slot != 13) {
      const int4 o = g.leaf_origin[f];
      const int64_t ni = (int64_t)o.x + 8 * (slot / 9 - 1), nj = (int64_t)o.y + 8 * ((slot / 3) % 3 - 1),
                    nk = (int64_t)o.z + 8 * (slot % 3 - 1);
      nl = -1;
      if (ni >= INT32_MIN && ni <= INT32_MAX && nj >= INT32_MIN && nj <= INT32_MAX && nk >= INT32_MIN &&
          nk <= INT32_MAX)
        nl = find_leaf(g, (int32_t)ni, (int32_t)nj, (int32_t)nk);
    }
    nbr[e] = nl;
  }
}

}  // namespace

// ------------------------------------------------------------------------------ host side

// One workspace block holds every temporary of a build (the host pays for each allocator
// call while the device waits on it after a read-back; the block is reused across builds);
// released on every exit path.
struct Arena {
  hipStream_t s;
  const igc_allocator* a;
  Workspace ws;
  char* base = nullptr;
  size_t used = 0, cap = 0;
  std::vector<std::pair<void*, size_t>> extra;  // rare oversized pieces
  Arena(hipStream_t st, const igc_allocator* al) : s(st), a(al) {}
  ~Arena() {
    for (const auto& e : extra) dev_free(e.first, e.second, s, a);
    ws_release(&ws, s);
  }
  int reserve(size_t bytes) {
    const int rc = ws_acquire(&ws, bytes, s, "igc_grid_build: workspace", a);
    base = (char*)ws.p;
    cap = bytes;
    return rc;
  }
  template <class T>
  T* take(size_t bytes) {
    T* p = (T*)(base + used);
    used = align_up(used + bytes, 256);
    return used <= cap ? p : nullptr;
  }
  template <class T>
  int get_extra(T** out, size_t bytes, const char* what) {
    const int rc = dev_alloc((void**)out, bytes, s, what, a);
    if (rc == IGC_OK) extra.push_back({(void*)*out, bytes});
    return rc;
  }
};

// Workgroups of the grid-stride passes (measured: 512 for both was 11% slower on the band and
// large builds; 2048 for the key pass slower than 1024, its per-workgroup histograms grow).
constexpr int kHistBlocks = 1024;  // workgroups of the key / histogram passes
constexpr int kTileBlocks = 2048;  // workgroups of the tile pass

// The build with a host read-back after the tile pass (the tile count and key bits choose the
// sort) and after the counts (they size the topology): any number of root tiles.
int build_grid_synced(const int32_t* d_ijk, int64_t n_in, hipStream_t s, igc_grid* g) {

  // Root table (keys, then upper-node rows): first capacity from an estimate, then the size
  // that always suffices (U <= n_in) - the capacity retry. It is built in the workspace and
  // copied into the grid's block once the block is allocated.
  uint64_t full_cap = 16;
  while (full_cap < 2ull * (uint64_t)n_in) full_cap <<= 1;
  uint64_t cap = std::min<uint64_t>(full_cap, 1ull << 16);
  if (const char* e = std::getenv("IGC_TEST_INITIAL_CAPACITY")) {
    const uint64_t want = std::strtoull(e, nullptr, 10);
    cap = 1;
    while (cap < want) cap <<= 1;
  }

  // Workspace sizes depend on n_in only (the tile lists of more than kSmallSort tiles, and a
  // root table grown by the retry, are allocated on their own).
  const int64_t tiles = (n_in + kTileKeys - 1) / kTileKeys;
  const int64_t sort_tiles = (n_in + kSortTile - 1) / kSortTile;
  const size_t ws = align_up(sizeof(BuildState), 256) + align_up((size_t)kTileBlocks * 32, 256) +
                    align_up(2 * kMaxPasses * kMaxBins * 4, 256) + align_up((size_t)kHistBlocks * kHistWidth * 4, 256) +
                    2 * align_up((size_t)n_in * 8, 256) + 2 * align_up((size_t)sort_tiles * kMaxBins * 4, 256) +
                    align_up((size_t)tiles * 8, 256) + align_up((size_t)tiles * 32, 256) +
                    2 * align_up((size_t)kSmallSort * 8, 256) + align_up((size_t)cap * 12, 256);
  Arena ar(s, grid_alloc(g));
  int rc = ar.reserve(ws);
  if (rc) return rc;
  BuildState* st = ar.take<BuildState>(sizeof(BuildState));
  uint64_t* partial = ar.take<uint64_t>((size_t)kTileBlocks * 32);
  uint32_t* hist = ar.take<uint32_t>(2 * kMaxPasses * kMaxBins * 4);
  uint32_t* hpart = ar.take<uint32_t>((size_t)kHistBlocks * kHistWidth * 4);
  uint64_t* ka = ar.take<uint64_t>((size_t)n_in * 8);
  uint64_t* kb = ar.take<uint64_t>((size_t)n_in * 8);
  uint32_t* rcnt = ar.take<uint32_t>((size_t)sort_tiles * kMaxBins * 4);
  uint32_t* roff = ar.take<uint32_t>((size_t)sort_tiles * kMaxBins * 4);
  uint64_t* bcounts = ar.take<uint64_t>((size_t)tiles * 8);
  uint64_t* bprefix = ar.take<uint64_t>((size_t)tiles * 32);
  uint64_t* tile_list = ar.take<uint64_t>((size_t)kSmallSort * 8);
  uint64_t* tile_tmp = ar.take<uint64_t>((size_t)kSmallSort * 8);
  uint64_t* root_keys = ar.take<uint64_t>((size_t)cap * 12);
  if (!root_keys) return set_error(IGC_ERR_INTERNAL, "igc_grid_build: workspace layout");
  BuildState* hd = nullptr;  // the staging buffer as kernels write it
  BuildState* h = (BuildState*)host_staging(sizeof(BuildState), (void**)&hd);
  if (!h || !hd) return set_error(IGC_ERR_OOM, "igc_grid_build: pinned staging buffer");

  for (int attempt = 0;; ++attempt) {
    k_init_root<<<grid_for((int64_t)cap, 256, 4096), 256, 0, s>>>(st, root_keys, (int64_t)cap);
    IGC_HIP(hipGetLastError(), "igc_grid_build: init launch");
    const uint32_t limit = (uint32_t)std::min<uint64_t>(cap, 4096);
    const int nbt = grid_for((n_in + 3) / 4, 256, kTileBlocks);
    k_tile_insert<<<nbt, 256, 0, s>>>(d_ijk, n_in, root_keys, (uint32_t)(cap - 1), limit, partial, st, tile_list,
                                      (uint32_t)kSmallSort);
    IGC_HIP(hipGetLastError(), "igc_grid_build: tile insert launch");
    k_reduce_bits<<<1, 256, 0, s>>>(partial, nbt, st, hd);  // also publishes the state to h
    IGC_HIP(hipGetLastError(), "igc_grid_build: tile bits launch");
    IGC_HIP(hipStreamSynchronize(s), "igc_grid_build: tile pass");
    if (!h->overflow) break;
    if (cap >= full_cap || attempt >= 2)
      return set_error(IGC_ERR_CAPACITY, "igc_grid_build: root table overflow after retries");
    cap = full_cap;
    if ((rc = ar.get_extra(&root_keys, cap * 12, "igc_grid_build: root table"))) return rc;
  }
  int32_t* root_vals = (int32_t*)(root_keys + cap);
  const int64_t U = h->n_tiles;
  const uint64_t off_var = h->off_or ^ h->off_and;
  const uint64_t key_var = h->key_or ^ h->key_and;
  if (U < 1 || (uint64_t)U > (1ull << 27))
    return set_error(U < 1 ? IGC_ERR_INTERNAL : IGC_ERR_RANGE, "igc_grid_build: root tile count out of range");

  // Up to kSmallSort tiles the tile pass has listed them already; more are compacted from the table.
  if (U > kSmallSort) {
    if ((rc = ar.get_extra(&tile_list, U * sizeof(uint64_t), "igc_grid_build: tile list"))) return rc;
    if ((rc = ar.get_extra(&tile_tmp, U * sizeof(uint64_t), "igc_grid_build: tile list"))) return rc;
    k_tile_compact<<<grid_for((int64_t)cap, 256, 1024), 256, 0, s>>>(root_keys, (uint32_t)cap, tile_list, (uint32_t)U,
                                                                     st);
    IGC_HIP(hipGetLastError(), "igc_grid_build: tile compaction launch");
  }
  uint64_t* tiles_sorted = tile_tmp;
  if (U <= kSmallSort) {
    k_sort_rank_small<<<1, 1024, 0, s>>>(tile_list, tile_tmp, (int)U, root_keys, root_vals, (uint32_t)(cap - 1), st,
                                         (int64_t)U);
    IGC_HIP(hipGetLastError(), "igc_grid_build: tile sort launch");
  } else {
    const PassSpec tps = pass_spec(key_var);
    const int nbh = grid_for(U, 256, kHistBlocks);
    k_hist<<<nbh, 256, 0, s>>>(tile_list, U, tps, hpart);
    IGC_HIP(hipGetLastError(), "igc_grid_build: tile histogram launch");
    const int twidth = tps.passes << tps.bits;
    k_hist_reduce<<<(twidth + 15) / 16, 256, 0, s>>>(hpart, nbh, twidth, hist + kMaxPasses * kMaxBins);
    IGC_HIP(hipGetLastError(), "igc_grid_build: tile histogram reduce launch");
    uint32_t* tcnt = nullptr;
    const int64_t ttiles = (U + kSortTile - 1) / kSortTile;
    if ((rc = ar.get_extra(&tcnt, (size_t)2 * ttiles * kMaxBins * 4, "igc_grid_build: tile radix counts"))) return rc;
    if ((rc = radix_sort(tile_list, tile_tmp, U, tps, hist + kMaxPasses * kMaxBins, tcnt, tcnt + ttiles * kMaxBins, ttiles,
                         &st->guard, s, &tiles_sorted)))
      return rc;
    k_tile_rank<<<grid_for(U, 256, 1024), 256, 0, s>>>(tiles_sorted, U, root_keys, root_vals, (uint32_t)(cap - 1), st);
    IGC_HIP(hipGetLastError(), "igc_grid_build: tile rank launch");
  }

  // key2, its histograms and its sort over the varying bit span.
  const SortPlan plan = make_sort_plan(h->off_or, h->off_and, (uint64_t)U, 0);
  const BitRuns runs = plan.kf.runs;
  const PassSpec ps = plan.ps;
  const int nbk = grid_for((n_in + 3) / 4, 256, kHistBlocks);
  k_key2<<<nbk, 256, 0, s>>>(d_ijk, n_in, root_keys, root_vals, (uint32_t)(cap - 1), tiles_sorted, U, ka, ps, runs,
                             hpart, st);
  IGC_HIP(hipGetLastError(), "igc_grid_build: key pass launch");
  if (ps.passes > 0) {
    const int width = ps.passes << ps.bits;
    k_hist_reduce<<<(width + 15) / 16, 256, 0, s>>>(hpart, nbk, width, hist);
    IGC_HIP(hipGetLastError(), "igc_grid_build: histogram reduce launch");
  }
  uint64_t* sorted = ka;
  if ((rc = radix_sort(ka, kb, n_in, ps, hist, rcnt, roff, sort_tiles, &st->guard, s, &sorted))) return rc;
  // The sorted keys stay compacted: leaf, lower and upper boundaries are compared at the
  // compacted positions of leaf-part bits 0, 12 and 27, and the register pass expands a key
  // only where it starts a leaf.
  const KeyForm kf = plan.kf;

  // Counts, then the read-back that sizes the topology.
  const int64_t nb = tiles;
  k_count<<<(unsigned)nb, kThreads, 0, s>>>(sorted, n_in, bcounts, kf.cs_lower, kf.cs_upper);
  IGC_HIP(hipGetLastError(), "igc_grid_build: count launch");
  k_scan_blocks<<<1, 1024, 0, s>>>(bcounts, nb, bprefix, st, hd);  // also publishes the state to h
  IGC_HIP(hipGetLastError(), "igc_grid_build: block scan launch");
  IGC_HIP(hipStreamSynchronize(s), "igc_grid_build: sort and count");
  if (h->guard) return set_error(IGC_ERR_INTERNAL, "igc_grid_build: device bounds check failed before registration");
  const int64_t F = (int64_t)h->counts[1], Lw = (int64_t)h->counts[2];
  if ((int64_t)h->counts[3] != U || F < 1 || F > n_in || Lw > F)
    return set_error(IGC_ERR_INTERNAL, "igc_grid_build: inconsistent node counts");

  // Topology block (zeroed with one fill: masks start empty).
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t o_upm = carve(U * 512 * 8), o_lom = carve(Lw * 64 * 8), o_leaf = carve(F * sizeof(LeafRec)),
               zero_end = off, o_root_list = carve(U * 8), o_upo = carve(U * 16), o_upp = carve(U * 512 * 2),
               o_upf = carve(U * 4), o_loo = carve(Lw * 16), o_lop = carve(Lw * 64 * 2), o_lof = carve(Lw * 4),
               o_lfo = carve(F * 16), o_nbr = carve(F * 27 * 4), o_root = carve(cap * 12);
  char* blk = nullptr;
  if ((rc = dev_alloc((void**)&blk, off, s, "igc_grid_build: topology", grid_alloc(g)))) return rc;
  g->block = blk;
  g->bytes = off;
  g->root_keys = (uint64_t*)(blk + o_root);
  g->root_vals = (int32_t*)(g->root_keys + cap);
  g->root_cap = (uint32_t)cap;
  g->root_list = (uint64_t*)(blk + o_root_list);
  g->upper_origin = (int4*)(blk + o_upo);
  g->upper_mask = (uint64_t*)(blk + o_upm);
  g->upper_pre = (uint16_t*)(blk + o_upp);
  g->upper_first = (uint32_t*)(blk + o_upf);
  g->lower_origin = (int4*)(blk + o_loo);
  g->lower_mask = (uint64_t*)(blk + o_lom);
  g->lower_pre = (uint16_t*)(blk + o_lop);
  g->lower_first = (uint32_t*)(blk + o_lof);
  g->leaf = (LeafRec*)(blk + o_leaf);
  g->leaf_origin = (int4*)(blk + o_lfo);
  g->leaf_nbr = (int32_t*)(blk + o_nbr);
  g->n_leaf = F;
  g->n_lower = Lw;
  g->n_upper = U;
  g->sort_passes = ps.passes;
  // cap * 12 bytes rounded up to whole words: both root-table regions are padded to 256 bytes.
  const int64_t root_words = (int64_t)((cap * 12 + 7) / 8);
  k_fill_copy_u64<<<grid_for((int64_t)(zero_end / 8) + root_words, 256, 4096), 256, 0, s>>>(
      (uint64_t*)blk, (int64_t)(zero_end / 8), g->root_keys, root_keys, root_words);
  IGC_HIP(hipGetLastError(), "igc_grid_build: topology initialisation launch");

  Topo t{F,           Lw,           U,          &st->guard,     &st->cap_over, tiles_sorted,
         g->root_list, g->upper_origin, g->upper_mask, g->upper_first, g->lower_origin, g->lower_mask,
         g->lower_first, g->leaf,     g->leaf_origin};
  k_register<<<(unsigned)nb, kThreads, 0, s>>>(sorted, n_in, bprefix, t, kf);
  IGC_HIP(hipGetLastError(), "igc_grid_build: register launch");
  const int64_t groups = (F + kLeafGroup - 1) / kLeafGroup;
  uint64_t* gsum = bprefix;  // the block prefixes are consumed by the register pass
  if ((size_t)groups * 8 > (size_t)tiles * 32) return set_error(IGC_ERR_INTERNAL, "igc_grid_build: leaf scan workspace");
  // Node prefixes and the leaf neighbour table (neither reads the leaves' rows) go before the
  // leaf scan, so that the group scan, which publishes N, follows every kernel that can set
  // the guard.
  const int64_t nbl = (Lw + 3) / 4;
  k_node_prefix<<<(unsigned)(nbl + (U + 3) / 4), 256, 0, s>>>(g->lower_mask, g->lower_pre, Lw, nbl, g->upper_mask,
                                                             g->upper_pre, U, nullptr);
  IGC_HIP(hipGetLastError(), "igc_grid_build: node prefix launch");
  k_leaf_neighbors<<<grid_for(F * 27, 256, 8192), 256, 0, s>>>(g->view(), g->leaf_nbr, nullptr);
  IGC_HIP(hipGetLastError(), "igc_grid_build: leaf neighbour launch");
  k_leaf_count<<<(unsigned)groups, 256, 0, s>>>(g->leaf, F, gsum, nullptr);
  IGC_HIP(hipGetLastError(), "igc_grid_build: leaf count launch");
  k_scan_groups<<<1, 1024, 0, s>>>(gsum, groups, st, hd);  // also publishes the state (N) to h
  IGC_HIP(hipGetLastError(), "igc_grid_build: leaf scan launch");
  if (groups > 1) {
    k_leaf_offset<<<(unsigned)groups, 256, 0, s>>>(g->leaf, F, gsum, nullptr);
    IGC_HIP(hipGetLastError(), "igc_grid_build: leaf offset launch");
  }
  // Last read-back: the voxel count.
  IGC_HIP(hipStreamSynchronize(s), "igc_grid_build: registration");
  if (h->guard || h->cap_over)
    return set_error(IGC_ERR_INTERNAL, "igc_grid_build: device bounds check failed in registration");
  const int64_t N = (int64_t)h->counts[0];
  if (N < F || N > n_in) return set_error(IGC_ERR_INTERNAL, "igc_grid_build: inconsistent voxel count");
  g->n_voxels = N;
  return IGC_OK;
}

// ------------------------------------------------------------------------------ counted build
//
// The build with one host read-back (DriveRT, "Counts kept on the GPU"), for scenes of at most
// kSmallSort root tiles. The tile pass's state stays on the device: the tiles are ranked from
// the device count, a one-thread kernel derives the sort plan (key compaction and passes of
// 8- or 9-bit digits) from the OR / AND of the keys, the radix passes are launched up to the largest
// count and skip themselves past the plan's (the key pass writes into the buffer that makes the
// last pass end in the first), and the counts N, F, Lw, U come out of the count pass on the
// device. The topology is sized from estimates (rows per coordinate of the last build in this
// process); a row past one sets cap_over and the build runs again with the exact counts it
// reported (DriveRT, "Compilation and deployment": results are never truncated). A scene with
// more tiles falls back to the synced build.
namespace {

constexpr uint32_t kCountedRoot = 2 * kSmallSort;  // root table slots of the counted build

struct BuildHint {
  double leaf = 0.25, lower = 1.0 / 64.0;  // leaves, lower nodes per input coordinate
  int64_t upper = 32;
  int digit_bits = 8;  // 9 when the last key span took fewer 9-bit passes than 8-bit ones
};
std::mutex g_hint_mu;
BuildHint g_hint;

enum CountedStatus { kBuilt = 0, kFallBack = 1, kRepeat = 2 };

template <int BITS>
int build_grid_counted(const int32_t* d_ijk, int64_t n_in, hipStream_t s, igc_grid* g, int64_t capF, int64_t capLw,
                       int64_t capU, int* status, int64_t exact[3]) {
  constexpr int kCountedHist = kCountedPasses << BITS;
  *status = kFallBack;
  uint64_t cap = kCountedRoot;
  if (const char* e = std::getenv("IGC_TEST_INITIAL_CAPACITY")) {  // forces the synced build's retries
    const uint64_t want = std::strtoull(e, nullptr, 10);
    cap = 1;
    while (cap < want) cap <<= 1;
  }
  const int64_t tiles = (n_in + kTileKeys - 1) / kTileKeys;
  const int64_t sort_tiles = (n_in + kSortTile - 1) / kSortTile;
  const int64_t groups = (capF + kLeafGroup - 1) / kLeafGroup;
  const size_t ws = align_up(sizeof(BuildState), 256) + align_up(sizeof(SortPlan), 256) +
                    align_up((size_t)kTileBlocks * 32, 256) + align_up((size_t)kMaxPasses * kMaxBins * 4, 256) +
                    align_up((size_t)kHistBlocks * kCountedHist * 4, 256) + 2 * align_up((size_t)n_in * 8, 256) +
                    2 * align_up((size_t)sort_tiles * kMaxBins * 4, 256) + align_up((size_t)tiles * 8, 256) +
                    align_up((size_t)tiles * 32, 256) + align_up((size_t)groups * 8, 256) +
                    2 * align_up((size_t)kSmallSort * 8, 256) + align_up((size_t)cap * 12, 256);
  Arena ar(s, grid_alloc(g));
  int rc = ar.reserve(ws);
  if (rc) return rc;
  BuildState* st = ar.take<BuildState>(sizeof(BuildState));
  SortPlan* plan = ar.take<SortPlan>(sizeof(SortPlan));
  uint64_t* partial = ar.take<uint64_t>((size_t)kTileBlocks * 32);
  uint32_t* hist = ar.take<uint32_t>((size_t)kMaxPasses * kMaxBins * 4);
  uint32_t* hpart = ar.take<uint32_t>((size_t)kHistBlocks * kCountedHist * 4);
  uint64_t* ka = ar.take<uint64_t>((size_t)n_in * 8);
  uint64_t* kb = ar.take<uint64_t>((size_t)n_in * 8);
  uint32_t* rcnt = ar.take<uint32_t>((size_t)sort_tiles * kMaxBins * 4);
  uint32_t* roff = ar.take<uint32_t>((size_t)sort_tiles * kMaxBins * 4);
  uint64_t* bcounts = ar.take<uint64_t>((size_t)tiles * 8);
  uint64_t* bprefix = ar.take<uint64_t>((size_t)tiles * 32);
  uint64_t* gsum = ar.take<uint64_t>((size_t)groups * 8);
  uint64_t* tile_list = ar.take<uint64_t>((size_t)kSmallSort * 8);
  uint64_t* tile_tmp = ar.take<uint64_t>((size_t)kSmallSort * 8);
  uint64_t* root_keys = ar.take<uint64_t>((size_t)cap * 12);
  if (!root_keys) return set_error(IGC_ERR_INTERNAL, "igc_grid_build: workspace layout");
  int32_t* root_vals = (int32_t*)(root_keys + cap);
  BuildState* hd = nullptr;
  BuildState* h = (BuildState*)host_staging(sizeof(BuildState), (void**)&hd);
  if (!h || !hd) return set_error(IGC_ERR_OOM, "igc_grid_build: pinned staging buffer");

  // Tiles, their ranks and the sort plan, all on the device.
  k_init_root<<<grid_for((int64_t)cap, 256, 4096), 256, 0, s>>>(st, root_keys, (int64_t)cap);
  IGC_HIP(hipGetLastError(), "igc_grid_build: init launch");
  const int nbt = grid_for((n_in + 3) / 4, 256, kTileBlocks);
  k_tile_insert<<<nbt, 256, 0, s>>>(d_ijk, n_in, root_keys, (uint32_t)(cap - 1), (uint32_t)cap, partial, st, tile_list,
                                    (uint32_t)kSmallSort);
  IGC_HIP(hipGetLastError(), "igc_grid_build: tile insert launch");
  k_reduce_bits<<<1, 256, 0, s>>>(partial, nbt, st, hd);
  IGC_HIP(hipGetLastError(), "igc_grid_build: tile bits launch");
  // More tiles than upper-node rows: the table is emptied (no lookup can return a row past the
  // upper arrays), the rest of the build does no work, and it is repeated with the exact count.
  k_sort_rank_small<<<1, 1024, 0, s>>>(tile_list, tile_tmp, -1, root_keys, root_vals, (uint32_t)(cap - 1), st, capU);
  IGC_HIP(hipGetLastError(), "igc_grid_build: tile sort launch");
  k_make_plan<<<1, 64, 0, s>>>(st, plan, BITS);
  IGC_HIP(hipGetLastError(), "igc_grid_build: sort plan launch");

  // Keys, their sort and the counts.
  const int nbk = grid_for((n_in + 3) / 4, 256, kHistBlocks);
  k_key2<<<nbk, 256, 0, s>>>(d_ijk, n_in, root_keys, root_vals, (uint32_t)(cap - 1), tile_tmp, kSmallSort, ka,
                             PassSpec{0, 0, BITS}, BitRuns{}, hpart, st, plan, kCountedHist, kb);
  IGC_HIP(hipGetLastError(), "igc_grid_build: key pass launch");
  k_hist_reduce<<<(kCountedHist + 15) / 16, 256, 0, s>>>(hpart, nbk, kCountedHist, hist);
  IGC_HIP(hipGetLastError(), "igc_grid_build: histogram reduce launch");
  for (int p = 0; p < kCountedPasses; ++p) {
    radix_pass<BITS>(ka, kb, n_in, 0, hist + ((size_t)p << BITS), rcnt, roff, sort_tiles, &st->guard, p == 0, s,
                     nullptr, plan, p);
    IGC_HIP(hipGetLastError(), "igc_grid_build: radix pass launch");
  }
  k_count<<<(unsigned)tiles, kThreads, 0, s>>>(ka, n_in, bcounts, 0, 0, plan);
  IGC_HIP(hipGetLastError(), "igc_grid_build: count launch");
  k_scan_blocks<<<1, 1024, 0, s>>>(bcounts, tiles, bprefix, st, hd);
  IGC_HIP(hipGetLastError(), "igc_grid_build: block scan launch");

  // Topology sized from the estimates (zeroed masks, the root table copied in).
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const int64_t F = capF, Lw = capLw, U = capU;
  const size_t o_upm = carve(U * 512 * 8), o_lom = carve(Lw * 64 * 8), o_leaf = carve(F * sizeof(LeafRec)),
               zero_end = off, o_root_list = carve(U * 8), o_upo = carve(U * 16), o_upp = carve(U * 512 * 2),
               o_upf = carve(U * 4), o_loo = carve(Lw * 16), o_lop = carve(Lw * 64 * 2), o_lof = carve(Lw * 4),
               o_lfo = carve(F * 16), o_nbr = carve(F * 27 * 4), o_root = carve(cap * 12);
  char* blk = nullptr;
  if ((rc = dev_alloc((void**)&blk, off, s, "igc_grid_build: topology", grid_alloc(g)))) return rc;
  g->block = blk;
  g->bytes = off;
  g->root_keys = (uint64_t*)(blk + o_root);
  g->root_vals = (int32_t*)(g->root_keys + cap);
  g->root_cap = (uint32_t)cap;
  g->root_list = (uint64_t*)(blk + o_root_list);
  g->upper_origin = (int4*)(blk + o_upo);
  g->upper_mask = (uint64_t*)(blk + o_upm);
  g->upper_pre = (uint16_t*)(blk + o_upp);
  g->upper_first = (uint32_t*)(blk + o_upf);
  g->lower_origin = (int4*)(blk + o_loo);
  g->lower_mask = (uint64_t*)(blk + o_lom);
  g->lower_pre = (uint16_t*)(blk + o_lop);
  g->lower_first = (uint32_t*)(blk + o_lof);
  g->leaf = (LeafRec*)(blk + o_leaf);
  g->leaf_origin = (int4*)(blk + o_lfo);
  g->leaf_nbr = (int32_t*)(blk + o_nbr);
  g->n_leaf = F;  // capacities until the read-back
  g->n_lower = Lw;
  g->n_upper = U;
  const int64_t root_words = (int64_t)((cap * 12 + 7) / 8);
  k_fill_copy_u64<<<grid_for((int64_t)(zero_end / 8) + root_words, 256, 4096), 256, 0, s>>>(
      (uint64_t*)blk, (int64_t)(zero_end / 8), g->root_keys, root_keys, root_words);
  IGC_HIP(hipGetLastError(), "igc_grid_build: topology initialisation launch");

  Topo t{F,           Lw,           U,          &st->guard,     &st->cap_over, tile_tmp,
         g->root_list, g->upper_origin, g->upper_mask, g->upper_first, g->lower_origin, g->lower_mask,
         g->lower_first, g->leaf,     g->leaf_origin};
  k_register<<<(unsigned)tiles, kThreads, 0, s>>>(ka, n_in, bprefix, t, KeyForm{21, 36, BitRuns{}}, plan);
  IGC_HIP(hipGetLastError(), "igc_grid_build: register launch");
  const uint64_t* dc = st->counts;
  const int64_t nbl = (Lw + 3) / 4;
  k_node_prefix<<<(unsigned)(nbl + (U + 3) / 4), 256, 0, s>>>(g->lower_mask, g->lower_pre, Lw, nbl, g->upper_mask,
                                                             g->upper_pre, U, dc);
  IGC_HIP(hipGetLastError(), "igc_grid_build: node prefix launch");
  k_leaf_neighbors<<<grid_for(F * 27, 256, 8192), 256, 0, s>>>(g->view(), g->leaf_nbr, dc);
  IGC_HIP(hipGetLastError(), "igc_grid_build: leaf neighbour launch");
  k_leaf_count<<<(unsigned)std::max<int64_t>(groups, 1), 256, 0, s>>>(g->leaf, F, gsum, dc);
  IGC_HIP(hipGetLastError(), "igc_grid_build: leaf count launch");
  k_scan_groups<<<1, 1024, 0, s>>>(gsum, std::max<int64_t>(groups, 1), st, hd);  // publishes the state
  IGC_HIP(hipGetLastError(), "igc_grid_build: leaf scan launch");
  if (groups > 1) {
    k_leaf_offset<<<(unsigned)groups, 256, 0, s>>>(g->leaf, F, gsum, dc);
    IGC_HIP(hipGetLastError(), "igc_grid_build: leaf offset launch");
  }

  IGC_HIP(hipStreamSynchronize(s), "igc_grid_build: the read-back");  // the one synchronisation
  auto drop_block = [&]() {
    dev_free(g->block, g->bytes, s, grid_alloc(g));
    g->block = nullptr;
    g->bytes = 0;
  };
  g->host_syncs += 1;
  if (h->overflow || h->n_tiles == 0 || h->n_tiles > (uint32_t)kSmallSort) {
    drop_block();
    *status = kFallBack;
    return IGC_OK;
  }
  if ((int64_t)h->n_tiles > U) {  // the tile count is exact; leaves and lower nodes were not counted
    drop_block();
    exact[0] = std::max<int64_t>(F, (int64_t)h->n_tiles);
    exact[1] = std::max<int64_t>(Lw, (int64_t)h->n_tiles);
    exact[2] = (int64_t)h->n_tiles;
    *status = kRepeat;
    return IGC_OK;
  }
  // F, Lw, U come from the count pass; N from the leaves' popcounts (partial when registration
  // stopped at an estimate, so it is checked only after that case).
  const int64_t N = (int64_t)h->counts[0], Fx = (int64_t)h->counts[1], Lwx = (int64_t)h->counts[2],
                Ux = (int64_t)h->counts[3];
  if (h->guard) return set_error(IGC_ERR_INTERNAL, "igc_grid_build: device bounds check failed");
  if ((int64_t)h->n_tiles != Ux || Fx < 1 || Fx > n_in || Lwx > Fx || Ux > Lwx)
    return set_error(IGC_ERR_INTERNAL, "igc_grid_build: inconsistent node counts");
  if (h->cap_over || Fx > F || Lwx > Lw || Ux > U) {
    drop_block();
    exact[0] = Fx;
    exact[1] = Lwx;
    exact[2] = Ux;
    *status = kRepeat;
    return IGC_OK;
  }
  if (N < Fx || N > n_in) return set_error(IGC_ERR_INTERNAL, "igc_grid_build: inconsistent voxel count");
  g->n_voxels = N;
  g->n_leaf = Fx;
  g->n_lower = Lwx;
  g->n_upper = Ux;
  g->sort_passes = (int32_t)h->sort_passes;
  {
    std::lock_guard<std::mutex> lk(g_hint_mu);
    g_hint.leaf = (double)Fx / (double)n_in;
    g_hint.lower = (double)Lwx / (double)n_in;
    g_hint.upper = Ux;
    const int span = (int)h->sort_span;
    g_hint.digit_bits = (span + 8) / 9 < (span + 7) / 8 ? 9 : 8;
  }
  *status = kBuilt;
  return IGC_OK;
}

}  // namespace

int build_grid(const int32_t* d_ijk, int64_t n_in, hipStream_t s, igc_grid* g) {
  g->n_input = n_in;
  if (n_in == 0) {
    // No device work. A grid built with an allocator still owns one (minimal) block from it.
    if (grid_alloc(g)) {
      const int rc = dev_alloc(&g->block, 256, s, "igc_grid_build: topology", grid_alloc(g));
      if (rc) return rc;
      g->bytes = 256;
    }
    return IGC_OK;
  }
  BuildHint hint;
  {
    std::lock_guard<std::mutex> lk(g_hint_mu);
    hint = g_hint;
  }
  const double n = (double)n_in;
  int64_t capF = std::min<int64_t>(n_in, (int64_t)std::ceil(hint.leaf * n * 1.25) + 256);
  int64_t capLw = std::min<int64_t>(capF, (int64_t)std::ceil(hint.lower * n * 1.25) + 64);
  int64_t capU = std::min<int64_t>({(int64_t)kSmallSort, capLw, 2 * hint.upper + 8});
  for (int attempt = 0; attempt < 2; ++attempt) {
    int status = kFallBack;
    int64_t exact[3] = {0, 0, 0};
    const int rc = hint.digit_bits == 9 ? build_grid_counted<9>(d_ijk, n_in, s, g, capF, capLw, capU, &status, exact)
                                        : build_grid_counted<8>(d_ijk, n_in, s, g, capF, capLw, capU, &status, exact);
    if (rc != IGC_OK) return rc;
    if (status == kBuilt) return IGC_OK;
    if (status == kFallBack) break;
    capF = exact[0];
    capLw = exact[1];
    capU = exact[2];
  }
  const int rc = build_grid_synced(d_ijk, n_in, s, g);
  g->host_syncs += 3;
  return rc;
}


// ------------------------------------------------------------------------------ derived grids
//
// Output grids of strided / transposed 3x3x3 convolutions built from the input grid's leaves,
// with every count kept on the device (DriveRT, "Counts kept on the GPU": a chain of strided
// layers needs one host synchronisation, not one per layer).
//
// Per axis an output coordinate y and an input coordinate x are related when |x - s y| <= 1
// (strided) or |y - s x| <= 1 (transposed); y is active iff some active x is related to it on
// all three axes (offsets d in {-1, 0, 1}^3). The relation is separable, so one input leaf's
// contribution to one output leaf comes from 8-bit row operations on its mask: output row
// (yi, yj) ORs the input rows (xi, xj) related to it, and the k bits of that row map through
// the k relation.
//  1. Records: one wave per (input leaf, output-leaf slot) writes the slot's 512-bit mask and
//     origin (or marks it empty); a non-empty record inserts its root tile into the new
//     grid's root table.
//  2. The root tiles are sorted and ranked in one workgroup (up to 4096 tiles).
//  3. Record r gets key ((tile rank << 27 | upper child << 12 | lower child) << IB) | r, an
//     empty one ~0; a radix sort over the rank and child bits puts the records in canonical
//     leaf order, records of one output leaf next to each other.
//  4. Leaf / lower / upper starts are counted over the sorted keys and scanned (F, Lw, U); the
//     register pass writes the nodes top-down and ORs every record's mask into its leaf.
//  5. Node prefixes, the leaf neighbour table, leaf rows and N follow as in the coordinate
//     build, each bounded by the counts on the device.
// Node arrays are sized from estimates made on the host. A stage that outgrows one sets a
// flag; after the one read-back the chain runs again from that stage with the exact counts it
// reported (DriveRT, "Compilation and deployment": buffers start from an estimated capacity
// and the invocation is repeated with larger ones; results are never truncated).

namespace {

struct Derive {
  int32_t s[3];
  int32_t tr;    // transposed
  int32_t L[3];  // output-leaf slots per axis and input leaf
};

// floor(a / b) for b in {1, 2, 3, 8}: each case divides by a constant (a multiply, not a
// 64-bit division routine).
__device__ __forceinline__ int64_t floor_div(int64_t a, int32_t b) {
  if (b == 1) return a;
  if (b == 2) return a >> 1;
  if (b == 8) return a >> 3;
  return a >= 0 ? a / 3 : -((-a + 2) / 3);
}

// Output span [lo, hi] on one axis of the input span [x0, x0 + 7].
__device__ __forceinline__ void derive_span(int64_t x0, int32_t s, int32_t tr, int64_t* lo, int64_t* hi) {
  if (tr) {
    *lo = (int64_t)s * x0 - 1;
    *hi = (int64_t)s * (x0 + 7) + 1;
  } else {
    *lo = -floor_div(1 - x0, s);  // ceil((x0 - 1) / s)
    *hi = floor_div(x0 + 8, s);
  }
}

// Bits t in [0, 8) of the input positions x0 + t related to the output Y + l on one axis,
// with c = s Y - x0 (strided) or c = Y - s x0 (transposed), so that only small integers occur.
__device__ __forceinline__ uint32_t related_bits(int32_t c, int32_t l, int32_t s, int32_t tr) {
  uint32_t m = 0;
#pragma unroll
  for (int d = -1; d <= 1; ++d) {
    int32_t t;
    if (tr) {
      const int32_t z = c + l - d;  // s (x - x0) when s divides it; |z| < 64
      const int32_t zq = s == 1 ? z : s == 2 ? (z >> 1) : (int32_t)floor_div(z, 3);
      if (zq * s != z) continue;
      t = zq;
    } else {
      t = c + s * l + d;
    }
    if (t >= 0 && t < 8) m |= 1u << t;
  }
  return m;
}

// Step 1. One wave per input leaf f (f below the input's leaf count, read from in_counts[1]
// when the input is itself a derived grid): its mask words are read once (lanes 0..7, then
// shuffled), and for each of its output-leaf slots that the leaf's output span reaches, the
// wave computes the slot's 512-bit mask (lane = output row (yi, yj)) into record f * S + slot.
// Slots out of reach, or whose mask is empty, are records with origin.w = 0.
__global__ __launch_bounds__(256) void k_derive_records(const LeafRec* __restrict__ leaf,
                                                        const int4* __restrict__ origin, int64_t F_cap,
                                                        const uint64_t* in_counts, Derive dv,
                                                        int4* __restrict__ rec_origin, uint64_t* __restrict__ rec_mask,
                                                        uint64_t* __restrict__ root_keys, uint32_t root_mask,
                                                        uint64_t* __restrict__ tile_list, BuildState* st) {
  const int S = dv.L[0] * dv.L[1] * dv.L[2];
  const int64_t f = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int64_t F = F_cap;
  if (in_counts && (int64_t)in_counts[1] < F) F = (int64_t)in_counts[1];
  if (blockIdx.x == 0 && threadIdx.x == 0) st->n_rec = (uint64_t)(F * S);
  if (f >= F) return;  // records past the input's leaves: later kernels stop at n_rec
  const int lane = lane_id();
  const int4 o = origin[f];
  const int64_t x0[3] = {o.x, o.y, o.z};
  const uint64_t my_word = lane < 8 ? leaf[f].mask[lane] : 0ull;
  uint64_t m8[8];
#pragma unroll
  for (int xi = 0; xi < 8; ++xi) m8[xi] = shfl64(my_word, xi);
  int64_t Y0[3];
  int n[3];
  bool in_range[3][4];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    int64_t lo, hi;
    derive_span(x0[a], dv.s[a], dv.tr, &lo, &hi);
    Y0[a] = floor_div(lo, 8) * 8;
    n[a] = (int)((hi - Y0[a]) / 8) + 1;  // output leaves the span reaches (at most L[a])
    if (n[a] > dv.L[a]) n[a] = dv.L[a];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t y = Y0[a] + 8 * q;
      in_range[a][q] = y >= (int64_t)INT32_MIN && y <= (int64_t)INT32_MAX - 7;
    }
  }
  const int l = lane & 7, yi = lane >> 3, yj = lane & 7;
  uint64_t last_tile = kEmptyKey;  // lane 0: the root tile inserted last
  // Slots out of reach stay empty records (lanes 0 .. S-1 write their origins).
  if (lane < S) {
    const int qi = lane / (dv.L[1] * dv.L[2]), qj = (lane / dv.L[2]) % dv.L[1], qk = lane % dv.L[2];
    if (qi >= n[0] || qj >= n[1] || qk >= n[2]) rec_origin[f * S + lane] = make_int4(0, 0, 0, 0);
  }
  for (int qi = 0; qi < n[0]; ++qi) {
    const int32_t ci = (int32_t)(dv.tr ? Y0[0] + 8 * qi - (int64_t)dv.s[0] * x0[0]
                                       : (int64_t)dv.s[0] * (Y0[0] + 8 * qi) - x0[0]);
    const uint32_t mi = (uint32_t)__shfl((int)related_bits(ci, l, dv.s[0], dv.tr), yi, 64);
    for (int qj = 0; qj < n[1]; ++qj) {
      const int32_t cj = (int32_t)(dv.tr ? Y0[1] + 8 * qj - (int64_t)dv.s[1] * x0[1]
                                         : (int64_t)dv.s[1] * (Y0[1] + 8 * qj) - x0[1]);
      const uint32_t mj = (uint32_t)__shfl((int)related_bits(cj, l, dv.s[1], dv.tr), yj, 64);
      uint64_t sel = 0;  // the bytes (input rows xj) related to yj
#pragma unroll
      for (int xj = 0; xj < 8; ++xj) sel |= ((mj >> xj) & 1u) ? (0xFFull << (8 * xj)) : 0ull;
      uint64_t acc = 0;
#pragma unroll
      for (int xi = 0; xi < 8; ++xi) acc |= ((mi >> xi) & 1u) ? (m8[xi] & sel) : 0ull;
      acc |= acc >> 32;
      acc |= acc >> 16;
      acc |= acc >> 8;
      const uint32_t b = (uint32_t)acc & 0xFFu;  // input k bits reaching this output row
      for (int qk = 0; qk < n[2]; ++qk) {
        const int32_t ck = (int32_t)(dv.tr ? Y0[2] + 8 * qk - (int64_t)dv.s[2] * x0[2]
                                           : (int64_t)dv.s[2] * (Y0[2] + 8 * qk) - x0[2]);
        const uint32_t rk = related_bits(ck, l, dv.s[2], dv.tr);
        uint32_t r = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) r |= (b & (uint32_t)__shfl((int)rk, t, 64)) ? (1u << t) : 0u;
        // Mask word yi of the output leaf: bits yj * 8 + k from the 8 lanes of row yi.
        uint64_t v = (uint64_t)r << (8 * yj);
        v |= shfl_xor64(v, 1);
        v |= shfl_xor64(v, 2);
        v |= shfl_xor64(v, 4);
        const int slot = (qi * dv.L[1] + qj) * dv.L[2] + qk;
        const int64_t w = f * S + slot;
        const bool any = __ballot(r != 0u) != 0ull;
        const bool ok = any && in_range[0][qi] && in_range[1][qj] && in_range[2][qk];
        if (ok && yj == 0) rec_mask[w * 8 + yi] = v;
        if (lane == 0) {
          const int4 yo = make_int4((int32_t)(Y0[0] + 8 * qi), (int32_t)(Y0[1] + 8 * qj), (int32_t)(Y0[2] + 8 * qk),
                                    ok ? 1 : 0);
          rec_origin[w] = ok ? yo : make_int4(0, 0, 0, 0);
          if (ok) {
            // The slots of one input leaf nearly always share a root tile: insert a key once
            // per run of equal keys (inserting a present key changes nothing).
            const uint64_t tk = tile_key(yo.x, yo.y, yo.z);
            if (tk != last_tile) {
              insert_tile(root_keys, root_mask, root_mask + 1u, tk, st, tile_list, (uint32_t)kSmallSort);
              last_tile = tk;
            }
          } else if (any) {
            atomicOr(&st->range, 1u);
          }
        }
      }
    }
  }
}

// Step 3. Sort keys of the records and the digit histograms of their sort.
__global__ __launch_bounds__(256) void k_derive_keys(const int4* __restrict__ rec_origin, int64_t R,
                                                     const uint64_t* __restrict__ root_keys,
                                                     const int32_t* __restrict__ root_vals, uint32_t root_mask, int ib,
                                                     int32_t rank_cap, PassSpec ps, uint64_t* __restrict__ keys,
                                                     uint32_t* __restrict__ hist, BuildState* st) {
  __shared__ uint32_t s_hist[kHistWidth];
  for (int x = threadIdx.x; x < (ps.passes << ps.bits); x += blockDim.x) s_hist[x] = 0;
  // A stage already over capacity (its table emptied) only writes empty keys: the rest of its
  // kernels then do no work, and the chain is repeated.
  const bool dead = st->cap_over != 0u;
  if ((int64_t)st->n_rec < R) R = (int64_t)st->n_rec;
  __syncthreads();
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R; r += (int64_t)gridDim.x * blockDim.x) {
    const int4 o = rec_origin[r];
    uint64_t k = ~0ull;
    if (o.w && !dead) {
      const int64_t slot = probe_slot(root_keys, root_mask, tile_key(o.x, o.y, o.z), st);
      if (slot >= 0 && root_vals[slot] >= rank_cap) {
        atomicOr(&st->cap_over, 1u);  // more tiles than the key has rank bits for (the host widens it)
      } else if (slot >= 0) {
        const uint32_t ui = (uint32_t)o.x, uj = (uint32_t)o.y, uk = (uint32_t)o.z;
        const uint64_t up = (((ui >> 7) & 31u) << 10) | (((uj >> 7) & 31u) << 5) | ((uk >> 7) & 31u);
        const uint64_t lo = (((ui >> 3) & 15u) << 8) | (((uj >> 3) & 15u) << 4) | ((uk >> 3) & 15u);
        k = ((((uint64_t)root_vals[slot] << 27) | (up << 12) | lo) << ib) | (uint64_t)r;
      }
    }
    keys[r] = k;
    hist_add(s_hist, k, ps);
  }
  hist_flush(s_hist, hist, ps);
}

// Leaf / lower / upper starts of a sorted record key (packed as in start_flags); the empty
// records (~0) sort last and start nothing.
__device__ __forceinline__ uint64_t derive_flags(uint64_t key, uint64_t prev, bool first, int ib) {
  if (key == ~0ull) return 0;
  if (first) return 0x0001000100010000ull;
  return ((uint64_t)((key >> ib) != (prev >> ib)) << 16) |
         ((uint64_t)((key >> (ib + 12)) != (prev >> (ib + 12))) << 32) |
         ((uint64_t)((key >> (ib + 27)) != (prev >> (ib + 27))) << 48);
}

// Step 4a. Per block of 256 sorted keys (one per thread), the leaf / lower / upper starts.
__global__ __launch_bounds__(256) void k_derive_count(const uint64_t* __restrict__ keys, int64_t n, int ib,
                                                      uint64_t* __restrict__ block_counts, const BuildState* st) {
  __shared__ uint64_t s_tmp[4];
  if ((int64_t)st->n_rec < n) n = (int64_t)st->n_rec;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t c = e < n ? derive_flags(keys[e], e > 0 ? keys[e - 1] : 0ull, e == 0, ib) : 0ull;
  uint64_t total;
  block_excl_scan64<256>(c, s_tmp, &total);
  if (threadIdx.x == 0) block_counts[blockIdx.x] = total;
}

// Step 4b. Registration, one sorted key per thread: node rows from the scanned block counts,
// nodes written top-down. The records of one output leaf are consecutive; a wave ORs the masks
// of each run of equal leaves with shuffles, and the first lane of a run ORs them into the leaf.
// Rows past a capacity set cap_over and write nothing.
__global__ __launch_bounds__(256) void k_derive_register(const uint64_t* __restrict__ keys, int64_t n,
                                                         const uint64_t* __restrict__ prefix, int ib,
                                                         const int4* __restrict__ rec_origin,
                                                         const uint64_t* __restrict__ rec_mask, Topo t,
                                                         BuildState* st) {
  __shared__ uint64_t s_tmp[4];
  const int lane = lane_id();
  if ((int64_t)st->n_rec < n) n = (int64_t)st->n_rec;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t key = e < n ? keys[e] : ~0ull;
  const uint64_t prev = e > 0 && e - 1 < n ? keys[e - 1] : 0ull;
  const uint64_t f = e < n ? derive_flags(key, prev, e == 0, ib) : 0ull;
  const uint64_t incl = block_excl_scan64<256>(f, s_tmp, nullptr) + f;
  const int64_t lf = (int64_t)prefix[blockIdx.x * 4 + 1] + (int64_t)((incl >> 16) & 0xFFFF) - 1;
  const int64_t lw = (int64_t)prefix[blockIdx.x * 4 + 2] + (int64_t)((incl >> 32) & 0xFFFF) - 1;
  const int64_t u = (int64_t)prefix[blockIdx.x * 4 + 3] + (int64_t)((incl >> 48) & 0xFFFF) - 1;
  const bool valid = key != ~0ull;
  const bool fits = valid && lf < t.n_leaf && lw < t.n_lower && u < t.n_upper;
  if (valid && !fits) atomicOr(&st->cap_over, 1u);
  const uint64_t r = key & ((1ull << ib) - 1ull);
  const uint64_t leafkey = key >> ib;
  // Lanes d ahead hold the same leaf iff their leaf key is equal (runs are contiguous).
  uint64_t m[8];
#pragma unroll
  for (int wd = 0; wd < 8; ++wd) m[wd] = fits ? rec_mask[r * 8 + wd] : 0ull;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t ok = shfl64(leafkey, lane + d < 64 ? lane + d : lane);
    const bool same = lane + d < 64 && ok == leafkey;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const uint64_t o = shfl64(m[wd], lane + d < 64 ? lane + d : lane);
      m[wd] |= same ? o : 0ull;
    }
  }
  const uint64_t lk_prev = shfl64(leafkey, lane > 0 ? lane - 1 : 0);
  if (!fits) return;
  if ((f >> 16) & 1 || lane == 0 || lk_prev != leafkey) {
#pragma unroll
    for (int wd = 0; wd < 8; ++wd)
      if (m[wd]) atomicOr((unsigned long long*)&t.leaf[lf].mask[wd], m[wd]);
  }
  if (!(f & 0x0001000100010000ull)) return;
  const int4 o = rec_origin[r];
  const uint32_t ui = (uint32_t)o.x, uj = (uint32_t)o.y, uk = (uint32_t)o.z;
  if ((f >> 48) & 1) {
    t.root_list[u] = tile_key(o.x, o.y, o.z);
    t.upper_origin[u] = make_int4(o.x & ~4095, o.y & ~4095, o.z & ~4095, 0);
    t.upper_first[u] = (uint32_t)lw;
  }
  if ((f >> 32) & 1) {
    const uint32_t cu = (((ui >> 7) & 31u) << 10) | (((uj >> 7) & 31u) << 5) | ((uk >> 7) & 31u);
    atomicOr((unsigned long long*)&t.upper_mask[u * 512 + (cu >> 6)], 1ull << (cu & 63u));
    t.lower_origin[lw] = make_int4(o.x & ~127, o.y & ~127, o.z & ~127, 0);
    t.lower_first[lw] = (uint32_t)lf;
  }
  if ((f >> 16) & 1) {
    const uint32_t cl = (((ui >> 3) & 15u) << 8) | (((uj >> 3) & 15u) << 4) | ((uk >> 3) & 15u);
    atomicOr((unsigned long long*)&t.lower_mask[lw * 64 + (cl >> 6)], 1ull << (cl & 63u));
    t.leaf_origin[lf] = make_int4(o.x, o.y, o.z, 0);
  }
}

}  // namespace

namespace {

// Output values on one axis reached from `n` consecutive input values (the input span of a
// leaf, n = 8, or of a root tile, n = 4096), and how many aligned blocks of n they can touch.
int64_t span_len(int64_t n, int32_t s, int32_t tr) { return tr ? (int64_t)s * (n - 1) + 3 : (n + 1) / s + 1; }
int span_blocks(int64_t n, int32_t s, int32_t tr) { return (int)((span_len(n, s, tr) - 1 + n - 1) / n + 1); }

// Node count estimate of a derived grid from its input's: per axis the output span of one
// node over the node size; strided grids at least half the input's (sparse inputs shrink
// less than dense ones); 1.5x room for strided, none for transposed (the volume growth
// already bounds a band's).
int64_t derive_estimate(int64_t n_in, int64_t unit, const int32_t* s, int32_t tr, int64_t cap) {
  double g = 1.0;
  for (int a = 0; a < 3; ++a) g *= (double)span_len(unit, s[a], tr) / (double)unit;
  if (!tr) g = std::max(g, 0.5) * 1.5;
  const double e = std::ceil(g * (double)n_in) + 16.0;
  return std::max<int64_t>(1, std::min<int64_t>(cap, e > 9e18 ? cap : (int64_t)e));
}

struct DeriveStage {
  Derive dv{};
  int64_t F_in = 0, Lw_in = 0, U_in = 0;  // input capacities (exact for the chain's input)
  int64_t R = 0;                           // records
  int64_t F = 0, Lw = 0, U = 0;            // output capacities
  uint32_t root = 0;                       // root table capacity (power of two)
  int ib = 0, rb = 0;                      // record-index bits and tile-rank bits of a key
  bool exact = false;                      // capacities are the counts a previous run reported
};

size_t derive_topology_bytes(const DeriveStage& d, size_t* zero_end) {
  size_t off = 0;
  auto carve = [&](size_t bytes) { off = align_up(off + bytes, 256); };
  carve(d.U * 512 * 8);
  carve(d.Lw * 64 * 8);
  carve(d.F * sizeof(LeafRec));
  *zero_end = off;
  carve(d.U * 8);
  carve(d.U * 16);
  carve(d.U * 512 * 2);
  carve(d.U * 4);
  carve(d.Lw * 16);
  carve(d.Lw * 64 * 2);
  carve(d.Lw * 4);
  carve(d.F * 16);
  carve(d.F * 27 * 4);
  carve((size_t)d.root * 12);
  return off;
}

// Carves the topology arrays of g from its block (same layout as the coordinate build).
void derive_carve(const DeriveStage& d, igc_grid* g) {
  char* blk = (char*)g->block;
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    char* p = blk + off;
    off = align_up(off + bytes, 256);
    return p;
  };
  g->upper_mask = (uint64_t*)carve(d.U * 512 * 8);
  g->lower_mask = (uint64_t*)carve(d.Lw * 64 * 8);
  g->leaf = (LeafRec*)carve(d.F * sizeof(LeafRec));
  g->root_list = (uint64_t*)carve(d.U * 8);
  g->upper_origin = (int4*)carve(d.U * 16);
  g->upper_pre = (uint16_t*)carve(d.U * 512 * 2);
  g->upper_first = (uint32_t*)carve(d.U * 4);
  g->lower_origin = (int4*)carve(d.Lw * 16);
  g->lower_pre = (uint16_t*)carve(d.Lw * 64 * 2);
  g->lower_first = (uint32_t*)carve(d.Lw * 4);
  g->leaf_origin = (int4*)carve(d.F * 16);
  g->leaf_nbr = (int32_t*)carve(d.F * 27 * 4);
  g->root_keys = (uint64_t*)carve((size_t)d.root * 12);
  g->root_vals = (int32_t*)(g->root_keys + d.root);
  g->root_cap = d.root;
  g->n_leaf = d.F;  // capacities until the read-back
  g->n_lower = d.Lw;
  g->n_upper = d.U;
}

// Temporaries of one stage, carved from the chain's workspace.
struct DeriveWs {
  int4* rec_origin;
  uint64_t* rec_mask;
  uint64_t *ka, *kb;
  uint32_t *hpart, *hist, *cnt, *off;
  uint64_t *bcounts, *bprefix, *gsum;
  uint64_t *tile_list, *tile_tmp;
  int64_t sort_tiles, nbh, nb, groups;
};

size_t derive_ws_bytes(const DeriveStage& d, DeriveWs* w, char* base) {
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off = align_up(off + bytes, 256);
    return p;
  };
  const int64_t R = std::max<int64_t>(d.R, 1);
  w->sort_tiles = (R + kSortTile - 1) / kSortTile;
  w->nbh = grid_for(R, 256, kHistBlocks);
  w->nb = (R + 255) / 256;
  w->groups = (d.F + kLeafGroup - 1) / kLeafGroup;
  w->rec_origin = (int4*)carve(R * 16);
  w->rec_mask = (uint64_t*)carve(R * 64);
  w->ka = (uint64_t*)carve(R * 8);
  w->kb = (uint64_t*)carve(R * 8);
  w->hpart = (uint32_t*)carve((size_t)w->nbh * kHistWidth * 4);
  w->hist = (uint32_t*)carve((size_t)kMaxPasses * kMaxBins * 4);
  w->cnt = (uint32_t*)carve((size_t)w->sort_tiles * kMaxBins * 4);
  w->off = (uint32_t*)carve((size_t)w->sort_tiles * kMaxBins * 4);
  w->bcounts = (uint64_t*)carve((size_t)w->nb * 8);
  w->bprefix = (uint64_t*)carve((size_t)w->nb * 32);
  w->gsum = (uint64_t*)carve((size_t)std::max<int64_t>(w->groups, 1) * 8);
  w->tile_list = (uint64_t*)carve((size_t)kSmallSort * 8);
  w->tile_tmp = (uint64_t*)carve((size_t)kSmallSort * 8);
  return off;
}

// Enqueues one stage: `in` (its counts on the device in in_counts when it is itself derived)
// to `out`, whose block is allocated and carved. st: this stage's device state, hd its
// pinned host copy.
int derive_enqueue(const igc_grid* in, const uint64_t* in_counts, const DeriveStage& d, const DeriveWs& w,
                   igc_grid* out, BuildState* st, BuildState* hd, hipStream_t s) {
  k_init_root<<<grid_for((int64_t)d.root, 256, 4096), 256, 0, s>>>(st, out->root_keys, (int64_t)d.root);
  IGC_HIP(hipGetLastError(), "igc_conv_grid: init launch");
  size_t zero_end = 0;
  derive_topology_bytes(d, &zero_end);
  int rc = fill_u64((uint64_t*)out->block, (int64_t)(zero_end / 8), 0ull, s);
  if (rc) return rc;
  if (d.R > 0) {
    k_derive_records<<<(unsigned)((d.F_in + 3) / 4), 256, 0, s>>>(in->leaf, in->leaf_origin, d.F_in, in_counts, d.dv,
                                                               w.rec_origin, w.rec_mask, out->root_keys,
                                                               d.root - 1u, w.tile_list, st);
    IGC_HIP(hipGetLastError(), "igc_conv_grid: record launch");
  }
  k_sort_rank_small<<<1, 1024, 0, s>>>(w.tile_list, w.tile_tmp, -1, out->root_keys, out->root_vals, d.root - 1u, st,
                                       d.U);
  IGC_HIP(hipGetLastError(), "igc_conv_grid: tile sort launch");
  const int key_bits = d.rb + 27;
  const PassSpec ps = pass_spec(((1ull << key_bits) - 1ull) << d.ib);
  uint64_t* sorted = w.ka;
  if (d.R > 0) {
    k_derive_keys<<<(unsigned)w.nbh, 256, 0, s>>>(w.rec_origin, d.R, out->root_keys, out->root_vals, d.root - 1u, d.ib,
                                                  (int32_t)(1 << (d.rb - 1)), ps, w.ka, w.hpart, st);
    IGC_HIP(hipGetLastError(), "igc_conv_grid: key launch");
    const int width = ps.passes << ps.bits;
    k_hist_reduce<<<(width + 15) / 16, 256, 0, s>>>(w.hpart, (int)w.nbh, width, w.hist);
    IGC_HIP(hipGetLastError(), "igc_conv_grid: histogram reduce launch");
    if ((rc = radix_sort(w.ka, w.kb, d.R, ps, w.hist, w.cnt, w.off, w.sort_tiles, &st->guard, s, &sorted, &st->n_rec)))
      return rc;
    k_derive_count<<<(unsigned)w.nb, 256, 0, s>>>(sorted, d.R, d.ib, w.bcounts, st);
    IGC_HIP(hipGetLastError(), "igc_conv_grid: count launch");
  }
  k_scan_blocks<<<1, 1024, 0, s>>>(w.bcounts, d.R > 0 ? w.nb : 0, w.bprefix, st, hd);
  IGC_HIP(hipGetLastError(), "igc_conv_grid: block scan launch");
  if (d.R > 0) {
    Topo t{d.F,           d.Lw,          d.U,           &st->guard,      &st->cap_over, nullptr,
           out->root_list, out->upper_origin, out->upper_mask, out->upper_first, out->lower_origin, out->lower_mask,
           out->lower_first, out->leaf,   out->leaf_origin};
    k_derive_register<<<(unsigned)w.nb, 256, 0, s>>>(sorted, d.R, w.bprefix, d.ib, w.rec_origin, w.rec_mask, t,
                                                          st);
    IGC_HIP(hipGetLastError(), "igc_conv_grid: register launch");
  }
  const uint64_t* dc = st->counts;
  const int64_t nbl = (d.Lw + 3) / 4;
  k_node_prefix<<<(unsigned)(nbl + (d.U + 3) / 4), 256, 0, s>>>(out->lower_mask, out->lower_pre, d.Lw, nbl,
                                                                out->upper_mask, out->upper_pre, d.U, dc);
  IGC_HIP(hipGetLastError(), "igc_conv_grid: node prefix launch");
  k_leaf_neighbors<<<grid_for(d.F * 27, 256, 8192), 256, 0, s>>>(out->view(), out->leaf_nbr, dc);
  IGC_HIP(hipGetLastError(), "igc_conv_grid: leaf neighbour launch");
  k_leaf_count<<<(unsigned)std::max<int64_t>(w.groups, 1), 256, 0, s>>>(out->leaf, d.F, w.gsum, dc);
  IGC_HIP(hipGetLastError(), "igc_conv_grid: leaf count launch");
  k_scan_groups<<<1, 1024, 0, s>>>(w.gsum, std::max<int64_t>(w.groups, 1), st, hd);  // publishes the state
  IGC_HIP(hipGetLastError(), "igc_conv_grid: leaf scan launch");
  if (w.groups > 1) {
    k_leaf_offset<<<(unsigned)w.groups, 256, 0, s>>>(out->leaf, d.F, w.gsum, dc);
    IGC_HIP(hipGetLastError(), "igc_conv_grid: leaf offset launch");
  }
  return IGC_OK;
}

int bits_for(int64_t n) {  // bits that hold 0 .. n-1 (at least 1)
  int b = 1;
  while (b < 63 && (1ll << b) < n) ++b;
  return b;
}

}  // namespace

bool derive_supported(const igc_grid* in, const int32_t* stride, int32_t transposed) {
  const int32_t tr = transposed ? 1 : 0;
  int64_t tiles = std::max<int64_t>(in->n_upper, 1), S = 1;
  for (int a = 0; a < 3; ++a) {
    tiles *= span_blocks(4096, stride[a], tr);
    S *= span_blocks(8, stride[a], tr);
  }
  if (tiles > kSmallSort) return false;
  const int ib = 64 - 27 - (bits_for(std::max<int64_t>(tiles, 2)) + 1);
  return in->n_leaf * S < (1ll << ib);
}

int derive_chain(const igc_grid* in, int n, const int32_t* strides, const int32_t* transposed, hipStream_t s,
                 igc_grid** outs) {
  std::vector<DeriveStage> d((size_t)n);
  auto plan = [&](int k) {  // capacities of stage k from stage k-1's (or the input's)
    DeriveStage& c = d[(size_t)k];
    const int32_t* st = strides + 3 * k;
    c.dv.tr = transposed[k] ? 1 : 0;
    int S = 1;
    int64_t tiles = 1;
    for (int a = 0; a < 3; ++a) {
      c.dv.s[a] = st[a];
      c.dv.L[a] = span_blocks(8, st[a], c.dv.tr);
      S *= c.dv.L[a];
      tiles *= span_blocks(4096, st[a], c.dv.tr);
    }
    if (k == 0) {
      c.F_in = in->n_leaf;
      c.Lw_in = in->n_lower;
      c.U_in = in->n_upper;
    } else {
      c.F_in = d[(size_t)k - 1].F;
      c.Lw_in = d[(size_t)k - 1].Lw;
      c.U_in = d[(size_t)k - 1].U;
    }
    c.R = c.F_in * S;
    if (!c.exact) {
      c.F = derive_estimate(c.F_in, 8, st, c.dv.tr, std::max<int64_t>(c.R, 1));
      c.Lw = std::min(c.F, derive_estimate(c.Lw_in, 128, st, c.dv.tr, std::max<int64_t>(c.R, 1)));
      c.U = std::min<int64_t>({(int64_t)kSmallSort, std::max<int64_t>(c.U_in, 1) * tiles, c.F});
      uint32_t root = 64;
      while ((int64_t)root < 2 * c.U) root <<= 1;
      c.root = std::max(c.root, root);
    }
    c.rb = bits_for(std::max<int64_t>(c.U, 2)) + 1;  // rank < U, one spare bit keeps real keys below ~0
    c.ib = 64 - 27 - c.rb;
  };
  for (int k = 0; k < n; ++k) {
    plan(k);
    if (d[(size_t)k].R >= (1ll << d[(size_t)k].ib))
      return set_error(IGC_ERR_UNSUPPORTED, "igc_conv_grid: too many output-leaf records for one derived grid");
  }
  // Device states of every stage (a later stage reads its input's counts from them) and their
  // pinned read-back copies.
  struct States {
    BuildState* p = nullptr;
    size_t bytes;
    hipStream_t s;
    const igc_allocator* a;
    ~States() {
      if (p) dev_free(p, bytes, s, a);
    }
  } states{nullptr, align_up(sizeof(BuildState) * (size_t)n, 256), s, grid_alloc(outs[0])};
  {
    const int rc = dev_alloc((void**)&states.p, states.bytes, s, "igc_conv_grid: chain state", states.a);
    if (rc) return rc;
  }
  BuildState* hd = nullptr;
  BuildState* h = (BuildState*)host_staging(sizeof(BuildState) * (size_t)n, (void**)&hd);
  if (!h || !hd) return set_error(IGC_ERR_OOM, "igc_conv_grid: pinned staging buffer");

  int first = 0, syncs = 0;
  for (int attempt = 0; attempt <= 2 * n + 2; ++attempt) {
    // Output blocks of stages first .. n-1.
    for (int k = first; k < n; ++k) {
      igc_grid* g = outs[k];
      if (g->block) {
        dev_free(g->block, g->bytes, s, grid_alloc(g));
        g->block = nullptr;
        g->bytes = 0;
      }
      size_t zero_end = 0;
      const size_t bytes = derive_topology_bytes(d[(size_t)k], &zero_end);
      int rc = dev_alloc(&g->block, bytes, s, "igc_conv_grid: topology", grid_alloc(g));
      if (rc) return rc;
      g->bytes = bytes;
      derive_carve(d[(size_t)k], g);
    }
    // One workspace for the largest stage (stages run in stream order).
    size_t ws_bytes = 0;
    DeriveWs w{};
    for (int k = first; k < n; ++k) ws_bytes = std::max(ws_bytes, derive_ws_bytes(d[(size_t)k], &w, nullptr));
    Workspace wsb;
    int rc = ws_acquire(&wsb, ws_bytes, s, "igc_conv_grid: workspace", grid_alloc(outs[0]));
    if (rc) return rc;
    char* base = (char*)wsb.p;
    for (int k = first; k < n && rc == IGC_OK; ++k) {
      derive_ws_bytes(d[(size_t)k], &w, base);
      const igc_grid* src = k == 0 ? in : outs[k - 1];
      const uint64_t* in_counts = k == 0 ? nullptr : states.p[k - 1].counts;
      rc = derive_enqueue(src, in_counts, d[(size_t)k], w, outs[k], &states.p[k], hd + k, s);
    }
    if (rc == IGC_OK) {
      const hipError_t e = hipStreamSynchronize(s);  // the chain's one read-back
      ++syncs;
      if (e != hipSuccess) rc = hip_status(e, "igc_conv_grid: synchronize");
    }
    ws_release(&wsb, s);
    if (rc) return rc;
    int bad = -1;
    for (int k = first; k < n; ++k) {
      const BuildState& r = h[k];
      if (r.range) return set_error(IGC_ERR_RANGE, "igc_conv_grid: an output coordinate leaves the int32 range");
      if (r.n_tiles > (uint32_t)kSmallSort)
        return set_error(IGC_ERR_UNSUPPORTED, "igc_conv_grid: more than 4096 root tiles in a derived grid");
      DeriveStage& c = d[(size_t)k];
      if (!r.overflow && (int64_t)r.n_tiles > c.U) {  // more root tiles than planned: exact count next time
        c.U = (int64_t)r.n_tiles;
        c.F = std::max(c.F, c.U);
        c.Lw = std::max(c.Lw, c.U);
        while ((int64_t)c.root < 2 * c.U) c.root <<= 1;
        c.exact = true;
        bad = k;
        break;
      }
      if (r.overflow) {  // root table too small: the tiles were not all inserted
        c.root <<= 2;
        c.U = std::min<int64_t>(kSmallSort, std::max<int64_t>(c.U, (int64_t)r.n_tiles) * 2);
        bad = k;
        break;
      }
      if (r.cap_over) {
        c.F = std::max<int64_t>(1, (int64_t)r.counts[1]);
        c.Lw = std::max<int64_t>(1, (int64_t)r.counts[2]);
        c.U = std::max<int64_t>(1, (int64_t)r.counts[3]);
        c.exact = true;
        bad = k;
        break;
      }
      if (r.guard) return set_error(IGC_ERR_INTERNAL, "igc_conv_grid: device bounds check failed");
      const int64_t N = (int64_t)r.counts[0], F = (int64_t)r.counts[1], Lw = (int64_t)r.counts[2],
                    U = (int64_t)r.counts[3];
      if (F > c.F || Lw > c.Lw || U > c.U || (int64_t)r.n_tiles != U || (F > 0) != (N > 0) || N > 512 * F)
        return set_error(IGC_ERR_INTERNAL, "igc_conv_grid: inconsistent derived counts");
    }
    if (bad < 0) {
      for (int k = 0; k < n; ++k) {
        const BuildState& r = h[k];
        igc_grid* g = outs[k];
        g->n_voxels = (int64_t)r.counts[0];
        g->n_leaf = (int64_t)r.counts[1];
        g->n_lower = (int64_t)r.counts[2];
        g->n_upper = (int64_t)r.counts[3];
        g->n_input = k == 0 ? in->n_voxels : outs[k - 1]->n_voxels;
        g->sort_passes = 0;
        g->host_syncs = syncs;
      }
      return IGC_OK;
    }
    // Later stages are planned again from the corrected capacities.
    for (int k = bad; k < n; ++k) plan(k);
    for (int k = bad; k < n; ++k)
      if (d[(size_t)k].R >= (1ll << d[(size_t)k].ib))
        return set_error(IGC_ERR_UNSUPPORTED, "igc_conv_grid: too many output-leaf records for one derived grid");
    first = bad;
  }
  return set_error(IGC_ERR_CAPACITY, "igc_conv_grid: derived grid capacities still too small after retries");
}

}  // namespace igc
