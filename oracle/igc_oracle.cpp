// CPU oracle for the IndexGrid build, the coordinate -> index query, the neighbour
// (kernel) map and the 3x3x3 submanifold sparse convolution.
//
// TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
// CPU-baseline leg may load this library. It shares no code, header, table or helper
// with the HIP library: it is written from the definitions below and nothing else.
//
// Every result here has a plain definition, so the oracle is that definition written
// out with standard containers and loops:
//
//  * IndexGrid, "IndexGrid: separating topology from values" in the fVDB paper notes
//    (woaixuexisr.github.io, notes on "fVDB: A Deep-Learning Framework for Sparse, Large
//    Scale, and High Performance Spatial Intelligence"): a VDB tree with a hashed root and
//    dense child nodes of fanout 32, 16 and 8 per axis (4096^3, 128^3 and 8^3 voxels per
//    node, "core method" section) that returns, for an active voxel, an index into an
//    external linear array. Only active voxels are indexed.
//  * The linear order is the order the GPU build of the same notes produces ("GPU-
//    accelerated IndexGrid build"): coordinates grouped by 4096^3 root tile (the 64-bit
//    key of i,j,k each shifted right by 12 and packed 21+21+21 bits), then by the in-tile
//    upper / lower / leaf offsets. Written here as a lexicographic tuple comparison.
//  * Leaf encoding ("IndexGrid" section): index = leaf offset + active count of the
//    preceding 64-bit mask words (bitmask prefix sum) + popcount of the masked word.
//  * Neighbour map (DriveRT page, "Shared neighbour maps"; fVDB notes, sparse-conv
//    operators): for each output row and each kernel offset, the row of the input voxel at
//    coordinate + offset, or -1.
//  * Submanifold convolution (fVDB notes, sparse-conv operators): outputs exist exactly at
//    the active input voxels; out(x) = sum over offsets d of W[d]^T in(x + d), where
//    inactive neighbours contribute zero. Accumulated in double precision.
//
// Readings where the pages are silent (each one is also listed in the design notes):
//  * key layout: i in the most significant 21-bit field, k in the least; the >>12 is a
//    logical shift of the 32-bit two's-complement pattern.
//  * child order inside every node is x-major: child = (x * n + y) * n + z.
//  * the leaf's 512 bits are 8 words of 64; word = i & 7, bit = (j & 7) * 8 + (k & 7).
//  * prefix[w], w = 1..7, is the active count of words 0..w-1, packed 9 bits each at bit
//    9 * (w - 1) of one 64-bit word (7 * 9 = 63 bits); the leaf offset is a 64-bit word.
//  * offsets are enumerated o = (di+1)*9 + (dj+1)*3 + (dk+1) by the callers; the map
//    takes any list of offsets.
//  * neighbour coordinates that leave the int32 range are absent (no wrap-around).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

struct Coord {
  int32_t i, j, k;
  bool operator==(const Coord& o) const { return i == o.i && j == o.j && k == o.k; }
};

struct CoordHash {
  size_t operator()(const Coord& c) const {
    uint64_t h = (uint64_t)(uint32_t)c.i;
    h = h * 0x9E3779B97F4A7C15ull ^ (uint64_t)(uint32_t)c.j;
    h = h * 0xC2B2AE3D27D4EB4Full ^ (uint64_t)(uint32_t)c.k;
    h ^= h >> 29;
    return (size_t)(h * 0x165667B19E3779F9ull);
  }
};

// Per-axis fields of one coordinate at each tree level (fanouts 32, 16, 8).
inline uint32_t tile_of(int32_t x) { return (uint32_t)x >> 12; }        // 4096 voxels per root tile
inline uint32_t upper_child(int32_t x) { return ((uint32_t)x & 4095u) >> 7; }  // 32 lowers per axis
inline uint32_t lower_child(int32_t x) { return ((uint32_t)x & 127u) >> 3; }   // 16 leaves per axis
inline uint32_t leaf_voxel(int32_t x) { return (uint32_t)x & 7u; }             // 8 voxels per axis

// Lexicographic comparison of the tuples
//   (tile_i, tile_j, tile_k, upper_i, upper_j, upper_k, lower_i, lower_j, lower_k, leaf_i, leaf_j, leaf_k)
bool canonical_less(const Coord& a, const Coord& b) {
  const uint32_t ta[12] = {tile_of(a.i),     tile_of(a.j),     tile_of(a.k),
                           upper_child(a.i), upper_child(a.j), upper_child(a.k),
                           lower_child(a.i), lower_child(a.j), lower_child(a.k),
                           leaf_voxel(a.i),  leaf_voxel(a.j),  leaf_voxel(a.k)};
  const uint32_t tb[12] = {tile_of(b.i),     tile_of(b.j),     tile_of(b.k),
                           upper_child(b.i), upper_child(b.j), upper_child(b.k),
                           lower_child(b.i), lower_child(b.j), lower_child(b.k),
                           leaf_voxel(b.i),  leaf_voxel(b.j),  leaf_voxel(b.k)};
  return std::lexicographical_compare(ta, ta + 12, tb, tb + 12);
}

inline int32_t node_origin(int32_t x, uint32_t size) { return (int32_t)((uint32_t)x & ~(size - 1u)); }

struct OracleGrid {
  std::vector<Coord> voxels;                                // active voxels in linear-index order
  std::unordered_map<Coord, int64_t, CoordHash> index;      // coordinate -> linear index

  // Topology in tree (depth-first) order.
  std::vector<uint64_t> root_key;         // [U]   packed tile key of each upper node
  std::vector<int32_t> upper_origin;      // [U,3]
  std::vector<uint64_t> upper_mask;       // [U,512] child mask, bit = (ui*32+uj)*32+uk
  std::vector<uint32_t> upper_first;      // [U]   first lower node of the upper node
  std::vector<int32_t> lower_origin;      // [Lw,3]
  std::vector<uint64_t> lower_mask;       // [Lw,64] child mask, bit = (li*16+lj)*16+lk
  std::vector<uint32_t> lower_first;      // [Lw]  first leaf of the lower node
  std::vector<int32_t> leaf_origin;       // [F,3]
  std::vector<uint64_t> leaf_mask;        // [F,8] voxel mask, word = fi, bit = fj*8+fk
  std::vector<uint64_t> leaf_offset;      // [F]   linear index of the leaf's first active voxel
  std::vector<uint64_t> leaf_prefix;      // [F]   7 x 9-bit active counts of the preceding words
};

}  // namespace

extern "C" {

// Builds the oracle grid from n coordinates int32[n,3] (any order, duplicates allowed).
// Returns nullptr only if n < 0 or coords is null with n > 0.
void* orc_build(const int32_t* coords, int64_t n) {
  if (n < 0 || (n > 0 && coords == nullptr)) return nullptr;
  auto* g = new OracleGrid();

  // Dedupe: one entry per distinct coordinate.
  std::unordered_map<Coord, int64_t, CoordHash> seen;
  seen.reserve((size_t)n * 2 + 16);
  std::vector<Coord> uniq;
  for (int64_t r = 0; r < n; ++r) {
    Coord c{coords[3 * r], coords[3 * r + 1], coords[3 * r + 2]};
    if (seen.emplace(c, 0).second) uniq.push_back(c);
  }
  seen.clear();

  // Linear order.
  std::sort(uniq.begin(), uniq.end(), canonical_less);
  g->voxels = std::move(uniq);
  g->index.reserve(g->voxels.size() * 2 + 16);
  for (size_t r = 0; r < g->voxels.size(); ++r) g->index.emplace(g->voxels[r], (int64_t)r);

  // Topology: walk the voxels in order; a new node starts where its key prefix changes.
  bool have = false;
  Coord prev{0, 0, 0};
  for (size_t r = 0; r < g->voxels.size(); ++r) {
    const Coord c = g->voxels[r];
    const bool new_upper = !have || tile_of(c.i) != tile_of(prev.i) || tile_of(c.j) != tile_of(prev.j) ||
                           tile_of(c.k) != tile_of(prev.k);
    const bool new_lower = new_upper || upper_child(c.i) != upper_child(prev.i) ||
                           upper_child(c.j) != upper_child(prev.j) || upper_child(c.k) != upper_child(prev.k);
    const bool new_leaf = new_lower || lower_child(c.i) != lower_child(prev.i) ||
                          lower_child(c.j) != lower_child(prev.j) || lower_child(c.k) != lower_child(prev.k);
    if (new_upper) {
      const uint64_t key = ((uint64_t)tile_of(c.i) << 42) | ((uint64_t)tile_of(c.j) << 21) | (uint64_t)tile_of(c.k);
      g->root_key.push_back(key);
      g->upper_origin.insert(g->upper_origin.end(),
                             {node_origin(c.i, 4096), node_origin(c.j, 4096), node_origin(c.k, 4096)});
      g->upper_mask.insert(g->upper_mask.end(), 512, 0ull);
      g->upper_first.push_back((uint32_t)(g->lower_first.size()));
    }
    if (new_lower) {
      const size_t u = g->root_key.size() - 1;
      const uint32_t child = (upper_child(c.i) * 32u + upper_child(c.j)) * 32u + upper_child(c.k);
      g->upper_mask[u * 512 + child / 64] |= 1ull << (child % 64);
      g->lower_origin.insert(g->lower_origin.end(),
                             {node_origin(c.i, 128), node_origin(c.j, 128), node_origin(c.k, 128)});
      g->lower_mask.insert(g->lower_mask.end(), 64, 0ull);
      g->lower_first.push_back((uint32_t)(g->leaf_offset.size()));
    }
    if (new_leaf) {
      const size_t l = g->lower_first.size() - 1;
      const uint32_t child = (lower_child(c.i) * 16u + lower_child(c.j)) * 16u + lower_child(c.k);
      g->lower_mask[l * 64 + child / 64] |= 1ull << (child % 64);
      g->leaf_origin.insert(g->leaf_origin.end(), {node_origin(c.i, 8), node_origin(c.j, 8), node_origin(c.k, 8)});
      g->leaf_mask.insert(g->leaf_mask.end(), 8, 0ull);
      g->leaf_offset.push_back((uint64_t)r);
      g->leaf_prefix.push_back(0);
    }
    const size_t f = g->leaf_offset.size() - 1;
    g->leaf_mask[f * 8 + leaf_voxel(c.i)] |= 1ull << (leaf_voxel(c.j) * 8u + leaf_voxel(c.k));
    prev = c;
    have = true;
  }
  // Bitmask prefix sums.
  for (size_t f = 0; f < g->leaf_offset.size(); ++f) {
    uint64_t packed = 0, running = 0;
    for (int w = 1; w < 8; ++w) {
      running += (uint64_t)__builtin_popcountll(g->leaf_mask[f * 8 + w - 1]);
      packed |= running << (9 * (w - 1));
    }
    g->leaf_prefix[f] = packed;
  }
  return g;
}

void orc_free(void* h) { delete static_cast<OracleGrid*>(h); }

// counts[0..3] = N (active voxels), F (leaves), Lw (lower nodes), U (upper nodes).
void orc_counts(const void* h, int64_t* counts) {
  const auto* g = static_cast<const OracleGrid*>(h);
  counts[0] = (int64_t)g->voxels.size();
  counts[1] = (int64_t)g->leaf_offset.size();
  counts[2] = (int64_t)g->lower_first.size();
  counts[3] = (int64_t)g->root_key.size();
}

// Copies the topology into caller buffers sized from orc_counts (any pointer may be null).
void orc_export(const void* h, uint64_t* root_key, int32_t* upper_origin, uint64_t* upper_mask,
                uint32_t* upper_first, int32_t* lower_origin, uint64_t* lower_mask, uint32_t* lower_first,
                int32_t* leaf_origin, uint64_t* leaf_mask, uint64_t* leaf_offset, uint64_t* leaf_prefix) {
  const auto* g = static_cast<const OracleGrid*>(h);
  auto put = [](auto* dst, const auto& v) {
    if (dst && !v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(v[0]));
  };
  put(root_key, g->root_key);
  put(upper_origin, g->upper_origin);
  put(upper_mask, g->upper_mask);
  put(upper_first, g->upper_first);
  put(lower_origin, g->lower_origin);
  put(lower_mask, g->lower_mask);
  put(lower_first, g->lower_first);
  put(leaf_origin, g->leaf_origin);
  put(leaf_mask, g->leaf_mask);
  put(leaf_offset, g->leaf_offset);
  put(leaf_prefix, g->leaf_prefix);
}

// Active voxel coordinates int32[N,3] in linear-index order.
void orc_active_ijk(const void* h, int32_t* out) {
  const auto* g = static_cast<const OracleGrid*>(h);
  for (size_t r = 0; r < g->voxels.size(); ++r) {
    out[3 * r] = g->voxels[r].i;
    out[3 * r + 1] = g->voxels[r].j;
    out[3 * r + 2] = g->voxels[r].k;
  }
}

// Linear index of each query coordinate, -1 if it is not an active voxel.
void orc_ijk_to_index(const void* h, const int32_t* q, int64_t m, int32_t* out) {
  const auto* g = static_cast<const OracleGrid*>(h);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < m; ++r) {
    auto it = g->index.find(Coord{q[3 * r], q[3 * r + 1], q[3 * r + 2]});
    out[r] = it == g->index.end() ? -1 : (int32_t)it->second;
  }
}

// map[o, r] (int32[K, N]) = index of voxel r + offsets[o], or -1.
// nbmask (uint32[N], may be null) gets bit o set when map[o, r] >= 0 (K <= 32).
void orc_kernel_map(const void* h, const int32_t* offsets, int32_t K, int32_t* map, uint32_t* nbmask) {
  const auto* g = static_cast<const OracleGrid*>(h);
  const int64_t N = (int64_t)g->voxels.size();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < N; ++r) {
    const Coord c = g->voxels[r];
    uint32_t bits = 0;
    for (int32_t o = 0; o < K; ++o) {
      const int64_t ni = (int64_t)c.i + offsets[3 * o];
      const int64_t nj = (int64_t)c.j + offsets[3 * o + 1];
      const int64_t nk = (int64_t)c.k + offsets[3 * o + 2];
      int32_t found = -1;
      if (ni >= INT32_MIN && ni <= INT32_MAX && nj >= INT32_MIN && nj <= INT32_MAX && nk >= INT32_MIN &&
          nk <= INT32_MAX) {
        auto it = g->index.find(Coord{(int32_t)ni, (int32_t)nj, (int32_t)nk});
        if (it != g->index.end()) found = (int32_t)it->second;
      }
      map[(int64_t)o * N + r] = found;
      if (found >= 0 && o < 32) bits |= 1u << o;
    }
    if (nbmask) nbmask[r] = bits;
  }
}

// Submanifold convolution for the output rows `rows` (int64[n_rows]; null = all N rows in
// order): out[t, co] = sum_o sum_ci feats[map[o, rows[t]], ci] * w[o, ci, co] over map >= 0,
// in double precision. feats float32[N, cin], w float32[K, cin, cout], out double[n_rows, cout].
void orc_conv(const int32_t* map, int64_t N, int32_t K, const float* feats, int32_t cin, const float* w,
              int32_t cout, const int64_t* rows, int64_t n_rows, double* out) {
  const int64_t R = rows ? n_rows : N;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t t = 0; t < R; ++t) {
    const int64_t r = rows ? rows[t] : t;
    double* acc = out + t * cout;
    for (int32_t co = 0; co < cout; ++co) acc[co] = 0.0;
    for (int32_t o = 0; o < K; ++o) {
      const int32_t s = map[(int64_t)o * N + r];
      if (s < 0) continue;
      for (int32_t ci = 0; ci < cin; ++ci) {
        const double x = (double)feats[(int64_t)s * cin + ci];
        const float* wr = w + ((int64_t)o * cin + ci) * cout;
        for (int32_t co = 0; co < cout; ++co) acc[co] += x * (double)wr[co];
      }
    }
  }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
