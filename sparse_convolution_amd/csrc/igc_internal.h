// Internal data layout of the IndexGrid on the device and the lookups every kernel shares.
//
// Tree (fVDB notes, "core method"): a hashed root of 4096^3 tiles, upper nodes with 32^3
// children, lower nodes with 16^3 children, leaves of 8^3 voxels. As in the IndexGrid
// ("IndexGrid: separating topology from values"), nodes store topology only and the leaf
// turns a coordinate into a row of an external feature array with a mask test, a prefix
// count and a popcount of the masked word.
//
// Internal nodes are stored the same way as leaves: a child bit mask plus per-word prefix
// counts, so child c of node n is first[n] + prefix[n][c/64] + popcount(mask[n][c/64] below
// bit c%64). Children of a node are consecutive in the depth-first order, which is what
// makes this compact form possible; it replaces a dense child table (128 KB per upper node,
// 16 KB per lower node) by 5 KB and 640 B.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace igc {

constexpr uint64_t kEmptyKey = ~0ull;  // packed tile keys use 62 bits, so ~0 never occurs

// Leaf index record: 8 mask words + first row + 7 packed 9-bit prefix counts = 80 bytes.
struct LeafRec {
  uint64_t mask[8];
  uint64_t offset;
  uint64_t prefix;
};
static_assert(sizeof(LeafRec) == 80, "leaf index record is 80 bytes");

// Read-only view of a built grid, passed to kernels by value.
struct GridView {
  const uint64_t* root_keys;    // [cap] hash slots (kEmptyKey = free)
  const int32_t* root_vals;     // [cap] upper node of the slot's tile
  uint32_t root_mask;           // cap - 1 (cap is a power of two)
  const uint64_t* upper_mask;   // [U*512]
  const uint16_t* upper_pre;    // [U*512]
  const uint32_t* upper_first;  // [U]
  const uint64_t* lower_mask;   // [Lw*64]
  const uint16_t* lower_pre;    // [Lw*64]
  const uint32_t* lower_first;  // [Lw]
  const LeafRec* leaf;          // [F]
  const int4* leaf_origin;      // [F] (i, j, k, 0)
  const int32_t* leaf_nbr;      // [F*27] leaf at origin + 8*(di,dj,dk), slot (di+1)*9+(dj+1)*3+(dk+1), -1 absent
  int64_t n_voxels;
  int64_t n_leaf;
};

// 64-bit mix (the splitmix64 finaliser) used for the root hash.
__host__ __device__ inline uint32_t hash_tile(uint64_t k) {
  k ^= k >> 30;
  k *= 0xBF58476D1CE4E5B9ull;
  k ^= k >> 27;
  k *= 0x94D049BB133111EBull;
  k ^= k >> 31;
  return (uint32_t)k;
}

// Packed root-tile key: each coordinate's 32-bit pattern shifted right by 12, i in the
// most significant 21-bit field.
__host__ __device__ inline uint64_t tile_key(int32_t i, int32_t j, int32_t k) {
  return ((uint64_t)((uint32_t)i >> 12) << 42) | ((uint64_t)((uint32_t)j >> 12) << 21) |
         (uint64_t)((uint32_t)k >> 12);
}

// In-tile offset: upper child (15 bits) << 21 | lower child (12 bits) << 9 | leaf voxel (9 bits).
__host__ __device__ inline uint64_t tile_offset(int32_t i, int32_t j, int32_t k) {
  const uint32_t ui = (uint32_t)i, uj = (uint32_t)j, uk = (uint32_t)k;
  const uint64_t up = (((ui >> 7) & 31u) << 10) | (((uj >> 7) & 31u) << 5) | ((uk >> 7) & 31u);
  const uint64_t lo = (((ui >> 3) & 15u) << 8) | (((uj >> 3) & 15u) << 4) | ((uk >> 3) & 15u);
  const uint64_t lf = ((ui & 7u) << 6) | ((uj & 7u) << 3) | (uk & 7u);
  return (up << 21) | (lo << 9) | lf;
}

__device__ inline int32_t find_upper(const GridView& g, uint64_t key) {
  uint32_t s = hash_tile(key) & g.root_mask;
  for (uint32_t p = 0; p <= g.root_mask; ++p) {
    const uint64_t k = g.root_keys[s];
    if (k == key) return g.root_vals[s];
    if (k == kEmptyKey) return -1;
    s = (s + 1) & g.root_mask;
  }
  return -1;
}

// Row of the child bit c of a compact node (mask / prefix / first), or -1.
__device__ inline int32_t node_child(const uint64_t* mask, const uint16_t* pre, uint32_t first, uint32_t c) {
  const uint64_t w = mask[c >> 6];
  const uint64_t bit = 1ull << (c & 63u);
  if (!(w & bit)) return -1;
  return (int32_t)(first + pre[c >> 6] + (uint32_t)__popcll(w & (bit - 1ull)));
}

// Leaf containing (i, j, k), or -1.
__device__ inline int32_t find_leaf(const GridView& g, int32_t i, int32_t j, int32_t k) {
  const int32_t u = find_upper(g, tile_key(i, j, k));
  if (u < 0) return -1;
  const uint32_t ui = (uint32_t)i, uj = (uint32_t)j, uk = (uint32_t)k;
  const uint32_t cu = (((ui >> 7) & 31u) << 10) | (((uj >> 7) & 31u) << 5) | ((uk >> 7) & 31u);
  const int32_t l = node_child(g.upper_mask + (size_t)u * 512, g.upper_pre + (size_t)u * 512, g.upper_first[u], cu);
  if (l < 0) return -1;
  const uint32_t cl = (((ui >> 3) & 15u) << 8) | (((uj >> 3) & 15u) << 4) | ((uk >> 3) & 15u);
  return node_child(g.lower_mask + (size_t)l * 64, g.lower_pre + (size_t)l * 64, g.lower_first[l], cl);
}

// Row of voxel n = (x*8 + y)*8 + z of a leaf given its 8 words, offset and packed prefix.
// The two branches: the bit test, and word 0 having no prefix field.
__device__ inline int32_t leaf_row(const uint64_t* mask, uint64_t offset, uint64_t prefix, uint32_t n) {
  const uint32_t w = n >> 6;
  const uint64_t word = mask[w];
  const uint64_t bit = 1ull << (n & 63u);
  if (!(word & bit)) return -1;
  const uint32_t pre = w ? (uint32_t)(prefix >> (9u * (w - 1u))) & 511u : 0u;
  return (int32_t)(offset + pre + (uint32_t)__popcll(word & (bit - 1ull)));
}

}  // namespace igc
