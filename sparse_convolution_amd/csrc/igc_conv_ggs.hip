// Gather-GEMM-scatter submanifold convolution, bf16 inputs / weights / outputs with fp32
// accumulation on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// fVDB notes, "accelerated operators for sparse convolution", third case: work is tiled over
// consecutive output rows, a workgroup-local buffer replaces global scatter, and for each of
// the 27 stencil offsets the tile's (input, output) pairs feed a tensor-core GEMM, with the
// pairs of each offset padded to a multiple of 16 rows.
//
// gfx950 form, in two kernels:
//
// k_ggs_plan, one workgroup per span of 256, 1024 or 4096 consecutive output rows: each row's
// 27-bit neighbour mask (bit o set when the kernel map has a neighbour at offset o) is read
// from the map, the span's rows are sorted by that mask (in a configurable bit order) and cut
// into tiles of 256, and for every offset a 16-bit mask records which 16-row blocks of a tile
// hold at least one pair. Sorting groups rows with the same neighbour set (DriveRT, "Kernels
// selected per GPU": rows sorted by their 27-bit neighbour mask give threads uniform work), so
// the pages' per-offset pair lists padded to 16 become "the blocks whose bit is set", and each
// tile computes only its own group of offsets; span and bit order are chosen per layer
// (igc_tuning_load).
//
// k_conv_ggs_bf16, one workgroup per tile x BN output channels (or per half tile: 128 rows of a
// plan tile with their own offset group, chosen per layer, so that two workgroups share a CU),
// output-stationary: the fp32 accumulators of the 256 x BN tile stay in registers for the whole reduction, so
// every offset's product is "scattered" into registers and each output row is written once,
// with no atomics and a fixed summation order (deterministic). The reduction runs over chunks
// (used offset, KC input channels): the tile's input rows of that offset are gathered by the
// kernel map (absent neighbours read a zero row) into LDS next to the matching BN x KC slice
// of W[o]^T, and each wave multiplies its (256/WM) x (BN/WN) sub-tile with 16x16x32 MFMAs,
// skipping the chunks in which none of its 16-row blocks has a pair at that offset. Both operands go from global
// memory straight into LDS (global_load_lds_dwordx4: no staging registers, which the 256 x 256
// accumulators leave none of); the next chunk's loads are in flight while the current chunk is
// multiplied (two LDS stages, one barrier per chunk). The tile's map entries of every used
// offset are staged in LDS once, so the gather never waits on the map. The output tile is
// staged through LDS and leaves as whole rows.
//
// Staged rows are unpadded and their 16-byte granules XOR-swizzled by row, so the rows read
// together by one fragment load fall on distinct banks. Workgroups are numbered so that each
// of the eight XCDs (each with its own L2) walks a contiguous range of row tiles: neighbouring
// output rows gather neighbouring input rows, and those stay in one L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;  // output rows per tile (= threads per workgroup)
constexpr int kNOff = 27;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));  // inf / nan
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Block index -> tile index such that XCD x (blocks x, x+8, ...) gets a contiguous range.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t nblk) {
  const int64_t x = bid & 7, q = nblk >> 3, rem = nblk & 7;
  return x * q + (x < rem ? x : rem) + (bid >> 3);
}

// Wt[o][n][k] = W[o][k][n] (bf16 as 16-bit words).
// wt[o][n][k] = w[o][k][n], by workgroup b of nb (256 threads each).
__device__ __forceinline__ void transpose_w(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt, int cin,
                                            int cout, int64_t b, int64_t nb) {
  const int64_t total = 27ll * cin * cout;
  for (int64_t e = b * 256 + threadIdx.x; e < total; e += nb * 256) {
    const int64_t o = e / ((int64_t)cin * cout);
    const int64_t rem = e - o * cin * cout;
    const int64_t n = rem / cin, k = rem - n * cin;
    wt[e] = w[(o * cin + k) * cout + n];
  }
}

// Row order of the tiles (the plan). Rows are sorted by their 27-bit neighbour mask within
// spans of SPAN consecutive rows (DriveRT, "Kernels selected per GPU": rows sorted by the mask
// execute the same work), and the sorted rows are cut into tiles of 256:
//   perm[q] = output row at sorted position q (-1 past N; positions below n_pos only), and
//   blk[tile*27 + o] bit b = some row at sorted positions [16b, 16b+16) of the tile has a
//   neighbour at o.
// A tile then computes only its own group of offsets (those with a bit in blk), and a wider span
// makes the groups smaller at the cost of gathering from a wider stretch of rows; the span and
// the bit order of the key (which offsets are the most significant) are configuration values
// measured per layer. The key of local row r is (the complemented mask with offset order[i] at
// bit 26 - i) << log2(SPAN) | r: equal masks stay in row order, rows without neighbours (and
// the padding past N) sort last. A map entry counts as a neighbour when it lies in [0, n_in).
// Rows with skip[row] != 0 (per-leaf dispatch: another path writes them) count as having none.
//
// One workgroup of 256 threads per span, K = SPAN / 256 keys per thread in registers. Spans of
// 1024 and 4096 rows sort with every compare-exchange between two registers of one thread: a
// layout keeps RB = log2(K) consecutive bits [lo, lo + RB) of a key's position in the register
// number and the other bits in the thread number, and moves to the group of bits the next
// stages need by writing every key to LDS at its position and reading the new layout back
// (22 such moves for 4096 rows, in place of 57 cross-lane and 18 LDS stages). Spans of 256
// rows (one key per thread) exchange across lanes and through LDS. Then each 16-row block's
// masks are OR-reduced across its lanes and lane o < 27 sets offset o's bits of four blocks.
struct BitOrder {
  uint8_t o[kNOff];  // o[i]: offset at key bit 26 - i
};

template <int SPAN>
__global__ __launch_bounds__(256) void k_ggs_plan(const int32_t* __restrict__ map, int64_t N, int64_t n_in,
                                                 int32_t* __restrict__ perm, int64_t n_pos,
                                                 uint16_t* __restrict__ blk, const uint8_t* __restrict__ skip,
                                                 BitOrder bo, int64_t n_plan, const uint16_t* __restrict__ w,
                                                 uint16_t* __restrict__ wt, int cin, int cout) {
  // Workgroups past the plan's transpose the weights for the conv (independent work in the same
  // launch, one dependent launch fewer per conv).
  if ((int64_t)blockIdx.x >= n_plan) {
    transpose_w(w, wt, cin, cout, (int64_t)blockIdx.x - n_plan, (int64_t)gridDim.x - n_plan);
    return;
  }
  constexpr int T = 256, TB = 8;
  constexpr int K = SPAN / T;
  constexpr int RB = K == 16 ? 4 : K == 4 ? 2 : 0;
  constexpr int LB = SPAN == 256 ? 8 : SPAN == 1024 ? 10 : 12;
  constexpr int NT = SPAN / kBM;  // tiles per span
  static_assert(SPAN == 256 || SPAN == 1024 || SPAN == 4096, "span");
  __shared__ uint64_t s_x[SPAN + SPAN / 32];
  __shared__ uint32_t s_mask[SPAN];
  __shared__ uint32_t s_blk[NT][kNOff];
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int64_t base = (int64_t)blockIdx.x * SPAN;
  for (int x = t; x < NT * kNOff; x += T) (&s_blk[0][0])[x] = 0u;

  // Masks of local rows q * T + t (coalesced map reads; the loop is not unrolled so that only
  // one row's 27 loads hold registers), then key q of thread t from its own masks.
#pragma unroll 1
  for (int q = 0; q < K; ++q) {
    const int local = q * T + t;
    const int64_t row = base + local;
    uint32_t mask = 0;
    if (row < N && !(skip && skip[row])) {
      int32_t v[kNOff];
#pragma unroll
      for (int o = 0; o < kNOff; ++o) v[o] = map[(size_t)o * (size_t)N + row];
#pragma unroll
      for (int o = 0; o < kNOff; ++o) mask |= ((uint64_t)(int64_t)v[o] < (uint64_t)n_in ? 1u : 0u) << o;
    }
    s_mask[local] = mask;
  }
  uint64_t key[K];
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int local = q * T + t;
    const uint32_t mask = s_mask[local];
    uint64_t pk = 0;
#pragma unroll
    for (int b = 0; b < kNOff; ++b) pk |= (uint64_t)((~mask >> bo.o[b]) & 1u) << (kNOff - 1 - b);
    key[q] = (pk << LB) | (uint64_t)local;
  }

  if constexpr (K == 1) {
    for (int k = 2; k <= SPAN; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        uint64_t other;
        if (j < 64) {
          other = shfl_xor64(key[0], j);
        } else {
          __syncthreads();
          s_x[t] = key[0];
          __syncthreads();
          other = s_x[t ^ j];
        }
        const bool asc = (t & k) == 0, lower = (t & j) == 0;
        const uint64_t a = key[0];
        key[0] = (lower == asc) ? (a < other ? a : other) : (a < other ? other : a);
      }
    }
  } else {
    // Position of key q of thread t in layout lo: bits [lo, lo + RB) from q, the rest from t.
    auto slot = [](int p) { return p + (p >> 5); };  // one spare word per 32 keys against bank conflicts
    auto tpart = [&](int l) { return (t & ((1 << l) - 1)) | ((t >> l) << (l + RB)); };
    int lo = TB;  // the load's layout: position q * T + t
    auto remap = [&](int nlo) {
      const int tp = tpart(lo);
      __syncthreads();
#pragma unroll
      for (int q = 0; q < K; ++q) s_x[slot(tp | (q << lo))] = key[q];
      __syncthreads();
      const int tn = tpart(nlo);
#pragma unroll
      for (int q = 0; q < K; ++q) key[q] = s_x[slot(tn | (q << nlo))];
      lo = nlo;
    };
    for (int k = 2; k <= SPAN; k <<= 1) {
      for (int b = __builtin_ctz(k) - 1; b >= 0; --b) {
        if (b < lo || b >= lo + RB) remap(b - RB + 1 > 0 ? b - RB + 1 : 0);
        const int tp = tpart(lo);
        // Partners differ in register bit d = b - lo (a compile-time stride per case).
        auto cx = [&](auto dc) {
          constexpr int qb = 1 << decltype(dc)::value;
#pragma unroll
          for (int q = 0; q < K; ++q) {
            if (q & qb) continue;
            const bool asc = ((tp | (q << lo)) & k) == 0;
            const uint64_t x = key[q], y = key[q | qb];
            const bool sw = (x > y) == asc;
            key[q] = sw ? y : x;
            key[q | qb] = sw ? x : y;
          }
        };
        switch (b - lo) {
          case 0: cx(std::integral_constant<int, 0>{}); break;
          case 1: cx(std::integral_constant<int, 1>{}); break;
          case 2: if constexpr (RB > 2) cx(std::integral_constant<int, (RB > 2 ? 2 : 0)>{}); break;
          default: if constexpr (RB > 3) cx(std::integral_constant<int, (RB > 3 ? 3 : 0)>{}); break;
        }
      }
    }
    if (lo != TB) remap(TB);
  }

  // Sorted position p = q * T + t: its row, and its tile's block bits (a wave holds 64
  // consecutive positions, four 16-row blocks of one tile).
  __syncthreads();
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int p = q * T + t;
    const int local = (int)(key[q] & (uint64_t)(SPAN - 1));
    const int64_t row = base + local;
    if (base + p < n_pos) perm[base + p] = row < N ? (int32_t)row : -1;
    uint32_t m = s_mask[local];
    m |= (uint32_t)__shfl_xor((int)m, 1);
    m |= (uint32_t)__shfl_xor((int)m, 2);
    m |= (uint32_t)__shfl_xor((int)m, 4);
    m |= (uint32_t)__shfl_xor((int)m, 8);
    const uint32_t g0 = __builtin_amdgcn_readlane(m, 0), g1 = __builtin_amdgcn_readlane(m, 16);
    const uint32_t g2 = __builtin_amdgcn_readlane(m, 32), g3 = __builtin_amdgcn_readlane(m, 48);
    const int tl = p / kBM, quarter = (p % kBM) / 64;
    if (lane < kNOff) {
      const uint32_t bits = ((g0 >> lane) & 1u) | (((g1 >> lane) & 1u) << 1) | (((g2 >> lane) & 1u) << 2) |
                            (((g3 >> lane) & 1u) << 3);
      if (bits) atomicOr(&s_blk[tl][lane], bits << (4 * quarter));
    }
  }
  __syncthreads();
  for (int x = t; x < NT * kNOff; x += T) {
    const int tl = x / kNOff, o = x % kNOff;
    const int64_t tile = base / kBM + tl;
    if (tile * kBM < n_pos) blk[(size_t)tile * kNOff + o] = (uint16_t)s_blk[tl][o];
  }
}

// Natural order (offset o at key bit o) and the class order (corners, then edges, faces and
// the centre, the rarest neighbours most significant).
BitOrder bit_order(int which) {
  BitOrder b{};
  if (which == 0) {
    for (int i = 0; i < kNOff; ++i) b.o[i] = (uint8_t)(kNOff - 1 - i);
    return b;
  }
  int n = 0;
  for (int cls = 3; cls >= 0; --cls)
    for (int o = 0; o < kNOff; ++o) {
      const int nz = (o / 9 != 1) + ((o / 3) % 3 != 1) + (o % 3 != 1);
      if (nz == cls) b.o[n++] = (uint8_t)o;
    }
  return b;
}

// With w non-null, 256 more workgroups of the same launch write wt[o][n][k] = w[o][k][n].
hipError_t launch_plan(int span, int order, const int32_t* map, int64_t N, int64_t n_in, int32_t* perm,
                       uint16_t* blk, const uint8_t* skip, hipStream_t s, const uint16_t* w = nullptr,
                       uint16_t* wt = nullptr, int cin = 0, int cout = 0) {
  const int64_t n_pos = (N + kBM - 1) / kBM * kBM;
  if (n_pos == 0) return hipSuccess;
  const BitOrder bo = bit_order(order);
  const int64_t n_plan = (N + span - 1) / span;
  const unsigned grid = (unsigned)(n_plan + (w ? 256 : 0));
  if (span == 4096)
    k_ggs_plan<4096><<<grid, 256, 0, s>>>(map, N, n_in, perm, n_pos, blk, skip, bo, n_plan, w, wt, cin, cout);
  else if (span == 1024)
    k_ggs_plan<1024><<<grid, 256, 0, s>>>(map, N, n_in, perm, n_pos, blk, skip, bo, n_plan, w, wt, cin, cout);
  else
    k_ggs_plan<256><<<grid, 256, 0, s>>>(map, N, n_in, perm, n_pos, blk, skip, bo, n_plan, w, wt, cin, cout);
  return hipGetLastError();
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Gathered in place of an absent neighbour's row (any channel slice of up to 1024 channels).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[1024];

// 16-byte granule g of staged row r sits at granule g ^ swz(r): with 8 granules per row (64
// channels) the eight rows read together by one fragment load land on eight distinct 4-bank
// groups; with 4 granules per row (32 channels) pairs of rows share a bank half, so rows are
// swizzled in pairs.
template <int SEG>
__device__ __forceinline__ int stage_swz(int r) {
  return SEG == 8 ? (r & 7) : ((r >> 1) & 3);
}

// vmcnt(n): wait until at most n vector-memory operations of this wave are outstanding.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// BN output channels per workgroup, KC input channels per chunk, WM waves along the rows
// (NWV / WM along the channels), NST LDS stages (NST - 1 chunks of loads in flight), NWV waves,
// TBM output rows per workgroup: a whole plan tile (kBM) or a part of one (its rows and their
// 16-row block bits).
template <int BN, int KC, int WM, int NST, int NWV, int TBM>
__global__ __launch_bounds__(64 * NWV) void k_conv_ggs_bf16(const int32_t* __restrict__ map, int64_t N, int64_t n_in,
                                                       const int32_t* __restrict__ perm,
                                                       const uint16_t* __restrict__ blk,
                                                       const uint16_t* __restrict__ feats,
                                                       const uint16_t* __restrict__ wt, int cin, int cout,
                                                       uint16_t* __restrict__ out, int64_t col_tiles) {
  constexpr int NT = 64 * NWV;  // threads
  constexpr int WN = NWV / WM;
  constexpr int MW = TBM / WM;  // rows per wave
  constexpr int NW = BN / WN;   // channels per wave
  constexpr int MI = MW / 16, NI = NW / 16;
  constexpr int SEG = KC / 8;                 // 16-byte granules per staged row
  constexpr int ROWB = KC * 2;                // bytes per staged row
  constexpr int RPI = 64 / SEG;               // rows filled by one wave-wide LDS load
  constexpr int AI = TBM / RPI / NWV;         // A loads per wave and chunk
  constexpr int BI = BN / RPI / NWV;          // B loads per wave and chunk
  constexpr int A_BYTES = TBM * ROWB, B_BYTES = BN * ROWB;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int OUT_ROWS = 128 * BN * 2 <= STAGE_BYTES ? 128 : (64 * BN * 2 <= STAGE_BYTES ? 64 : 32);
  constexpr int NPASS = TBM / OUT_ROWS;
  constexpr int OG = BN / 8;                  // 16-byte granules per output row
  static_assert(MI >= 1 && NI >= 1 && AI >= 1 && BI >= 1, "tile shape");
  static_assert(OUT_ROWS * BN * 2 <= STAGE_BYTES && OG >= 8, "output pass fits one stage");
  static_assert(NST >= 2 && NST <= 6, "stages");
  constexpr int LPC = AI + BI;  // loads per wave and chunk
  static_assert((NST - 2) * LPC < 64, "vmcnt range");
  // Stages as separate objects: the compiler then sees that the loads into one stage never
  // feed the fragment reads of another and does not wait for them.
  __shared__ uint4 s_st0[STAGE_BYTES / 16];
  __shared__ uint4 s_st1[STAGE_BYTES / 16];
  __shared__ uint4 s_st2[NST > 2 ? STAGE_BYTES / 16 : 1];
  __shared__ uint4 s_st3[NST > 3 ? STAGE_BYTES / 16 : 1];
  __shared__ uint4 s_st4[NST > 4 ? STAGE_BYTES / 16 : 1];
  __shared__ uint4 s_st5[NST > 5 ? STAGE_BYTES / 16 : 1];
  __shared__ int32_t s_perm[TBM];
  __shared__ __align__(16) int32_t s_map[kNOff][TBM];
  __shared__ uint16_t s_blk[kNOff];
  __shared__ uint16_t s_blku[kNOff];  // s_blk of the u-th used offset
  __shared__ int s_nused;
  __shared__ uint32_t s_used;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t t_lin = xcd_tile(blockIdx.x, gridDim.x);
  // Rows [part * TBM, (part + 1) * TBM) of plan tile `tile` and their 16-row block bits.
  constexpr int PARTS = kBM / TBM;
  static_assert(PARTS * TBM == kBM && TBM % 16 == 0, "tile rows");
  const int64_t wtile = t_lin / col_tiles;
  const int64_t tile = wtile / PARTS;
  const int part = (int)(wtile % PARTS);
  const int n0 = (int)(t_lin % col_tiles) * BN;

  for (int r = tid; r < TBM; r += NT) s_perm[r] = perm[tile * kBM + part * TBM + r];
  if (tid < kNOff)
    s_blk[tid] = (uint16_t)((blk[tile * kNOff + tid] >> (part * (TBM / 16))) & ((1u << (TBM / 16)) - 1u));
  __syncthreads();
  if (tid < 64) {
    // The used offsets' block bits in ascending offset order: one ballot over lanes 0..26 of
    // wave 0, each written at its rank.
    const uint32_t b = tid < kNOff ? s_blk[tid] : 0u;
    const uint64_t used = __ballot(b != 0u);
    if (b) {
      const int rank = __popcll(used & ((1ull << tid) - 1ull));
      s_blku[rank] = (uint16_t)b;
    }
    if (tid == 0) {
      s_nused = __popcll(used);
      s_used = (uint32_t)used;
    }
  }
  __syncthreads();

  // The tile's kernel-map entries of every used offset, in sorted-row order, go to LDS once:
  // all loads are issued before the first wait, so the map's latency is paid once per tile.
  // An entry outside [0, n_in) is stored as -1 (absent): the gather never leaves the input.
  // Layout: row u holds the u-th used offset, and the AI entries one lane gathers per chunk
  // (rows (w*AI + q)*RPI + l, q < AI) are adjacent, so one vector read fetches them.
  constexpr int RPI_ = 64 / (KC / 8), AI_ = TBM / RPI_ / NWV;
  auto mslot = [&](int row) {
    const int w = row / (AI_ * RPI_), rem = row % (AI_ * RPI_);
    return (w * RPI_ + rem % RPI_) * AI_ + rem / RPI_;
  };
  {
    // TBM rows x 27 offsets over NT threads: thread t takes row t % TBM and every
    // (NT / TBM)-th offset starting at t / TBM.
    constexpr int OSTEP = NT / TBM;
    constexpr int OPT = (kNOff + OSTEP - 1) / OSTEP;
    const int row = tid % TBM, o0 = tid / TBM;
    const int32_t myrow = s_perm[row];
    const uint32_t used = myrow >= 0 ? s_used : 0u;
    int32_t v[OPT];
    // Branch-free: unused entries load element 0 and are replaced by -1.
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int o = o0 + OSTEP * i;
      v[i] = (o < kNOff && ((used >> o) & 1u)) ? map[(size_t)o * (size_t)N + myrow] : map[0];
    }
    const uint32_t listed = s_used;
    const int slot = mslot(row);
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int o = o0 + OSTEP * i;
      if (o < kNOff && ((listed >> o) & 1u))
        s_map[__popc(listed & ((1u << o) - 1u))][slot] =
            ((used >> o) & 1u) && (uint64_t)(int64_t)v[i] < (uint64_t)n_in ? v[i] : -1;
    }
  }
  __syncthreads();

  const int ksl = cin / KC;  // chunks per offset
  const int nchunks = s_nused * ksl;

  // This lane's staged rows: row (wave*AI + q)*RPI + lane/SEG, granule slot lane%SEG, which
  // holds the row's granule (lane%SEG) ^ swz (the swizzle is the same for every q).
  const int gran = (lane % SEG) ^ ((lane >> 3) & (SEG - 1));
  const uint16_t* bptr = wt + (size_t)(n0 + wave * BI * RPI + lane / SEG) * cin + gran * 8;
  // What one chunk's loads need from LDS (its offset, channel slice and this lane's map entries),
  // read one chunk ahead: the reads are in flight while the current chunk is multiplied, so the
  // loads are issued without waiting on LDS.
  struct Pend {
    int o, kc;
    int32_t src[AI];
  };
  const uint16_t* const zrow = g_zero_row + gran * 8;
  static_assert(RPI_ == RPI && AI_ == AI && (AI == 2 || AI == 4), "map slots");
  typedef int32_t i32xAI __attribute__((ext_vector_type(AI)));
  // The chunks in order, as (u-th used offset, channel slice k): the fetch stream walks them one
  // by one, keeping its offset as the lowest bit of the not yet passed used offsets (scalar
  // registers, no LDS read and no division per chunk).
  const int nused = s_nused;
  uint32_t f_mask = __builtin_amdgcn_readfirstlane(s_used);
  int f_u = 0, f_k = 0;
  auto fetch_next = [&]() {
    Pend p;
    const int u = f_u < nused ? f_u : (nused > 0 ? nused - 1 : 0);  // past the end: never issued
    p.o = f_mask ? __builtin_ctz(f_mask) : 0;
    p.kc = f_k * KC;
    const i32xAI src = *(const i32xAI*)&s_map[u][(wave * RPI + lane / SEG) * AI];
#pragma unroll
    for (int q = 0; q < AI; ++q) p.src[q] = src[q];
    if (++f_k == ksl) {
      f_k = 0;
      ++f_u;
      f_mask &= f_mask - 1u;
    }
    return p;
  };
  auto issue = [&](const Pend& p, uint4* st) {
    const int o = p.o, kc = p.kc;
#pragma unroll
    for (int q = 0; q < AI; ++q) {
      const uint16_t* ap = (p.src[q] >= 0 ? feats + (size_t)p.src[q] * cin + gran * 8 : zrow) + kc;
      __builtin_amdgcn_global_load_lds((const glb_void*)ap, (lds_void*)(st + (wave * AI + q) * 64), 16, 0, 0);
    }
    const uint16_t* bsrc = bptr + (size_t)o * cout * cin + kc;
#pragma unroll
    for (int q = 0; q < BI; ++q)
      __builtin_amdgcn_global_load_lds((const glb_void*)(bsrc + (size_t)q * RPI * cin),
                                       (lds_void*)(st + A_BYTES / 16 + (wave * BI + q) * 64), 16, 0, 0);
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fsw = stage_swz<SEG>(frow);  // row bases are multiples of 16
  // The compute stream's position (the chunk after the one being multiplied) and that chunk's
  // 16-row block bits at its offset (all of the tile's; each wave uses its own).
  int v_u = 0, v_k = 0;
  auto blocks_next = [&]() -> uint32_t {
    if (++v_k == ksl) {
      v_k = 0;
      ++v_u;
    }
    return v_u < nused ? (uint32_t)s_blku[v_u] : 0u;
  };
  // Multiplies chunk c (this wave's blocks vm) from stage st.
  auto compute = [&](uint32_t vm, const uint4* st) {
    const char* A = (const char*)st;
    const char* B = A + A_BYTES;
    constexpr int KST = KC / 32;
    // Fragments of k-step t+1 are read while the MFMAs of k-step t run; blocks without pairs
    // at this offset skip their MFMAs (their fragments are read anyway).
    bf16x8 a[2][MI], b[2][NI];
    auto frags = [&](int t, int d) {
      const int slot = (((t * 4) + (lane >> 4)) ^ fsw) * 16;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) b[d][ni] = *(const bf16x8*)(B + (wn * NW + ni * 16 + frow) * ROWB + slot);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) a[d][mi] = *(const bf16x8*)(A + (wm * MW + mi * 16 + frow) * ROWB + slot);
    };
    if (vm) {
      // Schedule (one basic block): the reads of k-step 0, then its MFMAs with the reads of
      // k-step 1 issued between them (after the first two), then the MFMAs of k-step 1; each
      // wait for reads then overlaps MFMAs already issued. Blocks without a pair at this offset
      // gathered the zero row (their products add nothing), so no block is skipped.
      frags(0, 0);
#pragma unroll
      for (int t = 0; t < KST; ++t) {
        if (t + 1 < KST) frags(t + 1, (t + 1) & 1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t & 1][mi], b[t & 1][ni], acc[mi][ni], 0, 0, 0);
      }
      constexpr int NR = MI + NI;         // reads of one k-step
      constexpr int NM = MI * NI;         // MFMAs of one k-step
      constexpr int PER = (NM - 2) / NR;  // MFMAs between consecutive reads
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
      for (int t = 0; t < KST; ++t) {
        if (t + 1 < KST) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, NM - 2 - NR * PER, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        }
      }
    }
  };
  // Waits until chunk c+1 has landed while the chunks after it, up to `last`, stay in flight
  // (every chunk issues exactly LPC loads per wave, and vmcnt retires them in order).
  auto wait_next = [&](int ahead) {
    if (NST > 5 && ahead >= 4) wait_vmcnt<(NST > 5 ? 4 * LPC : 0)>();
    else if (NST > 4 && ahead >= 3) wait_vmcnt<(NST > 4 ? 3 * LPC : 0)>();
    else if (NST > 3 && ahead >= 2) wait_vmcnt<(NST > 3 ? 2 * LPC : 0)>();
    else if (NST > 2 && ahead >= 1) wait_vmcnt<(NST > 2 ? LPC : 0)>();
    else wait_vmcnt<0>();
  };
  // Stage i (i < NST); with the pipeline loops unrolled every use names one object.
  auto stage = [&](int i) -> uint4* {
    return i == 0 ? s_st0 : i == 1 ? s_st1 : i == 2 ? s_st2 : i == 3 ? s_st3 : i == 4 ? s_st4 : s_st5;
  };
  // One chunk: start filling the stage freed by the previous chunk with chunk c+NST-1,
  // multiply chunk c, wait for chunk c+1 and meet the other waves.
  // pend: the LDS reads of chunk c+NST-1 (read during the previous chunk); vcur: chunk c's blocks.
  Pend pend;
  uint32_t vcur = 0;
  auto step = [&](int c, const uint4* cur, uint4* fill) {
    const uint32_t vm = __builtin_amdgcn_readfirstlane((vcur >> (wm * MI)) & ((1u << MI) - 1u));
    if (c + NST - 1 < nchunks) issue(pend, fill);
    pend = fetch_next();  // chunk c + NST
    vcur = blocks_next();  // chunk c + 1
    compute(vm, cur);
    const int last = (c + NST - 1 < nchunks ? c + NST - 1 : nchunks - 1);
    wait_next(last - (c + 1));
    __syncthreads();
  };

  // Prologue: chunks 0 .. NST-2 in flight, wait for chunk 0.
#pragma unroll
  for (int q = 0; q < NST - 1; ++q) {
    const Pend p = fetch_next();  // chunk q
    if (q < nchunks) issue(p, stage(q));
  }
  pend = fetch_next();  // chunk NST - 1
  vcur = nused > 0 ? (uint32_t)s_blku[0] : 0u;
  wait_next((nchunks < NST - 1 ? nchunks : NST - 1) - 1);
  __syncthreads();
  // Chunk c is in stage c % NST; the stage it fills is the one chunk c-1 used.
  for (int c = 0; c < nchunks; c += NST) {
#pragma unroll
    for (int q = 0; q < NST; ++q)
      if (q == 0 || c + q < nchunks) step(c + q, stage(q), stage((q + NST - 1) % NST));
  }

  // Output: rows in passes of OUT_ROWS through stage 0, granules swizzled by row; D layout of
  // a 16x16 block: lane holds column lane%16 of rows 4*(lane/16) + j.
  uint16_t* O = (uint16_t*)s_st0;
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int rb = wm * MW + mi * 16;
      if (rb / OUT_ROWS == p) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = rb - p * OUT_ROWS + (lane >> 4) * 4 + j;
            const int col = wn * NW + ni * 16 + frow;
            O[row * BN + (((col >> 3) ^ (row & 7)) << 3) + (col & 7)] = f32_to_bf16_rne(acc[mi][ni][j]);
          }
      }
    }
    __syncthreads();
    for (int s = tid; s < OUT_ROWS * OG; s += NT) {
      const int row = s / OG, g = s % OG;
      const int32_t r = s_perm[p * OUT_ROWS + row];
      if (r >= 0)
        *(uint4*)(out + (size_t)r * cout + n0 + g * 8) = *(const uint4*)&O[row * BN + ((g ^ (row & 7)) << 3)];
    }
    __syncthreads();
  }
}

template <int BN, int KC, int WM, int NST, int NWV, int TBM = kBM>
void launch_main(int64_t n_tiles, int64_t col_tiles, const int32_t* map, int64_t N, int64_t n_in, const int32_t* perm,
                 const uint16_t* blk, const void* feats, const uint16_t* wt, int cin, int cout, void* out,
                 hipStream_t s) {
  k_conv_ggs_bf16<BN, KC, WM, NST, NWV, TBM><<<(unsigned)(n_tiles * (kBM / TBM) * col_tiles), 64 * NWV, 0, s>>>(
      map, N, n_in, perm, blk, (const uint16_t*)feats, wt, cin, cout, (uint16_t*)out, col_tiles);
}

}  // namespace

// Per-leaf dispatch: skip[r] = 1 for every row r of a leaf with at least min_count active
// voxels, 0 for the others. One wave per leaf (rows offset .. offset + count of the leaf).
__global__ __launch_bounds__(256) void k_dense_rows(const LeafRec* __restrict__ leaf, int64_t F, int64_t N,
                                                    uint32_t min_count, uint8_t* __restrict__ skip) {
  const int64_t f = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (f >= F) return;
  const int lane = lane_id();
  uint32_t c = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) c += (uint32_t)__popcll(leaf[f].mask[w]);
  const uint64_t off = leaf[f].offset;
  const uint8_t v = c >= min_count ? 1 : 0;
  for (uint32_t t = (uint32_t)lane; t < c; t += 64)
    if (off + t < (uint64_t)N) skip[off + t] = v;
}

int launch_ggs_plan(const int32_t* d_map, int64_t N, int32_t* perm, uint16_t* blk, hipStream_t s,
                    const uint8_t* skip) {
  const int64_t n_tiles = (N + kBM - 1) / kBM;
  if (n_tiles == 0) return IGC_OK;
  IGC_HIP(launch_plan(256, 0, d_map, N, N, perm, blk, skip, s), "igc_sparse_conv: plan launch");
  return IGC_OK;
}

bool ggs_conv_supported(int32_t dtype, int32_t cin, int32_t cout) {
  return dtype == IGC_BF16 && cin >= 32 && cin <= 1024 && cin % 32 == 0 && cout >= 64 && cout <= 1024 &&
         cout % 64 == 0;
}

namespace {
struct GgsLayout {
  int64_t n_tiles = 0;
  size_t wt_bytes = 0, perm_bytes = 0, blk_bytes = 0, skip_bytes = 0;
  size_t total() const { return wt_bytes + perm_bytes + blk_bytes + skip_bytes; }
};

GgsLayout ggs_layout(int64_t N, int32_t cin, int32_t cout, bool with_skip) {
  GgsLayout L;
  L.n_tiles = (N + kBM - 1) / kBM;
  L.wt_bytes = align_up((size_t)27 * cin * cout * 2, 256);
  L.perm_bytes = align_up((size_t)L.n_tiles * kBM * 4, 256);
  L.blk_bytes = align_up((size_t)L.n_tiles * kNOff * 2, 256);
  L.skip_bytes = with_skip ? align_up((size_t)N, 256) : 0;
  return L;
}
}  // namespace

size_t ggs_scratch_bytes(int64_t N, int32_t cin, int32_t cout, bool with_skip) {
  return ggs_layout(N, cin, cout, with_skip).total();
}

int launch_conv_ggs(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                    const void* d_w, int32_t cout, void* d_out, hipStream_t s, uint32_t dense_min, int64_t n_in,
                    void* scratch) {
  (void)dtype;
  const int64_t N = g->n_voxels;
  if (n_in < 0) n_in = N;
  const GgsLayout L = ggs_layout(N, cin, cout, dense_min != 0);
  const int64_t n_tiles = L.n_tiles;
  Workspace wsb;
  if (!scratch) {
    int rc = ws_acquire(&wsb, L.total(), s, "igc_sparse_conv: gather-GEMM-scatter workspace", grid_alloc(g));
    if (rc) return rc;
  }
  char* ws = scratch ? (char*)scratch : (char*)wsb.p;
  uint16_t* wt = (uint16_t*)ws;
  int32_t* perm = (int32_t*)(ws + L.wt_bytes);
  uint16_t* blk = (uint16_t*)(ws + L.wt_bytes + L.perm_bytes);
  uint8_t* skip = dense_min ? (uint8_t*)(ws + L.wt_bytes + L.perm_bytes + L.blk_bytes) : nullptr;
  hipError_t e = hipSuccess;
  if (skip) {
    k_dense_rows<<<(unsigned)((g->n_leaf + 3) / 4), 256, 0, s>>>(g->leaf, g->n_leaf, N, dense_min, skip);
    e = hipGetLastError();
  }
  const GgsTuning tu = ggs_tuning(cin, cout, N, g->n_leaf);
  if (e == hipSuccess && n_tiles > 0) {
    e = launch_plan(tu.span, tu.order, d_map, N, n_in, perm, blk, skip, s, (const uint16_t*)d_w, wt, cin, cout);
  }
  if (e == hipSuccess && n_tiles > 0) {
    // 64-channel chunks where cin allows, unless the layer's rule asks for 32-channel chunks.
    const bool k64 = cin % 64 == 0 && tu.kc != 32;
    // Tile shapes measured on MI355X: 256 x 256 with eight waves (two per SIMD, each 128 rows
    // by 64 channels: 64 rows by 128 is 0.5% slower on 128 -> 256), 256 x 128 with sixteen
    // (each 32 rows by 64 channels: 1.6% faster on 128 -> 128 than 64 by 32), 256 x 64 with
    // eight (each 32 rows by all 64 channels: 2% faster on 64 -> 64 than 64 by 32); 32-channel
    // chunks when cin is not a multiple of 64 or the layer's rule asks for them. 256 x 64 with
    // 32-channel chunks on four waves takes 70 KB of LDS, so two workgroups share a CU and one's
    // gather latency overlaps the other's work: 64 -> 64 on 17M voxels 7.92 -> 7.07 ms and on
    // 48M 22.3 -> 19.8 ms, 128 -> 64 on 17M 12.9 -> 11.8 ms, but 256 -> 64 on 17M 23.6 -> 25.3 ms
    // and 128 -> 64 on 204k voxels 0.136 -> 0.147 ms; hence a per-layer choice.
    const int64_t n256 = cout / 256, n128 = cout / 128, n64 = cout / 64;
    // A layer's rule may ask for narrower output tiles (more workgroups, each gathering the
    // same input rows for fewer channels).
    int bn = cout % 256 == 0 && k64 ? 256 : cout % 128 == 0 ? 128 : 64;
    if (tu.bn > 0 && tu.bn < bn && cout % tu.bn == 0) bn = tu.bn;
    // Half tiles (a rule's `h`): each workgroup takes 128 rows of a 256-row plan tile and only the
    // offsets those rows have. At 128 and 64 channels the stages then fit two workgroups per CU
    // (at 256 the tile stays whole). Measured with 64-channel chunks on 8 waves: 128 -> 128 on
    // 204k voxels 0.157 -> 0.140 ms, 64 -> 128 0.106 -> 0.089 ms, 128 -> 128 on 17M 15.4 -> 15.3
    // ms; with 32-channel chunks on 4 waves 64 -> 64 on 17M 7.08 -> 6.77 ms.
    const bool half = tu.rows == 128 && bn <= 128;
    if (bn == 256) {
      launch_main<256, 64, 2, 2, 8>(n_tiles, n256, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
    } else if (bn == 128 && k64) {
      if (half)
        launch_main<128, 64, 4, 2, 8, 128>(n_tiles, n128, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
      else
        launch_main<128, 64, 8, 2, 16>(n_tiles, n128, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
    } else if (bn == 128) {
      if (half)
        launch_main<128, 32, 2, 2, 4, 128>(n_tiles, n128, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
      else
        launch_main<128, 32, 2, 2, 8>(n_tiles, n128, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
    } else if (k64) {
      if (half)
        launch_main<64, 64, 4, 2, 4, 128>(n_tiles, n64, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
      else
        launch_main<64, 64, 8, 2, 8>(n_tiles, n64, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
    } else {
      if (half)
        launch_main<64, 32, 2, 2, 4, 128>(n_tiles, n64, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
      else
        launch_main<64, 32, 4, 2, 4>(n_tiles, n64, d_map, N, n_in, perm, blk, d_feats, wt, cin, cout, d_out, s);
    }
    e = hipGetLastError();
  }
  ws_release(&wsb, s);
  if (e != hipSuccess) return hip_status(e, "igc_sparse_conv: gather-GEMM-scatter launch");
  return IGC_OK;
}

}  // namespace igc
