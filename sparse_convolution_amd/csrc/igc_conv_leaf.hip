// Leaf-local submanifold convolution, fp32 (v_mfma_f32_16x16x4_f32, fp32 products and sums).
//
// fVDB notes, "accelerated operators for sparse convolution", first case: for low channel
// counts the convolution is bandwidth-bound, so regularity wins over sparsity: each 8^3 leaf
// plus a one-voxel halo (a 10^3 window) is densified in on-chip memory and a regular local
// dense convolution runs on the matrix units, with no auxiliary index structure.
//
// gfx950 form: one workgroup per leaf. It takes the 3x3x3 block of leaves from the grid's
// neighbour table, fills a 10 x 10 x 10 x cin window in LDS from the leaf records (inactive or
// absent cells are zero), and keeps W in registers (or LDS when it does not fit). Every
// neighbour read is then an LDS address computed from the voxel's position - the kernel map
// is not used. Output rows are produced only for the leaf's
// active voxels: they are compacted in row order, taken 16 at a time as the M dimension of a
// 16x16x4 fp32 MFMA whose A operand is read straight from the window at the shifted cell of
// each offset, K = 27 offsets x cin and N = cout (padded to 16). The result rows of one leaf
// are consecutive output rows. Leaves are numbered so that each XCD walks a contiguous range
// of leaves, which keeps the halo re-reads of neighbouring leaves in that XCD's L2.
#include <hip/hip_runtime.h>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t xcd_block(int64_t bid, int64_t nblk) {
  const int64_t x = bid & 7, q = nblk >> 3, rem = nblk & 7;
  return x * q + (x < rem ? x : rem) + (bid >> 3);
}

// Leaf records of the 3x3x3 block of leaves around leaf f (slot 13 = f) from the grid's
// neighbour table into LDS (threads 0..26); an absent leaf is an empty record.
__device__ __forceinline__ void load_leaf_block(const GridView& g, int64_t f, int tid, uint64_t (*s_mask)[8],
                                                uint64_t* s_off, uint64_t* s_pre) {
  if (tid < 27) {
    const int32_t nl = g.leaf_nbr[f * 27 + tid];
    if (nl >= 0) {
      const LeafRec& L = g.leaf[nl];
      for (int q = 0; q < 8; ++q) s_mask[tid][q] = L.mask[q];
      s_off[tid] = L.offset;
      s_pre[tid] = L.prefix;
    } else {
      for (int q = 0; q < 8; ++q) s_mask[tid][q] = 0;
      s_off[tid] = 0;
      s_pre[tid] = 0;
    }
  }
}

// Positions of slot 13's active voxels in row order, and their count (one wave).
__device__ __forceinline__ void compact_leaf(int lane, const uint64_t (*s_mask)[8], uint16_t* s_pos,
                                             uint32_t* s_count) {
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t count = 0;
  for (int q = 0; q < 8; ++q) {
    const uint64_t word = s_mask[13][q];
    if ((word >> lane) & 1ull) s_pos[count + (uint32_t)__popcll(word & lt)] = (uint16_t)(q * 64 + lane);
    count += (uint32_t)__popcll(word);
  }
  if (lane == 0) *s_count = count;
}

// Rotation of the 4-channel granules of window cell c: granule j of a cell is stored at granule
// (j + win_rot<CIN>(c)) mod CIN/4. Cells 64/CIN apart start on the same LDS bank, so without it
// the 16 rows of an MFMA operand read (16 cells, one granule each) meet on a few banks; with it
// consecutive groups of 64/CIN cells use different granules.
template <int CIN>
__device__ __forceinline__ int win_rot(int c) {
  return CIN >= 8 ? (c / (64 / CIN)) & (CIN / 4 - 1) : 0;
}

// fp32 window [1000 cells][CIN]: cell (x+1, y+1, z+1) for leaf-local x, y, z in [-1, 8] holds
// the features of that voxel (granules rotated by win_rot), zero where it is inactive or its
// leaf is absent.
template <int CIN>
__device__ __forceinline__ void fill_window_f32(float* s_win, const uint64_t (*s_mask)[8], const uint64_t* s_off,
                                                const uint64_t* s_pre, const float* __restrict__ feats, uint64_t n_rows,
                                                int tid) {
  for (int c = tid; c < 1000; c += 256) {
    const int x = c / 100 - 1, y = (c / 10) % 10 - 1, z = c % 10 - 1;  // leaf-local, in [-1, 8]
    const int slot = ((x >> 3) + 1) * 9 + ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
    const uint32_t q = (uint32_t)(x & 7);
    const uint64_t bit = 1ull << ((uint32_t)((y & 7) << 3) | (uint32_t)(z & 7));
    const uint64_t word = s_mask[slot][q];
    float4* dst = (float4*)&s_win[c * CIN];
    if (word & bit) {
      const uint32_t pre = q ? (uint32_t)(s_pre[slot] >> (9u * (q - 1u))) & 511u : 0u;
      const uint64_t r0 = s_off[slot] + pre + (uint32_t)__popcll(word & (bit - 1ull));
      const uint64_t row = r0 < n_rows ? r0 : 0;  // never past the feature array
      const float4* src = (const float4*)(feats + row * CIN);
      const int rot = win_rot<CIN>(c);
#pragma unroll
      for (int v = 0; v < CIN / 4; ++v) dst[(v + rot) & (CIN / 4 - 1)] = src[v];
    } else {
#pragma unroll
      for (int v = 0; v < CIN / 4; ++v) dst[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

template <int CIN, int COUT>
__global__ __launch_bounds__(256) void k_conv_leaf_f32_wide(GridView g, const float* __restrict__ feats,
                                                       const float* __restrict__ w, float* __restrict__ out) {
  constexpr int COUTP = (COUT + 15) / 16 * 16;
  constexpr int NS = COUTP / 16;  // 16-column MFMA slabs
  constexpr int KS = CIN / 4;     // 4-channel MFMA steps per offset
  // W fragments stay in registers when they fit (108 per lane at 16 -> 16 or 16 -> 8);
  // otherwise in LDS.
  constexpr bool kWRegs = NS * 27 * KS <= 112;
  __shared__ __attribute__((aligned(16))) float s_win[1000 * CIN];
  __shared__ float s_w[kWRegs ? 1 : 27 * CIN * COUTP];
  __shared__ uint64_t s_mask[27][8];
  __shared__ uint64_t s_off[27];
  __shared__ uint64_t s_pre[27];
  __shared__ uint16_t s_pos[512];
  __shared__ uint32_t s_count;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int rl = lane & 15;  // A row / B column / D column
  const int kq = lane >> 4;  // A column / B row / D row group
  const int64_t f = xcd_block(blockIdx.x, gridDim.x);

  load_leaf_block(g, f, tid, s_mask, s_off, s_pre);
  float wreg[kWRegs ? 27 * KS * NS : 1];
  if constexpr (kWRegs) {
#pragma unroll
    for (int o = 0; o < 27; ++o)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const int col = ns * 16 + rl;
          wreg[(o * KS + ks) * NS + ns] = col < COUT ? w[(o * CIN + ks * 4 + kq) * COUT + col] : 0.f;
        }
  } else {
    for (int e = tid; e < 27 * CIN * COUTP; e += 256) {
      const int col = e % COUTP;
      s_w[e] = col < COUT ? w[(e / COUTP) * COUT + col] : 0.f;
    }
  }
  __syncthreads();

  // Compacted active positions of this leaf (wave 0), and the window (all threads).
  if (wave == 0) compact_leaf(lane, s_mask, s_pos, &s_count);
  fill_window_f32<CIN>(s_win, s_mask, s_off, s_pre, feats, (uint64_t)g.n_voxels, tid);
  __syncthreads();

  const uint32_t count = s_count;
  const uint64_t base = s_off[13];
  for (uint32_t g0 = (uint32_t)wave * 16; g0 < count; g0 += 64) {
    const uint32_t t = g0 + rl;
    const uint32_t p = s_pos[t < count ? t : 0];
    const int px = (int)(p >> 6), py = (int)((p >> 3) & 7u), pz = (int)(p & 7u);
    const int cell0 = (px * 10 + py) * 10 + pz;  // window cell of offset (-1,-1,-1)
    f32x4 acc[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[ns] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A value of step i = o KS + ks. With one column block the reads run PF steps ahead of
    // their MFMAs, held there by scheduling barriers (the compiler's own schedule keeps two in
    // flight); with two, each read already feeds two MFMAs and the prefetch measured slower.
    auto aval = [&](int i) -> float {
      const int o = i / KS, ks = i % KS;
      const int cell = cell0 + (o / 9) * 100 + ((o / 3) % 3) * 10 + o % 3;
      const int rot = win_rot<CIN>(cell);
      return s_win[cell * CIN + (((ks + rot) & (KS - 1)) << 2) + kq];
    };
    constexpr int STEPS = 27 * KS;
    auto step = [&](int i, float a) {
      const int o = i / KS, ks = i % KS;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        float b;
        if constexpr (kWRegs) b = wreg[(o * KS + ks) * NS + ns];
        else b = s_w[(o * CIN + ks * 4 + kq) * COUTP + ns * 16 + rl];
        acc[ns] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[ns], 0, 0, 0);
      }
    };
    if constexpr (NS == 1) {
      constexpr int PF = 8;
      float ring[PF];
#pragma unroll
      for (int d = 0; d < PF; ++d) ring[d] = aval(d);
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        const float a = ring[i % PF];
        if (i + PF < STEPS) ring[i % PF] = aval(i + PF);
        step(i, a);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int o = 0; o < 27; ++o) {
        const int cell = cell0 + (o / 9) * 100 + ((o / 3) % 3) * 10 + o % 3;
        const int rot = win_rot<CIN>(cell);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const float a = s_win[cell * CIN + (((ks + rot) & (KS - 1)) << 2) + kq];
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
            float b;
            if constexpr (kWRegs) b = wreg[(o * KS + ks) * NS + ns];
            else b = s_w[(o * CIN + ks * 4 + kq) * COUTP + ns * 16 + rl];
            acc[ns] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[ns], 0, 0, 0);
          }
        }
      }
    }
    // D: lane holds column lane%16 of rows 4*(lane/16) + j.
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t r = g0 + (uint32_t)kq * 4 + j;
        const int col = ns * 16 + rl;
        if (r < count && col < COUT) out[(base + r) * COUT + col] = acc[ns][j];
      }
  }
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Round to nearest even (finite inputs), as a 16-bit pattern.
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_value(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// v = hi + mid + lo exactly (three bf16 values of 8 significant bits each): each residual is
// exact in fp32, and the last one has at most 8 significant bits left.
__device__ __forceinline__ void split3(float v, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = bf16_bits_rne(v);
  const float r1 = v - bf16_value(hi);
  mid = bf16_bits_rne(r1);
  const float r2 = r1 - bf16_value(mid);
  lo = bf16_bits_rne(r2);
}

// split3 of two values at once with the hardware's round-to-nearest-even conversion
// (v_cvt_pk_bf16_f32); value a in the low halves of the three words, b in the high halves.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split3x2(float a, float b, uint32_t& hw, uint32_t& mw, uint32_t& lw) {
  const f32x2 v = {a, b};
  hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  const f32x2 r1 = v - f32x2{__uint_as_float(hw << 16), __uint_as_float(hw & 0xFFFF0000u)};
  mw = __builtin_bit_cast(uint32_t, __builtin_convertvector(r1, bf16x2));
  const f32x2 r2 = r1 - f32x2{__uint_as_float(mw << 16), __uint_as_float(mw & 0xFFFF0000u)};
  lw = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2));
}

// Window cell offset of stencil offset o relative to the cell of offset (-1,-1,-1).
__device__ __forceinline__ int cell_delta(int o) { return (o / 9) * 100 + ((o / 3) % 3) * 10 + o % 3; }

// fp32 leaf conv on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16). Same structure as the
// fp32-MFMA form above: one workgroup per leaf, the 10^3 window in LDS, active voxels taken 16
// at a time as the M dimension. Every fp32 operand is split into three bf16 parts whose sum is
// exact (split3), and the product a*b is summed as the six partial products with index sum <= 2
// (a2 b0, a1 b1, a0 b2, a1 b0, a0 b1, a0 b0), each exact in fp32 and accumulated in fp32; the
// three dropped terms are below 2^-24 of |a b|, the size of fp32 rounding (the split-bf16
// scheme of Henry, Tang & Heinecke, "Leveraging the bfloat16 artificial intelligence datatype
// for higher-precision computations", 2019). The window holds the three splits of every cell,
// made once when the window is filled, and W's splits stay in registers. K = 27 offsets x CIN runs in chunks of 32: lane group g = lane/16 holds
// k = 8g..8g+7 of a chunk, i.e. one offset's 8 channels (CIN 8) or two offsets' 4 channels
// (CIN 4); offsets past 26 are zero.
template <int CIN, int COUT>
__global__ __launch_bounds__(256) void k_conv_leaf_f32(GridView g, const float* __restrict__ feats,
                                                       const float* __restrict__ w, float* __restrict__ out) {
  static_assert(CIN == 4 || CIN == 8, "channel layout of the split form");
  constexpr int COUTP = (COUT + 15) / 16 * 16;
  constexpr int NS = COUTP / 16;
  constexpr int OPG = 8 / CIN;                   // offsets per lane group and chunk
  constexpr int NCH = (27 * CIN + 31) / 32;      // chunks of 32 k values
  constexpr int CS = 3 * CIN;                    // bf16 elements per window cell (three splits)
  constexpr int WSP = NCH * 3 * NS * 64 * 8;     // bf16 elements of W's splits (staged before the window)
  __shared__ __attribute__((aligned(16))) uint16_t s_win[1000 * CS > WSP ? 1000 * CS : WSP];
  __shared__ uint64_t s_mask[27][8];
  __shared__ uint64_t s_off[27];
  __shared__ uint64_t s_pre[27];
  __shared__ uint16_t s_pos[512];
  __shared__ uint32_t s_count;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int rl = lane & 15;  // A row / B column / D column
  const int kg = lane >> 4;  // k group of A and B, row group of D
  const int64_t f = xcd_block(blockIdx.x, gridDim.x);

  load_leaf_block(g, f, tid, s_mask, s_off, s_pre);

  // W splits for this lane: chunk q, split s, column slab ns -> 8 bf16 (k = 8 kg .. 8 kg + 7).
  // Every wave needs the same fragments: wave w splits the (q, ns) pairs with (q*NS+ns) % 4 ==
  // w into LDS (the window's space, filled afterwards), and all waves then load all of them.
  int dcell[NCH][OPG];
#pragma unroll
  for (int q = 0; q < NCH; ++q)
#pragma unroll
    for (int h = 0; h < OPG; ++h) {
      const int o = (q * 32 + kg * 8) / CIN + h;
      dcell[q][h] = cell_delta(o < 27 ? o : 0);
    }
  bf16x8* s_wsp = (bf16x8*)s_win;
  for (int pr = wave; pr < NCH * NS; pr += 4) {
    const int q = pr / NS, ns = pr % NS;
    const int col = ns * 16 + rl;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = q * 32 + kg * 8 + e;  // k = o * CIN + ci
      v[e] = (k < 27 * CIN && col < COUT) ? w[(size_t)k * COUT + col] : 0.f;
    }
    bf16x8 h, m, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t hs, ms, ls;
      split3(v[e], hs, ms, ls);
      h[e] = __builtin_bit_cast(__bf16, hs);
      m[e] = __builtin_bit_cast(__bf16, ms);
      l[e] = __builtin_bit_cast(__bf16, ls);
    }
    s_wsp[((q * 3 + 0) * NS + ns) * 64 + lane] = h;
    s_wsp[((q * 3 + 1) * NS + ns) * 64 + lane] = m;
    s_wsp[((q * 3 + 2) * NS + ns) * 64 + lane] = l;
  }
  __syncthreads();
  bf16x8 wb[NCH][3][NS];
#pragma unroll
  for (int q = 0; q < NCH; ++q)
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) wb[q][sp][ns] = s_wsp[((q * 3 + sp) * NS + ns) * 64 + lane];
  __syncthreads();

  // Compacted active positions of this leaf (wave 0), and the split window (all threads).
  if (wave == 0) compact_leaf(lane, s_mask, s_pos, &s_count);
  // Window: up to four cells per thread; all their feature loads are issued before the first
  // split so that their latencies overlap.
  constexpr int CPT = (1000 + 255) / 256;
  float v[CPT][CIN];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    const int x = c / 100 - 1, y = (c / 10) % 10 - 1, z = c % 10 - 1;  // leaf-local, in [-1, 8]
    const int slot = ((x >> 3) + 1) * 9 + ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
    const uint32_t q = (uint32_t)(x & 7);
    const uint64_t bit = 1ull << ((uint32_t)((y & 7) << 3) | (uint32_t)(z & 7));
    const uint64_t word = c < 1000 ? s_mask[slot][q] : 0ull;
    if (word & bit) {
      const uint32_t pre = q ? (uint32_t)(s_pre[slot] >> (9u * (q - 1u))) & 511u : 0u;
      const uint64_t r0 = s_off[slot] + pre + (uint32_t)__popcll(word & (bit - 1ull));
      const uint64_t row = r0 < (uint64_t)g.n_voxels ? r0 : 0;  // never past the feature array
      const float4* src = (const float4*)(feats + row * CIN);
#pragma unroll
      for (int j = 0; j < CIN / 4; ++j) {
        const float4 t = src[j];
        v[i][4 * j] = t.x; v[i][4 * j + 1] = t.y; v[i][4 * j + 2] = t.z; v[i][4 * j + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < CIN; ++j) v[i][j] = 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    if (c >= 1000) break;
    uint32_t hw[CIN / 2], mw[CIN / 2], lw[CIN / 2];
#pragma unroll
    for (int j = 0; j < CIN / 2; ++j) split3x2(v[i][2 * j], v[i][2 * j + 1], hw[j], mw[j], lw[j]);
    uint16_t* dst = &s_win[c * CS];
    if constexpr (CIN == 8) {
      *(uint4*)&dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *(uint4*)&dst[8] = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      *(uint4*)&dst[16] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    } else {
      *(uint2*)&dst[0] = make_uint2(hw[0], hw[1]);
      *(uint2*)&dst[4] = make_uint2(mw[0], mw[1]);
      *(uint2*)&dst[8] = make_uint2(lw[0], lw[1]);
    }
  }
  __syncthreads();

  const uint32_t count = s_count;
  const uint64_t base = s_off[13];
  for (uint32_t g0 = (uint32_t)wave * 16; g0 < count; g0 += 64) {
    const uint32_t t = g0 + rl;
    const uint32_t p = s_pos[t < count ? t : 0];
    const int cell0 = (int)((p >> 6) * 100 + ((p >> 3) & 7u) * 10 + (p & 7u));  // cell of offset (-1,-1,-1)
    f32x4 acc[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[ns] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The three split fragments of chunk q (k past 27 CIN reads the cell of offset 0, a real
    // neighbour, against zero W splits).
    auto frag3 = [&](int q, bf16x8* a) {
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        if constexpr (CIN == 8) {
          a[sp] = *(const bf16x8*)&s_win[(cell0 + dcell[q][0]) * CS + sp * CIN];
        } else {
          const uint2 v0 = *(const uint2*)&s_win[(cell0 + dcell[q][0]) * CS + sp * CIN];
          const uint2 v1 = *(const uint2*)&s_win[(cell0 + dcell[q][1]) * CS + sp * CIN];
          a[sp] = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
        }
      }
    };
    // Fragments are read RING - 1 chunks ahead of their MFMAs, held there by scheduling
    // barriers (the compiler's own schedule reuses one register quad and waits on each read).
    constexpr int RING = 3;
    bf16x8 ring[RING][3];
#pragma unroll
    for (int d = 0; d < RING - 1; ++d)
      if (d < NCH) frag3(d, ring[d]);
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      if (q + RING - 1 < NCH) frag3(q + RING - 1, ring[(q + RING - 1) % RING]);
      const bf16x8* a = ring[q % RING];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        f32x4 c = acc[ns];
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], wb[q][0][ns], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], wb[q][1][ns], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], wb[q][2][ns], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], wb[q][0][ns], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], wb[q][1][ns], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], wb[q][0][ns], c, 0, 0, 0);
        acc[ns] = c;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // D: lane holds column lane%16 of rows 4*(lane/16) + j.
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t r = g0 + (uint32_t)kg * 4 + j;
        const int col = ns * 16 + rl;
        if (r < count && col < COUT) out[(base + r) * COUT + col] = acc[ns][j];
      }
  }
}

// Weight gradient of the leaf-local convolution, fp32 data (v_mfma_f32_16x16x4_f32):
// dW[o][ci][co] = sum over active voxels v of X[v + offset o][ci] dY[v][co], X zero where
// inactive. A workgroup walks a contiguous run of leaves; for each it fills the fp32 10^3 window
// of X as the forward does and stages the leaf's dY rows (consecutive output rows) in LDS. The
// MFMA's M dimension is the flattened pair m = o * CIN + ci (27 CIN, padded to 16), N the output
// channels (padded to 16) and K the leaf's active voxels, four per step: the A operand is one
// window read at the voxel's shifted cell, the B operand one dY read. Wave w takes the K steps
// w, w + 4, ... of every leaf with all M blocks, so one step issues MB x NS independent MFMAs,
// and keeps its sums in registers across the run. At the end the four waves' sums are added in
// LDS in wave order and the workgroup writes its partial dW; the partials of all workgroups are
// added in a fixed order afterwards.
template <int CIN, int COUT>
__global__ __launch_bounds__(256) void k_wgrad_leaf_f32(GridView g, int64_t n_leaf, int64_t leaves_per_group,
                                                        const float* __restrict__ feats,
                                                        const float* __restrict__ dout, float* __restrict__ part) {
  constexpr int MB = (27 * CIN + 15) / 16;  // 16-row M blocks
  constexpr int NS = (COUT + 15) / 16;      // 16-column N slabs
  constexpr int CPT = (1000 + 255) / 256;   // window cells per thread
  constexpr int DPT = (512 * COUT / 4 + 255) / 256;  // dY float4s per thread
  static_assert(MB * NS * 256 <= 1000 * CIN, "the cross-wave sum fits in the window");
  __shared__ __attribute__((aligned(16))) float s_win[1000 * CIN];
  __shared__ __attribute__((aligned(16))) float s_dy[512 * COUT];
  __shared__ uint64_t s_mask[27][8];
  __shared__ uint64_t s_off[27];
  __shared__ uint64_t s_pre[27];
  __shared__ uint16_t s_cell[512];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int rl = lane & 15;  // A row (m) / B column (n) / D column
  const int kq = lane >> 4;  // A column / B row (k) / D row group
  const int64_t grp = xcd_block(blockIdx.x, gridDim.x);

  // Window offset (cells * CIN + channel) of this lane's A row in each M block, -1 for padding
  // rows (o > 26).
  int aoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + rl;
    aoff[mb] = m < 27 * CIN ? cell_delta(m / CIN) * CIN + m % CIN : -1;
  }
  f32x4 acc[MB][NS];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[mb][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t f0 = grp * leaves_per_group;
  const int64_t f1 = f0 + leaves_per_group < n_leaf ? f0 + leaves_per_group : n_leaf;
  for (int64_t f = f0; f < f1; ++f) {
    __syncthreads();  // the previous leaf's window, dY and cell reads are done
    load_leaf_block(g, f, tid, s_mask, s_off, s_pre);
    __syncthreads();
    uint32_t count = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) count += (uint32_t)__popcll(s_mask[13][q]);
    const uint32_t cnt4 = (count + 3u) & ~3u;
    // All window and dY loads are issued before the first LDS store.
    float4 v[CPT][CIN / 4];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int x = c / 100 - 1, y = (c / 10) % 10 - 1, z = c % 10 - 1;  // leaf-local, in [-1, 8]
      const int slot = ((x >> 3) + 1) * 9 + ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
      const uint32_t q = (uint32_t)(x & 7);
      const uint64_t bit = 1ull << ((uint32_t)((y & 7) << 3) | (uint32_t)(z & 7));
      const uint64_t word = c < 1000 ? s_mask[slot][q] : 0ull;
      if (word & bit) {
        const uint32_t pre = q ? (uint32_t)(s_pre[slot] >> (9u * (q - 1u))) & 511u : 0u;
        const uint64_t r0 = s_off[slot] + pre + (uint32_t)__popcll(word & (bit - 1ull));
        const uint64_t row = r0 < (uint64_t)g.n_voxels ? r0 : 0;  // never past the feature array
        const float4* src = (const float4*)(feats + row * CIN);
#pragma unroll
        for (int j = 0; j < CIN / 4; ++j) v[i][j] = src[j];
      } else {
#pragma unroll
        for (int j = 0; j < CIN / 4; ++j) v[i][j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    // The leaf's dY rows are rows s_off[13] .. + count - 1; rows count .. cnt4 - 1 are zero.
    const float4* dsrc = (const float4*)(dout + s_off[13] * COUT);
    float4 d[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const uint32_t e = (uint32_t)tid + 256u * i;
      d[i] = e < count * (COUT / 4) ? dsrc[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (wave == 0) {
      // Window cell of offset (-1,-1,-1) for each active voxel, in row order.
      const uint64_t lt = (1ull << lane) - 1ull;
      uint32_t n = 0;
      for (int q = 0; q < 8; ++q) {
        const uint64_t word = s_mask[13][q];
        if ((word >> lane) & 1ull)
          s_cell[n + (uint32_t)__popcll(word & lt)] = (uint16_t)(q * 100 + (lane >> 3) * 10 + (lane & 7));
        n += (uint32_t)__popcll(word);
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c < 1000) {
#pragma unroll
        for (int j = 0; j < CIN / 4; ++j) ((float4*)&s_win[c * CIN])[j] = v[i][j];
      }
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const uint32_t e = (uint32_t)tid + 256u * i;
      if (e < cnt4 * (COUT / 4)) ((float4*)s_dy)[e] = d[i];
    }
    __syncthreads();
    // Two K steps per round (t0 and t0 + 16), every read of both issued before their MFMAs:
    // a step is a chain of LDS reads (cell, then window), which one step alone leaves exposed.
    // Voxels past cnt4 (the second step of the last round) read dY as zero.
    for (uint32_t t0 = (uint32_t)wave * 4; t0 < count; t0 += 32) {
      float a[2][MB], b[2][NS];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t t = t0 + 16u * h + (uint32_t)kq;
        const int cell0 = s_cell[t < count ? t : 0u];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const int col = ns * 16 + rl;
          b[h][ns] = col < COUT && t < cnt4 ? s_dy[t * COUT + col] : 0.f;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) a[h][mb] = aoff[mb] >= 0 ? s_win[cell0 * CIN + aoff[mb]] : 0.f;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int ns = 0; ns < NS; ++ns)
            acc[mb][ns] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[h][mb], b[h][ns], acc[mb][ns], 0, 0, 0);
    }
  }
  // Cross-wave sum in the window's space, fragment-major: wave 0 stores, waves 1..3 add in turn.
  __syncthreads();
  f32x4* s_sum = (f32x4*)s_win;
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          f32x4* p = &s_sum[(mb * NS + ns) * 64 + lane];
          *p = w == 0 ? acc[mb][ns] : *p + acc[mb][ns];
        }
    }
    __syncthreads();
  }
  // D: lane holds column lane%16 of rows 4*(lane/16) + j. Wave w writes M blocks w, w + 4, ...
  float* dst = part + grp * (int64_t)(27 * CIN * COUT);
  for (int mb = wave; mb < MB; mb += 4)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const f32x4 r = s_sum[(mb * NS + ns) * 64 + lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = mb * 16 + kq * 4 + j;
        const int col = ns * 16 + rl;
        if (m < 27 * CIN && col < COUT) dst[m * COUT + col] = r[j];
      }
    }
}

template <int CIN, int COUT>
int launch_leaf(const igc_grid* g, const void* d_feats, const void* d_w, void* d_out, hipStream_t s) {
  // Split-bf16 form for 4 or 8 input channels and up to 32 (CIN 4) / 16 (CIN 8) outputs, whose
  // W splits fit in registers; the fp32-MFMA form for the wider shapes.
  constexpr bool split = (CIN == 4 && COUT <= 32) || (CIN == 8 && COUT <= 16);
  if constexpr (split) {
    k_conv_leaf_f32<CIN, COUT><<<(unsigned)g->n_leaf, 256, 0, s>>>(g->view(), (const float*)d_feats,
                                                                  (const float*)d_w, (float*)d_out);
    IGC_HIP(hipGetLastError(), "igc_sparse_conv: leaf launch");
  } else {
    k_conv_leaf_f32_wide<CIN, COUT><<<(unsigned)g->n_leaf, 256, 0, s>>>(g->view(), (const float*)d_feats,
                                                                       (const float*)d_w, (float*)d_out);
    IGC_HIP(hipGetLastError(), "igc_sparse_conv: leaf launch");
  }
  return IGC_OK;
}

// ---------------------------------------------------------------- bf16 leaf window ("brick")
//
// fVDB notes, "accelerated operators for sparse convolution": the brick backend densifies small
// output windows with their halo and runs a dense convolution on the tensor cores, for feature
// depths of 32 to 64 at high neighbour occupancy. gfx950 form: the window is a whole leaf's
// 10^3 halo in LDS as bf16 (2 KB per channel: 32 KB for 16 channels, 128 KB for 64), zeros where
// inactive; the M dimension of v_mfma_f32_16x16x32_bf16 is the leaf's active voxels 16 at a
// time (inactive outputs of the window are not computed), K = 27 offsets x CIN, N = COUT in
// 16-column blocks, fp32 accumulation, bf16 output (round to nearest even).

__device__ __forceinline__ uint16_t bf16_out_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));  // inf / nan
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// wt[n][k] = W[k][n] for k = o CIN + ci < 27 CIN, zero up to the padded K (a multiple of 32): a
// lane's B fragment (8 consecutive k of one column) is one 16-byte load.
template <int CIN, int COUT>
__global__ void k_leaf_wt_bf16(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt) {
  constexpr int KP = (27 * CIN + 31) / 32 * 32;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < COUT * KP; e += gridDim.x * blockDim.x) {
    const int n = e / KP, k = e % KP;
    wt[e] = k < 27 * CIN ? w[(size_t)k * COUT + n] : (uint16_t)0;
  }
}

// 16-byte granule g of window cell c sits at granule g ^ bf16_swz<GPC>(c): eight consecutive
// cells (one 128-byte LDS row's worth of fragment reads) then fall on distinct banks.
template <int GPC>
__device__ __forceinline__ int bf16_swz(int c) {
  return (c / (8 / GPC)) & (GPC - 1);
}

// One workgroup per leaf. Wave w takes column block w % NS and the row blocks w / NS, w / NS +
// 4 / NS, ...; its B fragments (W^T, one per k-step) stay in registers, and each k-step is one
// 16-byte window read and one MFMA. K runs in steps of 32: lane group kg = lane / 16 holds k =
// 32 q + 8 kg .. + 7, i.e. 8 channels of one offset (CIN 64: offset q / 2, channels 32 (q % 2)
// + 8 kg ..; CIN 32: offset q; CIN 16: offset 2 q + kg / 2); k past 27 CIN (CIN 16: the second
// half of the last step) reads offset 0's cell against zero W.
template <int CIN, int COUT>
__global__ __launch_bounds__(256) void k_conv_leaf_bf16(GridView g, const uint16_t* __restrict__ feats,
                                                        const uint16_t* __restrict__ wt, uint16_t* __restrict__ out,
                                                        uint32_t min_count) {
  static_assert(CIN == 16 || CIN == 32 || CIN == 64, "window cells of two, four or eight 16-byte granules");
  static_assert(COUT == 16 || COUT == 32 || COUT == 64, "column blocks per wave");
  constexpr int NS = COUT / 16;
  constexpr int KP = (27 * CIN + 31) / 32 * 32;
  constexpr int NCH = KP / 32;
  constexpr int GPC = CIN / 8;
  constexpr int RSTEP = 4 / NS;
  __shared__ uint4 s_win[1000 * GPC];
  __shared__ uint64_t s_mask[27][8];
  __shared__ uint64_t s_off[27];
  __shared__ uint64_t s_pre[27];
  __shared__ uint16_t s_pos[512];
  __shared__ uint32_t s_count;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int rl = lane & 15;  // A row / B column / D column
  const int kg = lane >> 4;  // k group of A and B, row group of D
  const int ns = wave % NS;
  const int64_t f = xcd_block(blockIdx.x, gridDim.x);
  if (min_count) {  // per-leaf dispatch: sparser leaves belong to the other path (uniform exit)
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) c += (uint32_t)__popcll(g.leaf[f].mask[w]);
    if (c < min_count) return;
  }

  // B fragments of this wave's column block (in flight while the leaf records arrive).
  bf16x8 wb[NCH];
  const uint16_t* wrow = wt + (size_t)(ns * 16 + rl) * KP + kg * 8;
#pragma unroll
  for (int q = 0; q < NCH; ++q) wb[q] = *(const bf16x8*)(wrow + q * 32);
  // k-step q, lane group kg: offset q and granule kg (CIN 32), offset 2 q + kg / 2 and granule
  // kg % 2 (CIN 16), or offset q / 2 and granule 4 (q % 2) + kg (CIN 64).
  const int gran = CIN == 16 ? (kg & 1) : kg;
  const int ohalf = CIN == 16 ? (kg >> 1) : 0;
  load_leaf_block(g, f, tid, s_mask, s_off, s_pre);
  __syncthreads();

  // Compacted active positions (wave 0) and the window (all threads; every feature load of a
  // thread is issued before the first LDS store).
  if (wave == 0) compact_leaf(lane, s_mask, s_pos, &s_count);
  constexpr int CPT = (1000 + 255) / 256;
  uint4 v[CPT][GPC];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    const int x = c / 100 - 1, y = (c / 10) % 10 - 1, z = c % 10 - 1;  // leaf-local, in [-1, 8]
    const int slot = ((x >> 3) + 1) * 9 + ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
    const uint32_t q = (uint32_t)(x & 7);
    const uint64_t bit = 1ull << ((uint32_t)((y & 7) << 3) | (uint32_t)(z & 7));
    const uint64_t word = c < 1000 ? s_mask[slot][q] : 0ull;
    if (word & bit) {
      const uint32_t pre = q ? (uint32_t)(s_pre[slot] >> (9u * (q - 1u))) & 511u : 0u;
      const uint64_t r0 = s_off[slot] + pre + (uint32_t)__popcll(word & (bit - 1ull));
      const uint64_t row = r0 < (uint64_t)g.n_voxels ? r0 : 0;  // never past the feature array
      const uint4* src = (const uint4*)(feats + row * CIN);
#pragma unroll
      for (int j = 0; j < GPC; ++j) v[i][j] = src[j];
    } else {
#pragma unroll
      for (int j = 0; j < GPC; ++j) v[i][j] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    if (c < 1000) {
#pragma unroll
      for (int j = 0; j < GPC; ++j) s_win[c * GPC + (j ^ bf16_swz<GPC>(c))] = v[i][j];
    }
  }
  __syncthreads();

  const uint32_t count = s_count;
  const uint64_t base = s_off[13];
  for (uint32_t rb = (uint32_t)(wave / NS); rb * 16 < count; rb += RSTEP) {
    const uint32_t t = rb * 16 + rl;
    const uint32_t p = s_pos[t < count ? t : 0];
    const int cell0 = (int)((p >> 6) * 100 + ((p >> 3) & 7u) * 10 + (p & 7u));  // cell of offset (-1,-1,-1)
    // A fragment of k-step q: a window read at a constant cell distance from cell0.
    auto frag = [&](int q) -> bf16x8 {
      int dc, gq = gran;
      if constexpr (CIN == 64) {
        dc = cell_delta(q >> 1);
        gq = ((q & 1) << 2) | gran;
      } else if constexpr (CIN == 32) {
        dc = cell_delta(q);
      } else {
        const int o0 = 2 * q, o1 = 2 * q + 1 < 27 ? 2 * q + 1 : 0;
        dc = ohalf ? cell_delta(o1) : cell_delta(o0);
      }
      const int c = cell0 + dc;
      return __builtin_bit_cast(bf16x8, s_win[c * GPC + (gq ^ bf16_swz<GPC>(c))]);
    };
    // The reads run PF k-steps ahead of their MFMA, held there by scheduling barriers (the
    // compiler's own schedule keeps two in flight, and each MFMA then waits for most of an LDS
    // round trip).
    constexpr int PF = CIN == 16 ? 8 : 6;  // measured: 6 is 0.6% faster than 8 at 32 -> 32
    bf16x8 ring[PF];
#pragma unroll
    for (int d = 0; d < PF; ++d) ring[d] = frag(d);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const bf16x8 a = ring[q % PF];
      if (q + PF < NCH) ring[q % PF] = frag(q + PF);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wb[q], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep each read PF steps ahead of its MFMA
    }
    // D: lane holds column lane%16 of rows 4*(lane/16) + j.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t r = rb * 16 + (uint32_t)kg * 4 + j;
      if (r < count) out[(base + r) * COUT + ns * 16 + rl] = bf16_out_rne(acc[j]);
    }
  }
}

template <int CIN, int COUT>
int launch_leaf_bf16(const igc_grid* g, const void* d_feats, const void* d_w, void* d_out, hipStream_t s,
                     uint32_t min_count, void* scratch) {
  constexpr int KP = (27 * CIN + 31) / 32 * 32;
  Workspace wsb;
  if (!scratch) {
    int rc = ws_acquire(&wsb, (size_t)COUT * KP * 2, s, "igc_sparse_conv: leaf W transpose", grid_alloc(g));
    if (rc) return rc;
  }
  uint16_t* wt = (uint16_t*)(scratch ? scratch : wsb.p);
  k_leaf_wt_bf16<CIN, COUT><<<(COUT * KP + 255) / 256, 256, 0, s>>>((const uint16_t*)d_w, wt);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    k_conv_leaf_bf16<CIN, COUT><<<(unsigned)g->n_leaf, 256, 0, s>>>(g->view(), (const uint16_t*)d_feats, wt,
                                                                   (uint16_t*)d_out, min_count);
    e = hipGetLastError();
  }
  ws_release(&wsb, s);
  if (e != hipSuccess) return hip_status(e, "igc_sparse_conv: bf16 leaf launch");
  return IGC_OK;
}

template <int CIN, int COUT>
int launch_wgrad_leaf_t(const igc_grid* g, const void* d_feats, const void* d_dout, float* part, int64_t groups,
                        hipStream_t s) {
  const int64_t lpg = (g->n_leaf + groups - 1) / groups;
  k_wgrad_leaf_f32<CIN, COUT><<<(unsigned)groups, 256, 0, s>>>(g->view(), g->n_leaf, lpg, (const float*)d_feats,
                                                               (const float*)d_dout, part);
  IGC_HIP(hipGetLastError(), "igc_sparse_conv_backward: leaf weight-gradient launch");
  return IGC_OK;
}

}  // namespace

bool leaf_conv_supported(int32_t dtype, int32_t cin, int32_t cout) {
  if (dtype == IGC_BF16) {
    switch (cin * 1000 + cout) {
      case 16016: case 16032: case 16064: case 32016: case 32032: case 32064: case 64016: case 64032: case 64064:
        return true;
      default:
        return false;
    }
  }
  if (dtype != IGC_F32) return false;
  switch (cin * 1000 + cout) {
    case 4008: case 4016: case 4032: case 8008: case 8016: case 8032: case 16016:
    case 8004: case 16004: case 16008:  // the input-gradient shapes of 4 -> 8, 4 -> 16, 8 -> 16
      return true;
    default:
      return false;
  }
}

size_t leaf_scratch_bytes(int32_t dtype, int32_t cin, int32_t cout) {
  if (dtype != IGC_BF16) return 0;  // the fp32 kernels split W per workgroup, in LDS
  return align_up((size_t)cout * (size_t)((27 * cin + 31) / 32 * 32) * 2, 256);
}

int launch_conv_leaf(const igc_grid* g, const void* d_feats, int32_t dtype, int32_t cin, const void* d_w,
                     int32_t cout, void* d_out, hipStream_t s, uint32_t min_count, void* scratch) {
  if (min_count && dtype != IGC_BF16) return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv: per-leaf dispatch dtype");
  if (dtype == IGC_BF16) {
    switch (cin * 1000 + cout) {
      case 16016: return launch_leaf_bf16<16, 16>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 16032: return launch_leaf_bf16<16, 32>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 16064: return launch_leaf_bf16<16, 64>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 32016: return launch_leaf_bf16<32, 16>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 32032: return launch_leaf_bf16<32, 32>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 32064: return launch_leaf_bf16<32, 64>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 64016: return launch_leaf_bf16<64, 16>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 64032: return launch_leaf_bf16<64, 32>(g, d_feats, d_w, d_out, s, min_count, scratch);
      case 64064: return launch_leaf_bf16<64, 64>(g, d_feats, d_w, d_out, s, min_count, scratch);
      default: return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv: bf16 leaf path shape");
    }
  }
  switch (cin * 1000 + cout) {
    case 4008: return launch_leaf<4, 8>(g, d_feats, d_w, d_out, s);
    case 4016: return launch_leaf<4, 16>(g, d_feats, d_w, d_out, s);
    case 4032: return launch_leaf<4, 32>(g, d_feats, d_w, d_out, s);
    case 8008: return launch_leaf<8, 8>(g, d_feats, d_w, d_out, s);
    case 8016: return launch_leaf<8, 16>(g, d_feats, d_w, d_out, s);
    case 8032: return launch_leaf<8, 32>(g, d_feats, d_w, d_out, s);
    case 16016: return launch_leaf<16, 16>(g, d_feats, d_w, d_out, s);
    case 8004: return launch_leaf<8, 4>(g, d_feats, d_w, d_out, s);
    case 16004: return launch_leaf<16, 4>(g, d_feats, d_w, d_out, s);
    case 16008: return launch_leaf<16, 8>(g, d_feats, d_w, d_out, s);
    default: return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv: leaf path shape");
  }
}

bool wgrad_leaf_supported(int32_t cin, int32_t cout) {
  switch (cin * 1000 + cout) {
    case 4004: case 4008: case 4016: case 4032: case 8004: case 8008: case 8016: case 8032:
    case 16004: case 16008: case 16016:
      return true;
    default:
      return false;
  }
}

int64_t wgrad_leaf_groups(const igc_grid* g) {
  // About eight workgroups per CU, each over a run of consecutive leaves; every group has at
  // least one leaf. Measured on 7,732 leaves (ms, 1024 -> 2048 groups): 8 -> 8 0.310 -> 0.294,
  // 4 -> 16 0.207 -> 0.201, 8 -> 16 0.324 -> 0.321; 4096 and 8192 groups are slower (the partial
  // blocks to reduce grow with them).
  const int64_t want = 2048;
  if (g->n_leaf <= want) return g->n_leaf;
  const int64_t lpg = (g->n_leaf + want - 1) / want;
  return (g->n_leaf + lpg - 1) / lpg;
}

int launch_wgrad_leaf(const igc_grid* g, const void* d_feats, int32_t cin, const void* d_dout, int32_t cout,
                      float* part, int64_t groups, hipStream_t s) {
  switch (cin * 1000 + cout) {
    case 4004: return launch_wgrad_leaf_t<4, 4>(g, d_feats, d_dout, part, groups, s);
    case 4008: return launch_wgrad_leaf_t<4, 8>(g, d_feats, d_dout, part, groups, s);
    case 4016: return launch_wgrad_leaf_t<4, 16>(g, d_feats, d_dout, part, groups, s);
    case 4032: return launch_wgrad_leaf_t<4, 32>(g, d_feats, d_dout, part, groups, s);
    case 8004: return launch_wgrad_leaf_t<8, 4>(g, d_feats, d_dout, part, groups, s);
    case 8008: return launch_wgrad_leaf_t<8, 8>(g, d_feats, d_dout, part, groups, s);
    case 8016: return launch_wgrad_leaf_t<8, 16>(g, d_feats, d_dout, part, groups, s);
    case 8032: return launch_wgrad_leaf_t<8, 32>(g, d_feats, d_dout, part, groups, s);
    case 16004: return launch_wgrad_leaf_t<16, 4>(g, d_feats, d_dout, part, groups, s);
    case 16008: return launch_wgrad_leaf_t<16, 8>(g, d_feats, d_dout, part, groups, s);
    case 16016: return launch_wgrad_leaf_t<16, 16>(g, d_feats, d_dout, part, groups, s);
    default: return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv_backward: leaf weight-gradient shape");
  }
}

}  // namespace igc
