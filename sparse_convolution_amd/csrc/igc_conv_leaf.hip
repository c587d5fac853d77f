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

template <int CIN, int COUT>
__global__ __launch_bounds__(256) void k_conv_leaf_f32(GridView g, const float* __restrict__ feats,
                                                       const float* __restrict__ w, float* __restrict__ out) {
  constexpr int COUTP = (COUT + 15) / 16 * 16;
  constexpr int NS = COUTP / 16;  // 16-column MFMA slabs
  constexpr int KS = CIN / 4;     // 4-channel MFMA steps per offset
  // W fragments stay in registers when they fit (54 per lane at 8 -> 16); otherwise in LDS.
  constexpr bool kWRegs = NS * 27 * KS <= 64;
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

  // Leaf records of the 3x3x3 block (slot 13 = this leaf) from the grid's neighbour table.
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
  if (wave == 0) {
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t count = 0;
    for (int q = 0; q < 8; ++q) {
      const uint64_t word = s_mask[13][q];
      if ((word >> lane) & 1ull) s_pos[count + (uint32_t)__popcll(word & lt)] = (uint16_t)(q * 64 + lane);
      count += (uint32_t)__popcll(word);
    }
    if (lane == 0) s_count = count;
  }
  for (int c = tid; c < 1000; c += 256) {
    const int x = c / 100 - 1, y = (c / 10) % 10 - 1, z = c % 10 - 1;  // leaf-local, in [-1, 8]
    const int slot = ((x >> 3) + 1) * 9 + ((y >> 3) + 1) * 3 + ((z >> 3) + 1);
    const uint32_t q = (uint32_t)(x & 7);
    const uint64_t bit = 1ull << ((uint32_t)((y & 7) << 3) | (uint32_t)(z & 7));
    const uint64_t word = s_mask[slot][q];
    float4* dst = (float4*)&s_win[c * CIN];
    if (word & bit) {
      const uint32_t pre = q ? (uint32_t)(s_pre[slot] >> (9u * (q - 1u))) & 511u : 0u;
      const uint64_t row = s_off[slot] + pre + (uint32_t)__popcll(word & (bit - 1ull));
      const float4* src = (const float4*)(feats + row * CIN);
#pragma unroll
      for (int v = 0; v < CIN / 4; ++v) dst[v] = src[v];
    } else {
#pragma unroll
      for (int v = 0; v < CIN / 4; ++v) dst[v] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
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
#pragma unroll
    for (int o = 0; o < 27; ++o) {
      const int cell = cell0 + (o / 9) * 100 + ((o / 3) % 3) * 10 + o % 3;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float a = s_win[cell * CIN + ks * 4 + kq];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          float b;
          if constexpr (kWRegs) b = wreg[(o * KS + ks) * NS + ns];
          else b = s_w[(o * CIN + ks * 4 + kq) * COUTP + ns * 16 + rl];
          acc[ns] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[ns], 0, 0, 0);
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

template <int CIN, int COUT>
int launch_leaf(const igc_grid* g, const void* d_feats, const void* d_w, void* d_out, hipStream_t s) {
  k_conv_leaf_f32<CIN, COUT><<<(unsigned)g->n_leaf, 256, 0, s>>>(g->view(), (const float*)d_feats, (const float*)d_w,
                                                                 (float*)d_out);
  IGC_HIP(hipGetLastError(), "igc_sparse_conv: leaf launch");
  return IGC_OK;
}

}  // namespace

bool leaf_conv_supported(int32_t dtype, int32_t cin, int32_t cout) {
  if (dtype != IGC_F32) return false;
  switch (cin * 1000 + cout) {
    case 4008: case 4016: case 4032: case 8008: case 8016: case 8032: case 16016:
      return true;
    default:
      return false;
  }
}

int launch_conv_leaf(const igc_grid* g, const void* d_feats, int32_t dtype, int32_t cin, const void* d_w,
                     int32_t cout, void* d_out, hipStream_t s) {
  (void)dtype;
  switch (cin * 1000 + cout) {
    case 4008: return launch_leaf<4, 8>(g, d_feats, d_w, d_out, s);
    case 4016: return launch_leaf<4, 16>(g, d_feats, d_w, d_out, s);
    case 4032: return launch_leaf<4, 32>(g, d_feats, d_w, d_out, s);
    case 8008: return launch_leaf<8, 8>(g, d_feats, d_w, d_out, s);
    case 8016: return launch_leaf<8, 16>(g, d_feats, d_w, d_out, s);
    case 8032: return launch_leaf<8, 32>(g, d_feats, d_w, d_out, s);
    case 16016: return launch_leaf<16, 16>(g, d_feats, d_w, d_out, s);
    default: return set_error(IGC_ERR_UNSUPPORTED, "igc_sparse_conv: leaf path shape");
  }
}

}  // namespace igc
