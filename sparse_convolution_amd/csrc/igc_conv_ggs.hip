// Gather-GEMM-scatter submanifold convolution, bf16 inputs / weights / outputs with fp32
// accumulation on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// fVDB notes, "accelerated operators for sparse convolution", third case: work is tiled over
// consecutive output rows, a workgroup-local buffer replaces global scatter, and for each of
// the 27 stencil offsets the tile's (input, output) pairs feed a tensor-core GEMM.
//
// The gfx950 form used here is output-stationary: a workgroup owns BM = 128 consecutive
// output rows and BN output channels and keeps their fp32 accumulators in registers for the
// whole reduction, so the "scatter" of every offset's product lands in registers and the
// output is written once (no atomics, deterministic). For each offset that at least one row
// of the tile uses, and each 32-channel slice of the input, the tile gathers its 128 input
// rows by the kernel map (absent neighbours read as zeros) into LDS next to the matching
// 32 x BN slice of W[o], and four waves run 32x32x16 MFMAs on 64 x BN/2 sub-tiles. The next
// slice is fetched into registers while the current one is multiplied (two LDS buffers, one
// barrier per slice). Offsets that no row of the tile uses are skipped entirely, which is the
// pages' per-offset pair packing at tile granularity.
//
// Rows are padded to 80 bytes in LDS so that eight lanes reading 16 bytes of eight
// consecutive rows hit distinct banks. Workgroups are numbered so that each of the eight
// XCDs (each with its own L2) walks a contiguous range of row tiles: neighbouring output
// rows gather neighbouring input rows, and those stay in one L2.
#include <hip/hip_runtime.h>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;    // output rows per workgroup
constexpr int kBK = 32;     // input channels per slice
constexpr int kLD = kBK + 8;  // LDS row stride in bf16 (80 bytes)

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
__global__ void k_transpose_w(const uint16_t* __restrict__ w, uint16_t* __restrict__ wt, int cin, int cout) {
  const int64_t total = 27ll * cin * cout;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t o = e / ((int64_t)cin * cout);
    const int64_t rem = e - o * cin * cout;
    const int64_t n = rem / cin, k = rem - n * cin;
    wt[e] = w[(o * cin + k) * cout + n];
  }
}

template <int BN>
__global__ __launch_bounds__(256) void k_conv_ggs_bf16(const int32_t* __restrict__ map, int64_t N,
                                                       const uint16_t* __restrict__ feats,
                                                       const uint16_t* __restrict__ wt, int cin, int cout,
                                                       uint16_t* __restrict__ out, int64_t col_tiles) {
  constexpr int NB = BN / 64;  // 32-column MFMA blocks per wave
  __shared__ int32_t s_map[27][kBM];
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kBM * kLD];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][BN * kLD];
  __shared__ uint32_t s_used;
  __shared__ uint8_t s_olist[27];
  __shared__ int s_nused;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int64_t t_lin = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t r0 = (t_lin / col_tiles) * kBM;
  const int64_t n0 = (t_lin % col_tiles) * BN;

  if (tid == 0) s_used = 0;
  __syncthreads();
  uint32_t used = 0;
  for (int idx = tid; idx < 27 * kBM; idx += 256) {
    const int o = idx / kBM, r = idx - o * kBM;
    const int32_t v = r0 + r < N ? map[(size_t)o * (size_t)N + r0 + r] : -1;
    s_map[o][r] = v;
    if (v >= 0) used |= 1u << o;
  }
  if (used) atomicOr(&s_used, used);
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int o = 0; o < 27; ++o)
      if ((s_used >> o) & 1u) s_olist[n++] = (uint8_t)o;
    s_nused = n;
  }
  __syncthreads();

  const int kslices = cin / kBK;
  const int nchunks = s_nused * kslices;

  // Loader: A has 128 rows x 4 segments of 16 B (2 per thread); B has BN rows x 4 (NB per thread).
  uint4 ra[2], rb[NB];
  auto load = [&](int c) {
    const int o = s_olist[c / kslices];
    const int kc = (c % kslices) * kBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = tid + 256 * i;
      const int row = slot >> 2, seg = slot & 3;
      const int32_t src = s_map[o][row];
      ra[i] = src >= 0 ? *(const uint4*)(feats + (size_t)src * cin + kc + seg * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int slot = tid + 256 * i;
      const int n = slot >> 2, seg = slot & 3;
      rb[i] = *(const uint4*)(wt + ((size_t)o * cout + n0 + n) * cin + kc + seg * 8);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = tid + 256 * i;
      *(uint4*)&s_a[buf][(slot >> 2) * kLD + (slot & 3) * 8] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int slot = tid + 256 * i;
      *(uint4*)&s_b[buf][(slot >> 2) * kLD + (slot & 3) * 8] = rb[i];
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][NB];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.f;

  if (nchunks > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  const int arow = lane & 31, akg = (lane >> 5) * 8;
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) load(c + 1);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += 16) {
      bf16x8 a[2], b[NB];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *(const bf16x8*)&s_a[buf][(wm * 64 + mi * 32 + arow) * kLD + ks + akg];
#pragma unroll
      for (int ni = 0; ni < NB; ++ni)
        b[ni] = *(const bf16x8*)&s_b[buf][(wn * (BN / 2) + ni * 32 + arow) * kLD + ks + akg];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NB; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    if (c + 1 < nchunks) store(buf ^ 1);
    __syncthreads();
  }

  // D layout of the 32x32 block: lane holds column lane%32, rows 8i + 4(lane/32) + j.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < NB; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t row = r0 + wm * 64 + mi * 32 + 8 * i + (lane >> 5) * 4 + j;
          const int64_t col = n0 + wn * (BN / 2) + ni * 32 + (lane & 31);
          if (row < N) out[row * cout + col] = f32_to_bf16_rne(acc[mi][ni][4 * i + j]);
        }
}

}  // namespace

bool ggs_conv_supported(int32_t dtype, int32_t cin, int32_t cout) {
  return dtype == IGC_BF16 && cin >= 32 && cin <= 1024 && cin % 32 == 0 && cout >= 64 && cout <= 1024 &&
         cout % 64 == 0;
}

int launch_conv_ggs(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                    const void* d_w, int32_t cout, void* d_out, hipStream_t s) {
  (void)dtype;
  const int64_t N = g->n_voxels;
  uint16_t* wt = nullptr;
  int rc = dev_alloc((void**)&wt, (size_t)27 * cin * cout * 2, s, "igc_sparse_conv: transposed weights");
  if (rc) return rc;
  k_transpose_w<<<256, 256, 0, s>>>((const uint16_t*)d_w, wt, cin, cout);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    const int64_t row_tiles = (N + kBM - 1) / kBM;
    if (cout % 128 == 0) {
      const int64_t col_tiles = cout / 128;
      k_conv_ggs_bf16<128><<<(unsigned)(row_tiles * col_tiles), 256, 0, s>>>(
          d_map, N, (const uint16_t*)d_feats, wt, cin, cout, (uint16_t*)d_out, col_tiles);
    } else {
      const int64_t col_tiles = cout / 64;
      k_conv_ggs_bf16<64><<<(unsigned)(row_tiles * col_tiles), 256, 0, s>>>(
          d_map, N, (const uint16_t*)d_feats, wt, cin, cout, (uint16_t*)d_out, col_tiles);
    }
    e = hipGetLastError();
  }
  dev_free(wt, s);
  if (e != hipSuccess) return hip_status(e, "igc_sparse_conv: gather-GEMM-scatter launch");
  return IGC_OK;
}

}  // namespace igc
