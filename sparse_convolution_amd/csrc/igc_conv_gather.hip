// General-shape path of the 3x3x3 sparse convolution and its weight gradient, for the channel
// counts and dtypes the tuned paths do not take (fVDB notes, "accelerated operators for sparse
// convolution": the convolution as a sum over the kernel map's (input, output) pairs; this is
// that sum written out per output row).
//
// k_conv_gather: one lane per output row and a slice of up to 32 output channels (the slice is
// the grid's second dimension). For each offset with a neighbour the lane reads the neighbour's
// input row channel by channel and multiplies it into its accumulators with the weights
// W[o, ci, co0 .. co0 + 31], which are the same for every lane of the wave: k_pack_w first
// writes them as fp32 in aligned runs of 8, 16 or 32 words (zero past cout), so the kernel reads
// them with scalar loads and one weight feeds 64 rows. fp32 accumulation in the order (o, ci),
// so results are deterministic; bf16 outputs are rounded to nearest even.
//
// k_wgrad_gather: partial dW per (chunk of rows, tile of up to 64 x 64 channels, offset), rows
// staged 64 at a time in LDS (the gathered input rows of that offset and the output-gradient
// rows) and multiplied in 4 x 4 register blocks, summed in fp32 in a fixed order; the chunks are
// then summed in fp64 in a fixed order by the weight-gradient reduction. Small layers (a first
// layer's few input channels) take k_wgrad_gather_all instead: one workgroup covers all 27
// offsets of its rows, so each output-gradient row is staged once instead of once per offset.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

constexpr int kNOffG = 27;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) == 0x7F800000u) {
    *p = (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));  // inf / nan
    return;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  *p = (uint16_t)(u >> 16);
}

// wp[((o * cin + ci) * slices + sl) * COB + j] = W[o, ci, sl * COB + j] in fp32, zero past cout:
// every (offset, input channel, slice) run of weights is COB aligned words.
template <typename T>
__global__ void k_pack_w(const T* __restrict__ w, float* __restrict__ wp, int cin, int cout, int slices, int cob) {
  const int64_t total = (int64_t)kNOffG * cin * slices * cob;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(e % cob);
    const int64_t r = e / cob;
    const int sl = (int)(r % slices);
    const int64_t oc = r / slices;  // o * cin + ci
    const int co = sl * cob + j;
    wp[e] = co < cout ? to_f32(w[oc * cout + co]) : 0.f;
  }
}

// VEC: input rows are 16-byte aligned and a whole number of 16-byte granules (8 bf16 or 4 fp32
// channels), read one granule per load.
template <typename T, int COB, bool VEC>
__global__ __launch_bounds__(256) void k_conv_gather(const int32_t* __restrict__ map, int64_t N, int64_t n_in,
                                                     const T* __restrict__ feats, int cin,
                                                     const float* __restrict__ wp, int cout, int slices,
                                                     T* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= N) return;
  const int sl = blockIdx.y;
  float acc[COB];
#pragma unroll
  for (int j = 0; j < COB; ++j) acc[j] = 0.f;
  for (int o = 0; o < kNOffG; ++o) {
    const int32_t src = map[(size_t)o * (size_t)N + row];
    if (src < 0 || (int64_t)src >= n_in) continue;  // absent, or outside the input rows
    const T* fr = feats + (size_t)src * cin;
    const float* wo = wp + ((size_t)o * cin * slices + sl) * COB;  // wave-uniform: scalar loads
    // Eight input channels per step: their loads are in flight together.
    for (int c0 = 0; c0 < cin; c0 += 8) {
      float f[8];
      if constexpr (VEC && sizeof(T) == 2) {
        const uint4 q = *(const uint4*)(fr + c0);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[2 * k] = __uint_as_float(u[k] << 16);
          f[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
        }
      } else if constexpr (VEC) {
        const float4 a = *(const float4*)(fr + c0);
        const float4 b = c0 + 4 < cin ? *(const float4*)(fr + c0 + 4) : float4{0.f, 0.f, 0.f, 0.f};
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = c0 + k < cin ? to_f32(fr[c0 + k]) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (c0 + k < cin) {
          const float* wr = wo + (size_t)(c0 + k) * slices * COB;
#pragma unroll
          for (int j = 0; j < COB; ++j) acc[j] = fmaf(f[k], wr[j], acc[j]);
        }
      }
    }
  }
  const int co0 = sl * COB;
  T* y = out + (size_t)row * cout + co0;
#pragma unroll
  for (int j = 0; j < COB; ++j)
    if (co0 + j < cout) store_out(y + j, acc[j]);
}

constexpr int kWgStage = 64;  // rows staged per step
constexpr int kWgTile = 64;   // input and output channels per tile

// part[(chunk * 27 + o) * cin * cout + ci * cout + co] = sum over the chunk's rows r with
// map[o, r] in [0, n_in) of feats[map[o, r], ci] * dout[r, co], for one tile of up to 64 input x
// 64 output channels. A thread owns 4 x 4 of the tile; the T threads that cover the tile form a
// group, and the 256 / T groups of the workgroup take the staged rows in turn (row k goes to
// group k mod G), so small tiles keep every thread busy. The groups' sums are added in group
// order at the end: the result does not depend on timing.
template <typename T>
__global__ __launch_bounds__(256) void k_wgrad_gather(const int32_t* __restrict__ map, int64_t N, int64_t n_in,
                                                      const T* __restrict__ feats, const T* __restrict__ dout,
                                                      int cin, int cout, int ci_tiles, int co_tiles,
                                                      int64_t rows_per_chunk, float* __restrict__ part) {
  __shared__ __align__(16) float s_x[kWgStage][kWgTile];
  __shared__ __align__(16) float s_d[kWgStage][kWgTile];
  __shared__ int32_t s_src[kWgStage];
  const int tid = threadIdx.x;
  int64_t b = blockIdx.x;
  const int o = (int)(b % kNOffG);  // the 27 offsets of one row range run next to each other
  b /= kNOffG;
  const int cot = (int)(b % co_tiles);
  b /= co_tiles;
  const int cit = (int)(b % ci_tiles);
  const int64_t chunk = b / ci_tiles;
  const int ci0 = cit * kWgTile, co0 = cot * kWgTile;
  const int CI = cin - ci0 < kWgTile ? cin - ci0 : kWgTile;
  const int CO = cout - co0 < kWgTile ? cout - co0 : kWgTile;
  const int TI = (CI + 3) / 4, TJ = (CO + 3) / 4, TT = TI * TJ, NG = 256 / TT;
  const int g = tid / TT, t = tid % TT, ti = t / TJ, tj = t % TJ;
  const int64_t r0 = chunk * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < N ? r0 + rows_per_chunk : N;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
  for (int64_t base = r0; base < r1; base += kWgStage) {
    __syncthreads();
    if (tid < kWgStage) {
      const int64_t r = base + tid;
      const int32_t src = r < r1 ? map[(size_t)o * (size_t)N + r] : -1;
      s_src[tid] = src >= 0 && (int64_t)src < n_in ? src : -1;
    }
    __syncthreads();
    // Rows without a neighbour at o (and past the chunk) stage zeros on both sides. Columns past
    // CI / CO are not written: they only reach accumulators that are never stored.
    for (int i = tid; i < kWgStage * CI; i += 256) {
      const int k = i / CI, c = i - k * CI;
      const int32_t src = s_src[k];
      s_x[k][c] = src >= 0 ? to_f32(feats[(size_t)src * cin + ci0 + c]) : 0.f;
    }
    for (int i = tid; i < kWgStage * CO; i += 256) {
      const int k = i / CO, c = i - k * CO;
      s_d[k][c] = s_src[k] >= 0 ? to_f32(dout[(size_t)(base + k) * cout + co0 + c]) : 0.f;
    }
    __syncthreads();
    if (g < NG) {
      for (int k = g; k < kWgStage; k += NG) {
        const float4 x = *(const float4*)&s_x[k][4 * ti];
        const float4 d = *(const float4*)&s_d[k][4 * tj];
        const float xv[4] = {x.x, x.y, x.z, x.w}, dv[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(xv[a], dv[c], acc[a][c]);
      }
    }
  }
  // Sum the groups in order: group g's 4 x 4 block of thread t goes to s_x as 16 words.
  float* red = &s_x[0][0];  // 256 threads x 16 words = the size of s_x
  __syncthreads();
  if (g < NG) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) red[(size_t)tid * 16 + a * 4 + c] = acc[a][c];
  }
  __syncthreads();
  if (tid < TT) {
    float sum[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sum[e] = red[(size_t)tid * 16 + e];
    for (int q = 1; q < NG; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[e] += red[((size_t)q * TT + tid) * 16 + e];
    float* dst = part + ((size_t)chunk * kNOffG + o) * (size_t)cin * cout;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ci = ci0 + 4 * ti + a;
      if (4 * ti + a < CI)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (4 * tj + c < CO) dst[(size_t)ci * cout + co0 + 4 * tj + c] = sum[a * 4 + c];
    }
  }
}

int gather_cob(int cout) { return cout <= 8 ? 8 : cout <= 16 ? 16 : 32; }

template <typename T>
hipError_t launch_gather_t(const int32_t* map, int64_t N, int64_t n_in, const void* feats, int cin, const void* w,
                           int cout, void* out, float* wp, hipStream_t s) {
  const int cob = gather_cob(cout), slices = (cout + cob - 1) / cob;
  const int64_t packed = (int64_t)kNOffG * cin * slices * cob;
  k_pack_w<T><<<(unsigned)std::min<int64_t>((packed + 255) / 256, 4096), 256, 0, s>>>((const T*)w, wp, cin, cout,
                                                                                    slices, cob);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)slices);
  const T* f = (const T*)feats;
  T* y = (T*)out;
  const bool vec = ((uintptr_t)feats & 15u) == 0 && ((size_t)cin * sizeof(T)) % 16 == 0;
  if (vec) {
    if (cob == 8) k_conv_gather<T, 8, true><<<grid, 256, 0, s>>>(map, N, n_in, f, cin, wp, cout, slices, y);
    else if (cob == 16) k_conv_gather<T, 16, true><<<grid, 256, 0, s>>>(map, N, n_in, f, cin, wp, cout, slices, y);
    else k_conv_gather<T, 32, true><<<grid, 256, 0, s>>>(map, N, n_in, f, cin, wp, cout, slices, y);
  } else {
    if (cob == 8) k_conv_gather<T, 8, false><<<grid, 256, 0, s>>>(map, N, n_in, f, cin, wp, cout, slices, y);
    else if (cob == 16) k_conv_gather<T, 16, false><<<grid, 256, 0, s>>>(map, N, n_in, f, cin, wp, cout, slices, y);
    else k_conv_gather<T, 32, false><<<grid, 256, 0, s>>>(map, N, n_in, f, cin, wp, cout, slices, y);
  }
  return hipGetLastError();
}

// Small layers: 27 * ceil(cin / 4) * ceil(cout / 4) <= 256 and cin <= CM (4 or 8). One
// workgroup per chunk of rows covers all 27 offsets, and thread (o, ti, tj) owns the 4 x 4 block
// (4 ti.., 4 tj..) of offset o, summing the chunk's rows in order. Per 64-row step the gathered
// input rows of every offset and the output-gradient rows (once) are staged in LDS. Same partial
// layout as k_wgrad_gather.
template <typename T, int CM>
__global__ __launch_bounds__(256) void k_wgrad_gather_all(const int32_t* __restrict__ map, int64_t N, int64_t n_in,
                                                          const T* __restrict__ feats, const T* __restrict__ dout,
                                                          int cin, int cout, int64_t rows_per_chunk,
                                                          float* __restrict__ part) {
  __shared__ __align__(16) float s_x[kNOffG][kWgStage][CM];
  __shared__ __align__(16) float s_d[kWgStage][kWgTile];
  const int tid = threadIdx.x;
  const int TI = (cin + 3) / 4, TJ = (cout + 3) / 4, TT = TI * TJ;
  const int o = tid / TT, t = tid % TT, ti = t / TJ, tj = t % TJ;
  const int64_t chunk = blockIdx.x;
  const int64_t r0 = chunk * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < N ? r0 + rows_per_chunk : N;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
  for (int64_t base = r0; base < r1; base += kWgStage) {
    __syncthreads();
    // Input rows of every (offset, row) of the step; absent neighbours and columns past cin
    // stage zeros.
    for (int i = tid; i < kNOffG * kWgStage; i += 256) {
      const int o2 = i / kWgStage, k = i - o2 * kWgStage;
      const int64_t r = base + k;
      int32_t src = r < r1 ? map[(size_t)o2 * (size_t)N + r] : -1;
      if (src < 0 || (int64_t)src >= n_in) src = -1;
#pragma unroll
      for (int c = 0; c < CM; ++c) s_x[o2][k][c] = src >= 0 && c < cin ? to_f32(feats[(size_t)src * cin + c]) : 0.f;
    }
    // Output-gradient rows, once for all offsets. Columns past cout are not written: they only
    // reach accumulators that are never stored.
    for (int i = tid; i < kWgStage * cout; i += 256) {
      const int k = i / cout, c = i - k * cout;
      const int64_t r = base + k;
      s_d[k][c] = r < r1 ? to_f32(dout[(size_t)r * cout + c]) : 0.f;
    }
    __syncthreads();
    if (o < kNOffG) {
      for (int k = 0; k < kWgStage; ++k) {
        const float4 x = *(const float4*)&s_x[o][k][4 * ti];
        const float4 d = *(const float4*)&s_d[k][4 * tj];
        const float xv[4] = {x.x, x.y, x.z, x.w}, dv[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(xv[a], dv[c], acc[a][c]);
      }
    }
  }
  if (o < kNOffG) {
    float* dst = part + ((size_t)chunk * kNOffG + o) * (size_t)cin * cout;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ci = 4 * ti + a;
      if (ci < cin)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (4 * tj + c < cout) dst[(size_t)ci * cout + 4 * tj + c] = acc[a][c];
    }
  }
}

// The shapes k_wgrad_gather_all takes, and its input-channel bound.
int wgrad_all_cm(int32_t cin, int32_t cout) {
  if (cin < 1 || cout < 1 || cout > kWgTile || kNOffG * ((cin + 3) / 4) * ((cout + 3) / 4) > 256) return 0;
  return cin <= 4 ? 4 : cin <= 8 ? 8 : 0;
}

}  // namespace

bool gather_conv_supported(int32_t dtype, int32_t cin, int32_t cout) {
  return (dtype == IGC_F32 || dtype == IGC_BF16) && cin >= 1 && cin <= kGatherMaxChannels && cout >= 1 &&
         cout <= kGatherMaxChannels;
}

size_t gather_scratch_bytes(int32_t cin, int32_t cout) {
  const int cob = gather_cob(cout);
  return align_up((size_t)kNOffG * cin * ((cout + cob - 1) / cob) * cob * 4, 256);
}

int launch_conv_gather(const igc_grid* g, const int32_t* d_map, int64_t N, int64_t n_in, const void* d_feats,
                       int32_t dtype, int32_t cin, const void* d_w, int32_t cout, void* d_out, hipStream_t s,
                       void* scratch) {
  if (N == 0) return IGC_OK;
  Workspace wsb;
  if (!scratch) {
    const int rc = ws_acquire(&wsb, gather_scratch_bytes(cin, cout), s, "igc_sparse_conv: general-shape weights",
                              grid_alloc(g));
    if (rc) return rc;
  }
  float* wp = (float*)(scratch ? scratch : wsb.p);
  const hipError_t e =
      dtype == IGC_BF16 ? launch_gather_t<uint16_t>(d_map, N, n_in, d_feats, cin, d_w, cout, d_out, wp, s)
                        : launch_gather_t<float>(d_map, N, n_in, d_feats, cin, d_w, cout, d_out, wp, s);
  if (!scratch) ws_release(&wsb, s);
  IGC_HIP(e, "igc_sparse_conv: general-shape launch");
  return IGC_OK;
}

int launch_wgrad_gather(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                        const void* d_dout, int32_t cout, float* d_dw, hipStream_t s) {
  const int64_t N = g->n_voxels;
  const int64_t E = (int64_t)kNOffG * cin * cout;
  if (const int cm = wgrad_all_cm(cin, cout)) {
    // All offsets per workgroup: about 8192 workgroups of 64 to 8192 rows, at most 256 MiB of
    // partial sums.
    int64_t chunks = 8192;
    if (chunks < (N + 8191) / 8192) chunks = (N + 8191) / 8192;
    const int64_t cap = ((int64_t)256 << 20) / (E * 4);
    if (chunks > cap) chunks = cap;
    if (chunks > (N + kWgStage - 1) / kWgStage) chunks = (N + kWgStage - 1) / kWgStage;
    if (chunks < 1) chunks = 1;
    const int64_t rpc = (N + chunks - 1) / chunks;
    chunks = (N + rpc - 1) / rpc;
    Workspace wsb;
    int rc = ws_acquire(&wsb, (size_t)chunks * E * 4, s, "igc_sparse_conv_backward: general-shape wgrad partials",
                        grid_alloc(g));
    if (rc) return rc;
    float* part = (float*)wsb.p;
    const bool bf = dtype == IGC_BF16;
    if (bf && cm == 4)
      k_wgrad_gather_all<uint16_t, 4><<<(unsigned)chunks, 256, 0, s>>>(
          d_map, N, N, (const uint16_t*)d_feats, (const uint16_t*)d_dout, cin, cout, rpc, part);
    else if (bf)
      k_wgrad_gather_all<uint16_t, 8><<<(unsigned)chunks, 256, 0, s>>>(
          d_map, N, N, (const uint16_t*)d_feats, (const uint16_t*)d_dout, cin, cout, rpc, part);
    else if (cm == 4)
      k_wgrad_gather_all<float, 4><<<(unsigned)chunks, 256, 0, s>>>(d_map, N, N, (const float*)d_feats,
                                                                    (const float*)d_dout, cin, cout, rpc, part);
    else
      k_wgrad_gather_all<float, 8><<<(unsigned)chunks, 256, 0, s>>>(d_map, N, N, (const float*)d_feats,
                                                                    (const float*)d_dout, cin, cout, rpc, part);
    const hipError_t e = hipGetLastError();
    rc = e != hipSuccess ? hip_status(e, "igc_sparse_conv_backward: general-shape wgrad launch")
                         : launch_wgrad_reduce(part, chunks, E, d_dw, s);
    ws_release(&wsb, s);
    return rc;
  }
  const int ci_tiles = (cin + kWgTile - 1) / kWgTile, co_tiles = (cout + kWgTile - 1) / kWgTile;
  // About 4096 workgroups, at most 8192 rows per chunk (the fp32 part of the sum), at least 64,
  // and at most 256 MiB of partial sums.
  int64_t chunks = 4096 / ((int64_t)kNOffG * ci_tiles * co_tiles);
  if (chunks < (N + 8191) / 8192) chunks = (N + 8191) / 8192;
  const int64_t cap = ((int64_t)256 << 20) / (E * 4);
  if (chunks > cap) chunks = cap;
  if (chunks < 1) chunks = 1;
  if (chunks > (N + kWgStage - 1) / kWgStage) chunks = (N + kWgStage - 1) / kWgStage;
  const int64_t rpc = (N + chunks - 1) / chunks;
  chunks = (N + rpc - 1) / rpc;
  Workspace wsb;
  int rc = ws_acquire(&wsb, (size_t)chunks * E * 4, s, "igc_sparse_conv_backward: general-shape wgrad partials",
                      grid_alloc(g));
  if (rc) return rc;
  float* part = (float*)wsb.p;
  const unsigned blocks = (unsigned)(chunks * kNOffG * ci_tiles * co_tiles);
  if (dtype == IGC_BF16)
    k_wgrad_gather<uint16_t><<<blocks, 256, 0, s>>>(d_map, N, N, (const uint16_t*)d_feats, (const uint16_t*)d_dout,
                                                    cin, cout, ci_tiles, co_tiles, rpc, part);
  else
    k_wgrad_gather<float><<<blocks, 256, 0, s>>>(d_map, N, N, (const float*)d_feats, (const float*)d_dout, cin, cout,
                                                 ci_tiles, co_tiles, rpc, part);
  const hipError_t e = hipGetLastError();
  rc = e != hipSuccess ? hip_status(e, "igc_sparse_conv_backward: general-shape wgrad launch")
                       : launch_wgrad_reduce(part, chunks, E, d_dw, s);
  ws_release(&wsb, s);
  return rc;
}

}  // namespace igc
