// Backward pass of the submanifold convolution (the operator of the fVDB notes' "accelerated
// operators for sparse convolution", differentiated; the notes list training support for these
// backends as future work).
//
// Forward: Y[r] = sum over o with map[o, r] >= 0 of W[o]^T X[map[o, r]].
//
// dgrad: dX[s] = sum over the pairs (o, r) with map[o, r] = s of W[o] dY[r]. For the 27 offsets
// of a 3x3x3 kernel the map is symmetric under negation (map[o, r] = s <=> map[26 - o, s] = r),
// so dX is the forward convolution of dY with W~[o] = W[26 - o]^T (k_flip_w) over the same map
// and grid: both forward paths serve as they are.
//
// wgrad: dW[o] = sum over r with map[o, r] >= 0 of X[map[o, r]] dY[r]^T, a reduction over all
// rows. Work is split over (offset, chunk of row tiles, channel block); each workgroup writes
// its partial block and k_wgrad_reduce adds the partials of all chunks in a fixed order, in
// fp64, so the result does not depend on scheduling.
//  - bf16: on the matrix cores (v_mfma_f32_16x16x32_bf16) with K = rows. Rows are taken in the
//    mask-sorted order of the gather-GEMM-scatter plan, 64 at a time; a 64-row stage that has
//    no pair at the workgroup's offset is skipped. The stage's gathered input rows and output
//    gradients are written to LDS transposed (channel-major, rows contiguous), so both MFMA
//    operands are 16-byte reads of 8 consecutive rows.
//  - fp32: the leaf-local kernel (k_wgrad_leaf_f32, fp32 MFMA over each leaf's window) for the
//    leaf path's shapes, otherwise plain fp32 FMAs over 64-row stages in LDS.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "igc_host.h"
#include "igc_internal.h"
#include "igc_wave.h"

namespace igc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kNOff = 27;
constexpr int kTileRows = 256;  // rows of a plan tile
constexpr int kStage = 64;      // rows staged at a time
constexpr int kLdT = kStage + 8;  // LDS row stride of the transposed stages (bf16): 144 bytes

// wf[o][co][ci] = w[26 - o][ci][co].
template <typename T>
__global__ void k_flip_w(const T* __restrict__ w, T* __restrict__ wf, int cin, int cout) {
  const int64_t total = (int64_t)kNOff * cin * cout;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t o = e / ((int64_t)cin * cout);
    const int64_t rem = e - o * cin * cout;
    const int64_t co = rem / cin, ci = rem - co * cin;
    wf[e] = w[((kNOff - 1 - o) * cin + ci) * cout + co];
  }
}

// Workgroup index -> (offset, chunk, m block, n block); the 27 offsets of one (chunk, block)
// are neighbours, so the chunk's output-gradient rows are re-read from L2.
struct WgradSplit {
  int64_t chunks, mblocks, nblocks;
  __device__ void decode(int64_t id, int& o, int64_t& chunk, int& mb, int& nb) const {
    o = (int)(id % kNOff);
    int64_t rest = id / kNOff;
    nb = (int)(rest % nblocks);
    rest /= nblocks;
    mb = (int)(rest % mblocks);
    chunk = rest / mblocks;
  }
};

// Partial dW blocks of MB input x NB output channels per (offset, chunk of tiles), bf16 data.
// NWV waves in 2 x (NWV/2), each (MB/2) x (NB/(NWV/2)) with 16x16x32 MFMAs. The stages (64 rows of a
// tile that hold at least one pair at the offset) are software-pipelined through registers:
// while the MFMAs consume stage i from LDS, the thread's loads for the next stages are in
// flight - the input and output-gradient rows of stage i+1, the source rows (kernel map) of
// stage i+2 and the row order of stage i+3. Thread tid stages rows 2 (tid % 32) and
// 2 (tid % 32) + 1 of a stage, for the 8-channel granules tid / 32 + (NT / 32) j.
// At least three waves per SIMD: the 128 x 128 block then keeps its accumulators in 146 VGPRs
// instead of spreading to 180 VGPR + AGPR, and three workgroups share a CU instead of two (each
// stage waits on its gathers; more workgroups overlap those waits). Measured: 128 -> 256 on 48M
// voxels 215 -> 195 ms, 128 -> 128 on 17M 36.2 -> 33.8 ms and on 204k 0.269 -> 0.239 ms; the
// smaller blocks already run six or eight waves per SIMD. Four waves spill.
template <int MB, int NB, int NWV>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(3))) void k_wgrad_bf16(const int32_t* __restrict__ map, int64_t N,
                                                    const int32_t* __restrict__ perm,
                                                    const uint16_t* __restrict__ blk,
                                                    const uint16_t* __restrict__ feats,
                                                    const uint16_t* __restrict__ dout, int cin, int cout,
                                                    int64_t n_tiles, int64_t tiles_per_chunk, WgradSplit sp,
                                                    float* __restrict__ part) {
  constexpr int NT = 64 * NWV;               // threads
  constexpr int WNW = NWV / 2;               // waves along the output channels
  constexpr int MI = MB / 32, NI = NB / WNW / 16;  // 16-blocks per wave
  constexpr int GS = NT / 32;                // granule step of a thread's staging items
  constexpr int XG = MB / 8, DG = NB / 8;    // 8-channel granules of a row
  constexpr int XI = (32 * XG + NT - 1) / NT, DI = (32 * DG + NT - 1) / NT;  // staging items per thread
  static_assert(MI >= 1 && NI >= 1, "block shape");
  __shared__ __attribute__((aligned(16))) uint16_t s_xt[MB * kLdT];  // [channel][row]
  __shared__ __attribute__((aligned(16))) uint16_t s_dt[NB * kLdT];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const int pr = tid & 31;
  int o, mb, nb;
  int64_t chunk;
  sp.decode(blockIdx.x, o, chunk, mb, nb);
  const int c0 = mb * MB, n0 = nb * NB;
  const int64_t t0 = chunk * tiles_per_chunk;
  const int64_t t1 = t0 + tiles_per_chunk < n_tiles ? t0 + tiles_per_chunk : n_tiles;
  const int32_t* map_o = map + (size_t)o * (size_t)N;

  // Stage cursor over the chunk: code t * 4 + st of the next stage with a pair, -1 past the end.
  int64_t ct = t0;
  int cst = -1;
  uint32_t cbits = t0 < t1 ? blk[t0 * kNOff + o] : 0u;
  uint32_t nbits = t0 + 1 < t1 ? blk[(t0 + 1) * kNOff + o] : 0u;
  auto next_stage = [&]() -> int64_t {
    while (ct < t1) {
      if (++cst == 4) {
        cst = 0;
        ++ct;
        cbits = nbits;
        nbits = ct + 1 < t1 ? blk[(ct + 1) * kNOff + o] : 0u;
        if (ct >= t1) break;
      }
      if ((cbits >> (cst * 4)) & 0xFu) return ct * 4 + cst;
    }
    return -1;
  };
  auto load_perm = [&](int64_t sc, int32_t& r0, int32_t& r1) {
    if (sc >= 0) {
      const int2 v = *(const int2*)&perm[(sc >> 2) * kTileRows + (sc & 3) * kStage + 2 * pr];
      r0 = v.x;
      r1 = v.y;
    } else {
      r0 = r1 = -1;
    }
  };
  auto load_src = [&](int32_t r, int32_t& src) { src = r >= 0 ? map_o[r] : -1; };
  uint4 xa[XI], xb[XI], da[DI], db[DI];  // stage data: rows 2 pr (a) and 2 pr + 1 (b)
  auto load_data = [&](int32_t r0, int32_t r1, int32_t s0, int32_t s1) {
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int g = (tid >> 5) + GS * j;
      const bool ok = 32 * XG >= NT || g < XG;
      xa[j] = ok && s0 >= 0 ? *(const uint4*)(feats + (size_t)s0 * cin + c0 + g * 8) : make_uint4(0, 0, 0, 0);
      xb[j] = ok && s1 >= 0 ? *(const uint4*)(feats + (size_t)s1 * cin + c0 + g * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < DI; ++j) {
      const int g = (tid >> 5) + GS * j;
      const bool ok = 32 * DG >= NT || g < DG;
      da[j] = ok && s0 >= 0 ? *(const uint4*)(dout + (size_t)r0 * cout + n0 + g * 8) : make_uint4(0, 0, 0, 0);
      db[j] = ok && s1 >= 0 ? *(const uint4*)(dout + (size_t)r1 * cout + n0 + g * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  // Transposed store: channel c of granule g gets the pair (row 2 pr, row 2 pr + 1) as one word.
  auto store_pair = [&](uint16_t* dst, int g, const uint4& a, const uint4& b) {
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t lo = (av[c >> 1] >> ((c & 1) * 16)) & 0xFFFFu, hi = (bv[c >> 1] >> ((c & 1) * 16)) & 0xFFFFu;
      *(uint32_t*)&dst[(g * 8 + c) * kLdT + 2 * pr] = lo | (hi << 16);
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prologue: data of the first stage, source rows of the second, row order of the third.
  int64_t cur = next_stage();
  int64_t nx1 = next_stage();
  int64_t nx2 = next_stage();
  int32_t r0, r1, s0, s1;
  load_perm(cur, r0, r1);
  load_src(r0, s0);
  load_src(r1, s1);
  load_data(r0, r1, s0, s1);
  int32_t m_r0, m_r1, m_s0, m_s1;  // stage nx1
  load_perm(nx1, m_r0, m_r1);
  load_src(m_r0, m_s0);
  load_src(m_r1, m_s1);
  int32_t p_r0, p_r1;  // stage nx2
  load_perm(nx2, p_r0, p_r1);

  const int frow = lane & 15, fk = (lane >> 4) * 8;
  while (cur >= 0) {
    __syncthreads();  // the previous stage's LDS reads are done
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int g = (tid >> 5) + GS * j;
      if (32 * XG >= NT || g < XG) store_pair(s_xt, g, xa[j], xb[j]);
    }
#pragma unroll
    for (int j = 0; j < DI; ++j) {
      const int g = (tid >> 5) + GS * j;
      if (32 * DG >= NT || g < DG) store_pair(s_dt, g, da[j], db[j]);
    }
    // Loads for the next stages.
    load_data(m_r0, m_r1, m_s0, m_s1);
    m_r0 = p_r0;
    m_r1 = p_r1;
    load_src(m_r0, m_s0);
    load_src(m_r1, m_s1);
    const int64_t nx3 = next_stage();
    load_perm(nx3, p_r0, p_r1);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kStage; ks += 32) {
      bf16x8 a[MI], b[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        a[mi] = *(const bf16x8*)&s_xt[(wm * (MB / 2) + mi * 16 + frow) * kLdT + ks + fk];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        b[ni] = *(const bf16x8*)&s_dt[(wn * (NB / WNW) + ni * 16 + frow) * kLdT + ks + fk];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    cur = nx1;
    nx1 = nx2;
    nx2 = nx3;
  }
  // D layout: lane holds column lane%16 of rows 4*(lane/16) + j.
  float* dst = part + ((size_t)chunk * kNOff + o) * (size_t)cin * cout;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = c0 + wm * (MB / 2) + mi * 16 + (lane >> 4) * 4 + j;
        const int n = n0 + wn * (NB / WNW) + ni * 16 + frow;
        dst[(size_t)m * cout + n] = acc[mi][ni][j];
      }
}

// dw[e] = sum over chunks c of part[c * E + e], in fp64 and in a fixed order: thread group q
// of NG adds the chunks c = q, q + NG, ... in increasing order, then the NG group sums are added
// in order of q. A workgroup covers 256 / NG consecutive elements.
template <int NG>
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ part, int64_t chunks, int64_t E,
                                                      float* __restrict__ dw) {
  constexpr int EL = 256 / NG;
  __shared__ double s_sum[NG][EL];
  const int el = threadIdx.x % EL, q = threadIdx.x / EL;
  const int64_t e = (int64_t)blockIdx.x * EL + el;
  double acc = 0.0;
  if (e < E) {
#pragma unroll 8
    for (int64_t c = q; c < chunks; c += NG) acc += (double)part[c * E + e];
  }
  s_sum[q][el] = acc;
  __syncthreads();
  if (q == 0 && e < E) {
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < NG; ++k) t += s_sum[k][el];
    dw[e] = (float)t;
  }
}

}  // namespace

int launch_wgrad_reduce(const float* part, int64_t chunks, int64_t E, float* dw, hipStream_t s) {
  // Few elements and many chunks: more threads per element.
  if (E >= 65536 || chunks <= 64)
    k_wgrad_reduce<8><<<(unsigned)((E + 31) / 32), 256, 0, s>>>(part, chunks, E, dw);
  else
    k_wgrad_reduce<32><<<(unsigned)((E + 7) / 8), 256, 0, s>>>(part, chunks, E, dw);
  IGC_HIP(hipGetLastError(), "igc_sparse_conv_backward: weight-gradient reduction launch");
  return IGC_OK;
}

namespace {

template <int MB, int NB, int NWV>
int launch_wgrad_bf16(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t cin,
                      const void* d_dout, int32_t cout, float* d_dw, hipStream_t s) {
  const int64_t N = g->n_voxels;
  const int64_t n_tiles = (N + kTileRows - 1) / kTileRows;
  WgradSplit sp;
  sp.mblocks = cin / MB;
  sp.nblocks = cout / NB;
  // Chunks of tiles per workgroup: about 32768 workgroups, so that the work per workgroup and
  // the last round of workgroups even out (measured against about 2048: 128 -> 256 on 48M
  // voxels 191 -> 157 ms, 64 -> 64 on 17M 17.0 -> 13.8 ms, 128 -> 128 on 17M 32.7 -> 27.2 ms);
  // at least 11 tiles per chunk, since on small grids the partial blocks and their reduction
  // take over (128 -> 128 on 204k voxels: 0.236 ms at 11 tiles per chunk, 0.255 at 5, 0.351
  // at 3, and 0.281 at 23); and at most 4 GiB of partial blocks. The chunking depends only on
  // the grid's size and the channel counts, so results stay run-to-run identical.
  const int64_t E = (int64_t)kNOff * cin * cout;
  const int64_t per_chunk = (int64_t)kNOff * sp.mblocks * sp.nblocks;  // workgroups per chunk
  int64_t tpc = (n_tiles * per_chunk + 32767) / 32768;
  if (tpc < 11) tpc = 11;
  const int64_t max_chunks = std::max<int64_t>(1, ((int64_t)1 << 32) / (E * 4));
  if ((n_tiles + tpc - 1) / tpc > max_chunks) tpc = (n_tiles + max_chunks - 1) / max_chunks;
  const int64_t chunks = (n_tiles + tpc - 1) / tpc;
  sp.chunks = chunks;
  const size_t perm_bytes = align_up((size_t)n_tiles * kTileRows * 4, 256);
  const size_t blk_bytes = align_up((size_t)n_tiles * kNOff * 2, 256);
  const size_t part_bytes = align_up((size_t)chunks * E * 4, 256);
  Workspace wsb;
  int rc = ws_acquire(&wsb, perm_bytes + blk_bytes + part_bytes, s, "igc_sparse_conv_backward: wgrad workspace",
                      grid_alloc(g));
  if (rc) return rc;
  char* ws = (char*)wsb.p;
  int32_t* perm = (int32_t*)ws;
  uint16_t* blk = (uint16_t*)(ws + perm_bytes);
  float* part = (float*)(ws + perm_bytes + blk_bytes);
  rc = launch_ggs_plan(d_map, N, perm, blk, s);
  hipError_t e = hipSuccess;
  if (rc == IGC_OK) {
    k_wgrad_bf16<MB, NB, NWV><<<(unsigned)(kNOff * chunks * sp.mblocks * sp.nblocks), 64 * NWV, 0, s>>>(
        d_map, N, perm, blk, (const uint16_t*)d_feats, (const uint16_t*)d_dout, cin, cout, n_tiles, tpc, sp, part);
    e = hipGetLastError();
    if (e != hipSuccess) rc = hip_status(e, "igc_sparse_conv_backward: wgrad launch");
    else rc = launch_wgrad_reduce(part, chunks, E, d_dw, s);
  }
  ws_release(&wsb, s);
  return rc;
}

int launch_wgrad_f32(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t cin, const void* d_dout,
                     int32_t cout, float* d_dw, hipStream_t s) {
  const int64_t E = (int64_t)kNOff * cin * cout;
  if (wgrad_leaf_supported(cin, cout)) {
    const int64_t groups = wgrad_leaf_groups(g);
    Workspace wsb;
    int rc = ws_acquire(&wsb, (size_t)groups * E * 4, s, "igc_sparse_conv_backward: wgrad partials", grid_alloc(g));
    if (rc) return rc;
    float* part = (float*)wsb.p;
    rc = launch_wgrad_leaf(g, d_feats, cin, d_dout, cout, part, groups, s);
    if (rc == IGC_OK) rc = launch_wgrad_reduce(part, groups, E, d_dw, s);
    ws_release(&wsb, s);
    return rc;
  }
  // Row chunks on the general-shape kernel (4 x 4 register blocks): 55.7 ms against 387 ms for
  // one workgroup per (offset, chunk) with a thread per weight, fp32 32 -> 32 on the band scene.
  return launch_wgrad_gather(g, d_map, d_feats, IGC_F32, cin, d_dout, cout, d_dw, s);
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) p[e] = v;
}

}  // namespace

int fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return IGC_OK;
  const int64_t b = (n + 255) / 256;
  k_fill_u32<<<(unsigned)(b < 2048 ? b : 2048), 256, 0, s>>>(p, n, v);
  IGC_HIP(hipGetLastError(), "fill kernel launch");
  return IGC_OK;
}

bool wgrad_supported(int32_t dtype, int32_t cin, int32_t cout) {
  return wgrad_tuned_supported(dtype, cin, cout) || gather_conv_supported(dtype, cin, cout);
}

bool wgrad_tuned_supported(int32_t dtype, int32_t cin, int32_t cout) {
  if (dtype == IGC_BF16) return cin >= 32 && cin % 32 == 0 && cin <= 1024 && cout >= 64 && cout % 64 == 0 && cout <= 1024;
  return dtype == IGC_F32 && cin >= 1 && cout >= 1 && cin <= 64 && cout <= 64 && cin * cout <= 1024;
}

int launch_conv_backward(const igc_grid* g, const int32_t* d_map, const void* d_feats, int32_t dtype, int32_t cin,
                         const void* d_w, int32_t cout, const void* d_dout, void* d_dfeats, float* d_dw,
                         int32_t dgrad_path, hipStream_t s) {
  const size_t esize = dtype == IGC_BF16 ? 2 : 4;
  if (d_dfeats) {
    void* wf = nullptr;
    const size_t wf_bytes = (size_t)kNOff * cin * cout * esize;
    int rc = dev_alloc(&wf, wf_bytes, s, "igc_sparse_conv_backward: flipped weights", grid_alloc(g));
    if (rc) return rc;
    if (dtype == IGC_BF16)
      k_flip_w<uint16_t><<<256, 256, 0, s>>>((const uint16_t*)d_w, (uint16_t*)wf, cin, cout);
    else
      k_flip_w<float><<<256, 256, 0, s>>>((const float*)d_w, (float*)wf, cin, cout);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      dev_free(wf, wf_bytes, s, grid_alloc(g));
      return hip_status(e, "igc_sparse_conv_backward: weight flip launch");
    }
    // dX = forward conv of dY (cout channels) with W~ (cout -> cin).
    rc = dgrad_path == IGC_PATH_LEAF     ? launch_conv_leaf(g, d_dout, dtype, cout, wf, cin, d_dfeats, s)
         : dgrad_path == IGC_PATH_GATHER ? launch_conv_gather(g, d_map, g->n_voxels, g->n_voxels, d_dout, dtype, cout,
                                                              wf, cin, d_dfeats, s)
                                         : launch_conv_ggs(g, d_map, d_dout, dtype, cout, wf, cin, d_dfeats, s);
    dev_free(wf, wf_bytes, s, grid_alloc(g));
    if (rc) return rc;
  }
  if (d_dw) {
    // Shapes the tuned kernels do not take run on the general-shape kernel (IGC_TEST_WGRAD_FORM =
    // "general" sends every shape there: tests and measurements).
    const char* form = std::getenv("IGC_TEST_WGRAD_FORM");
    if (!wgrad_tuned_supported(dtype, cin, cout) || (form && !std::strcmp(form, "general")))
      return launch_wgrad_gather(g, d_map, d_feats, dtype, cin, d_dout, cout, d_dw, s);
    if (dtype == IGC_BF16) {
      // 128 x 256 blocks on 8 waves (85 FLOP per staged byte instead of 64) measured slower on
      // the large workload (222 ms against 214): staging is not bound by the L2 feed.
      if (cin % 128 == 0 && cout % 128 == 0)
        return launch_wgrad_bf16<128, 128, 4>(g, d_map, d_feats, cin, d_dout, cout, d_dw, s);
      if (cin % 64 == 0) return launch_wgrad_bf16<64, 64, 4>(g, d_map, d_feats, cin, d_dout, cout, d_dw, s);
      return launch_wgrad_bf16<32, 64, 4>(g, d_map, d_feats, cin, d_dout, cout, d_dw, s);
    }
    return launch_wgrad_f32(g, d_map, d_feats, cin, d_dout, cout, d_dw, s);
  }
  return IGC_OK;
}

}  // namespace igc
