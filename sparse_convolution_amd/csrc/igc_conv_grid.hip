// Output grids of strided and transposed 3x3x3 convolutions, and the neighbour map between two
// grids (the grid-to-grid ops ConvGrid / ConvTransposeGrid in the op table of the "ONNX Runtime
// support for fVDB operations" proposal; DriveRT, "Shared neighbour maps" for two coordinate
// domains). Offsets d run over {-1, 0, 1}^3, o = (dx+1)*9 + (dy+1)*3 +
// (dz+1), and the stride s is per axis:
//   strided:    y is an output iff some input x = s*y + d; map[o, y] = in.index(s*y + d_o);
//   transposed: y is an output iff y = s*x + d for an input x; map[o, y] = in.index((y - d_o)/s)
//               where s divides y - d_o.
// The output grid is the IndexGrid build of a candidate list with a fixed number of entries,
// duplicates included (the build deduplicates): every candidate count is known on the host, so
// no compaction or extra read-back is needed.
//  - strided: per input leaf (origin O), the outputs y whose box [s y - 1, s y + 1] can meet the
//    leaf are y in [ceil((O - 1) / s), floor((O + 8) / s)], at most floor(9 / s) + 1 per axis;
//    each slot tests its box against the leaf's mask words and, if it misses, repeats an output
//    the leaf does produce (that of its first voxel). Leaves, not voxels, set the count.
//  - transposed: 27 slots per input voxel, y = s x + d.
#include <hip/hip_runtime.h>

#include "igc_host.h"
#include "igc_internal.h"

namespace igc {
namespace {

struct Stride3 {
  int32_t s[3];
};

// Candidate output coordinates of input voxel e: slots per axis (n0, n1, n2), row-major.
__global__ __launch_bounds__(256) void k_conv_candidates(const int32_t* __restrict__ ijk, int64_t n, Stride3 st,
                                                         int32_t transposed, int n0, int n1, int n2,
                                                         int32_t* __restrict__ out, uint32_t* __restrict__ flag) {
  const int slots = n0 * n1 * n2;
  const int64_t total = n * slots;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = e / slots;
    int slot = (int)(e - v * slots);
    const int js[3] = {slot / (n1 * n2), (slot / n2) % n1, slot % n2};
    int32_t y[3];
    bool ok = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const int64_t x = ijk[3 * v + a];
      const int64_t s = st.s[a];
      int64_t c;
      if (transposed) {
        c = s * x + (js[a] - 1);  // slot j <-> offset j - 1
      } else {
        // j-th offset d in {-1, 0, 1} with s | (x - d), or the first such offset.
        int64_t first = 0, pick = 0;
        int cnt = 0;
        for (int d = -1; d <= 1; ++d) {
          const int64_t z = x - d;
          if (((z % s) + s) % s == 0) {
            if (cnt == 0) first = z;
            if (cnt == js[a]) pick = z;
            ++cnt;
          }
        }
        const int64_t z = js[a] < cnt ? pick : first;
        c = z >= 0 ? z / s : -((-z) / s);  // exact: s divides z
        ok = ok && cnt > 0;
      }
      ok = ok && c >= INT32_MIN && c <= INT32_MAX;
      y[a] = (int32_t)c;
    }
    if (!ok) {
      atomicOr(flag, 1u);
      y[0] = y[1] = y[2] = 0;
    }
    out[3 * e] = y[0];
    out[3 * e + 1] = y[1];
    out[3 * e + 2] = y[2];
  }
}

__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Strided output candidates, R[0] x R[1] x R[2] slots per input leaf.
__global__ __launch_bounds__(256) void k_conv_candidates_leaf(GridView in, Stride3 st, int r0, int r1, int r2,
                                                              int32_t* __restrict__ out, uint32_t* __restrict__ flag) {
  const int slots = r0 * r1 * r2;
  const int64_t total = in.n_leaf * slots;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = e / slots;
    const int slot = (int)(e - f * slots);
    const int js[3] = {slot / (r1 * r2), (slot / r2) % r1, slot % r2};
    const int4 o4 = in.leaf_origin[f];
    const int64_t O[3] = {o4.x, o4.y, o4.z};
    const LeafRec& L = in.leaf[f];
    int64_t y[3];
    int lo[3], hi[3];
    bool hit = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const int64_t s = st.s[a];
      y[a] = -floor_div(-(O[a] - 1), s) + js[a];  // ceil((O - 1) / s) + slot
      hit = hit && y[a] <= floor_div(O[a] + 8, s);
      // The part of [s y - 1, s y + 1] inside the leaf, in leaf-local coordinates.
      const int64_t b0 = s * y[a] - 1 - O[a], b1 = s * y[a] + 1 - O[a];
      lo[a] = (int)(b0 < 0 ? 0 : b0);
      hi[a] = (int)(b1 > 7 ? 7 : b1);
      hit = hit && lo[a] <= hi[a];
    }
    if (hit) {
      // Bits (y, z) of the box in one mask word: rows y = lo1..hi1, columns z = lo2..hi2.
      const uint64_t zrow = ((1ull << (hi[2] - lo[2] + 1)) - 1ull) << lo[2];
      uint64_t pat = 0;
      for (int yy = lo[1]; yy <= hi[1]; ++yy) pat |= zrow << (8 * yy);
      bool any = false;
      for (int xx = lo[0]; xx <= hi[0]; ++xx) any = any || (L.mask[xx] & pat) != 0ull;
      hit = any;
    }
    if (!hit) {
      // The output of the leaf's first voxel x0: y0 = floor((x0 + 1) / s) has x0 in its box.
      int w = 0;
      while (w < 7 && L.mask[w] == 0ull) ++w;
      const int b = __ffsll((unsigned long long)L.mask[w]) - 1;
      const int64_t x0[3] = {O[0] + w, O[1] + (b >> 3), O[2] + (b & 7)};
#pragma unroll
      for (int a = 0; a < 3; ++a) y[a] = floor_div(x0[a] + 1, st.s[a]);
    }
    bool ok = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) ok = ok && y[a] >= INT32_MIN && y[a] <= INT32_MAX;
    if (!ok) atomicOr(flag, 1u);
    out[3 * e] = ok ? (int32_t)y[0] : 0;
    out[3 * e + 1] = ok ? (int32_t)y[1] : 0;
    out[3 * e + 2] = ok ? (int32_t)y[2] : 0;
  }
}

// map[o, r] for output voxel r (coordinates in row order) and the 27 offsets; one thread per
// output voxel, stores of one offset contiguous over the threads.
__global__ __launch_bounds__(256) void k_conv_map(GridView in, const int32_t* __restrict__ yijk, int64_t n_out,
                                                  Stride3 st, int32_t transposed, int32_t* __restrict__ map) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n_out; r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t y[3] = {yijk[3 * r], yijk[3 * r + 1], yijk[3 * r + 2]};
    for (int o = 0; o < 27; ++o) {
      const int d[3] = {o / 9 - 1, (o / 3) % 3 - 1, o % 3 - 1};
      int64_t q[3];
      bool ok = true;
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        const int64_t s = st.s[a];
        if (transposed) {
          const int64_t z = y[a] - d[a];
          const int64_t m = ((z % s) + s) % s;
          ok = ok && m == 0;
          q[a] = z >= 0 ? z / s : -((-z) / s);
        } else {
          q[a] = s * y[a] + d[a];
        }
        ok = ok && q[a] >= INT32_MIN && q[a] <= INT32_MAX;
      }
      int32_t idx = -1;
      if (ok) {
        const int32_t i = (int32_t)q[0], j = (int32_t)q[1], k = (int32_t)q[2];
        const int32_t f = find_leaf(in, i, j, k);
        if (f >= 0) {
          const LeafRec& L = in.leaf[f];
          idx = leaf_row(L.mask, L.offset, L.prefix,
                         (((uint32_t)i & 7u) << 6) | (((uint32_t)j & 7u) << 3) | ((uint32_t)k & 7u));
        }
      }
      map[(int64_t)o * n_out + r] = idx;
    }
  }
}

int grid_blocks(int64_t n, int64_t cap) {
  const int64_t b = (n + 255) / 256;
  return (int)(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

int conv_grid_slots(const int32_t* stride, int32_t transposed, int* n) {
  for (int a = 0; a < 3; ++a) {
    if (stride[a] < 1 || stride[a] > 3) return 0;
    n[a] = transposed ? 3 : (3 + stride[a] - 1) / stride[a];
  }
  return n[0] * n[1] * n[2];
}

int build_conv_grid(const igc_grid* in, const int32_t* stride, int32_t transposed, hipStream_t s, igc_grid* out) {
  int n[3];
  const int slots = conv_grid_slots(stride, transposed, n);
  if (slots == 0) return set_error(IGC_ERR_UNSUPPORTED, "igc_conv_grid: strides must be 1, 2 or 3");
  const int64_t N = in->n_voxels;
  if (N == 0) return build_grid(nullptr, 0, s, out);
  int R[3];
  for (int a = 0; a < 3; ++a) R[a] = 9 / stride[a] + 1;
  const int64_t n_cand = transposed ? N * slots : in->n_leaf * R[0] * R[1] * R[2];
  if (n_cand > INT32_MAX) return set_error(IGC_ERR_RANGE, "igc_conv_grid: candidate count exceeds 2^31-1");
  const size_t ijk_bytes = transposed ? align_up((size_t)N * 12, 256) : 0;
  const size_t cand_bytes = align_up((size_t)n_cand * 12, 256);
  char* ws = nullptr;
  const size_t ws_bytes = ijk_bytes + cand_bytes + 256;
  int rc = dev_alloc((void**)&ws, ws_bytes, s, "igc_conv_grid: workspace", grid_alloc(out));
  if (rc) return rc;
  int32_t* ijk = (int32_t*)ws;
  int32_t* cand = (int32_t*)(ws + ijk_bytes);
  uint32_t* flag = (uint32_t*)(ws + ijk_bytes + cand_bytes);
  rc = fill_u32(flag, 1, 0u, s);
  hipError_t e = hipSuccess;
  if (rc) {
    dev_free(ws, ws_bytes, s, grid_alloc(out));
    return rc;
  }
  Stride3 st{{stride[0], stride[1], stride[2]}};
  if (e == hipSuccess && transposed) {
    rc = launch_active_ijk(in, ijk, s);
    if (rc == IGC_OK) {
      k_conv_candidates<<<grid_blocks(n_cand, 8192), 256, 0, s>>>(ijk, N, st, transposed, n[0], n[1], n[2], cand, flag);
      e = hipGetLastError();
    }
  } else if (e == hipSuccess) {
    k_conv_candidates_leaf<<<grid_blocks(n_cand, 8192), 256, 0, s>>>(in->view(), st, R[0], R[1], R[2], cand, flag);
    e = hipGetLastError();
  }
  uint32_t h_flag = 0;
  if (e == hipSuccess && rc == IGC_OK) {
    e = hipMemcpyAsync(&h_flag, flag, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  if (e == hipSuccess && rc == IGC_OK && h_flag)
    rc = set_error(IGC_ERR_RANGE, "igc_conv_grid: an output coordinate leaves the int32 range");
  if (e == hipSuccess && rc == IGC_OK) {
    rc = build_grid(cand, n_cand, s, out);
    out->host_syncs += 1;  // the range flag's read-back
  }
  dev_free(ws, ws_bytes, s, grid_alloc(out));
  if (e != hipSuccess) return hip_status(e, "igc_conv_grid: candidates");
  return rc;
}

int launch_conv_map(const igc_grid* in, const igc_grid* out, const int32_t* stride, int32_t transposed,
                    int32_t* d_map, hipStream_t s) {
  const int64_t n_out = out->n_voxels;
  if (n_out == 0) return IGC_OK;
  Workspace wsb;
  int rc = ws_acquire(&wsb, (size_t)n_out * 12, s, "igc_conv_map: output coordinates", grid_alloc(out));
  if (rc) return rc;
  int32_t* ijk = (int32_t*)wsb.p;
  rc = launch_active_ijk(out, ijk, s);
  hipError_t e = hipSuccess;
  if (rc == IGC_OK) {
    Stride3 st{{stride[0], stride[1], stride[2]}};
    k_conv_map<<<grid_blocks(n_out, 16384), 256, 0, s>>>(in->view(), ijk, n_out, st, transposed, d_map);
    e = hipGetLastError();
  }
  ws_release(&wsb, s);
  if (rc) return rc;
  if (e != hipSuccess) return hip_status(e, "igc_conv_map: launch");
  return IGC_OK;
}

}  // namespace igc
