// Exercises every C entry point of the CPU oracle under AddressSanitizer / UndefinedBehavior-
// Sanitizer (built and run by tests/test_host_sanitizers.py): grids from random, duplicated,
// extreme (int32 limits) and empty coordinate sets, the topology export, coordinate and index
// queries, standard and custom kernel maps, and the convolution over all rows and a row subset.
// Exits non-zero on a failed consistency check; the sanitizers abort on any finding.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../oracle/igc_oracle.cpp"

static int fail(const char* what) {
  std::fprintf(stderr, "oracle driver: %s\n", what);
  return 1;
}

static int exercise(const std::vector<int32_t>& c, int cin, int cout) {
  const int64_t n = (int64_t)c.size() / 3;
  void* h = orc_build(n ? c.data() : nullptr, n);
  if (!h) return fail("orc_build returned null");
  int64_t k[4];
  orc_counts(h, k);
  const int64_t N = k[0], F = k[1], L = k[2], U = k[3];
  std::vector<uint64_t> root(U), umask(U * 512), lmask(L * 64), fmask(F * 8), foff(F), fpre(F);
  std::vector<int32_t> uo(U * 3), lo(L * 3), fo(F * 3);
  std::vector<uint32_t> uf(U), lf(L);
  orc_export(h, root.data(), uo.data(), umask.data(), uf.data(), lo.data(), lmask.data(), lf.data(), fo.data(),
             fmask.data(), foff.data(), fpre.data());
  std::vector<int32_t> ijk(N * 3);
  orc_active_ijk(h, ijk.data());
  // Every active voxel maps to its own row; shifted queries (some inactive, some past int32) too.
  std::vector<int32_t> idx(N);
  orc_ijk_to_index(h, ijk.data(), N, idx.data());
  for (int64_t r = 0; r < N; ++r)
    if (idx[r] != (int32_t)r) return fail("ijk_to_index is not the inverse of active_ijk");
  std::vector<int32_t> q(ijk);
  for (auto& v : q) v = v == INT32_MAX ? v : v + 1;
  orc_ijk_to_index(h, q.data(), N, idx.data());
  // Standard 27 offsets, with masks; then a custom list (K = 7, offsets up to +-2).
  std::vector<int32_t> off27;
  for (int o = 0; o < 27; ++o) off27.insert(off27.end(), {o / 9 - 1, (o / 3) % 3 - 1, o % 3 - 1});
  std::vector<int32_t> map(27 * N);
  std::vector<uint32_t> nb(N);
  orc_kernel_map(h, off27.data(), 27, map.data(), nb.data());
  for (int64_t r = 0; r < N; ++r)
    if (map[13 * N + r] != (int32_t)r) return fail("centre offset is not the identity");
  const int32_t off7[21] = {0, 0, 0, 2, 0, 0, -2, 0, 0, 0, 2, 0, 0, -2, 0, 0, 0, 2, 1, -1, 2};
  std::vector<int32_t> map7(7 * N);
  orc_kernel_map(h, off7, 7, map7.data(), nullptr);
  // Convolution over all rows and over a subset.
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  std::vector<float> f(N * cin), w(27 * cin * cout);
  for (auto& v : f) v = nd(rng);
  for (auto& v : w) v = nd(rng);
  std::vector<double> y(N * cout);
  orc_conv(map.data(), N, 27, f.data(), cin, w.data(), cout, nullptr, 0, y.data());
  std::vector<int64_t> rows;
  for (int64_t r = 0; r < N; r += 3) rows.push_back(r);
  std::vector<double> ys(rows.size() * cout);
  orc_conv(map.data(), N, 27, f.data(), cin, w.data(), cout, rows.data(), (int64_t)rows.size(), ys.data());
  for (size_t t = 0; t < rows.size(); ++t)
    for (int co = 0; co < cout; ++co)
      if (ys[t * cout + co] != y[rows[t] * cout + co]) return fail("row-subset conv differs");
  orc_free(h);
  return 0;
}

int main() {
  std::mt19937 rng(1);
  std::uniform_int_distribution<int32_t> u(-300, 300);
  std::vector<int32_t> c;
  for (int i = 0; i < 4000; ++i) c.insert(c.end(), {u(rng), u(rng) / 4, u(rng) / 16});
  for (int i = 0; i < 500; ++i) c.insert(c.end(), {c[3 * i], c[3 * i + 1], c[3 * i + 2]});  // duplicates
  if (exercise(c, 5, 7)) return 1;
  std::vector<int32_t> ext = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MIN, INT32_MIN, INT32_MIN, INT32_MAX, 0, INT32_MIN,
                              -1,        -1,        -1,        0,         0,         0,         INT32_MAX - 1, 0, 0};
  if (exercise(ext, 3, 2)) return 1;
  if (exercise({}, 4, 4)) return 1;
  std::printf("oracle driver: ok\n");
  return 0;
}
