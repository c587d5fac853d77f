// Per-layer configuration of the gather-GEMM-scatter row order (DriveRT, "Kernels selected per
// GPU": tile sizes, bit orders and offset groups are configuration values measured per layer
// on the target GPU; "Measurement and reproducibility": the selection is stored in a
// documented file). A rule maps a layer (input / output channels and the grid's leaf
// occupancy N / (512 F)) to the span over which rows are sorted by their neighbour mask and
// the bit order of that sort; without a matching rule the span is one tile (256 rows) in
// natural order.
//
// File format (text, one rule per line, '#' starts a comment, first matching rule wins):
//   ggs <cin|*> <cout|*> <occupancy_lo> <occupancy_hi> <span> <natural|class> [tile]
// with span 256, 1024 or 4096, lo <= occupancy < hi, and tile (output channels per workgroup)
// auto, 256, 128 or 64. A width of 128 or 64 may carry the suffix k32 (32-channel chunks:
// smaller LDS stages, two workgroups per CU at 64 channels) and then h (each workgroup takes
// half of a 256-row plan tile), e.g. 128h or 64k32h.
#include <cctype>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "igc_host.h"

namespace igc {
namespace {

struct Rule {
  int32_t cin = -1, cout = -1;  // -1: any
  double occ_lo = 0.0, occ_hi = 1e30;
  GgsTuning tu;
};

std::mutex g_mu;
std::vector<Rule> g_rules;

}  // namespace

GgsTuning ggs_tuning(int32_t cin, int32_t cout, int64_t n_voxels, int64_t n_leaf) {
  const double occ = n_leaf > 0 ? (double)n_voxels / (512.0 * (double)n_leaf) : 0.0;
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Rule& r : g_rules)
    if ((r.cin < 0 || r.cin == cin) && (r.cout < 0 || r.cout == cout) && occ >= r.occ_lo && occ < r.occ_hi) return r.tu;
  return GgsTuning{};
}

}  // namespace igc

using namespace igc;

extern "C" int igc_tuning_load(const char* path) {
  clear_error();
  if (!path) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_rules.clear();
    return IGC_OK;
  }
  FILE* f = std::fopen(path, "r");
  if (!f) return set_error(IGC_ERR_INVALID_ARG, std::string("igc_tuning_load: cannot open ") + path);
  std::vector<Rule> rules;
  // Whole lines of any length (the measured times are kept as long comment lines).
  std::string text;
  auto next_line = [&]() {
    text.clear();
    char chunk[512];
    while (std::fgets(chunk, sizeof chunk, f)) {
      text += chunk;
      if (text.back() == '\n') return true;
    }
    return !text.empty();
  };
  int lineno = 0;
  int rc = IGC_OK;
  while (next_line()) {
    ++lineno;
    const size_t hash = text.find('#');
    if (hash != std::string::npos) text.resize(hash);
    const char* line = text.c_str();
    char kind[16] = "", cin[16] = "", cout[16] = "", order[16] = "", tile[16] = "auto";
    double lo = 0, hi = 0;
    int span = 0, used = 0;
    const int n = std::sscanf(line, "%15s %15s %15s %lf %lf %d %15s %15s%n", kind, cin, cout, &lo, &hi, &span, order,
                              tile, &used);
    if (n <= 0) continue;  // blank or comment
    // Nothing may follow the last field (%n is only set when all eight fields were read).
    const char* rest = line + used;
    if (n == 7) {  // no tile: everything after the order must be blank
      const char* p = std::strstr(line, order);
      rest = p ? p + std::strlen(order) : line;
    }
    bool extra = false;
    for (const char* p = rest; *p; ++p) extra |= !std::isspace((unsigned char)*p);
    // Channel counts: "*" or a positive integer.
    auto channels = [](const char* t, int32_t* v) {
      if (!std::strcmp(t, "*")) return *v = -1, true;
      char* end = nullptr;
      const long x = std::strtol(t, &end, 10);
      return *v = (int32_t)x, end != t && *end == '\0' && x > 0 && x <= 1 << 20;
    };
    Rule r;
    const bool ch_ok = channels(cin, &r.cin) && channels(cout, &r.cout);
    const bool order_ok = !std::strcmp(order, "natural") || !std::strcmp(order, "class");
    // Tile: <auto|256|128|64>, then for 128 and 64 optionally "k32", then optionally "h".
    std::string tk(tile);
    const bool half = tk.size() > 1 && tk.back() == 'h';
    if (half) tk.pop_back();
    const bool k32 = tk.size() > 3 && tk.compare(tk.size() - 3, 3, "k32") == 0;
    if (k32) tk.resize(tk.size() - 3);
    const int bn = tk == "256" ? 256 : tk == "128" ? 128 : tk == "64" ? 64 : 0;
    const bool tile_ok = ((tk == "auto" || bn == 256) && !k32 && !half) || bn == 128 || bn == 64;
    if ((n != 7 && n != 8) || extra || std::strcmp(kind, "ggs") || !ch_ok ||
        !(span == 256 || span == 1024 || span == 4096) || !order_ok || !tile_ok || !(lo <= hi)) {
      rc = set_error(IGC_ERR_INVALID_ARG, "igc_tuning_load: " + std::string(path) + ":" + std::to_string(lineno) +
                                              ": expected 'ggs <cin|*> <cout|*> <occ_lo> <occ_hi> <256|1024|4096> "
                                              "<natural|class> [auto|256|128|64, 128/64 with k32 and/or h]'");
      break;
    }
    r.tu.bn = bn;
    r.tu.kc = k32 ? 32 : 0;
    r.tu.rows = half ? 128 : 0;
    r.occ_lo = lo;
    r.occ_hi = hi;
    r.tu.span = span;
    r.tu.order = std::strcmp(order, "class") ? 0 : 1;
    rules.push_back(r);
  }
  std::fclose(f);
  if (rc != IGC_OK) return rc;
  std::lock_guard<std::mutex> lk(g_mu);
  g_rules.swap(rules);
  return IGC_OK;
}
