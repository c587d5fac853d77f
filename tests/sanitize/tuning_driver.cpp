// Exercises the library's per-layer tuning-file parser (igc_tuning_load / ggs_tuning, host code of
// libigconv) under AddressSanitizer / UndefinedBehaviorSanitizer (built and run by
// tests/test_host_sanitizers.py): valid rules with wildcards and comments, every malformed form,
// unreadable paths, clearing, and loads racing with queries on four threads. The error-reporting
// functions of the library are replaced by the two below. Exits non-zero on a wrong result.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <thread>
#include <vector>

#include "igc_host.h"

namespace igc {
static thread_local std::string g_msg;
void clear_error() { g_msg.clear(); }
int set_error(int status, const std::string& msg) {
  g_msg = msg;
  return status;
}
}  // namespace igc

extern "C" int igc_tuning_load(const char* path);

static std::string write_file(const char* name, const char* text) {
  std::string p = std::string(std::getenv("SAN_TMP") ? std::getenv("SAN_TMP") : "/tmp") + "/" + name;
  FILE* f = std::fopen(p.c_str(), "w");
  std::fputs(text, f);
  std::fclose(f);
  return p;
}

static int check(bool ok, const char* what) {
  if (!ok) std::fprintf(stderr, "tuning driver: %s\n", what);
  return ok ? 0 : 1;
}

int main() {
  int bad = 0;
  // A comment line longer than the parser's read buffer, then rules (one with a 32-channel-chunk tile).
  const std::string text = "# comment line" + std::string(3000, 'x') + "\n"
                           "\n"
                           "ggs 128 256 0 0.5 4096 class auto   # trailing comment" + std::string(1000, 'y') + "\n"
                           "ggs 128 256 0.5 1e30 1024 natural 128\n"
                           "ggs 64 96 0 1e30 1024 class 64k32\n"
                           "ggs 96 128 0 1e30 256 natural 128h\n"
                           "ggs * 64 0 1e30 256 class 64\n"
                           "ggs * * 0 1e30 1024 natural\n";
  const std::string good = write_file("good.txt", text.c_str());
  bad += check(igc_tuning_load(good.c_str()) == 0, "valid file rejected");
  igc::GgsTuning t = igc::ggs_tuning(128, 256, 1000, 100);  // occupancy 1000 / 51200 < 0.5
  bad += check(t.span == 4096 && t.order == 1 && t.bn == 0, "first rule not matched");
  t = igc::ggs_tuning(128, 256, 51200, 100);  // occupancy 1.0
  bad += check(t.span == 1024 && t.order == 0 && t.bn == 128, "second rule not matched");
  t = igc::ggs_tuning(64, 96, 10, 10);
  bad += check(t.span == 1024 && t.order == 1 && t.bn == 64 && t.kc == 32, "32-channel-chunk rule not matched");
  t = igc::ggs_tuning(96, 128, 10, 10);
  bad += check(t.span == 256 && t.order == 0 && t.bn == 128 && t.kc == 0 && t.rows == 128, "half-tile rule not matched");
  t = igc::ggs_tuning(32, 64, 10, 10);
  bad += check(t.span == 256 && t.order == 1 && t.bn == 64, "wildcard cin not matched");
  t = igc::ggs_tuning(96, 96, 10, 10);
  bad += check(t.span == 1024 && t.bn == 0, "catch-all rule not matched");
  const char* malformed[] = {"ggs 128 256 0 1 512 class\n",       "ggs 128 256 0 1 256 diagonal\n",
                             "ggs 128 256 0 1 256 natural 96\n",  "ggs 128 256 zero 1 256 natural\n",
                             "ggs 128\n",                         "conv 128 256 0 1 256 natural\n",
                             "ggs -4 256 0 1 256 natural\n",      "ggs 128 256 0 1 256 natural auto extra\n",
                             "ggs 128 256 0 1 256 natural 256k32\n", "ggs 128 256 0 1 256 natural 256h\n"};
  for (size_t i = 0; i < sizeof malformed / sizeof malformed[0]; ++i) {
    const std::string p = write_file("bad.txt", malformed[i]);
    bad += check(igc_tuning_load(p.c_str()) != 0, "malformed line accepted");
    // A failed load leaves the previous table in place.
    bad += check(igc::ggs_tuning(128, 256, 1000, 100).span == 4096, "failed load changed the table");
  }
  bad += check(igc_tuning_load("/nonexistent/dir/rules.txt") != 0, "missing file accepted");
  bad += check(igc_tuning_load(nullptr) == 0, "clearing failed");
  t = igc::ggs_tuning(128, 256, 1000, 100);
  bad += check(t.span == 256 && t.order == 0 && t.bn == 0, "cleared table still matches");
  // Loads and queries from four threads at once (the table is guarded by a mutex).
  std::vector<std::thread> th;
  for (int k = 0; k < 4; ++k)
    th.emplace_back([&good, k] {
      for (int i = 0; i < 200; ++i) {
        if ((i + k) % 3 == 0) igc_tuning_load(good.c_str());
        else if ((i + k) % 7 == 0) igc_tuning_load(nullptr);
        else (void)igc::ggs_tuning(128, 256, 1000 + i, 100);
      }
    });
  for (auto& x : th) x.join();
  std::printf(bad ? "tuning driver: %d failures\n" : "tuning driver: ok\n", bad);
  return bad ? 1 : 0;
}
