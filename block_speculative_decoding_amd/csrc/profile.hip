// Optional per-kernel-group timing: HIP events recorded on the launching stream
// around each launch of one named group.  Disarmed by default; when disarmed
// the hooks cost one flag test.  Only used by tests and the benchmark.
#include <string.h>

#include <string>
#include <vector>

#include "../../include/dfspec.h"
#include "common.h"

namespace dfs {
namespace {
struct ProfState {
  bool on = false;
  std::string group;
  std::vector<hipEvent_t> ev;   // 2 per launch
  int max_launches = 0;
  int used = 0;
  int depth = 0;                // nesting of scopes of the armed group
};
ProfState g;
}  // namespace

void prof_before(const char* group, hipStream_t s) {
  if (!g.on || g.group != group) return;
  if (g.depth++ > 0) return;
  if (g.used < g.max_launches) hipEventRecord(g.ev[2 * g.used], s);
}

void prof_after(const char* group, hipStream_t s) {
  if (!g.on || g.group != group) return;
  if (--g.depth > 0) return;
  if (g.used < g.max_launches) {
    hipEventRecord(g.ev[2 * g.used + 1], s);
    ++g.used;
  }
}

}  // namespace dfs

extern "C" int dfs_profile_begin(const char* group, int32_t max_launches) {
  using dfs::g;
  if (!group || max_launches <= 0) return DFS_EINVAL;
  const size_t need = 2 * (size_t)max_launches;
  while (g.ev.size() < need) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return DFS_EHIP;
    g.ev.push_back(e);
  }
  g.group = group;
  g.max_launches = max_launches;
  g.used = 0;
  g.depth = 0;
  g.on = true;
  return DFS_OK;
}

extern "C" int dfs_profile_end(int32_t* launches, double* total_ms) {
  using dfs::g;
  if (!launches || !total_ms) return DFS_EINVAL;
  g.on = false;
  double tot = 0.0;
  for (int i = 0; i < g.used; ++i) {
    if (hipEventSynchronize(g.ev[2 * i + 1]) != hipSuccess) return DFS_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g.ev[2 * i], g.ev[2 * i + 1]) != hipSuccess) return DFS_EHIP;
    tot += ms;
  }
  *launches = g.used;
  *total_ms = tot;
  return DFS_OK;
}
