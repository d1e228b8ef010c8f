// Per-shape tuning table of the assignment kernel's tile configuration
// (host code only).  An entry maps an exact shape (dtype, D, N, B, K) to a
// compiled configuration; kmeans_tune fills it by timing, kmeans_tune_save /
// kmeans_tune_load persist it as text, FLASHKM_TUNE_CACHE names a file that is
// loaded once at the first lookup.
#include "kernels.h"
#include "workspace.h"

#include "flashkm.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

namespace fkm {

namespace {

struct Entry {
  int dt, D;
  int64_t N;
  int B, K;
  AssignConfig cfg;
  bool same_shape(const Entry& o) const { return dt == o.dt && D == o.D && N == o.N && B == o.B && K == o.K; }
};

std::mutex& table_mutex() {
  static std::mutex m;
  return m;
}
std::vector<Entry>& table() {
  static std::vector<Entry> t;
  return t;
}

void put_locked(const Entry& e) {
  for (Entry& x : table())
    if (x.same_shape(e)) {
      x.cfg = e.cfg;
      return;
    }
  table().push_back(e);
}

bool valid_shape(int dt, int D, int64_t N, int B, int K) {
  return (dt == DT_F32 || dt == DT_F16 || dt == DT_BF16) &&
         (D == 16 || D == 32 || D == 64 || D == 128 || D == 256) && B >= 1 && K >= 1 && N >= K;
}

// Parse a whole file; entries are added only if every line is valid.
int load_file(const char* path) {
  FILE* f = fopen(path, "r");
  if (!f) return fail(KM_EINVAL, "cannot open tuning table '%s'", path);
  std::vector<Entry> got;
  char line[512];
  int no = 0;
  int rc = KM_OK;
  while (fgets(line, sizeof line, f)) {
    ++no;
    char* hash = strchr(line, '#');
    if (hash) *hash = 0;
    char* p = line;
    while (*p == ' ' || *p == '\t' || *p == '\r' || *p == '\n') ++p;
    if (!*p) continue;
    int dt = 0, D = 0, B = 0, K = 0, pb = 0, w = 0;
    long long N = 0;
    char extra = 0;
    const int n = sscanf(p, "%d %d %lld %d %d %d %d %c", &dt, &D, &N, &B, &K, &pb, &w, &extra);
    if (n != 7) {
      rc = fail(KM_EINVAL, "%s:%d: expected 'dtype D N B K pb waves'", path, no);
      break;
    }
    if (!valid_shape(dt, D, N, B, K)) {
      rc = fail(KM_EINVAL, "%s:%d: unsupported shape", path, no);
      break;
    }
    const AssignConfig c{pb, w};
    if (!assign_config_compiled(dt, D, c)) {
      rc = fail(KM_EINVAL, "%s:%d: configuration pb=%d waves=%d is not compiled for this row size", path, no, pb, w);
      break;
    }
    got.push_back(Entry{dt, D, (int64_t)N, B, K, c});
  }
  fclose(f);
  if (rc != KM_OK) return rc;
  std::lock_guard<std::mutex> lock(table_mutex());
  for (const Entry& e : got) put_locked(e);
  return KM_OK;
}

void load_env_once() {
  static std::once_flag once;
  std::call_once(once, [] {
    if (const char* p = getenv("FLASHKM_TUNE_CACHE"))
      if (*p) {
        // a bad file leaves the table as it was and the caller's error text untouched
        char saved[512];
        memcpy(saved, err_buf(), sizeof saved);
        (void)load_file(p);
        memcpy(err_buf(), saved, sizeof saved);
      }
  });
}

}  // namespace

bool tune_lookup(int dt, int D, int64_t N, int B, int K, AssignConfig* cfg) {
  load_env_once();
  const Entry key{dt, D, N, B, K, {0, 0}};
  std::lock_guard<std::mutex> lock(table_mutex());
  for (const Entry& e : table())
    if (e.same_shape(key)) {
      *cfg = e.cfg;
      return true;
    }
  return false;
}

void tune_record(int dt, int D, int64_t N, int B, int K, AssignConfig cfg) {
  load_env_once();
  std::lock_guard<std::mutex> lock(table_mutex());
  put_locked(Entry{dt, D, N, B, K, cfg});
}

}  // namespace fkm

using namespace fkm;

extern "C" {

int kmeans_tune_save(const char* path) {
  err_buf()[0] = 0;
  if (!path) return fail(KM_EINVAL, "path is null");
  load_env_once();
  std::vector<Entry> snap;
  {
    std::lock_guard<std::mutex> lock(table_mutex());
    snap = table();
  }
  FILE* f = fopen(path, "w");
  if (!f) return fail(KM_EINVAL, "cannot open '%s' for writing", path);
  fprintf(f, "# flashkm assignment tuning table: dtype D N B K pb waves\n");
  for (const Entry& e : snap)
    fprintf(f, "%d %d %lld %d %d %d %d\n", e.dt, e.D, (long long)e.N, e.B, e.K, e.cfg.pb, e.cfg.waves);
  if (fclose(f) != 0) return fail(KM_EINVAL, "error writing '%s'", path);
  return KM_OK;
}

int kmeans_assign_configs(int32_t dtype, int32_t D, int32_t* pb, int32_t* waves, int32_t cap, int32_t* count) {
  err_buf()[0] = 0;
  if (!count || cap < 0 || (cap > 0 && (!pb || !waves)))
    return fail(KM_EINVAL, "count must be non-null, and pb and waves hold cap >= 0 entries");
  if (!valid_shape(dtype, D, 1, 1, 1)) return fail(KM_EUNSUPPORTED, "unsupported dtype %d or D=%d", dtype, D);
  AssignConfig all[8];
  const int n = assign_configs(dtype, D, all, 8);
  for (int i = 0; i < n && i < cap; ++i) {
    pb[i] = all[i].pb;
    waves[i] = all[i].waves;
  }
  *count = n;
  return KM_OK;
}

int kmeans_tune_load(const char* path) {
  err_buf()[0] = 0;
  if (!path) return fail(KM_EINVAL, "path is null");
  load_env_once();
  return load_file(path);
}

}  // extern "C"
