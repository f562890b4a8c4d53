// Error reporting, status strings and the kernel timer of libstreambp.
#include <stdarg.h>
#include <stdio.h>

#include <map>
#include <string>
#include <vector>

#include "common.h"

namespace sbp {

static thread_local std::string g_last_error;

sbp_status set_error(sbp_status s, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

// ---------------------------------------------------------------------------
// Kernel timer: hipEvents around every launch while enabled.
// ---------------------------------------------------------------------------
namespace {
struct Rec {
  const char* name;
  double flops, bytes;
  int e0, e1;
};
struct Entry {
  std::string name;
  int64_t launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};
struct Prof {
  bool on = false;
  std::vector<hipEvent_t> ev;
  int next = 0;
  std::vector<Rec> recs;
  std::vector<Entry> out;
};
Prof& prof() {
  static Prof p;
  return p;
}
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t st, double flops, double bytes)
    : slot(-1), stream(st) {
  Prof& P = prof();
  if (!P.on || P.next + 2 > (int)P.ev.size()) return;
  Rec r{name, flops, bytes, P.next, P.next + 1};
  P.next += 2;
  if (hipEventRecord(P.ev[r.e0], st) != hipSuccess) return;
  slot = (int)P.recs.size();
  P.recs.push_back(r);
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  Prof& P = prof();
  (void)hipEventRecord(P.ev[P.recs[slot].e1], stream);
}

}  // namespace sbp

using namespace sbp;

extern "C" {

const char* sbp_status_string(int32_t s) {
  switch (s) {
    case SBP_OK: return "SBP_OK";
    case SBP_ERR_INVALID_ARG: return "SBP_ERR_INVALID_ARG";
    case SBP_ERR_UNSUPPORTED: return "SBP_ERR_UNSUPPORTED";
    case SBP_ERR_WORKSPACE: return "SBP_ERR_WORKSPACE";
    case SBP_ERR_HIP: return "SBP_ERR_HIP";
    default: return "SBP_ERR_UNKNOWN";
  }
}

const char* sbp_last_error(void) { return g_last_error.c_str(); }

int32_t sbp_version(void) { return 100; }

sbp_status sbp_profile_begin(int32_t max_launches) {
  Prof& P = prof();
  if (max_launches < 1) return set_error(SBP_ERR_INVALID_ARG, "max_launches must be >= 1");
  const size_t need = 2 * (size_t)max_launches;
  while (P.ev.size() < need) {
    hipEvent_t e;
    SBP_HIP_CHECK(hipEventCreate(&e));
    P.ev.push_back(e);
  }
  P.next = 0;
  P.recs.clear();
  P.out.clear();
  P.on = true;
  return SBP_OK;
}

sbp_status sbp_profile_end(int32_t* count) {
  Prof& P = prof();
  P.on = false;
  std::map<std::string, size_t> index;
  for (const Rec& r : P.recs) {
    SBP_HIP_CHECK(hipEventSynchronize(P.ev[r.e1]));
    float ms = 0.f;
    SBP_HIP_CHECK(hipEventElapsedTime(&ms, P.ev[r.e0], P.ev[r.e1]));
    auto it = index.find(r.name);
    size_t k;
    if (it == index.end()) {
      k = P.out.size();
      index[r.name] = k;
      P.out.push_back(Entry{r.name});
    } else {
      k = it->second;
    }
    Entry& e = P.out[k];
    e.launches += 1;
    e.ms += ms;
    e.flops += r.flops;
    e.bytes += r.bytes;
  }
  P.recs.clear();
  if (count) *count = (int32_t)P.out.size();
  return SBP_OK;
}

sbp_status sbp_profile_entry(int32_t i, const char** name, int64_t* launches, double* total_ms,
                             double* flops, double* bytes) {
  Prof& P = prof();
  if (i < 0 || i >= (int32_t)P.out.size()) return set_error(SBP_ERR_INVALID_ARG, "no entry %d", i);
  const Entry& e = P.out[i];
  if (name) *name = e.name.c_str();
  if (launches) *launches = e.launches;
  if (total_ms) *total_ms = e.ms;
  if (flops) *flops = e.flops;
  if (bytes) *bytes = e.bytes;
  return SBP_OK;
}

}  // extern "C"
