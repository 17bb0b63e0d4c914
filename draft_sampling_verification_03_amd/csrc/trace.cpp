// Kernel timing records (see trace.h) and their C ABI accessors.
#include "trace.h"

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dspark.h"

namespace dspark {
namespace {

struct Record {
  const char *name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;
struct Entry {
  std::string name;
  double ms;
  int launches;
};
std::vector<Entry> g_summary;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle_records() {
  for (auto &r : g_records) {
    if (r.start) g_pool.push_back(r.start);
    if (r.stop) g_pool.push_back(r.stop);
  }
  g_records.clear();
}

}  // namespace

bool trace_on() { return g_on.load(std::memory_order_relaxed); }

void trace_events(const char *name, hipEvent_t *start, hipEvent_t *stop) {
  std::lock_guard<std::mutex> lock(g_mu);
  Record r{name, take_event(), take_event()};
  g_records.push_back(r);
  *start = r.start;
  *stop = r.stop;
}

}  // namespace dspark

using namespace dspark;

extern "C" {

dspark_status dspark_trace_enable(int on) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (on) {
    // waits for outstanding records before their events are reused
    for (auto &r : g_records)
      if (r.stop) (void)hipEventSynchronize(r.stop);
    recycle_records();
    g_summary.clear();
  }
  g_on.store(on != 0, std::memory_order_relaxed);
  return DSPARK_OK;
}

int dspark_trace_collect(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  std::map<std::string, Entry> agg;
  std::vector<std::string> order;
  for (auto &r : g_records) {
    float ms = 0.0f;
    if (!r.start || !r.stop || hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return -1;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = Entry{r.name, (double)ms, 1};
    } else {
      it->second.ms += ms;
      it->second.launches += 1;
    }
  }
  g_summary.clear();
  for (auto &n : order) g_summary.push_back(agg[n]);
  return (int)g_summary.size();
}

dspark_status dspark_trace_entry(int i, const char **name, double *total_ms, int *launches) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (i < 0 || i >= (int)g_summary.size() || !name || !total_ms || !launches)
    return DSPARK_ERR_VALUE;
  *name = g_summary[i].name.c_str();
  *total_ms = g_summary[i].ms;
  *launches = g_summary[i].launches;
  return DSPARK_OK;
}

}  // extern "C"
