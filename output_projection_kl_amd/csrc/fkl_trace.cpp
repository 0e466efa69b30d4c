// Event-based per-kernel timing for libfkl (see fkl_trace_enable in fkl.h).
#include <algorithm>
#include <atomic>
#include <cstring>
#include <iterator>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "fkl.h"
#include "fkl_internal.h"

namespace {

struct Record {
  std::string name;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  double flops = 0.0;
  double bytes = 0.0;
  uint64_t id = 0;
  bool closed = false;  // stop event recorded
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Record> g_records;
uint64_t g_next_id = 1;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_pool;

std::pair<hipEvent_t, hipEvent_t> take_events() {
  if (!g_pool.empty()) {
    auto e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return {nullptr, nullptr};
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return {nullptr, nullptr};
  }
  return {a, b};
}

}  // namespace

namespace fkl {

TraceScope::TraceScope(hipStream_t stream, const char* name, double flops, double bytes)
    : stream_(stream), id_(0) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  auto ev = take_events();
  if (!ev.first) return;
  if (hipEventRecord(ev.first, stream) != hipSuccess) {
    g_pool.push_back(ev);
    return;
  }
  Record r;
  r.name = name;
  r.start = ev.first;
  r.stop = ev.second;
  r.flops = flops;
  r.bytes = bytes;
  r.id = g_next_id++;
  id_ = r.id;
  g_records.push_back(r);
}

// The scope closes its own record, found by id: a concurrent fkl_trace_read
// takes only closed records, so an open one stays in g_records until here.
TraceScope::~TraceScope() {
  if (id_ == 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto it = g_records.rbegin(); it != g_records.rend(); ++it) {
    if (it->id == id_) {
      if (hipEventRecord(it->stop, stream_) == hipSuccess) it->closed = true;
      else {
        g_pool.emplace_back(it->start, it->stop);
        g_records.erase(std::next(it).base());
      }
      return;
    }
  }
}

}  // namespace fkl

extern "C" {

fkl_status fkl_trace_enable(int on) {
  g_enabled.store(on != 0);
  return FKL_OK;
}

fkl_status fkl_trace_read(fkl_kernel_stat* stats, int capacity, int* count) {
  if (capacity < 0 || (capacity > 0 && !stats)) return FKL_EINVAL;
  // Closed records only; scopes still open on other threads keep theirs.
  std::vector<Record> recs;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    std::vector<Record> open;
    for (auto& r : g_records) (r.closed ? recs : open).push_back(std::move(r));
    g_records.swap(open);
  }
  std::map<std::string, fkl_kernel_stat> agg;
  std::vector<std::string> order;
  fkl_status st = FKL_OK;
  for (auto& r : recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = FKL_EDEVICE;
    } else {
      auto it = agg.find(r.name);
      if (it == agg.end()) {
        fkl_kernel_stat k;
        std::memset(&k, 0, sizeof(k));
        std::strncpy(k.name, r.name.c_str(), sizeof(k.name) - 1);
        k.min_ms = 1e300;
        it = agg.emplace(r.name, k).first;
        order.push_back(r.name);
      }
      fkl_kernel_stat& k = it->second;
      k.launches += 1;
      k.total_ms += ms;
      k.min_ms = std::min(k.min_ms, static_cast<double>(ms));
      k.max_ms = std::max(k.max_ms, static_cast<double>(ms));
      k.flops += r.flops;
      k.bytes += r.bytes;
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& r : recs) g_pool.emplace_back(r.start, r.stop);
  }
  const int n = static_cast<int>(order.size());
  for (int i = 0; i < n && i < capacity; ++i) stats[i] = agg[order[i]];
  if (count) *count = n;
  return st;
}

}  // extern "C"
