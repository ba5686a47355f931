#include "profile.h"

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "ta_error.h"

namespace {

struct Pending {
  const char* name;
  hipEvent_t a, b;
};

struct Table {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  std::map<std::string, std::pair<double, int64_t>> totals;
  std::vector<std::string> order;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  // Folds finished records into the totals (blocks until they complete).
  void drain() {
    for (auto& p : pending) {
      float ms = 0.0f;
      if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
        auto it = totals.find(p.name);
        if (it == totals.end()) {
          order.push_back(p.name);
          totals[p.name] = {ms, 1};
        } else {
          it->second.first += ms;
          it->second.second += 1;
        }
      }
      pool.push_back(p.a);
      pool.push_back(p.b);
    }
    pending.clear();
  }
};

Table& table() {
  static Table t;
  return t;
}

}  // namespace

namespace ta {

ProfScope::ProfScope(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  Table& t = table();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on) return;
  start_ = t.get();
  if (start_ != nullptr && hipEventRecord(start_, stream_) != hipSuccess) {
    t.pool.push_back(start_);
    start_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (start_ == nullptr) return;
  Table& t = table();
  std::lock_guard<std::mutex> g(t.mu);
  hipEvent_t stop = t.get();
  if (stop == nullptr || hipEventRecord(stop, stream_) != hipSuccess) {
    t.pool.push_back(start_);
    if (stop) t.pool.push_back(stop);
    return;
  }
  t.pending.push_back({name_, start_, stop});
}

}  // namespace ta

extern "C" int tree_attn_profile_enable(int32_t on) {
  ta::clear_error();
  Table& t = table();
  std::lock_guard<std::mutex> g(t.mu);
  t.drain();
  t.totals.clear();
  t.order.clear();
  t.on = on != 0;
  return TA_OK;
}

extern "C" int tree_attn_profile_read(int32_t idx, char* name, int32_t name_cap, double* total_ms, int64_t* count) {
  ta::clear_error();
  Table& t = table();
  std::lock_guard<std::mutex> g(t.mu);
  t.drain();
  if (idx < 0 || idx >= (int32_t)t.order.size())
    return ta::fail(TA_EINVAL, "tree_attn_profile_read: index %d out of range (%zu entries)", idx, t.order.size());
  const std::string& n = t.order[idx];
  if (name != nullptr && name_cap > 0) {
    std::strncpy(name, n.c_str(), (size_t)name_cap - 1);
    name[name_cap - 1] = '\0';
  }
  if (total_ms != nullptr) *total_ms = t.totals[n].first;
  if (count != nullptr) *count = t.totals[n].second;
  return TA_OK;
}
