// Per-launch kernel timing (see timing.h): an event pool, the list of recorded
// launches and the C-ABI calls that switch it on and read it.
#include "timing.h"

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "qkv.h"

namespace qkv {

namespace {

struct Record {
  const char* name;
  hipEvent_t start, end;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;     // events reused across enable/read cycles
size_t g_used = 0;                  // events of the pool handed out since the last enable
std::vector<Record> g_records;

hipEvent_t take_event() {           // g_mu held
  if (g_used == g_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_used++];
}

}  // namespace

bool timing_enabled() { return g_on.load(std::memory_order_relaxed); }

TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : s_(s) {
  if (!timing_enabled()) return;
  std::lock_guard<std::mutex> lock(g_mu);
  Record r{name, take_event(), take_event()};
  if (!r.start || !r.end || hipEventRecord(r.start, s) != hipSuccess) return;
  slot_ = (int)g_records.size();
  g_records.push_back(r);
}

TimedLaunch::~TimedLaunch() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (hipEventRecord(g_records[slot_].end, s_) != hipSuccess) g_records[slot_].end = nullptr;
}

}  // namespace qkv

extern "C" {

int qkv_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lock(qkv::g_mu);
  qkv::g_records.clear();
  qkv::g_used = 0;
  qkv::g_on.store(on != 0);
  return QKV_OK;
}

int qkv_timing_read(int32_t max_kernels, qkv_kernel_time* out, int32_t* n_out) {
  if (!n_out || (max_kernels > 0 && !out)) return QKV_EINVAL;
  std::lock_guard<std::mutex> lock(qkv::g_mu);
  std::map<std::string, std::pair<int64_t, double>> acc;
  for (const qkv::Record& r : qkv::g_records) {
    if (!r.end) continue;
    if (hipEventSynchronize(r.end) != hipSuccess) return QKV_EDEVICE;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.start, r.end) != hipSuccess) return QKV_EDEVICE;
    auto& a = acc[r.name];
    a.first += 1;
    a.second += ms;
  }
  int32_t n = 0;
  for (const auto& kv : acc) {
    if (n < max_kernels) {
      std::memset(out[n].name, 0, sizeof out[n].name);
      std::strncpy(out[n].name, kv.first.c_str(), sizeof out[n].name - 1);
      out[n].launches = kv.second.first;
      out[n].total_ms = kv.second.second;
    }
    ++n;
  }
  *n_out = n;
  return QKV_OK;
}

}  // extern "C"
