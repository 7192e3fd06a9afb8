// Kernel timing instrumentation of the library (off by default).
//
// When enabled, every kernel the library enqueues is bracketed by a pair of HIP
// events recorded on the same stream; ssd_timing_read() waits for the recorded
// events and returns the summed device time and launch count per kernel kind.
// Events are pooled and reused; nothing is allocated on the device.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/ssd.h"
#include "launch.hpp"

namespace ssd {

namespace {

struct Pending {
  int kind;
  hipEvent_t a, b;
};

struct TimingState {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  double total_ms[kKernelKinds] = {};
  int64_t count[kKernelKinds] = {};
};

TimingState& st() {
  static TimingState s;
  return s;
}

hipEvent_t take_event(TimingState& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

const char* const kNames[kKernelKinds] = {
    "prepass", "walk_state", "scan", "walk_out", "conv_state_out", "conv_fwd",
    "chunk_states", "dstate", "scan_rev", "bwd_main", "conv_bwd", "dbc_reduce", "params",
    "scan_groups", "bwd_prepass", "linear", "decode", "rmsnorm"};

}  // namespace

TimingScope::TimingScope(int kind, hipStream_t s) : kind_(kind), s_(s) {
  TimingState& t = st();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.enabled) return;
  a_ = take_event(t);
  b_ = take_event(t);
  if (a_) hipEventRecord(static_cast<hipEvent_t>(a_), s_);
}

TimingScope::~TimingScope() {
  if (!a_ || !b_) return;
  TimingState& t = st();
  std::lock_guard<std::mutex> g(t.mu);
  hipEventRecord(static_cast<hipEvent_t>(b_), s_);
  t.pending.push_back(Pending{kind_, static_cast<hipEvent_t>(a_), static_cast<hipEvent_t>(b_)});
}

int64_t resident_blocks(const void* kernel, int threads) {
  struct Entry {
    const void* kernel;
    int threads, device;
    int64_t blocks;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry& e : cache)
      if (e.kernel == kernel && e.threads == threads && e.device == dev) return e.blocks;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  const int64_t blocks = static_cast<int64_t>(cus) * per_cu;
  std::lock_guard<std::mutex> lk(mu);
  cache.push_back(Entry{kernel, threads, dev, blocks});
  return blocks;
}

}  // namespace ssd

extern "C" {

ssd_status ssd_timing_enable(int on) {
  ssd::TimingState& t = ssd::st();
  std::lock_guard<std::mutex> g(t.mu);
  t.enabled = on != 0;
  for (int k = 0; k < ssd::kKernelKinds; ++k) {
    t.total_ms[k] = 0.0;
    t.count[k] = 0;
  }
  return SSD_OK;
}

ssd_status ssd_timing_read(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= ssd::kKernelKinds) return SSD_ERR_SHAPE;
  if (!total_ms || !launches) return SSD_ERR_NULL;
  ssd::TimingState& t = ssd::st();
  std::lock_guard<std::mutex> g(t.mu);
  for (const ssd::Pending& p : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess) return SSD_ERR_HIP;
    if (hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) return SSD_ERR_HIP;
    t.total_ms[p.kind] += ms;
    t.count[p.kind] += 1;
    t.pool.push_back(p.a);
    t.pool.push_back(p.b);
  }
  t.pending.clear();
  *total_ms = t.total_ms[kind];
  *launches = t.count[kind];
  return SSD_OK;
}

const char* ssd_timing_name(int kind) {
  if (kind < 0 || kind >= ssd::kKernelKinds) return "";
  return ssd::kNames[kind];
}

int ssd_timing_kinds(void) { return ssd::kKernelKinds; }

}  // extern "C"
