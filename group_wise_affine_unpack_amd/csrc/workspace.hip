// Per-(device, stream) scratch for the launchers that need device memory
// beyond their arguments: the GEMM pre-pass buffers, the GPTQ split-K
// partials and permuted activations.  Work on one stream runs in order, so a
// stream reuses its buffer call after call and no call allocates once the
// buffer is large enough; different streams get different buffers.  A
// buffer only grows (to the next power of two, at least 1 MiB); a grown-out
// buffer is kept, not freed, because a captured graph may still address it.
// Growing is refused while the stream is being captured, so a graph is
// captured after one eager call of the same shapes.  A captured graph keeps
// the address of the buffer of the stream it was captured on: its replays
// use that buffer whatever stream they run on.  release_workspaces() frees
// every cached and grown-out buffer at once.
// Also here: how many workgroups of a kernel the device holds at once, by
// which the launchers size their K splits.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "common.h"

namespace qaff {

namespace {

struct Workspace {
  void* p = nullptr;
  size_t cap = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// grown-out buffers, still valid for graphs that captured them: (device, pointer)
std::vector<std::pair<int, void*>> g_retired;

// (device, kernel, block, LDS) -> (CUs, resident workgroups per CU), under g_mu
std::map<std::tuple<int, const void*, int, size_t>, std::pair<int, int>> g_resident;

}  // namespace

namespace {
// A caller-provided scratch region that replaces the per-stream buffer for
// the calls made on this thread between scratch_override_begin and _end
// (the no-allocation entry point).  `need` records the largest request.
struct Override {
  bool on = false;
  void* p = nullptr;
  size_t cap = 0, need = 0;
};
thread_local Override g_over;
}  // namespace

void scratch_override_begin(void* p, size_t cap) { g_over = Override{true, p, cap, 0}; }

size_t scratch_override_end() {
  const size_t need = g_over.need;
  g_over = Override{};
  return need;
}

hipError_t stream_workspace(hipStream_t s, size_t bytes, void** out) {
  *out = nullptr;
  if (bytes == 0) return hipSuccess;
  if (g_over.on) {
    // never allocates: the region serves every request that fits
    g_over.need = std::max(g_over.need, bytes);
    if (bytes > g_over.cap) return hipErrorOutOfMemory;
    *out = g_over.p;
    return hipSuccess;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  Workspace& w = g_ws[{dev, s}];
  if (w.cap < bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    size_t cap = size_t(1) << 20;
    while (cap < bytes) cap <<= 1;
    void* p = nullptr;
    e = hipMalloc(&p, cap);
    if (e != hipSuccess) return e;
    if (w.p) g_retired.push_back({dev, w.p});
    w.p = p;
    w.cap = cap;
  }
  *out = w.p;
  return hipSuccess;
}

hipError_t release_workspaces(size_t* freed) {
  if (freed) *freed = 0;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ws.empty() && g_retired.empty()) return hipSuccess;  // nothing held: no HIP call
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  std::vector<std::pair<int, void*>> all;
  size_t bytes = 0;
  for (auto& kv : g_ws) {
    if (kv.second.p) all.push_back({kv.first.first, kv.second.p});
    bytes += kv.second.cap;
  }
  all.insert(all.end(), g_retired.begin(), g_retired.end());
  hipError_t first = hipSuccess;
  for (auto& dp : all) {
    // free on the buffer's own device
    hipError_t r = hipSetDevice(dp.first);
    if (r == hipSuccess) r = hipFree(dp.second);
    if (r != hipSuccess && first == hipSuccess) first = r;
  }
  g_ws.clear();
  g_retired.clear();
  const hipError_t r = hipSetDevice(cur);
  if (first == hipSuccess) first = r;
  if (freed) *freed = bytes;
  return first;
}

hipError_t resident_workgroups(const void* kernel, int block, size_t lds, int max_per_cu, int64_t* out) {
  *out = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_tuple(dev, kernel, block, lds);
  std::pair<int, int> r{0, 0};  // (CUs, resident per CU)
  bool known = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    const auto it = g_resident.find(key);
    if (it != g_resident.end()) {
      r = it->second;
      known = true;
    }
  }
  if (!known) {
    e = hipDeviceGetAttribute(&r.first, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&r.second, kernel, block, lds);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mu);
    g_resident[key] = r;
  }
  *out = (int64_t)r.first * std::min(r.second, max_per_cu);
  return hipSuccess;
}

}  // namespace qaff
