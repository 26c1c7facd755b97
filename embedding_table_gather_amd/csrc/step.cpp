// Graph-cached endpoint calls for small, repeated shapes: the serving pattern of
// the Perplexity blog "Fast embeddings on GPUs", section "Tulip" (one GPU graph
// per shape configuration, token counts padded to buckets of multiples of 64 or
// 256, captured lazily: an eager run on the first hit, capture and replay from
// the second), with the answer delivered into page-locked host memory behind an
// event (its lazy result tensors).  The public contract is in etg.h.
//
// Host I/O without copy operations: page-locked buffers that are mapped into the
// device's address space (hipHostGetDevicePointer succeeds) are read (token ids)
// and written (the top-k answer) by the kernels themselves, so a call is kernels
// only; buffers that are not mapped are copied with async memcpys instead.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <tuple>

#include "../../include/etg.h"
#include "etg_internal.hpp"

struct etg_step_cache {
  etg::TableDesc t;
  int64_t max_ids, ids_cap, max_batch;
  int32_t k;
  int32_t use_graphs;
  int32_t* d_ids;
  float* d_rows;
  const float* d_residual;
  int32_t* d_topk_ids;
  float* d_topk_scores;
  void* d_ws;
  size_t ws_bytes;
  int32_t* h_ids;  // [ETG_STEP_ID_SLOTS][ids_cap]
  int32_t* h_topk_ids;
  float* h_topk_scores;
  // device views of the page-locked buffers (null: not mapped, copies are used)
  bool mapped_looked_up = false;
  const int32_t* m_ids = nullptr;
  int32_t* m_topk_ids = nullptr;
  float* m_topk_scores = nullptr;
  struct Entry {
    int hits = 0;
    bool uncapturable = false;
    hipGraphExec_t exec = nullptr;
  };
  std::map<std::tuple<int, uint32_t, int64_t, int>, Entry> graphs;  // (operation, scale bits, shape, id slot)
  int64_t captured = 0, replays = 0;
  // id staging ring: slot s is rewritten only once the gather that last read it has run
  hipEvent_t slot_done[ETG_STEP_ID_SLOTS] = {};
  bool slot_pending[ETG_STEP_ID_SLOTS] = {};
  int64_t gathers = 0;
  std::mutex mu;  // calls on one cache are serialised
};

namespace {

constexpr int64_t kStepBucketSmall = 64, kStepBucketLarge = 256, kStepSmallLimit = 1024;

int64_t ids_bucket(int64_t n) {
  const int64_t b = n <= kStepSmallLimit ? kStepBucketSmall : kStepBucketLarge;
  return (n + b - 1) / b * b;
}

template <typename T>
T* device_view(T* host) {
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, (void*)host, 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return (T*)d;
}

void look_up_mappings(etg_step_cache* c) {
  if (c->mapped_looked_up) return;
  c->m_ids = device_view(c->h_ids);
  c->m_topk_ids = device_view(c->h_topk_ids);
  c->m_topk_scores = device_view(c->h_topk_scores);
  if (c->m_topk_ids == nullptr || c->m_topk_scores == nullptr) c->m_topk_ids = nullptr, c->m_topk_scores = nullptr;
  c->mapped_looked_up = true;
}

// One call: eager on the first hit of its configuration (and always when graphs
// are off or the stream cannot be captured), captured on the second, replayed
// after.  enqueue(s) puts the call's work on stream s and returns a HIP status.
template <typename F>
hipError_t run_cached(etg_step_cache* c, std::tuple<int, uint32_t, int64_t, int> key, hipStream_t stream, F enqueue) {
  if (!c->use_graphs || stream == nullptr) return enqueue(stream);
  etg_step_cache::Entry& e = c->graphs[key];
  e.hits++;
  if (e.uncapturable || (e.hits == 1 && e.exec == nullptr)) return enqueue(stream);
  if (e.exec == nullptr) {
    hipError_t st = hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal);
    if (st != hipSuccess) {
      e.uncapturable = true;
      (void)hipGetLastError();
      return enqueue(stream);
    }
    const hipError_t work = enqueue(stream);
    hipGraph_t graph = nullptr;
    st = hipStreamEndCapture(stream, &graph);
    if (work != hipSuccess || st != hipSuccess || graph == nullptr) {
      if (graph != nullptr) (void)hipGraphDestroy(graph);
      e.uncapturable = true;
      (void)hipGetLastError();
      return work != hipSuccess ? work : enqueue(stream);
    }
    st = hipGraphInstantiate(&e.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (st != hipSuccess) {
      e.exec = nullptr;
      e.uncapturable = true;
      (void)hipGetLastError();
      return enqueue(stream);
    }
    c->captured++;
  }
  c->replays++;
  return hipGraphLaunch(e.exec, stream);
}

}  // namespace

extern "C" {

int64_t etg_step_cache_ids_capacity(int64_t max_ids) {
  if (max_ids < 1 || max_ids > 2147483647LL) return -1;
  return ids_bucket(max_ids);
}

int64_t etg_step_cache_workspace(const etg_table* table, int64_t max_batch, int32_t k) {
  if (table == nullptr) return etg::set_error(ETG_EINVAL, "table handle is NULL");
  if (max_batch < 1 || max_batch > 65536)
    return etg::set_error(ETG_ESHAPE, "max_batch %lld outside [1, 65536]", (long long)max_batch);
  int64_t ws = 0;
  for (int64_t b = 1; b <= max_batch; b++) {
    const int64_t n = etg_logits_topk_workspace(table, b, k);
    if (n < 0) return n;
    ws = n > ws ? n : ws;
  }
  return ws;
}

int32_t etg_step_cache_create(const etg_table* table, int64_t max_ids, int64_t max_batch, int32_t k,
                              int32_t use_graphs, int32_t* d_ids, float* d_rows, const float* d_residual,
                              int32_t* d_topk_ids, float* d_topk_scores, void* d_workspace, size_t workspace_bytes,
                              int32_t* h_ids, int32_t* h_topk_ids, float* h_topk_scores, etg_step_cache** out) {
  if (out == nullptr) return etg::set_error(ETG_EINVAL, "out handle pointer is NULL");
  *out = nullptr;
  const int64_t cap = etg_step_cache_ids_capacity(max_ids);
  if (cap < 0) return etg::set_error(ETG_ESHAPE, "max_ids %lld outside [1, 2^31 - 1]", (long long)max_ids);
  const int64_t ws = etg_step_cache_workspace(table, max_batch, k);
  if (ws < 0) return (int32_t)ws;
  if (d_ids == nullptr || d_rows == nullptr || d_residual == nullptr || d_topk_ids == nullptr ||
      d_topk_scores == nullptr || d_workspace == nullptr || h_ids == nullptr || h_topk_ids == nullptr ||
      h_topk_scores == nullptr)
    return etg::set_error(ETG_EINVAL, "a buffer pointer is NULL");
  if ((uintptr_t)d_rows % 16 || (uintptr_t)d_workspace % 256 || (uintptr_t)d_ids % 4 || (uintptr_t)d_residual % 4 ||
      (uintptr_t)d_topk_ids % 4 || (uintptr_t)d_topk_scores % 4 || (uintptr_t)h_ids % 4 ||
      (uintptr_t)h_topk_ids % 4 || (uintptr_t)h_topk_scores % 4)
    return etg::set_error(ETG_EALIGN, "buffer alignment (rows 16, workspace 256, the others 4 bytes)");
  if (workspace_bytes < (size_t)ws)
    return etg::set_error(ETG_EWORKSPACE, "workspace has %zu bytes, needs %lld", workspace_bytes, (long long)ws);
  etg_step_cache* c = new (std::nothrow) etg_step_cache;
  if (c == nullptr) return etg::set_error(ETG_EINVAL, "out of host memory");
  c->t = table->d;
  c->max_ids = max_ids;
  c->ids_cap = cap;
  c->max_batch = max_batch;
  c->k = k;
  c->use_graphs = use_graphs != 0;
  c->d_ids = d_ids;
  c->d_rows = d_rows;
  c->d_residual = d_residual;
  c->d_topk_ids = d_topk_ids;
  c->d_topk_scores = d_topk_scores;
  c->d_ws = d_workspace;
  c->ws_bytes = workspace_bytes;
  c->h_ids = h_ids;
  c->h_topk_ids = h_topk_ids;
  c->h_topk_scores = h_topk_scores;
  *out = c;
  return ETG_OK;
}

int32_t etg_step_cache_destroy(etg_step_cache* c) {
  if (c == nullptr) return ETG_OK;
  for (auto& kv : c->graphs)
    if (kv.second.exec != nullptr) (void)hipGraphExecDestroy(kv.second.exec);
  for (hipEvent_t e : c->slot_done)
    if (e != nullptr) (void)hipEventDestroy(e);
  delete c;
  return ETG_OK;
}

int32_t etg_step_cache_stats(etg_step_cache* c, int64_t* graphs, int64_t* replays) {
  if (c == nullptr || graphs == nullptr || replays == nullptr) return etg::set_error(ETG_EINVAL, "a pointer is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  *graphs = c->captured;
  *replays = c->replays;
  return ETG_OK;
}

int32_t etg_step_gather(etg_step_cache* c, const int32_t* h_ids, int64_t n, float scale, void* stream) {
  if (c == nullptr || h_ids == nullptr) return etg::set_error(ETG_EINVAL, "cache or ids pointer is NULL");
  if (n < 1 || n > c->max_ids)
    return etg::set_error(ETG_ESHAPE, "n %lld outside [1, %lld]", (long long)n, (long long)c->max_ids);
  if (!(scale == scale) || scale - scale != 0.0f) return etg::set_error(ETG_ERANGE, "scale is not finite");
  // bad token ids are refused on the host, before anything is enqueued
  for (int64_t i = 0; i < n; i++)
    if ((uint32_t)h_ids[i] >= (uint64_t)c->t.V)
      return etg::set_error(ETG_ERANGE, "bad token id %d at position %lld (vocab %lld)", h_ids[i], (long long)i,
                            (long long)c->t.V);
  std::lock_guard<std::mutex> lock(c->mu);
  look_up_mappings(c);
  const int slot = (int)(c->gathers % ETG_STEP_ID_SLOTS);
  hipEvent_t& done = c->slot_done[slot];
  if (done == nullptr && hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess) {
    done = nullptr;
    return etg::set_error(ETG_EHIP, "event creation failed");
  }
  if (c->slot_pending[slot] && hipEventSynchronize(done) != hipSuccess)
    return etg::set_error(ETG_EHIP, "waiting for an earlier gather failed");
  c->slot_pending[slot] = false;
  const int64_t np = ids_bucket(n);
  int32_t* hs = c->h_ids + (size_t)slot * (size_t)c->ids_cap;
  // the bucket's padding ids are 0, a valid row whose output is not part of the answer
  std::memcpy(hs, h_ids, (size_t)n * sizeof(int32_t));
  std::memset(hs + n, 0, (size_t)(np - n) * sizeof(int32_t));
  uint32_t sbits;
  std::memcpy(&sbits, &scale, 4);
  const int32_t* ms = c->m_ids != nullptr ? c->m_ids + (size_t)slot * (size_t)c->ids_cap : nullptr;
  const auto key = std::make_tuple(0, sbits, np, slot);
  const hipError_t e = run_cached(c, key, (hipStream_t)stream, [&](hipStream_t s) {
    if (ms != nullptr) return etg::launch_gather(c->t, ms, np, scale, c->d_rows, nullptr, s);
    hipError_t st = hipMemcpyAsync(c->d_ids, hs, (size_t)np * sizeof(int32_t), hipMemcpyHostToDevice, s);
    if (st == hipSuccess) st = etg::launch_gather(c->t, c->d_ids, np, scale, c->d_rows, nullptr, s);
    return st;
  });
  if (e != hipSuccess) return etg::set_error(ETG_EHIP, "step gather failed: %s", hipGetErrorString(e));
  if (hipEventRecord(done, (hipStream_t)stream) != hipSuccess) return etg::set_error(ETG_EHIP, "event record failed");
  c->slot_pending[slot] = true;
  c->gathers++;
  return ETG_OK;
}

int32_t etg_step_logits(etg_step_cache* c, int64_t batch, void* event, void* stream) {
  if (c == nullptr) return etg::set_error(ETG_EINVAL, "cache is NULL");
  if (batch < 1 || batch > c->max_batch)
    return etg::set_error(ETG_ESHAPE, "batch %lld outside [1, %lld]", (long long)batch, (long long)c->max_batch);
  std::lock_guard<std::mutex> lock(c->mu);
  look_up_mappings(c);
  etg::LogitsPlan p;
  const char* why = "";
  const int32_t st0 = etg::plan_logits(c->t, batch, c->k, 0, &p, &why);
  if (st0 != 0) return etg::set_error(st0, "%s", why);
  const auto key = std::make_tuple(1, 0u, batch, 0);
  const size_t n = (size_t)batch * (size_t)c->k;
  const hipError_t e = run_cached(c, key, (hipStream_t)stream, [&](hipStream_t s) {
    if (c->m_topk_ids != nullptr)  // the kernels write the answer into host memory
      return etg::launch_logits_topk(c->t, p, c->d_residual, c->m_topk_ids, c->m_topk_scores, c->d_ws, s);
    hipError_t st = etg::launch_logits_topk(c->t, p, c->d_residual, c->d_topk_ids, c->d_topk_scores, c->d_ws, s);
    if (st == hipSuccess) st = hipMemcpyAsync(c->h_topk_ids, c->d_topk_ids, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (st == hipSuccess)
      st = hipMemcpyAsync(c->h_topk_scores, c->d_topk_scores, n * sizeof(float), hipMemcpyDeviceToHost, s);
    return st;
  });
  if (e != hipSuccess) return etg::set_error(ETG_EHIP, "step logits failed: %s", hipGetErrorString(e));
  if (event != nullptr && hipEventRecord((hipEvent_t)event, (hipStream_t)stream) != hipSuccess)
    return etg::set_error(ETG_EHIP, "event record failed");
  return ETG_OK;
}

}  // extern "C"
