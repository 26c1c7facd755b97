// C-ABI of libetg: argument checks, error messages, kernel dispatch.
// The public contract (argument meaning, layout, ownership, errors) is in etg.h.
#include "../../include/etg.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <new>

#include "etg_internal.hpp"


namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxHidden = 65536;
constexpr int64_t kMaxVocab = 2147483647;  // ids are 32-bit keys
constexpr int64_t kMaxBatch = 65536;
constexpr int32_t kMaxK = 64;

const char* dtype_name(int32_t dt) {
  switch (dt) {
    case ETG_F32: return "f32";
    case ETG_BF16: return "bf16";
    case ETG_Q8_0: return "q8_0";
    case ETG_F16: return "f16";
    default: return "?";
  }
}

int32_t check_logits_args(const etg_table* t, int64_t batch, int32_t k) {
  if (t == nullptr) return fail(ETG_EINVAL, "lm_head table handle is NULL");
  if (batch < 1 || batch > kMaxBatch)
    return fail(ETG_ESHAPE, "batch %lld outside [1, %lld]", (long long)batch, (long long)kMaxBatch);
  const int64_t kmax = t->d.V < kMaxK ? t->d.V : kMaxK;
  if (k < 1 || k > kmax) return fail(ETG_ERANGE, "k %d outside [1, %lld]", k, (long long)kmax);
  return ETG_OK;
}

}  // namespace

int32_t etg::set_error(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

extern "C" {

int32_t etg_version(void) { return 100; }

const char* etg_last_error(void) { return g_err; }

int64_t etg_row_bytes(int32_t dtype, int64_t hidden) {
  if (hidden < 1 || hidden > kMaxHidden) return -1;
  switch (dtype) {
    case ETG_F32: return hidden % 4 ? -1 : 4 * hidden;
    case ETG_BF16: return hidden % 8 ? -1 : 2 * hidden;
    case ETG_F16: return hidden % 8 ? -1 : 2 * hidden;
    case ETG_Q8_0: return hidden % 32 ? -1 : 34 * (hidden / 32);
    default: return -1;
  }
}

float etg_sqrt_d(int64_t hidden) {
  if (hidden < 1) return 0.0f;
  // sqrt in double is correctly rounded and 53 >= 2 * 24 + 2, so rounding it to
  // float gives the float nearest the exact root.
  return (float)std::sqrt((double)hidden);
}

int32_t etg_table_create(const void* d_rows, int32_t dtype, int64_t vocab, int64_t hidden, etg_table** out) {
  if (out == nullptr) return fail(ETG_EINVAL, "out handle pointer is NULL");
  *out = nullptr;
  if (d_rows == nullptr) return fail(ETG_EINVAL, "table rows pointer is NULL");
  if (dtype != ETG_F32 && dtype != ETG_BF16 && dtype != ETG_Q8_0 && dtype != ETG_F16)
    return fail(ETG_EDTYPE, "unknown dtype %d", dtype);
  if (vocab < 1 || vocab > kMaxVocab)
    return fail(ETG_ESHAPE, "vocab %lld outside [1, %lld]", (long long)vocab, (long long)kMaxVocab);
  const int64_t rb = etg_row_bytes(dtype, hidden);
  if (rb < 0)
    return fail(ETG_ESHAPE, "hidden %lld not storable as %s (multiple of %d, at most %lld)", (long long)hidden,
                dtype_name(dtype), dtype == ETG_F32 ? 4 : dtype == ETG_Q8_0 ? 32 : 8, (long long)kMaxHidden);
  if (!aligned(d_rows, 16)) return fail(ETG_EALIGN, "table rows pointer is not 16-byte aligned");
  etg_table* t = new (std::nothrow) etg_table;
  if (t == nullptr) return fail(ETG_EINVAL, "out of host memory");
  t->d.rows = (const uint8_t*)d_rows;
  t->d.dtype = dtype;
  t->d.V = vocab;
  t->d.hidden = hidden;
  t->d.row_bytes = rb;
  *out = t;
  return ETG_OK;
}

int32_t etg_table_destroy(etg_table* table) {
  delete table;
  return ETG_OK;
}

int32_t etg_embed_gather(const etg_table* t, const int32_t* d_ids, int64_t seq_len, float scale, float* d_out,
                         int32_t* d_bad_count, void* stream) {
  if (t == nullptr) return fail(ETG_EINVAL, "table handle is NULL");
  if (seq_len < 0 || seq_len > 2147483647LL)
    return fail(ETG_ESHAPE, "seq_len %lld outside [0, 2^31 - 1]", (long long)seq_len);
  if (seq_len == 0) return ETG_OK;
  if (d_ids == nullptr) return fail(ETG_EINVAL, "ids pointer is NULL");
  if (d_out == nullptr) return fail(ETG_EINVAL, "output pointer is NULL");
  if (!aligned(d_ids, 4)) return fail(ETG_EALIGN, "ids pointer is not 4-byte aligned");
  if (!aligned(d_out, 16)) return fail(ETG_EALIGN, "output pointer is not 16-byte aligned");
  if (d_bad_count != nullptr && !aligned(d_bad_count, 4))
    return fail(ETG_EALIGN, "bad-count pointer is not 4-byte aligned");
  if (!std::isfinite(scale)) return fail(ETG_ERANGE, "scale is not finite");
  hipError_t e = etg::launch_gather(t->d, d_ids, seq_len, scale, d_out, d_bad_count, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ETG_EHIP, "gather launch failed: %s", hipGetErrorString(e));
  return ETG_OK;
}

int64_t etg_wire_row_bytes(int32_t wire, int64_t hidden) {
  if (hidden < 1 || hidden > kMaxHidden) return -1;
  switch (wire) {
    case ETG_WIRE_F32: return 4 * hidden;
    case ETG_WIRE_F16: return 2 * hidden;
    case ETG_WIRE_I8: return hidden + 8;
    default: return -1;
  }
}

int32_t etg_embed_gather_wire(const etg_table* t, const int32_t* d_ids, int64_t seq_len, float scale, int32_t wire,
                              void* d_out, int32_t* d_bad_count, void* stream) {
  if (wire == ETG_WIRE_F32) return etg_embed_gather(t, d_ids, seq_len, scale, (float*)d_out, d_bad_count, stream);
  if (wire != ETG_WIRE_F16 && wire != ETG_WIRE_I8) return fail(ETG_ERANGE, "unknown wire format %d", wire);
  if (t == nullptr) return fail(ETG_EINVAL, "table handle is NULL");
  if (seq_len < 0 || seq_len > 2147483647LL)
    return fail(ETG_ESHAPE, "seq_len %lld outside [0, 2^31 - 1]", (long long)seq_len);
  if (seq_len == 0) return ETG_OK;
  if (d_ids == nullptr) return fail(ETG_EINVAL, "ids pointer is NULL");
  if (d_out == nullptr) return fail(ETG_EINVAL, "output pointer is NULL");
  if (!aligned(d_ids, 4)) return fail(ETG_EALIGN, "ids pointer is not 4-byte aligned");
  if (!aligned(d_out, 4)) return fail(ETG_EALIGN, "output pointer is not 4-byte aligned");
  if (d_bad_count != nullptr && !aligned(d_bad_count, 4))
    return fail(ETG_EALIGN, "bad-count pointer is not 4-byte aligned");
  if (!std::isfinite(scale)) return fail(ETG_ERANGE, "scale is not finite");
  hipError_t e = etg::launch_gather_wire(t->d, d_ids, seq_len, scale, wire, (uint8_t*)d_out, d_bad_count,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return fail(ETG_EHIP, "gather launch failed: %s", hipGetErrorString(e));
  return ETG_OK;
}

int64_t etg_logits_topk_workspace_ex(const etg_table* t, int64_t batch, int32_t k, int32_t path) {
  int32_t st = check_logits_args(t, batch, k);
  if (st != ETG_OK) return st;
  etg::LogitsPlan p;
  const char* why = "";
  st = etg::plan_logits(t->d, batch, k, path, &p, &why);
  if (st != ETG_OK) return fail(st, "%s", why);
  return (int64_t)p.ws_bytes;
}

int64_t etg_logits_topk_workspace(const etg_table* t, int64_t batch, int32_t k) {
  return etg_logits_topk_workspace_ex(t, batch, k, ETG_PATH_AUTO);
}

}  // extern "C"

namespace {

// Shared body of the logits entry points: argument checks, plan, launch.
// ids == nullptr selects the raw logits mode (k = 1 internally, no merge).
int32_t run_logits(const etg_table* t, const void* d_residual, int64_t batch, int32_t k, int32_t* d_topk_ids,
                   float* d_topk_scores, float* d_topk_probs, float temperature, float* d_logits,
                   void* d_workspace, size_t workspace_bytes, int32_t path, void* event_before, void* event_after,
                   void* stream, int32_t wire = ETG_WIRE_F32) {
  int32_t st = check_logits_args(t, batch, k);
  if (st != ETG_OK) return st;
  if (wire != ETG_WIRE_F32 && wire != ETG_WIRE_F16 && wire != ETG_WIRE_I8)
    return fail(ETG_ERANGE, "unknown wire format %d", wire);
  if (wire == ETG_WIRE_F16 && !aligned(d_residual, 2))
    return fail(ETG_EALIGN, "f16 residual pointer is not 2-byte aligned");
  const bool raw = d_topk_ids == nullptr;
  if (d_residual == nullptr || d_workspace == nullptr || (raw ? d_logits == nullptr : d_topk_scores == nullptr))
    return fail(ETG_EINVAL, "a residual, output or workspace pointer is NULL");
  if ((wire != ETG_WIRE_F16 && !aligned(d_residual, 4)) ||
      (!raw && (!aligned(d_topk_ids, 4) || !aligned(d_topk_scores, 4))) ||
      !aligned(d_topk_probs, 4) || !aligned(d_logits, 4))
    return fail(ETG_EALIGN, "residual and output pointers must be 4-byte aligned");
  if (!aligned(d_workspace, 256)) return fail(ETG_EALIGN, "workspace pointer is not 256-byte aligned");
  float lse_scale = 0.f;
  if (d_topk_probs != nullptr) {
    // c = log2(e) / T must be a finite positive float
    lse_scale = (float)(1.4426950408889634 / (double)temperature);
    if (!(temperature > 0.f) || !std::isfinite(temperature) || !std::isfinite(lse_scale) || !(lse_scale > 0.f))
      return fail(ETG_ERANGE, "temperature %g is not a finite value in [1e-37, 3.4e38]", (double)temperature);
  }
  etg::LogitsPlan p;
  const char* why = "";
  st = etg::plan_logits(t->d, batch, k, path, &p, &why, raw || d_topk_probs != nullptr);
  if (st != ETG_OK) return fail(st, "%s", why);
  if (workspace_bytes < p.ws_bytes)
    return fail(ETG_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, p.ws_bytes);
  hipError_t e = etg::launch_logits_topk(t->d, p, d_residual, d_topk_ids, d_topk_scores, d_workspace,
                                         (hipStream_t)stream, (hipEvent_t)event_before, (hipEvent_t)event_after,
                                         d_logits, d_topk_probs, lse_scale, wire);
  if (e != hipSuccess) return fail(ETG_EHIP, "logits launch failed: %s", hipGetErrorString(e));
  return ETG_OK;
}

}  // namespace

extern "C" {

int32_t etg_logits_topk_profiled(const etg_table* t, const float* d_residual, int64_t batch, int32_t k,
                                 int32_t* d_topk_ids, float* d_topk_scores, void* d_workspace,
                                 size_t workspace_bytes, int32_t path, void* event_before, void* event_after,
                                 void* stream) {
  if (d_topk_ids == nullptr) return fail(ETG_EINVAL, "ids pointer is NULL");
  return run_logits(t, d_residual, batch, k, d_topk_ids, d_topk_scores, nullptr, 0.f, nullptr, d_workspace,
                    workspace_bytes, path, event_before, event_after, stream);
}

int32_t etg_logits_topk_probs(const etg_table* t, const float* d_residual, int64_t batch, int32_t k,
                              float temperature, int32_t* d_topk_ids, float* d_topk_scores, float* d_topk_probs,
                              void* d_workspace, size_t workspace_bytes, int32_t path, void* stream) {
  if (d_topk_ids == nullptr || d_topk_probs == nullptr) return fail(ETG_EINVAL, "ids or probs pointer is NULL");
  return run_logits(t, d_residual, batch, k, d_topk_ids, d_topk_scores, d_topk_probs, temperature, nullptr,
                    d_workspace, workspace_bytes, path, nullptr, nullptr, stream);
}

int32_t etg_logits_topk_wire(const etg_table* t, const void* d_residual, int32_t wire, int64_t batch, int32_t k,
                             int32_t* d_topk_ids, float* d_topk_scores, void* d_workspace, size_t workspace_bytes,
                             int32_t path, void* stream) {
  if (d_topk_ids == nullptr) return fail(ETG_EINVAL, "ids pointer is NULL");
  return run_logits(t, d_residual, batch, k, d_topk_ids, d_topk_scores, nullptr, 0.f, nullptr, d_workspace,
                    workspace_bytes, path, nullptr, nullptr, stream, wire);
}

int64_t etg_logits_raw_workspace(const etg_table* t, int64_t batch, int32_t path) {
  return etg_logits_topk_workspace_ex(t, batch, 1, path);
}

int32_t etg_logits_raw(const etg_table* t, const float* d_residual, int64_t batch, float* d_logits,
                       void* d_workspace, size_t workspace_bytes, int32_t path, void* stream) {
  if (d_logits == nullptr) return fail(ETG_EINVAL, "logits pointer is NULL");
  return run_logits(t, d_residual, batch, 1, nullptr, nullptr, nullptr, 0.f, d_logits, d_workspace,
                    workspace_bytes, path, nullptr, nullptr, stream);
}

int32_t etg_logits_topk_ex(const etg_table* t, const float* d_residual, int64_t batch, int32_t k,
                           int32_t* d_topk_ids, float* d_topk_scores, void* d_workspace, size_t workspace_bytes,
                           int32_t path, void* stream) {
  return etg_logits_topk_profiled(t, d_residual, batch, k, d_topk_ids, d_topk_scores, d_workspace,
                                  workspace_bytes, path, nullptr, nullptr, stream);
}

int32_t etg_logits_topk_to_host(const etg_table* t, const float* d_residual, int64_t batch, int32_t k,
                                int32_t* d_topk_ids, float* d_topk_scores, void* d_workspace, size_t workspace_bytes,
                                int32_t path, int32_t* h_topk_ids, float* h_topk_scores, void* event,
                                void* stream) {
  if (h_topk_ids == nullptr || h_topk_scores == nullptr) return fail(ETG_EINVAL, "host result pointer is NULL");
  if (d_topk_scores == nullptr) return fail(ETG_EINVAL, "scores pointer is NULL");
  if (event == nullptr) return fail(ETG_EINVAL, "event is NULL");
  const int32_t st = etg_logits_topk_ex(t, d_residual, batch, k, d_topk_ids, d_topk_scores, d_workspace,
                                        workspace_bytes, path, stream);
  if (st != ETG_OK) return st;
  const size_t n = (size_t)batch * (size_t)k;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(h_topk_ids, d_topk_ids, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(h_topk_scores, d_topk_scores, n * sizeof(float), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipEventRecord((hipEvent_t)event, s);
  if (e != hipSuccess) return fail(ETG_EHIP, "result copy to host failed: %s", hipGetErrorString(e));
  return ETG_OK;
}

int32_t etg_hbm_read_probe(const void* d_src, int64_t bytes, uint32_t* d_sink, void* stream) {
  if (d_src == nullptr || d_sink == nullptr) return fail(ETG_EINVAL, "source or sink pointer is NULL");
  if (!aligned(d_src, 16)) return fail(ETG_EALIGN, "source pointer is not 16-byte aligned");
  if (!aligned(d_sink, 4)) return fail(ETG_EALIGN, "sink pointer is not 4-byte aligned");
  if (bytes <= 0 || bytes % 16 != 0) return fail(ETG_ESHAPE, "bytes %lld is not a positive multiple of 16",
                                                 (long long)bytes);
  hipError_t e = etg::launch_read_probe(d_src, bytes, d_sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ETG_EHIP, "read probe launch failed: %s", hipGetErrorString(e));
  return ETG_OK;
}

int32_t etg_hbm_write_probe(void* d_dst, int64_t bytes, uint32_t value, void* stream) {
  if (d_dst == nullptr) return fail(ETG_EINVAL, "destination pointer is NULL");
  if (!aligned(d_dst, 16)) return fail(ETG_EALIGN, "destination pointer is not 16-byte aligned");
  if (bytes <= 0 || bytes % 16 != 0) return fail(ETG_ESHAPE, "bytes %lld is not a positive multiple of 16",
                                                 (long long)bytes);
  hipError_t e = etg::launch_write_probe(d_dst, bytes, value, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ETG_EHIP, "write probe launch failed: %s", hipGetErrorString(e));
  return ETG_OK;
}

int32_t etg_logits_topk(const etg_table* t, const float* d_residual, int64_t batch, int32_t k, int32_t* d_topk_ids,
                        float* d_topk_scores, void* d_workspace, size_t workspace_bytes, void* stream) {
  return etg_logits_topk_ex(t, d_residual, batch, k, d_topk_ids, d_topk_scores, d_workspace, workspace_bytes,
                            ETG_PATH_AUTO, stream);
}

}  // extern "C"
