// Host-side declarations shared by the C-ABI layer and the kernel launchers of libetg.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace etg {

struct TableDesc {
  const uint8_t* rows;  // device pointer, 16-byte aligned
  int32_t dtype;        // 0 f32, 1 bf16, 2 Q8_0, 3 f16
  int64_t V;            // rows
  int64_t hidden;       // values per row
  int64_t row_bytes;
};

// Launch geometry and workspace layout of one etg_logits_topk call.  A pure
// function of (table shape, batch, k, path): the workspace size can be queried
// without a device.
struct LogitsPlan {
  int32_t path;          // 1 valu, 2 stream, 3 gemm, 4 wide, 5 q8, 6 row, 7 rank
  int32_t k;
  int64_t batch;
  // stream path
  int32_t nimg;          // residual operand images: 1 (hi+lo packed, 4 rows per pass), 2 (8 rows)
  int32_t nbc;           // residual rows per pass
  int32_t steps;         // 64-value K steps = ceil(hidden / 64) (wide: padded to the chunk)
  int32_t chunk;         // K steps of the residual image staged in LDS at a time
  int64_t ngroups;       // 8-row table groups = ceil(V / 8)
  int32_t max_groups;    // most 8-row groups one wave handles
  // gemm path
  int32_t tn;            // split residual columns per column tile (256)
  int32_t gemm_wn;       // waves along the columns (4: 2 x 4 waves)
  int32_t gemm_ring;     // LDS ring depths, table x 10 + residual (33 or 34)
  int32_t kpad;          // hidden rounded up to the K stage
  int32_t nct;           // column tiles of tn / 2 residual rows
  int32_t nvr;           // vocabulary ranges
  int32_t tiles_per_range;
  // rank path (the gemm kernel in ranking mode, then exact rescoring)
  int32_t kb;            // keys per vocabulary-range heap (or per wide-kernel block)
  int32_t rank_wide;     // 1: the wide kernel ranks (one pass of up to 256 rows), 0: the gemm kernel
  int32_t ngrp;          // column tiles that measure table row norms (a share of K each)
  size_t rescore_lds;    // dynamic LDS of the rescoring kernel
  // wide path
  int32_t ntile;         // 16-column N-tiles per pass (residual rows per pass / 16)
  // row path
  int32_t row_ni;        // KiB loads per table row
  // q8 path
  int32_t lpr_log2;      // log2 of the lanes that split one row's blocks
  int32_t q8_t;          // blocks per lane per row
  int32_t q8_chunks;     // 16-byte chunks per lane per step when rows are staged through LDS (0: not)
  int32_t q8_mfma;       // 1: the matrix-core kernel (stream.hip; nbc, steps, chunk, ngroups, max_groups)
  // valu and q8 paths
  int32_t rb;            // residual rows per pass (valu: 1, 2, 4 or 8; q8: 1 or 2)
  int64_t rows_per_blk;  // most table rows one block handles
  // common
  int32_t npass;         // batch passes (grid.y)
  int32_t nblk;          // blocks per pass
  int32_t ncand;         // candidate keys per residual row
  size_t lds_bytes;      // dynamic LDS of the main kernel
  size_t img_offset, img_bytes;    // bf16 residual operand (gemm and wide paths)
  size_t cand_offset, cand_bytes;  // u64 keys [batch][nblk][k]
  size_t aux_offset, aux_bytes;    // wide path: u64 top-k lower bound per residual row;
                                   // gemm path: per-thread running log-partition partials;
                                   // rank path: f32 squared row norm parts [ngrp][V] and block maxima
  int32_t nparts;                  // log-partition partials per residual row (= ncand / k)
  size_t lse_offset, lse_bytes;    // float2 partials [batch][nparts]
  size_t ws_bytes;
};

// Optional outputs of a logits call besides the top-k.
//  logits     [batch][V] f32 raw logits, the same values the top-k ranks (nullable)
//  lse        [batch][nparts] log-partition partials (m, s) of each block's
//             vocabulary slice: m = max logit, s = sum exp2((logit - m) lse_scale)
//             (nullable; (-inf, 0) for a slice with no rows)
//  lse_scale  log2(e) / temperature
//  aux        the plan's aux area of the workspace
//  wire       encoding of the residual rows (0 f32, 1 f16, 2 per-row symmetric i8)
struct LogitsExtras {
  float* logits = nullptr;
  float2* lse = nullptr;
  float lse_scale = 0.f;
  void* aux = nullptr;
  int32_t wire = 0;
};

// Returns 0 or a negative etg_status; fills *plan.  `why` receives a short reason.
// `extras`: the call also wants probabilities or raw logits (which the rank path
// does not produce).  With path 0 (auto) the workspace size covers both answers.
int32_t plan_logits(const TableDesc& t, int64_t batch, int32_t k, int32_t path, LogitsPlan* plan,
                    const char** why, bool extras = false);

hipError_t launch_gather(const TableDesc& t, const int32_t* ids, int64_t n, float scale,
                         float* out, int32_t* bad, hipStream_t stream);
// Gather with the rows written in wire format 1 (f16) or 2 (i8) to `out`.
hipError_t launch_gather_wire(const TableDesc& t, const int32_t* ids, int64_t n, float scale, int32_t wire,
                              uint8_t* out, int32_t* bad, hipStream_t stream);

// ev_before / ev_after (nullable) are recorded around the table-streaming kernel.
// With want_logits the raw logits go to `logits`; with `probs` (nullable) the
// merge also writes the softmax probabilities at log2(e) / lse_scale temperature;
// with ids == nullptr only the table kernel runs (raw logits mode).
hipError_t launch_logits_topk(const TableDesc& t, const LogitsPlan& p, const void* R,
                              int32_t* ids, float* scores, void* ws, hipStream_t stream,
                              hipEvent_t ev_before = nullptr, hipEvent_t ev_after = nullptr,
                              float* logits = nullptr, float* probs = nullptr, float lse_scale = 0.f,
                              int32_t wire = 0);

// Set the calling thread's etg_last_error() message and return `code` (etg_api.cpp).
int32_t set_error(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

constexpr size_t kMaxLds = 160 * 1024;
constexpr int kTargetBlocks = 256;  // one workgroup per MI355X compute unit

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Opt a kernel in to more than 64 KiB of dynamic LDS.
inline hipError_t set_dynamic_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

inline hipError_t record_event(hipEvent_t ev, hipStream_t stream) {
  return ev ? hipEventRecord(ev, stream) : hipSuccess;
}

// Per-path geometry (fill the path's fields and nblk, npass, lds_bytes,
// img_bytes, aux_bytes, ncand) and launchers of the table-streaming kernel
// (recording ev0 / ev1 around it).  stream.hip, wide.hip, gemm.hip (gemm and the ranking contraction), q8.hip,
// row.hip; the rank path's rescoring is in rank.hip.
int32_t plan_stream(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why);
int32_t plan_wide(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why, bool rank = false);
int32_t plan_gemm(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why);
int32_t plan_q8(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why);
int32_t plan_row(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why);
int32_t plan_rank(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why);
// Q8_0 tables with hidden a multiple of 256 through the matrix cores (stream.hip);
// plan_q8 and launch_q8 use it when it applies.
int32_t plan_stream_q8(const TableDesc& t, int64_t batch, int32_t k, LogitsPlan* p, const char** why);
hipError_t launch_stream_q8(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                            const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_stream(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand,
                         const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_wide(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* img, uint64_t* cand,
                       uint64_t* thr, const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_gemm(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* rs, uint64_t* cand,
                       const LogitsExtras& x, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_q8(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand, const LogitsExtras& x,
                     hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_row(const TableDesc& t, const LogitsPlan& p, const void* R, uint64_t* cand, const LogitsExtras& x,
                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
// The rank path writes ids / scores itself (its rescoring kernel replaces the merge):
// the gemm kernel ranks past 64 residual rows, the wide kernel up to 64.
hipError_t launch_wide_rank(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* img, uint64_t* cand,
                            const LogitsExtras& x, int32_t* ids, float* scores, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1);
// Rescoring and certificate of the rank path (rank.hip): candidate keys [batch][nranges][p.kb]
// of ranges of range_rows table rows, nrm2 [nnrm] upper bounds of the squared row norms,
// kpad the terms the ranking kernel accumulated per logit; sorted: each range's keys
// are in descending order.
hipError_t launch_rescore(const TableDesc& t, const LogitsPlan& p, const void* R, int wire, const uint64_t* cand,
                          int nranges, int64_t range_rows, const float* nrm2, int nnrm, int kpad, int32_t* ids,
                          float* scores, hipStream_t stream, int sorted);
int32_t rescore_waves(int64_t batch);
// Rank path constants (rank.hip): the residual row is kept in LDS by the rescoring;
// rank_norm_kernel reduces the row norm parts per block of kRankNormRows rows.
constexpr int kRankMaxHidden = 16384;
// Largest batch the rank path gives to the wide kernel (one pass of up to 256 rows).
constexpr int64_t kRankWideBatch = 256;
constexpr int kRankNormRows = 1024;
// Squared row norms from parts npart [ngrp][V]: nrm2[x] = the largest norm of rows
// [x kRankNormRows, (x + 1) kRankNormRows) (rank.hip).
hipError_t launch_rank_norm(const float* npart, int ngrp, int64_t V, float* nrm2, hipStream_t stream);
// Plain read stream of bytes (a multiple of 16) at src (16-byte aligned); sink
// (4 bytes) is written only if the XOR of the data equals a fixed word (probe.hip).
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
// Plain write stream: every 32-bit word of bytes (a multiple of 16) at dst
// (16-byte aligned) is set to value (probe.hip).
hipError_t launch_write_probe(void* dst, int64_t bytes, uint32_t value, hipStream_t stream);
size_t rescore_lds(int64_t hidden, int n, int nvr, int k, int64_t batch);
hipError_t launch_rank(const TableDesc& t, const LogitsPlan& p, const void* R, uint8_t* rs, uint64_t* cand,
                       const LogitsExtras& x, int32_t* ids, float* scores, hipStream_t stream, hipEvent_t ev0,
                       hipEvent_t ev1);

}  // namespace etg

// The opaque handle of etg.h: host metadata of a table in device memory.
struct etg_table {
  etg::TableDesc d;
};
