// libmsa C ABI: argument validation, workspace layout and the launch sequence of each entry
// point. The contract of every function is stated in include/msa.h.
//
// Launch sequences ("MiniMax goes sparse: decoding M3's attention from a single diagram",
// §1 Steps 1-2; §3 decode / prefill):
//   msa_decode_step   [append: new K/V row, that block's summary and score | score] (one launch) -> top-k
//                     -> attend -> split-K merge; for bf16, k <= 256 on long rows, split over
//                     several workgroups: [append | score + run maxima] -> select-and-attend -> merge
//   msa_prefill_chunk [append + summaries | tile queries] (one launch) -> score -> top-k (+diagonal)
//                     -> attend (-> merge of the list splits, for short chunks)
//   msa_prefill_attend  attend (the last launch of msa_prefill_chunk, over given lists)
//   msa_decode_step_noalloc  msa_decode_step's launches with a file-scope device array as the workspace
// Everything is enqueued on the caller's stream; nothing is allocated; validation precedes any
// HIP call, so an invalid call enqueues nothing.
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include <hip/hip_runtime.h>

#include "msa.h"
#include "common.h"
#include "kernels.h"

namespace {

using namespace msa;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t scores = 0, idx = 0, pages = 0, qtile = 0, part_o = 0, part_ml = 0, cmax = 0, total = 0;
  int row_stride = 0;   // scores per row
  int cstride = 0;      // run maxima per row (fused decode step)
  int bps = 1, nsplit = 0;
  bool fused = false;   // decode step: Step 1's TopK inside the attend launch
};

// A bf16 decode step with k <= kMaxFusedTopK and rows of at most kMaxFusedChunks scoring chunks
// selects inside its attend launch (launch_decode_select_attend); for k > 64 the rows must also
// hold at least 2k runs of kMaxRun blocks, so that the run-maximum bound leaves few candidates
// (1M tokens, k = 128: 38.9 -> 35.0 us per step; k = 256: 52.2 -> 46.6 us; 256k tokens, k = 256:
// 44.0 -> 42.8 us).
bool fused_decode(const msa_config* c, int row_stride) {
  return c->q_dtype == MSA_BF16 && c->top_k <= kMaxFusedTopK && row_stride <= kMaxFusedChunks * kScoreChunk &&
         (c->top_k <= 64 || row_stride >= 2 * kMaxRun * c->top_k);
}

// any_mode: the entry point does not read score_mode (msa_select_index)
msa_status check_config(const msa_config* c, bool any_mode = false) {
  if (c == nullptr) return MSA_ERR_INVALID_ARG;
  if (c->num_q_heads < 1 || c->num_kv_heads < 1 || c->num_q_heads % c->num_kv_heads != 0) return MSA_ERR_INVALID_ARG;
  if (c->top_k < 1) return MSA_ERR_INVALID_ARG;
  if (c->keep_sink < 0 || c->keep_local < 0 || (long long)c->keep_sink + c->keep_local > c->top_k)
    return MSA_ERR_INVALID_ARG;
  if (c->q_dtype != MSA_F32 && c->q_dtype != MSA_BF16) return MSA_ERR_INVALID_ARG;
  if (c->kv_dtype != MSA_F32 && c->kv_dtype != MSA_BF16) return MSA_ERR_INVALID_ARG;
  if (c->out_dtype != MSA_F32 && c->out_dtype != MSA_BF16) return MSA_ERR_INVALID_ARG;
  if (c->summary_dtype != MSA_F32 && c->summary_dtype != MSA_BF16) return MSA_ERR_INVALID_ARG;
  if (c->score_mode != MSA_SCORE_MEAN_KEY && c->score_mode != MSA_SCORE_MAX_TOKEN) return MSA_ERR_INVALID_ARG;
  if (!std::isfinite(c->softmax_scale) || !(c->softmax_scale > 0.f)) return MSA_ERR_INVALID_ARG;
  if (c->head_dim != MSA_HEAD_DIM || c->block_size != MSA_BLOCK) return MSA_ERR_UNSUPPORTED;
  if (c->top_k > MSA_MAX_TOP_K) return MSA_ERR_UNSUPPORTED;
  if (c->num_q_heads / c->num_kv_heads > MSA_MAX_GROUP) return MSA_ERR_UNSUPPORTED;
  if (c->num_kv_heads > MSA_MAX_KV_HEADS) return MSA_ERR_UNSUPPORTED;
  if (c->kv_dtype != c->q_dtype || c->out_dtype != c->q_dtype) return MSA_ERR_UNSUPPORTED;
  if (c->score_mode != MSA_SCORE_MEAN_KEY && !any_mode) return MSA_ERR_UNSUPPORTED;
  if (c->q_tile != MSA_BLOCK) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

// decode-side layouts (op = SELECT, ATTEND or DECODE)
Layout decode_layout(const msa_config* c, int op, int B, int max_len) {
  Layout L;
  const int Hkv = c->num_kv_heads, Hq = c->num_q_heads, k = c->top_k;
  const size_t rows = (size_t)B * Hkv;
  L.row_stride = (max_len + MSA_BLOCK - 1) / MSA_BLOCK;
  L.bps = decode_blocks_per_split(B, Hkv, k);
  L.nsplit = (k + L.bps - 1) / L.bps;
  const bool sel = op == MSA_OP_SELECT || op == MSA_OP_DECODE;
  const bool att = op == MSA_OP_ATTEND || op == MSA_OP_DECODE;
  size_t off = 0;
  if (sel) {
    L.scores = off; off += align256(rows * (size_t)(L.row_stride > 0 ? L.row_stride : 1) * sizeof(float));
  }
  if (op == MSA_OP_DECODE) {
    L.idx = off;   off += align256(rows * (size_t)k * sizeof(int32_t));
    L.pages = off; off += align256(rows * (size_t)k * sizeof(int32_t));
    // rows attended by one workgroup each (no split) keep the separate top-k launch: there the
    // fused selection sits in front of a long attend with nothing to overlap it (batch 32 over
    // mixed lengths up to 1M: a whole step of 181 us fused against 172 us unfused)
    L.fused = fused_decode(c, L.row_stride) && L.nsplit > 1;
    if (L.fused) {
      L.cstride = 2 * ((L.row_stride + kScoreChunk - 1) / kScoreChunk);   // two runs per scoring chunk
      L.cmax = off; off += align256(rows * (size_t)(L.cstride > 0 ? L.cstride : 1) * sizeof(float));
    }
  }
  if (att) {
    L.part_o = off;   off += align256((size_t)B * Hq * L.nsplit * kD * sizeof(float));
    L.part_ml = off;  off += align256((size_t)B * Hq * L.nsplit * 2 * sizeof(float));
  }
  L.total = off;
  return L;
}

Layout prefill_layout(const msa_config* c, int max_len, int T) {
  Layout L;
  const int Hkv = c->num_kv_heads, k = c->top_k;
  const int ntiles = (T + kP - 1) / kP;
  const size_t rows = (size_t)ntiles * Hkv;
  L.row_stride = (max_len + kP - 1) / kP;
  size_t off = 0;
  L.scores = off; off += align256(rows * (size_t)(L.row_stride > 0 ? L.row_stride : 1) * sizeof(float));
  L.qtile = off;  off += align256(rows * (size_t)kD * sizeof(float));
  L.idx = off;    off += align256(rows * (size_t)(k + 1) * sizeof(int32_t));
  L.nsplit = prefill_splits(T, c->num_q_heads, Hkv, k);   // split-K of short chunks' lists
  if (L.nsplit > 1) {
    const size_t units = (size_t)T * c->num_q_heads * L.nsplit;
    L.part_o = off;  off += align256(units * kD * sizeof(float));
    L.part_ml = off; off += align256(units * 2 * sizeof(float));
  }
  L.total = off;
  return L;
}

// one line per decode-side entry point when MSA_LOG is set (kernels.h): the arguments and the layout
void log_layout(const char* entry, const msa_config* c, int B, int max_len, const Layout& L, size_t ws_bytes,
                const char* extra) {
  if (!log_enabled()) return;
  log_call("%s: batch %d, max_seq_len %d, %d q / %d kv heads, top_k %d, %s; row stride %d, %d split(s) of %d "
           "block(s)%s; workspace %zu of %zu B%s",
           entry, B, max_len, c->num_q_heads, c->num_kv_heads, c->top_k, c->q_dtype == MSA_BF16 ? "bf16" : "f32",
           L.row_stride, L.nsplit, L.bps, L.fused ? ", top-k inside the attend launch" : "", L.total, ws_bytes, extra);
}

// MSA_DEVICE_CHECKS (kernels.h): the caller's lengths, page ids and, for attend, lists, checked on
// the device before anything else is enqueued
msa_status cache_check(const char* entry, const msa_kv_cache* c, int B, int max_len, const int32_t* idx, int k,
                       int Hkv, hipStream_t st) {
  if (!checks_enabled()) return MSA_OK;
  CheckArgs a;
  a.table = c->block_table;
  a.lens = c->seq_lens;
  a.B = B;
  a.max_blocks = c->max_blocks;
  a.max_len = max_len;
  a.num_pages = c->num_pages;
  a.idx = idx;
  a.k = k;
  a.Hkv = Hkv;
  const int r = device_check(entry, a, st);
  return r == 0 ? MSA_OK : r > 0 ? MSA_ERR_INVALID_ARG : MSA_ERR_HIP;
}

msa_status prefill_check(const char* entry, const msa_kv_cache* c, int len, hipStream_t st) {
  if (!checks_enabled()) return MSA_OK;
  CheckArgs a;
  a.table = c->block_table;
  a.fixed_len = len;
  a.B = 1;
  a.max_blocks = c->max_blocks;
  a.max_len = len;
  a.num_pages = c->num_pages;
  const int r = device_check(entry, a, st);
  return r == 0 ? MSA_OK : r > 0 ? MSA_ERR_INVALID_ARG : MSA_ERR_HIP;
}

template <typename T> T* at(void* ws, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off); }

msa_status check_cache(const msa_kv_cache* cache, bool need_kv, bool need_lens) {
  if (cache == nullptr || cache->summaries == nullptr || cache->block_table == nullptr) return MSA_ERR_INVALID_ARG;
  if (need_kv && (cache->k_pages == nullptr || cache->v_pages == nullptr)) return MSA_ERR_INVALID_ARG;
  if (need_lens && cache->seq_lens == nullptr) return MSA_ERR_INVALID_ARG;
  if (cache->num_pages < 0 || cache->max_blocks < 1) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

msa_status check_batch(const msa_kv_cache* cache, int B, int max_len) {
  if (B < 0 || max_len < 0) return MSA_ERR_INVALID_ARG;
  if (B > MSA_MAX_BATCH) return MSA_ERR_UNSUPPORTED;   // the batch is a grid dimension of 65535 at most
  if ((long long)max_len > (long long)cache->max_blocks * MSA_BLOCK) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

CacheArgs cache_args(const msa_config* cfg, const msa_kv_cache* c) {
  return CacheArgs{c->k_pages, c->v_pages, c->summaries, cfg->summary_dtype == MSA_BF16, c->block_table, c->seq_lens,
                   c->num_pages, c->max_blocks};
}

msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

#define MSA_TRY(expr)                        \
  do {                                       \
    const msa_status s_ = (expr);            \
    if (s_ != MSA_OK) return s_;             \
  } while (0)

// top-k of decode score rows on validated arguments; pages (page ids of the kept blocks,
// nullable) is the decode step's extra
msa_status run_topk(const msa_config* cfg, const msa_kv_cache* cache, int B, int max_len, float* scores,
                    int row_stride, int32_t* idx, int32_t* pages, hipStream_t st) {
  TopkArgs t{};
  t.scores = scores;
  t.row_stride = row_stride;
  t.idx = idx;
  t.idx_stride = cfg->top_k;
  t.rows = B * cfg->num_kv_heads;
  t.k = cfg->top_k;
  t.Hkv = cfg->num_kv_heads;
  t.lens = cache->seq_lens;
  t.max_len = max_len;
  t.base_blocks = 0;
  t.keep_sink = cfg->keep_sink;
  t.keep_local = cfg->keep_local;
  t.pages = pages;
  t.table = cache->block_table;
  t.max_blocks = cache->max_blocks;
  t.num_pages = cache->num_pages;
  return hip_status(launch_topk(t, st));
}

// Step 1 on validated arguments; the appended token (k_new / v_new, nullable) goes into the
// scoring launch
// pad: the scores go to a caller's buffer, which gets its -inf entries past each sequence's end
msa_status run_select(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int B, int max_len,
                      float* scores, int row_stride, int32_t* idx, int32_t* pages, const void* k_new,
                      const void* v_new, bool pad, hipStream_t st) {
  MSA_TRY(hip_status(launch_score_decode(cfg->q_dtype == MSA_BF16, q, cache_args(cfg, cache), B, cfg->num_q_heads,
                                         cfg->num_kv_heads, max_len, scores, row_stride, k_new, v_new, st, nullptr, 0,
                                         pad)));
  return run_topk(cfg, cache, B, max_len, scores, row_stride, idx, pages, st);
}

AttendArgs attend_args(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int B, int max_len,
                       const int32_t* idx, const int32_t* pages, void* out, float* lse, const Layout& L, void* ws);

// Step 2 on validated arguments
msa_status run_attend(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int B, int max_len,
                      const int32_t* idx, const int32_t* pages, void* out, float* lse, const Layout& L, void* ws,
                      hipStream_t st) {
  const AttendArgs a = attend_args(cfg, q, cache, B, max_len, idx, pages, out, lse, L, ws);
  return hip_status(launch_attend_decode(cfg->q_dtype == MSA_BF16, a, st));
}

AttendArgs attend_args(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int B, int max_len,
                       const int32_t* idx, const int32_t* pages, void* out, float* lse, const Layout& L, void* ws) {
  AttendArgs a{};
  a.q = q;
  a.kpool = cache->k_pages;
  a.vpool = cache->v_pages;
  a.table = cache->block_table;
  a.lens = cache->seq_lens;
  a.idx = idx;
  a.pages = pages;
  a.num_pages = cache->num_pages;
  a.max_blocks = cache->max_blocks;
  a.max_len = max_len;
  a.B = B;
  a.Hq = cfg->num_q_heads;
  a.Hkv = cfg->num_kv_heads;
  a.k = cfg->top_k;
  a.scale_log2 = cfg->softmax_scale * kLog2e;
  a.blocks_per_split = L.bps;
  a.nsplit = L.nsplit;
  a.part_o = at<float>(ws, L.part_o);
  a.part_ml = at<float>(ws, L.part_ml);
  a.out = out;
  a.lse = lse;
  return a;
}

// Argument checks of a decode step (both entry points) and its workspace layout
msa_status check_decode_step(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int B, int max_len,
                             const void* k_new, const void* v_new, const void* out, Layout* L) {
  MSA_TRY(check_config(cfg));
  MSA_TRY(check_cache(cache, true, true));
  MSA_TRY(check_batch(cache, B, max_len));
  if (q == nullptr || out == nullptr || ((k_new == nullptr) != (v_new == nullptr))) return MSA_ERR_INVALID_ARG;
  *L = decode_layout(cfg, MSA_OP_DECODE, B, max_len);
  if (L->nsplit > kMaxDecodeSplit) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

// A decode step on validated arguments with a workspace of at least L.total bytes. Every
// workspace byte the step reads is written earlier in the same step (scores, lists, page ids,
// split partials), so the workspace needs no clearing.
msa_status run_decode_step(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int B, int max_len,
                           const void* k_new, const void* v_new, int32_t* idx_out, float* scores_out, void* out,
                           float* lse_out, const Layout& L, void* ws, hipStream_t st) {
  float* scores = scores_out ? scores_out : at<float>(ws, L.scores);
  if (L.fused) {   // score (+ run maxima) -> select-and-attend -> merge
    float* cmax = at<float>(ws, L.cmax);
    MSA_TRY(hip_status(launch_score_decode(true, q, cache_args(cfg, cache), B, cfg->num_q_heads, cfg->num_kv_heads,
                                           max_len, scores, L.row_stride, k_new, v_new, st, cmax, L.cstride,
                                           scores_out != nullptr)));
    FusedArgs f{};
    f.att = attend_args(cfg, q, cache, B, max_len, nullptr, nullptr, out, lse_out, L, ws);
    f.scores = scores;
    f.row_stride = L.row_stride;
    f.cmax = cmax;
    f.keep_sink = cfg->keep_sink;
    f.keep_local = cfg->keep_local;
    f.cstride = L.cstride;
    f.idx_out = idx_out;
    return hip_status(launch_decode_select_attend(f, st));
  }
  int32_t* idx = idx_out ? idx_out : at<int32_t>(ws, L.idx);
  int32_t* pages = at<int32_t>(ws, L.pages);
  MSA_TRY(run_select(cfg, q, cache, B, max_len, scores, L.row_stride, idx, pages, k_new, v_new, scores_out != nullptr,
                     st));
  return run_attend(cfg, q, cache, B, max_len, idx, pages, out, lse_out, L, ws, st);
}

// The no-allocation decode step's workspace: one file-scope device array. Every GPU the library
// runs on holds its own copy (at its own address) until the process ends. In host code `scratch`
// names a host-side stand-in, never device memory: its device address on the current device is
// looked up once per device with hipGetSymbolAddress and only that address is handed to kernels.
// Calls that overlap in time on one GPU share this array and race.
__device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

msa_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MSA_OK;
}

// Step 2 of a prefill chunk on validated arguments; nsplit > 1: the lists split over that many
// workgroups, whose partials (part_o, part_ml) a merge launch combines
msa_status run_prefill_attend(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int past_len, int T,
                              const int32_t* idx, void* out, float* lse, int nsplit, float* part_o, float* part_ml,
                              hipStream_t st) {
  PrefillArgs p{};
  p.q = q;
  p.kpool = cache->k_pages;
  p.vpool = cache->v_pages;
  p.table = cache->block_table;
  p.idx = idx;
  p.num_pages = cache->num_pages;
  p.past_len = past_len;
  p.T = T;
  p.Hq = cfg->num_q_heads;
  p.Hkv = cfg->num_kv_heads;
  p.k = cfg->top_k;
  p.scale_log2 = cfg->softmax_scale * kLog2e;
  p.out = out;
  p.lse = lse;
  p.nsplit = nsplit;
  p.part_o = part_o;
  p.part_ml = part_ml;
  return hip_status(launch_attend_prefill(p, st));
}

}  // namespace

extern "C" {

msa_status msa_workspace_size(const msa_config* cfg, int32_t op, int32_t batch, int32_t max_seq_len,
                              int32_t chunk_len, size_t* bytes) {
  MSA_TRY(check_config(cfg));
  if (bytes == nullptr || batch < 0 || max_seq_len < 0) return MSA_ERR_INVALID_ARG;
  if (batch > MSA_MAX_BATCH) return MSA_ERR_UNSUPPORTED;
  switch (op) {
    case MSA_OP_SELECT:
    case MSA_OP_ATTEND:
    case MSA_OP_DECODE:
      {
        const Layout L = decode_layout(cfg, op, batch, max_seq_len);
        if (L.nsplit > kMaxDecodeSplit) return MSA_ERR_UNSUPPORTED;   // never: the split rule bounds it
        *bytes = L.total;
      }
      log_call("msa_workspace_size: op %d, batch %d, max_seq_len %d -> %zu B", op, batch, max_seq_len, *bytes);
      return MSA_OK;
    case MSA_OP_PREFILL:
      if (chunk_len < 1 || batch != 1 || max_seq_len < chunk_len) return MSA_ERR_INVALID_ARG;
      *bytes = prefill_layout(cfg, max_seq_len, chunk_len).total;
      log_call("msa_workspace_size: prefill, max_seq_len %d, chunk %d -> %zu B", max_seq_len, chunk_len, *bytes);
      return MSA_OK;
    default:
      return MSA_ERR_INVALID_ARG;
  }
}

msa_status msa_build_summaries(const msa_config* cfg, const msa_kv_cache* cache, int32_t batch,
                               int32_t max_seq_len, void* stream) {
  MSA_TRY(check_config(cfg));
  MSA_TRY(check_cache(cache, false, true));
  if (cache->k_pages == nullptr) return MSA_ERR_INVALID_ARG;
  MSA_TRY(check_batch(cache, batch, max_seq_len));
  if (batch == 0) return MSA_OK;
  MSA_TRY(cache_check("msa_build_summaries", cache, batch, max_seq_len, nullptr, 0, 0, (hipStream_t)stream));
  log_call("msa_build_summaries: batch %d, max_seq_len %d, %d kv heads, %s summaries", batch, max_seq_len,
           cfg->num_kv_heads, cfg->summary_dtype == MSA_BF16 ? "bf16" : "f32");
  return hip_status(launch_build_summaries(cfg->kv_dtype == MSA_BF16, cache_args(cfg, cache), batch, cfg->num_kv_heads,
                                           max_seq_len, (hipStream_t)stream));
}

msa_status msa_score(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int32_t batch,
                     int32_t max_seq_len, float* scores_out, void* stream) {
  MSA_TRY(check_config(cfg));
  MSA_TRY(check_cache(cache, false, true));
  MSA_TRY(check_batch(cache, batch, max_seq_len));
  if (q == nullptr || scores_out == nullptr) return MSA_ERR_INVALID_ARG;
  if (batch == 0) return MSA_OK;
  const int row_stride = (max_seq_len + MSA_BLOCK - 1) / MSA_BLOCK;
  MSA_TRY(cache_check("msa_score", cache, batch, max_seq_len, nullptr, 0, 0, (hipStream_t)stream));
  log_call("msa_score: batch %d, max_seq_len %d, %d q / %d kv heads, row stride %d", batch, max_seq_len,
           cfg->num_q_heads, cfg->num_kv_heads, row_stride);
  return hip_status(launch_score_decode(cfg->q_dtype == MSA_BF16, q, cache_args(cfg, cache), batch, cfg->num_q_heads,
                                        cfg->num_kv_heads, max_seq_len, scores_out, row_stride, nullptr, nullptr,
                                        (hipStream_t)stream));
}

msa_status msa_select(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int32_t batch,
                      int32_t max_seq_len, float* scores_out, int32_t* idx_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  MSA_TRY(check_config(cfg));
  MSA_TRY(check_cache(cache, false, true));
  MSA_TRY(check_batch(cache, batch, max_seq_len));
  if (q == nullptr || idx_out == nullptr) return MSA_ERR_INVALID_ARG;
  const Layout L = decode_layout(cfg, MSA_OP_SELECT, batch, max_seq_len);
  if (workspace_bytes < L.total || workspace == nullptr) return MSA_ERR_WORKSPACE;
  if (batch == 0) return MSA_OK;
  MSA_TRY(cache_check("msa_select", cache, batch, max_seq_len, nullptr, 0, 0, (hipStream_t)stream));
  log_layout("msa_select", cfg, batch, max_seq_len, L, workspace_bytes, "");
  float* scores = scores_out ? scores_out : at<float>(workspace, L.scores);
  return run_select(cfg, q, cache, batch, max_seq_len, scores, L.row_stride, idx_out, nullptr, nullptr, nullptr,
                    scores_out != nullptr, (hipStream_t)stream);
}

msa_status msa_select_index(const msa_config* cfg, const void* q_index, const void* index_keys, int32_t index_dim,
                            const msa_kv_cache* cache, int32_t batch, int32_t max_seq_len, float* scores_out,
                            int32_t* idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  MSA_TRY(check_config(cfg, true));
  if (cache == nullptr || cache->block_table == nullptr || cache->seq_lens == nullptr) return MSA_ERR_INVALID_ARG;
  if (cache->num_pages < 0 || cache->max_blocks < 1) return MSA_ERR_INVALID_ARG;
  MSA_TRY(check_batch(cache, batch, max_seq_len));
  if (q_index == nullptr || index_keys == nullptr || idx_out == nullptr) return MSA_ERR_INVALID_ARG;
  if (index_dim < 1) return MSA_ERR_INVALID_ARG;
  if (index_dim != 64 && index_dim != 128) return MSA_ERR_UNSUPPORTED;
  const Layout L = decode_layout(cfg, MSA_OP_SELECT, batch, max_seq_len);
  if (workspace_bytes < L.total || workspace == nullptr) return MSA_ERR_WORKSPACE;
  if (batch == 0) return MSA_OK;
  const hipStream_t st = (hipStream_t)stream;
  MSA_TRY(cache_check("msa_select_index", cache, batch, max_seq_len, nullptr, 0, 0, st));
  log_layout("msa_select_index", cfg, batch, max_seq_len, L, workspace_bytes, index_dim == 64 ? ", index dim 64" : ", index dim 128");
  float* scores = scores_out ? scores_out : at<float>(workspace, L.scores);
  MSA_TRY(hip_status(launch_score_index(cfg->q_dtype == MSA_BF16, q_index, index_keys, index_dim,
                                        cache_args(cfg, cache), batch, cfg->num_kv_heads, max_seq_len, scores,
                                        L.row_stride, st)));
  return run_topk(cfg, cache, batch, max_seq_len, scores, L.row_stride, idx_out, nullptr, st);
}

msa_status msa_attend(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int32_t batch,
                      int32_t max_seq_len, const int32_t* idx, void* out, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  MSA_TRY(check_config(cfg));
  MSA_TRY(check_cache(cache, true, true));
  MSA_TRY(check_batch(cache, batch, max_seq_len));
  if (q == nullptr || idx == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  const Layout L = decode_layout(cfg, MSA_OP_ATTEND, batch, max_seq_len);
  if (L.nsplit > kMaxDecodeSplit) return MSA_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total || workspace == nullptr) return MSA_ERR_WORKSPACE;
  if (batch == 0) return MSA_OK;
  const hipStream_t st = (hipStream_t)stream;
  MSA_TRY(cache_check("msa_attend", cache, batch, max_seq_len, idx, cfg->top_k, cfg->num_kv_heads, st));
  log_layout("msa_attend", cfg, batch, max_seq_len, L, workspace_bytes, "");
  return run_attend(cfg, q, cache, batch, max_seq_len, idx, nullptr, out, lse_out, L, workspace, st);
}

msa_status msa_decode_step(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int32_t batch,
                           int32_t max_seq_len, const void* k_new, const void* v_new, int32_t* idx_out,
                           float* scores_out, void* out, float* lse_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Layout L;
  MSA_TRY(check_decode_step(cfg, q, cache, batch, max_seq_len, k_new, v_new, out, &L));
  if (workspace_bytes < L.total || workspace == nullptr) return MSA_ERR_WORKSPACE;
  if (batch == 0) return MSA_OK;
  MSA_TRY(cache_check("msa_decode_step", cache, batch, max_seq_len, nullptr, 0, 0, (hipStream_t)stream));
  log_layout("msa_decode_step", cfg, batch, max_seq_len, L, workspace_bytes,
             k_new != nullptr ? ", appending a new token" : "");
  return run_decode_step(cfg, q, cache, batch, max_seq_len, k_new, v_new, idx_out, scores_out, out, lse_out, L,
                         workspace, (hipStream_t)stream);
}

msa_status msa_decode_step_noalloc(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int32_t batch,
                                   int32_t max_seq_len, const void* k_new, const void* v_new, int32_t* idx_out,
                                   float* scores_out, void* out, float* lse_out, void* stream) {
  Layout L;
  MSA_TRY(check_decode_step(cfg, q, cache, batch, max_seq_len, k_new, v_new, out, &L));
  if (L.total > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_WORKSPACE;
  if (batch == 0) return MSA_OK;
  void* ws = nullptr;
  MSA_TRY(scratch_of_current_device(&ws));
  MSA_TRY(cache_check("msa_decode_step_noalloc", cache, batch, max_seq_len, nullptr, 0, 0, (hipStream_t)stream));
  log_layout("msa_decode_step_noalloc", cfg, batch, max_seq_len, L, (size_t)MSA_NOALLOC_SCRATCH_BYTES,
             k_new != nullptr ? ", appending a new token; workspace = the per-GPU scratch array" : "; workspace = the per-GPU scratch array");
  return run_decode_step(cfg, q, cache, batch, max_seq_len, k_new, v_new, idx_out, scores_out, out, lse_out, L, ws,
                         (hipStream_t)stream);
}

msa_status msa_prefill_chunk(const msa_config* cfg, const void* q, const void* k_new, const void* v_new,
                             const msa_kv_cache* cache, int32_t past_len, int32_t T, int32_t* idx_out,
                             float* scores_out, void* out, float* lse_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  MSA_TRY(check_config(cfg));
  MSA_TRY(check_cache(cache, true, false));
  if (q == nullptr || k_new == nullptr || v_new == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (T < 1 || past_len < 0) return MSA_ERR_INVALID_ARG;
  if ((long long)past_len + T > (long long)cache->max_blocks * MSA_BLOCK) return MSA_ERR_INVALID_ARG;
  if (past_len % MSA_BLOCK != 0) return MSA_ERR_UNSUPPORTED;
  if (cfg->q_dtype != MSA_BF16) return MSA_ERR_UNSUPPORTED;
  const int max_len = past_len + T;
  const Layout L = prefill_layout(cfg, max_len, T);
  if (workspace_bytes < L.total || workspace == nullptr) return MSA_ERR_WORKSPACE;
  const hipStream_t st = (hipStream_t)stream;
  const int Hkv = cfg->num_kv_heads, Hq = cfg->num_q_heads;
  const int past_blocks = past_len / kP, ntiles = (T + kP - 1) / kP;
  const CacheArgs ca = cache_args(cfg, cache);
  float* qtile = at<float>(workspace, L.qtile);
  float* scores = scores_out ? scores_out : at<float>(workspace, L.scores);
  int32_t* idx = idx_out ? idx_out : at<int32_t>(workspace, L.idx);
  MSA_TRY(prefill_check("msa_prefill_chunk", cache, max_len, st));
  log_call("msa_prefill_chunk: past_len %d, T %d (%d tiles), %d q / %d kv heads, top_k %d; row stride %d; "
           "%d list split(s); workspace %zu of %zu B", past_len, T, ntiles, Hq, Hkv, cfg->top_k, L.row_stride, L.nsplit,
           L.total, workspace_bytes);

  MSA_TRY(hip_status(launch_prefill_prologue(true, ca, k_new, v_new, q, past_blocks, T, Hq, Hkv, qtile, st)));
  MSA_TRY(hip_status(launch_score_prefill(qtile, ca, past_blocks, ntiles, Hkv, scores, L.row_stride, st)));
  TopkArgs t{};
  t.scores = scores;
  t.row_stride = L.row_stride;
  t.idx = idx;
  t.idx_stride = cfg->top_k + 1;
  t.pages = nullptr;
  t.rows = ntiles * Hkv;
  t.k = cfg->top_k;
  t.Hkv = Hkv;
  t.lens = nullptr;
  t.max_len = max_len;
  t.base_blocks = past_blocks;
  t.keep_sink = cfg->keep_sink;
  t.keep_local = cfg->keep_local;
  MSA_TRY(hip_status(launch_topk(t, st)));
  return run_prefill_attend(cfg, q, cache, past_len, T, idx, out, lse_out, L.nsplit,
                            L.nsplit > 1 ? at<float>(workspace, L.part_o) : nullptr,
                            L.nsplit > 1 ? at<float>(workspace, L.part_ml) : nullptr, st);
}

msa_status msa_prefill_attend(const msa_config* cfg, const void* q, const msa_kv_cache* cache, int32_t past_len,
                              int32_t T, const int32_t* idx, void* out, float* lse_out, void* stream) {
  MSA_TRY(check_config(cfg));
  if (cache == nullptr || cache->block_table == nullptr || cache->k_pages == nullptr || cache->v_pages == nullptr)
    return MSA_ERR_INVALID_ARG;
  if (cache->num_pages < 0 || cache->max_blocks < 1) return MSA_ERR_INVALID_ARG;
  if (q == nullptr || idx == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (T < 1 || past_len < 0) return MSA_ERR_INVALID_ARG;
  if ((long long)past_len + T > (long long)cache->max_blocks * MSA_BLOCK) return MSA_ERR_INVALID_ARG;
  if (past_len % MSA_BLOCK != 0) return MSA_ERR_UNSUPPORTED;
  if (cfg->q_dtype != MSA_BF16) return MSA_ERR_UNSUPPORTED;
  MSA_TRY(prefill_check("msa_prefill_attend", cache, past_len + T, (hipStream_t)stream));
  log_call("msa_prefill_attend: past_len %d, T %d, %d q / %d kv heads, top_k %d", past_len, T, cfg->num_q_heads,
           cfg->num_kv_heads, cfg->top_k);
  return run_prefill_attend(cfg, q, cache, past_len, T, idx, out, lse_out, 1, nullptr, nullptr, (hipStream_t)stream);
}

const char* msa_status_string(msa_status status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG: a required pointer is null or a count/size is invalid";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: valid configuration that this library does not implement";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE: workspace is null or smaller than msa_workspace_size()";
    case MSA_ERR_HIP: return "MSA_ERR_HIP: a HIP kernel launch failed";
    default: return "unknown msa_status";
  }
}

}  // extern "C"
