// Internal launchers of libmsa (host side). Every launcher enqueues on `st` and returns the
// launch status; all argument validation happens before, in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Launch logging (diag.hip): with MSA_LOG set (non-empty, not "0"), entry points and kernel
// launches print one line each on stderr. log_launch's fmt describes the template parameters.
bool log_enabled();
void log_call(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void log_launch(const char* kernel, dim3 grid, int threads, size_t lds_bytes, const char* fmt, ...)
    __attribute__((format(printf, 5, 6)));

// Device-side checks of the caller's index data (diag.hip), on with MSA_DEVICE_CHECKS set
// (non-empty, not "0"): lens (or fixed_len when lens is null) against
// [0, min(max_len, max_blocks * 64)], the page ids of the visible blocks against [0, num_pages),
// and, when idx is given ([B][Hkv][k] attend lists), repeated valid entries in a row (rows of up to
// kCheckMaxBits blocks are checked in full). device_check returns 0 (clean, or checks off, or the
// stream is capturing), 1 (a violation, printed on stderr) or -1 (a HIP error). It synchronises st.
constexpr long long kCheckMaxBits = 1 << 18;   // 32 KiB of LDS bitmap per row
struct CheckArgs {
  const int32_t* table = nullptr;
  const int32_t* lens = nullptr;
  int fixed_len = 0;
  int B = 0, max_blocks = 0, max_len = 0, num_pages = 0;
  const int32_t* idx = nullptr;
  int k = 0, Hkv = 0;
};
bool checks_enabled();
int device_check(const char* entry, const CheckArgs& a, hipStream_t st);

struct CacheArgs {
  void* k;               // [num_pages][Hkv][64][128]
  void* v;
  void* S;               // [num_pages][Hkv][128] summaries: float, or bf16 when s_bf16
  bool s_bf16;
  const int32_t* table;  // [B][max_blocks]
  const int32_t* lens;   // [B] (decode paths)
  int num_pages;
  int max_blocks;
};

// ---- block summaries / append
hipError_t launch_build_summaries(bool bf16, const CacheArgs& c, int B, int Hkv, int max_len, hipStream_t st);
// prefill: append the chunk (K/V rows + the new blocks' summaries) and compute the tile index
// queries qtile [ceil(T/64)][Hkv][128] in one launch
hipError_t launch_prefill_prologue(bool bf16, const CacheArgs& c, const void* k_new, const void* v_new,
                                   const void* q, int past_blocks, int T, int Hq, int Hkv, float* qtile,
                                   hipStream_t st);

// ---- Step 1 scoring. scores rows are (b, g) [decode] or (tile, g) [prefill], row_stride floats each.
// k_new / v_new (nullable, [B][Hkv][128]): the decode step's new token, already counted in seq_lens.
// The same launch writes its K/V row at position seq_len-1, recomputes that block's summary from
// its keys and scores the block from the stored summary.
// cmax (nullable, [B][Hkv][cstride]): the largest score of each run of kMaxRun blocks j < n_b
// (two per scoring chunk), the appended block's excepted (-inf for a run with none);
// cstride >= 2 ceil(row_stride / kScoreChunk) (both runs of every scoring chunk are written)
// pad: also write -inf over the scores past n_b (a caller's score buffer); without it those
// entries are left as they are (the library's own consumers read a row only up to n_b). Run
// maxima past n_b are never written.
constexpr int kScoreChunk = 16;
constexpr int kMaxRun = 8;      // blocks per recorded maximum
hipError_t launch_score_decode(bool bf16, const void* q, const CacheArgs& c, int B, int Hq, int Hkv,
                               int max_len, float* scores, int row_stride, const void* k_new, const void* v_new,
                               hipStream_t st, float* cmax = nullptr, int cstride = 0, bool pad = true);
// index branch (single-head index keys [num_pages][64][index_dim], q_index [B][Hkv][index_dim],
// index_dim 64 or 128): block score = max over the block's valid tokens of <q_index[b][g], K_idx[t]>
hipError_t launch_score_index(bool bf16, const void* q_index, const void* index_keys, int index_dim,
                              const CacheArgs& c, int B, int Hkv, int max_len, float* scores, int row_stride,
                              hipStream_t st);
hipError_t launch_score_prefill(const float* qtile, const CacheArgs& c, int past_blocks, int ntiles, int Hkv,
                                float* scores, int row_stride, hipStream_t st);

// ---- Step 1 top-k
struct TopkArgs {
  float* scores;
  int row_stride;
  int32_t* idx;
  int idx_stride;      // top_k (decode) or top_k + 1 (prefill)
  int rows;
  int k;
  int Hkv;
  const int32_t* lens; // decode: n = ceil(clamp(lens[row / Hkv]) / 64); null -> prefill mode
  int max_len;
  int base_blocks;     // prefill: n = base_blocks + row / Hkv, and block n is appended
  // forced blocks: candidates j < keep_sink or j >= n - keep_local are always kept (counted in
  // k_eff; keep_sink + keep_local <= k)
  int keep_sink;
  int keep_local;
  // decode only (nullable): page ids of the kept blocks [rows][k] (-1 for padding or a bad page
  // id), translated through table [B][max_blocks]
  int32_t* pages;
  const int32_t* table;
  int max_blocks;
  int num_pages;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

// ---- Step 2, decode
struct AttendArgs {
  const void* q;        // [B][Hq][128]
  const void* kpool;    // pools
  const void* vpool;
  const int32_t* table;
  const int32_t* lens;
  const int32_t* idx;   // [B][Hkv][k]
  const int32_t* pages; // nullable [B][Hkv][k]: page ids of idx (else translated through table)
  int num_pages, max_blocks, max_len;
  int B, Hq, Hkv, k;
  float scale_log2;     // softmax_scale * log2(e)
  int blocks_per_split, nsplit;
  float* part_o;        // [B][Hq][nsplit][128]
  float* part_ml;       // [B][Hq][nsplit][2]
  void* out;            // [B][Hq][128]
  float* lse;           // nullable [B][Hq]
};
// Split-K partials one merge workgroup combines; decode_blocks_per_split keeps the split count
// ceil(k / blocks_per_split) at or below it for every (B, Hkv, k).
constexpr int kMaxDecodeSplit = 256;
int decode_blocks_per_split(int B, int Hkv, int k);
hipError_t launch_attend_decode(bool bf16, const AttendArgs& a, hipStream_t st);
// the split-K merge alone (bf16 output), for a.nsplit > 1
hipError_t launch_merge_bf16(const AttendArgs& a, hipStream_t st);

// ---- Steps 1 (TopK) and 2 of a bf16 decode step in one launch (then the merge when split):
// every attend workgroup selects its row's top-k from the scores and run maxima of the scoring
// launch and attends its split of the list. For k <= kMaxFusedTopK and rows of at most
// kMaxFusedChunks * kScoreChunk blocks (k > 64: rows of at least 2 k runs of kMaxRun blocks);
// forced sink / local blocks take a key above every score, and so does the maximum of every run
// that holds one.
constexpr int kMaxFusedTopK = 256;
constexpr int kMaxFusedChunks = 1024;
struct FusedArgs {
  AttendArgs att;        // idx / pages unused
  const float* scores;   // [B][Hkv][row_stride]
  int row_stride;
  const float* cmax;     // [B][Hkv][cstride]
  int cstride;
  int32_t* idx_out;      // nullable [B][Hkv][k]
  int keep_sink, keep_local;   // forced blocks: the first / last of each row's blocks
};
hipError_t launch_decode_select_attend(const FusedArgs& f, hipStream_t st);

// ---- Step 2, prefill (bf16, MFMA)
struct PrefillArgs {
  const void* q;        // [T][Hq][128] bf16
  const void* kpool;    // pools (bf16)
  const void* vpool;
  const int32_t* table; // [max_blocks] of the one sequence
  const int32_t* idx;   // [ntiles][Hkv][k+1]
  int num_pages, past_len, T, Hq, Hkv, k;
  float scale_log2;
  void* out;            // [T][Hq][128] bf16
  float* lse;           // nullable [T][Hq]
  int nsplit;           // workgroups per (tile, group) list: 1 writes out / lse; more write partials
  float* part_o;        // [T][Hq][nsplit][128]: O relative to the split's reference max (nsplit > 1)
  float* part_ml;       // [T][Hq][nsplit][2]: that max (log2 domain) and the split's sum l
};
// Short chunks leave the chip idle with one workgroup per (tile, group): their lists are split
// so that about kPrefillSplitTarget workgroups run (at least two list slots each), and a second
// launch merges the partials of every (token, head) row.
constexpr int kPrefillSplitTarget = 256;
int prefill_splits(int T, int Hq, int Hkv, int k);
// the attend launch, then (a.nsplit > 1) the merge launch
hipError_t launch_attend_prefill(const PrefillArgs& a, hipStream_t st);

}  // namespace msa
