/*
 * msa.h -- C ABI of libmsa: two-stage GQA block-sparse attention on MI355X (gfx950).
 *
 * The method: "MiniMax goes sparse: decoding M3's attention from a single diagram"
 * (atlascloud.ai blog; cited below as [MGS]), §1 "What the diagram shows".
 *   Step 1 (index branch): each GQA group scores the context's fixed-size blocks with one
 *     index query and keeps its top-k blocks -> one short index list per group and layer.
 *   Step 2 (sparse branch): every query head of the group runs ordinary softmax attention over
 *     the real K/V of the selected blocks only; the group's heads share one selection.
 * §3 of the same page: block size unstated (64 assumed); decode time is bound by KV-cache
 * bandwidth, while in prefill the index branch still scans the whole input.
 *
 * Readings fixed by this library where the page is silent:
 *   - block summary = fp32 mean of the block's valid keys (per KV head); block score =
 *     <index query, summary>, unscaled; index query = mean of the group's query heads (decode)
 *     or of the tile's rows x the group's heads (prefill, 64-query tiles);
 *   - top-k order = score descending, then logical block index ascending; -0 == +0;
 *     k_eff = min(top_k, number of candidate blocks); lists are written in ascending block
 *     order and padded with -1;
 *   - decode: all seq_lens[b] cached tokens are visible (the cache already holds the current
 *     token); prefill: candidates are the blocks strictly before a tile's diagonal block, the
 *     diagonal block is always appended, and key position <= query position inside it;
 *   - forced blocks ([MGS §2], third subtraction: the page guesses that an attention sink and a
 *     local block replaced the sliding window): off by default. With keep_sink = s and
 *     keep_local = l, candidates j < s and j >= n - l of a row's n candidates (decode: the
 *     sequence's blocks; prefill: the blocks before the diagonal) are always kept and count
 *     toward k_eff; the remaining k_eff - |forced| are chosen by the order above among the
 *     other candidates. s, l >= 0 and s + l <= top_k, else MSA_ERR_INVALID_ARG;
 *   - summary pool precision: fp32 by default. With summary_dtype = MSA_BF16 the pool holds bf16:
 *     a summary is the fp32 mean of the block's keys rounded to the nearest bf16 value (ties to
 *     even), and every score is computed from the stored bf16 summary. Halves the bytes Step 1
 *     reads in decode; the ranking then sees summaries rounded to 8 significant bits;
 *   - softmax: logits = softmax_scale * <q_h, k_t>, fp32 accumulation, lse in natural log.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; nothing is allocated or
 *     freed by the library and no state is kept between calls (reentrant). The one exception is
 *     msa_decode_step_noalloc, whose workspace is a per-GPU array inside the library (see there).
 *   - `stream` is a hipStream_t passed as void* (0 = the null stream). All work is enqueued
 *     asynchronously on it; no call synchronises the host or copies device data to the host.
 *   - batch <= MSA_MAX_BATCH (a larger batch returns MSA_ERR_UNSUPPORTED).
 *   - Arguments are validated on the host before anything is enqueued. An invalid call
 *     returns MSA_ERR_INVALID_ARG / MSA_ERR_UNSUPPORTED / MSA_ERR_WORKSPACE and enqueues
 *     nothing. A failed kernel launch returns MSA_ERR_HIP. No C++ exception crosses the ABI.
 *   - Device-side data is bounds-checked where it addresses memory: seq_lens are clamped to
 *     [0, min(max_seq_len, max_blocks * block_size)]; a page id outside [0, num_pages) is
 *     never dereferenced: its block scores -inf and contributes no tokens. A sequence with no
 *     visible token gets o = 0 and lse = -inf.
 *   - Non-finite q / K / V values are not supported and not checked.
 *   - Calls that share a workspace must not overlap in time (same stream, or synchronised).
 *   - Diagnostics, both off by default and read from the environment once per process (a value
 *     other than empty or "0" turns them on):
 *     MSA_LOG: every entry point prints one line with its arguments and chosen layout, and every
 *       kernel launch one line (kernel, template parameters, grid, threads, LDS), on stderr.
 *     MSA_DEVICE_CHECKS: every entry point that reads a paged cache first checks on the device
 *       what the kernels otherwise tolerate silently: seq_lens outside
 *       [0, min(max_seq_len, max_blocks * block_size)], a visible block's page id outside
 *       [0, num_pages), and (msa_attend) a valid block listed twice in one row. The first
 *       violation is printed on stderr and the call returns MSA_ERR_INVALID_ARG with nothing
 *       else enqueued. This mode synchronises the stream (the one exception to the rule above),
 *       allocates nothing, and stands aside while the stream is being captured into a graph.
 *
 * Layouts (row-major, element type per msa_config):
 *   q            decode [B][Hq][D]; prefill [T][Hq][D]
 *   K/V pools    [num_pages][Hkv][block_size][D]   (one page = one 64-token block of all heads)
 *   summaries    [num_pages][Hkv][D] float32 or bf16 (summary_dtype; kept equal to the block
 *                                                   means by msa_build_summaries and the append
 *                                                   paths)
 *   block_table  [B][max_blocks] int32             logical block -> page id
 *   seq_lens     [B] int32                         visible tokens per sequence
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msa_status {
    MSA_OK = 0,
    MSA_ERR_INVALID_ARG = 1,  /* null required pointer, bad count or size */
    MSA_ERR_UNSUPPORTED = 2,  /* valid but not implemented: head_dim != 128, block != 64, ... */
    MSA_ERR_WORKSPACE = 3,    /* workspace smaller than msa_workspace_size() */
    MSA_ERR_HIP = 4           /* a HIP launch failed */
} msa_status;

typedef enum msa_dtype { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

/* How the config-driven entry points summarise blocks for Step 1: MEAN_KEY only. MAX_TOKEN
 * (the diagram's Block Max Pool over a single-head index key) needs index keys and index
 * queries that msa_config does not carry; it is served by msa_select_index, and the other
 * entry points return MSA_ERR_UNSUPPORTED for it. */
typedef enum msa_score_mode { MSA_SCORE_MEAN_KEY = 0, MSA_SCORE_MAX_TOKEN = 1 } msa_score_mode;

typedef enum msa_op {
    MSA_OP_SELECT = 0, MSA_OP_ATTEND = 1, MSA_OP_DECODE = 2, MSA_OP_PREFILL = 3
} msa_op;

#define MSA_HEAD_DIM 128
#define MSA_BLOCK 64
#define MSA_MAX_TOP_K 4096
#define MSA_MAX_GROUP 8        /* Hq / Hkv */
#define MSA_MAX_KV_HEADS 64
#define MSA_MAX_BATCH 65535    /* sequences per decode / select / attend call */
#define MSA_NOALLOC_SCRATCH_BYTES (32u << 20)   /* workspace of msa_decode_step_noalloc, per GPU */

typedef struct msa_config {
    int32_t num_q_heads;      /* Hq */
    int32_t num_kv_heads;     /* Hkv <= MSA_MAX_KV_HEADS; Hq % Hkv == 0, Hq / Hkv <= MSA_MAX_GROUP */
    int32_t head_dim;         /* must be 128 */
    int32_t block_size;       /* must be 64 (== page size) */
    int32_t top_k;            /* 1 .. MSA_MAX_TOP_K blocks kept per group (per tile in prefill) */
    float softmax_scale;      /* logit scale > 0, 1/sqrt(head_dim) in the usual setting */
    int32_t q_dtype;          /* msa_dtype of q and k_new/v_new */
    int32_t kv_dtype;         /* msa_dtype of the K/V pools; must equal q_dtype */
    int32_t out_dtype;        /* msa_dtype of out; must equal q_dtype */
    int32_t score_mode;       /* msa_score_mode; MEAN_KEY */
    int32_t keep_local;       /* forced local blocks: the last keep_local candidates are always kept */
    int32_t q_tile;           /* prefill selection tile in query rows; must be 64 */
    int32_t keep_sink;        /* forced sink blocks: the first keep_sink candidates are always kept */
    int32_t summary_dtype;    /* msa_dtype of the summary pool: MSA_F32 (default) or MSA_BF16 */
} msa_config;

typedef struct msa_kv_cache {
    void* k_pages;            /* [num_pages][Hkv][64][128] kv_dtype */
    void* v_pages;            /* same */
    void* summaries;          /* [num_pages][Hkv][128] of cfg->summary_dtype (float32 or bf16) */
    const int32_t* block_table; /* [B][max_blocks] */
    const int32_t* seq_lens;  /* [B]; decode/select/attend/build only */
    int32_t num_pages;
    int32_t max_blocks;
} msa_kv_cache;

/* Workspace bytes needed by `op` for a batch of `batch` sequences of at most `max_seq_len`
 * tokens (prefill: batch = 1, max_seq_len = past_len + chunk_len, chunk_len = T).
 * Writes *bytes and returns MSA_OK, or an error for an invalid / unsupported config. */
msa_status msa_workspace_size(const msa_config* cfg, int32_t op, int32_t batch,
                              int32_t max_seq_len, int32_t chunk_len, size_t* bytes);

/* Setup helper (step 0 of Step 1): recompute summaries[page][g] = mean of the valid keys of
 * every block of every sequence, for b < batch. */
msa_status msa_build_summaries(const msa_config* cfg, const msa_kv_cache* cache, int32_t batch,
                               int32_t max_seq_len, void* stream);

/* Step 1 scoring alone ([MGS §1 Step 1] index branch, before TopK): scores_out[b][g][j] =
 * <mean of the group's query heads, summaries[block_table[b][j]][g]> for j < nb_b, -inf for
 * j in [nb_b, ceil(max_seq_len/64)) and for blocks whose page id is out of range.
 *   q           [batch][Hq][128] q_dtype
 *   scores_out  [batch][Hkv][ceil(max_seq_len/64)] float32 (required)
 * One kernel launch; no workspace. */
msa_status msa_score(const msa_config* cfg, const void* q, const msa_kv_cache* cache,
                     int32_t batch, int32_t max_seq_len, float* scores_out, void* stream);

/* Step 1 ([MGS §1 Step 1]): per (sequence b, KV group g) score every block j < nb_b with
 * <mean of the group's query heads, summary> and keep the top-k.
 *   q           [batch][Hq][128] q_dtype
 *   scores_out  nullable [batch][Hkv][ceil(max_seq_len/64)] float32; -inf past nb_b
 *   idx_out     [batch][Hkv][top_k] int32, ascending logical block ids, -1 padded  */
msa_status msa_select(const msa_config* cfg, const void* q, const msa_kv_cache* cache,
                      int32_t batch, int32_t max_seq_len, float* scores_out, int32_t* idx_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Step 1 as the diagram draws its index branch ([MGS §1 Step 1]: Index Q/K, token scores,
 * Block Max Pool, TopK). One index key per cached token, a single head shared by all groups,
 * paged with the same block_table as K; one index query per (sequence, group):
 *   scores_out[b][g][j] = max over the valid tokens t of block j of <q_index[b][g], K_idx[t]>
 * (unscaled, fp32 accumulation) for j < nb_b = ceil(seq_lens[b]/64); -inf for blocks whose
 * page id is outside [0, num_pages) and for j in [nb_b, ceil(max_seq_len/64)). The top-k
 * rule, k_eff, list order and padding are those of msa_select.
 *   q_index     [batch][Hkv][index_dim] q_dtype
 *   index_keys  [num_pages][64][index_dim] kv_dtype (page p holds the index keys of the
 *               block that block_table maps to p)
 *   index_dim   64 or 128 (other positive values: MSA_ERR_UNSUPPORTED)
 *   cache       only block_table, seq_lens, num_pages and max_blocks are read; K/V and
 *               summaries may be null
 *   scores_out  nullable [batch][Hkv][ceil(max_seq_len/64)] float32
 *   idx_out     [batch][Hkv][top_k] int32
 * cfg->score_mode is not read. Workspace: msa_workspace_size(cfg, MSA_OP_SELECT, ...). */
msa_status msa_select_index(const msa_config* cfg, const void* q_index, const void* index_keys,
                            int32_t index_dim, const msa_kv_cache* cache, int32_t batch,
                            int32_t max_seq_len, float* scores_out, int32_t* idx_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Step 2 ([MGS §1 Step 2]): every head of group g attends over the tokens of the blocks in
 * idx[b][g][:] (entries < 0 or >= nb_b are skipped; entries must not repeat), split-K across
 * blocks with an online softmax, then a log-sum-exp merge.
 *   idx      [batch][Hkv][top_k] int32
 *   out      [batch][Hq][128] out_dtype
 *   lse_out  nullable [batch][Hq] float32 (natural log) */
msa_status msa_attend(const msa_config* cfg, const void* q, const msa_kv_cache* cache,
                      int32_t batch, int32_t max_seq_len, const int32_t* idx, void* out,
                      float* lse_out, void* workspace, size_t workspace_bytes, void* stream);

/* One decode step ([MGS §1 Steps 1-2]; [MGS §3] decode). If k_new is given, first write
 * k_new/v_new [batch][Hkv][128] into position seq_lens[b]-1 of each sequence (its page must
 * already be in block_table) and recompute that block's summary; a sequence of length 0 takes
 * no token, and a page id out of range is never written. Then Step 1 and Step 2, with that
 * block scored from its new summary.
 * idx_out / scores_out / lse_out are nullable. */
msa_status msa_decode_step(const msa_config* cfg, const void* q, const msa_kv_cache* cache,
                           int32_t batch, int32_t max_seq_len, const void* k_new,
                           const void* v_new, int32_t* idx_out, float* scores_out, void* out,
                           float* lse_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* msa_decode_step for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, kernels, results and
 * errors as msa_decode_step, without the workspace arguments: the workspace is a file-scope
 * device array of MSA_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one per GPU, held until
 * the process ends. A call whose msa_workspace_size(cfg, MSA_OP_DECODE, batch, max_seq_len, 0)
 * exceeds that size returns MSA_ERR_WORKSPACE and enqueues nothing (e.g. batch 32 at 1M tokens
 * and 8 KV heads needs about 17 MiB; batch 1 fits up to 16M tokens). The call allocates nothing;
 * its first call on a device looks up that device's copy of the array (no allocation, no
 * enqueued work), so make one call on each device before capturing it in a graph if the capture
 * mode forbids such lookups. All calls on one GPU share the array: calls that overlap in time on
 * one GPU (different streams, or concurrent host threads without ordering) race and must not be
 * made. Nothing in the array needs to start at zero: every byte a step reads is written earlier
 * in the same step. */
msa_status msa_decode_step_noalloc(const msa_config* cfg, const void* q, const msa_kv_cache* cache,
                                   int32_t batch, int32_t max_seq_len, const void* k_new,
                                   const void* v_new, int32_t* idx_out, float* scores_out,
                                   void* out, float* lse_out, void* stream);

/* One prefill chunk of one sequence ([MGS §1 Steps 1-2]; [MGS §3] prefill): append T new
 * tokens (k_new/v_new [T][Hkv][128]) at positions past_len .. past_len+T-1 (pages already in
 * block_table[0]; past_len % 64 == 0), recompute the new blocks' summaries, select per
 * 64-query tile and group the top-k among the blocks before the tile's diagonal block, append
 * the diagonal block, and run causal attention over the selection (bf16 only, MFMA).
 *   q          [T][Hq][128] bf16;  out [T][Hq][128] bf16;  lse_out nullable [T][Hq] float32
 *   idx_out    nullable [ceil(T/64)][Hkv][top_k+1] int32 (k_eff ascending ids, the diagonal
 *              block, then -1 padding)
 *   scores_out nullable [ceil(T/64)][Hkv][past_len/64 + ceil(T/64)] float32, -inf for
 *              non-candidates
 * cache->seq_lens is not read or written. A short chunk (fewer than 256 (tile, group) attend
 * workgroups) splits each tile's list over several workgroups and merges their partial softmax
 * states in a second launch; msa_workspace_size(MSA_OP_PREFILL) then includes T * Hq * splits
 * partials of 130 floats, and the outputs equal the unsplit ones up to fp32 summation order. */
msa_status msa_prefill_chunk(const msa_config* cfg, const void* q, const void* k_new,
                             const void* v_new, const msa_kv_cache* cache, int32_t past_len,
                             int32_t T, int32_t* idx_out, float* scores_out, void* out,
                             float* lse_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Step 2 of a prefill chunk alone ([MGS §1 Step 2]; [MGS §3] prefill: the savings fall on this
 * main attention): causal attention of the chunk's T queries (positions past_len ..
 * past_len+T-1 of one sequence) over given per-tile lists, with the chunk's own K/V already in
 * the cache (e.g. written by msa_prefill_chunk). For tile tau and group g, with diagonal block
 * d = past_len/64 + tau: block d is always attended, causally (key position <= query position);
 * list entries j with 0 <= j < d and a page id in [0, num_pages) are attended in full; every
 * other entry (-1, d itself, blocks after d) is skipped. Entries must not repeat.
 *   q        [T][Hq][128] bf16;  out [T][Hq][128] bf16;  lse_out nullable [T][Hq] float32
 *   idx      [ceil(T/64)][Hkv][top_k+1] int32 (the layout msa_prefill_chunk writes)
 * Only block_table[0], num_pages and the K/V pools of the cache are read. No workspace. */
msa_status msa_prefill_attend(const msa_config* cfg, const void* q, const msa_kv_cache* cache,
                              int32_t past_len, int32_t T, const int32_t* idx, void* out,
                              float* lse_out, void* stream);

/* Static text for a status code. */
const char* msa_status_string(msa_status status);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
