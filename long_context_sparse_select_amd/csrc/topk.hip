// Step 1 top-k: keep the k best blocks of every (sequence, group) -- or (tile, group) -- row.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 1: TopK keeps
// the k highest-scoring blocks for the layer and the group and hands Step 2 a short index list.
// Readings: order = score descending, then block index ascending (-0 == +0); k_eff =
// min(k, n); the list is written in ascending block order and padded with -1; in prefill the
// tile's diagonal block is appended after the k_eff entries.
//
// One 1024-thread workgroup per row. Scores are compared as order-preserving 32-bit keys.
//  1. The scoring kernel has already counted the row's keys in a 4096-bin histogram of their
//     top 12 bits. A suffix scan over it finds bin b1 holding the k_eff-th largest key
//     (the histogram row is cleared here for the next call).
//  2. One pass over the row collects A = keys in bins above b1 and B = keys in bin b1 into LDS,
//     counting both exactly. If |A| < k_eff <= |A| + |B| and B fits in LDS, the answer is A plus
//     the k_eff - |A| best of B (ranked in LDS by the full order) -- correct whatever the
//     histogram said, because the counts are exact. Otherwise (a stale histogram, or very many
//     ties) an exact fallback finds the k_eff-th key by a bitwise search over the key space and
//     emits the selection with an ordered compaction.
//  3. The k_eff kept indices are sorted ascending by counting in LDS.
// The output is deterministic: it depends only on the scores.
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCapB = 2048;
constexpr int kMaxK = 4096;

// block-wide integer sum (all threads get it); s_tmp holds kWaves ints
__device__ int block_sum(int v, int* s_tmp) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) total += s_tmp[w];
  __syncthreads();
  return total;
}

// exclusive count of `pred` over threads in index order; *total gets the block's count
__device__ int block_excl_count(bool pred, int* s_tmp, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long m = __ballot(pred);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_tmp[wave] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = s_tmp[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

__global__ void __launch_bounds__(kThreads) k_topk(TopkArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ int32_t s_sel[kMaxK];
  __shared__ uint32_t s_bkey[kCapB];
  __shared__ int32_t s_bidx[kCapB];
  __shared__ int s_tmp[kWaves];
  __shared__ int s_b1, s_above, s_cntA, s_cntB;

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const bool prefill = a.lens == nullptr;
  int n;
  if (!prefill) {
    const int N = clamp_len(a.lens[row / a.Hkv], a.max_len);
    n = (N + kP - 1) / kP;
  } else {
    n = a.base_blocks + row / a.Hkv;
  }
  const int keff = min(a.k, n);
  const float* srow = a.scores + (long long)row * a.row_stride;
  int32_t* out = a.idx + (long long)row * a.idx_stride;
  uint32_t* grow = a.hist + (long long)row * kHistBins;

  for (int i = tid; i < kHistBins; i += kThreads) {
    s_hist[i] = grow[i];
    grow[i] = 0u;
  }
  if (tid == 0) { s_b1 = -1; s_above = 0; s_cntA = 0; s_cntB = 0; }
  __syncthreads();

  if (keff == n) {  // every candidate is kept
    for (int i = tid; i < a.idx_stride; i += kThreads) out[i] = i < n ? i : ((prefill && i == n) ? n : -1);
    return;
  }

  // ---- 1. bin of the k_eff-th largest key: thread t owns bins 4t .. 4t+3
  {
    const uint32_t c0 = s_hist[4 * tid], c1 = s_hist[4 * tid + 1], c2 = s_hist[4 * tid + 2], c3 = s_hist[4 * tid + 3];
    const uint32_t local = c0 + c1 + c2 + c3;
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t incl = local;  // inclusive suffix sum within the wave
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(incl, off);
      if (lane + off < 64) incl += y;
    }
    if (lane == 0) s_tmp[wave] = (int)incl;
    __syncthreads();
    uint32_t above = incl - local;
    for (int w = wave + 1; w < kWaves; ++w) above += (uint32_t)s_tmp[w];
    const uint32_t c[4] = {c0, c1, c2, c3};
    uint32_t run = above;
    for (int i = 3; i >= 0; --i) {
      if (run < (uint32_t)keff && run + c[i] >= (uint32_t)keff) { s_b1 = 4 * tid + i; s_above = (int)run; }
      run += c[i];
    }
  }
  __syncthreads();

  // ---- 2. one pass over the row
  const int b1 = s_b1;
  if (b1 >= 0) {
    for (int j = tid; j < n; j += kThreads) {
      const uint32_t key = order_key(srow[j]);
      const int bin = (int)(key >> (32 - kHistBits));
      if (bin > b1) {
        const int p = atomicAdd(&s_cntA, 1);
        if (p < keff) s_sel[p] = j;
      } else if (bin == b1) {
        const int p = atomicAdd(&s_cntB, 1);
        if (p < kCapB) { s_bkey[p] = key; s_bidx[p] = j; }
      }
    }
  }
  __syncthreads();
  const int cntA = s_cntA, cntB = s_cntB;
  const bool fast = b1 >= 0 && cntA < keff && cntA + cntB >= keff && cntB <= kCapB;

  if (fast) {
    const int need = keff - cntA;
    for (int e = tid; e < cntB; e += kThreads) {
      const uint32_t ke = s_bkey[e];
      const int je = s_bidx[e];
      int rank = 0;
      for (int f = 0; f < cntB; ++f) {
        const uint32_t kf = s_bkey[f];
        rank += (kf > ke) || (kf == ke && s_bidx[f] < je);
      }
      if (rank < need) s_sel[cntA + rank] = je;
    }
    __syncthreads();
    for (int e = tid; e < keff; e += kThreads) {
      const int v = s_sel[e];
      int pos = 0;
      for (int f = 0; f < keff; ++f) pos += s_sel[f] < v;
      out[pos] = v;
    }
  } else {
    // ---- exact fallback: T = largest key with count(key >= T) >= k_eff
    uint32_t T = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int c = 0;
      for (int j = tid; j < n; j += kThreads) c += order_key(srow[j]) >= cand;
      if (block_sum(c, s_tmp) >= keff) T = cand;
    }
    int gt = 0;
    for (int j = tid; j < n; j += kThreads) gt += order_key(srow[j]) > T;
    const int need_eq = keff - block_sum(gt, s_tmp);
    int run_eq = 0, run_sel = 0;
    for (int base = 0; base < n; base += kThreads) {
      const int j = base + tid;
      const uint32_t key = j < n ? order_key(srow[j]) : 0u;
      const bool is_gt = j < n && key > T;
      const bool is_eq = j < n && key == T;
      int tot_eq, tot_sel;
      const int eq_rank = run_eq + block_excl_count(is_eq, s_tmp, &tot_eq);
      const bool sel = is_gt || (is_eq && eq_rank < need_eq);
      const int pos = run_sel + block_excl_count(sel, s_tmp, &tot_sel);
      if (sel) out[pos] = j;
      run_eq += tot_eq;
      run_sel += tot_sel;
    }
  }
  for (int i = keff + tid; i < a.idx_stride; i += kThreads) out[i] = (prefill && i == keff) ? n : -1;
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  k_topk<<<a.rows, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
