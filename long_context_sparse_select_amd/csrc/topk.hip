// Step 1 top-k: keep the k best blocks of every (sequence, group) -- or (tile, group) -- row.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 1: TopK keeps
// the k highest-scoring blocks for the layer and the group and hands Step 2 a short index list.
// Readings: order = score descending, then block index ascending (-0 == +0); k_eff =
// min(k, n); the list is written in ascending block order and padded with -1; in prefill the
// tile's diagonal block is appended after the k_eff entries.
//
// One workgroup per row (1024 threads, or 512 for short rows); scores are compared as
// order-preserving 32-bit keys. Rows of up to 16 candidates per thread are held in registers
// (j = tid + NT i):
//  1. each thread's maximum is a group maximum; any value with k_eff group maxima at or above
//     it is a lower bound T0 of the k_eff-th largest key (each of those groups holds a key
//     >= T0). A 256-bin histogram of the group maxima -- linear in the score value between the
//     smallest and largest finite maximum, or linear in the key where that range is unusable --
//     finds the bin where the count from the top reaches k_eff; T0 = that bin's lower edge (less
//     a margin for the float binning), so >= k_eff keys are >= T0 -- whatever the data. Every
//     wave reads the bin off the histogram itself, so the bound costs two barriers;
//  2. the survivors (keys >= T0; typically a little over k) are gathered in LDS and ranked
//     exactly by (key desc, index asc); ranks < k_eff are kept;
//  3. the kept indices are sorted ascending by counting.
// Longer rows, or rows where too many keys tie at T0, take an exact fallback: a bitwise search
// for the k_eff-th key over the row in memory, then an ordered compaction.
// Decode rows also get each kept block's page id (for the attend kernel). The output depends
// only on the scores.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace msa {

namespace {

constexpr int kThreads = 1024;          // the largest workgroup (rows up to 16384 candidates)
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 16;                // candidates held per thread
constexpr int kCap = 2048;
constexpr int kBins = 256;
constexpr int kMaxK = 4096;
constexpr int kSmallK = 256;    // k_eff up to this uses the survivor path; larger k the exact select
constexpr int kRowRank = 512;   // survivors ranked 16 lanes each up to this count
constexpr int kLBins = 1024;    // bins per pass of the exact select
constexpr int kBinKeys = 512;   // exact select: a chosen bin of at most this many keys is finished in LDS

struct TopkShared {
  union {                             // one of the two per row, never both live
    unsigned long long comp[kCap + 2];  // survivors: (key << 32) | ~index, larger = better
    uint32_t bkeys[kBinKeys];           // exact select: the chosen bin's keys
  };
  int32_t sel[kMaxK + 4];
  int32_t selpg[kMaxK];
  uint32_t hist[kBins];
  uint32_t hbig[kLBins];             // exact select: histogram of the current key range
  int pre[kPer * kWaves];            // exact select: per (slot, wave) counts, then their prefixes
  uint32_t range[3];                 // exact select: lo, hi, keys above hi
  uint32_t red[3 * kWaves];
  int tmp[kWaves];
  int cnt;
};

__device__ __forceinline__ uint32_t select_key(const TopkArgs& a, int j, int n, float s) {
  return forced_or_key(j, n, a.keep_sink, a.keep_local, s);
}

__device__ __forceinline__ int page_of(const TopkArgs& a, int row, int j) {
  const int p = a.table[(long long)(row / a.Hkv) * a.max_blocks + j];
  return page_ok(p, a.num_pages) ? p : -1;
}

__device__ __forceinline__ void emit(const TopkArgs& a, int row, int pos, int j) {
  a.idx[(long long)row * a.idx_stride + pos] = j;
  if (a.pages != nullptr) a.pages[(long long)row * a.k + pos] = page_of(a, row, j);
}

template <int NT>
__device__ __forceinline__ void pad(const TopkArgs& a, int row, int keff, int n, bool prefill) {
  for (int i = keff + threadIdx.x; i < a.idx_stride; i += NT) {
    a.idx[(long long)row * a.idx_stride + i] = (prefill && i == keff) ? n : -1;
    if (a.pages != nullptr && i < a.k) a.pages[(long long)row * a.k + i] = -1;
  }
}

// exact selection straight from memory: T = k_eff-th largest key, then ordered compaction
template <int NT>
__device__ void select_fallback(const TopkArgs& a, const float* srow, int row, int n, int keff, TopkShared& sh) {
  const int tid = threadIdx.x;
  auto key_of = [&](int j) { return select_key(a, j, n, srow[j]); };
  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
    for (int j = tid; j < n; j += NT) c += key_of(j) >= cand;
    if (block_sum<NT>(c, sh.tmp) >= keff) T = cand;
  }
  int gt = 0;
  for (int j = tid; j < n; j += NT) gt += key_of(j) > T;
  const int need_eq = keff - block_sum<NT>(gt, sh.tmp);
  int run_eq = 0, run_sel = 0;
  for (int base = 0; base < n; base += NT) {
    const int j = base + tid;
    const uint32_t key = j < n ? key_of(j) : 0u;
    const bool is_gt = j < n && key > T;
    const bool is_eq = j < n && key == T;
    int tot_eq, tot_sel;
    const int eq_rank = run_eq + block_excl_count<NT>(is_eq, sh.tmp, &tot_eq);
    const bool sel = is_gt || (is_eq && eq_rank < need_eq);
    const int pos = run_sel + block_excl_count<NT>(sel, sh.tmp, &tot_sel);
    if (sel) emit(a, row, pos, j);
    run_eq += tot_eq;
    run_sel += tot_sel;
  }
}

// Exclusive prefixes, in ascending block order, of two predicates at once (slot i of thread t
// holds block t + NT*i, so the order is slot-major, then wave, then lane): per-(slot, wave) counts
// packed as (count of a) << 16 | (count of b) and scanned together (each total is at most 16,384,
// so neither half carries into the other). Two barriers.
template <int NT>
__device__ __forceinline__ void ordered_prefix_pair(const bool (&pa)[kPer], const bool (&pb)[kPer], int (&ra)[kPer],
                                                    int (&rb)[kPer], TopkShared& sh) {
  constexpr int kW = NT / 64, kE = kPer * kW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long ba[kPer], bb[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    ba[i] = __ballot(pa[i]);
    bb[i] = __ballot(pb[i]);
    if (lane == 0) sh.pre[i * kW + wave] = (__popcll(ba[i]) << 16) | __popcll(bb[i]);
  }
  __syncthreads();
  if (wave == 0) {
    int v[4], sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = 4 * lane + e < kE ? sh.pre[4 * lane + e] : 0; sum += v[e]; }
    int incl = sum;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int run = incl - sum;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * lane + e < kE) sh.pre[4 * lane + e] = run;
      run += v[e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pre = sh.pre[i * kW + wave];
    ra[i] = (pre >> 16) + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(ba[i] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ba[i], 0u));
    rb[i] = (pre & 0xffff) + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bb[i] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bb[i], 0u));
  }
}

// Bin of a key on a linear score scale from vlo (bins of 1/vscale): monotone in the key, with
// every key above +inf's (NaN payloads, the forced key) in the top bin and NaN below -inf in bin 0.
__device__ __forceinline__ uint32_t value_bin(uint32_t k, float vlo, float vscale) {
  const float t = (key_value(k) - vlo) * vscale;
  return k > kPosInfKey ? (uint32_t)(kLBins - 1) : (uint32_t)fminf(fmaxf(t, 0.f), (float)(kLBins - 1));
}

// Exact selection for large k on keys held in registers (slot i of thread t = block t + NT*i):
//  1. the k_eff-th largest key T by range refinement: a 1024-bin histogram of the keys in
//     [lo, hi], the bin where the count from the top reaches k_eff becomes the next range (a
//     32-bit key range takes at most 4 passes). The first pass bins score values linearly
//     instead of keys: order keys of typical scores bunch into a sliver of the key range, so a
//     key-linear first pass piles thousands of LDS atomics onto a few bins and leaves most keys
//     in the chosen one. A chosen value bin of at most kBinKeys keys (typically a few dozen) is
//     gathered into LDS and T is the key there with fewer than r = k_eff - (keys above the bin)
//     larger keys and at least r at or above it, one thread per key; a fuller bin is mapped back
//     to its exact key range by a min / max over the keys that fall in it and refined;
//  2. ordered compaction: keys > T, then the ties == T with the smallest block indices, written
//     at their rank in ascending block order (no sort needed); one prefix pass counts both.
template <int NT>
__device__ void select_large(const TopkArgs& a, int row, int n, int keff, const uint32_t (&key)[kPer],
                             const int32_t* trow, TopkShared& sh) {
  constexpr int kW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool valid[kPer];
  uint32_t kmx = 0u, kmn = 0xffffffffu, kfin = 0u;   // kfin: the largest key at or below +inf's
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    valid[i] = tid + NT * i < n;
    if (valid[i]) {
      kmx = max(kmx, key[i]);
      kmn = min(kmn, key[i]);
      if (key[i] <= kPosInfKey) kfin = max(kfin, key[i]);
    }
  }
  kmx = wave_max_u32(kmx);
  kmn = wave_min_u32(kmn);
  kfin = wave_max_u32(kfin);
  if (lane == 0) { sh.red[wave] = kmx; sh.red[kW + wave] = kmn; sh.red[2 * kW + wave] = kfin; }
  __syncthreads();
  uint32_t lo = 0xffffffffu, hi = 0u, fin = 0u, above = 0u;
#pragma unroll
  for (int w = 0; w < kW; ++w) {   // every thread reads the wave results (no second barrier)
    hi = max(hi, sh.red[w]);
    lo = min(lo, sh.red[kW + w]);
    fin = max(fin, sh.red[2 * kW + w]);
  }
  bool done = false;   // T (lo == hi) and `above` found through the chosen bin's keys in LDS
  const float vlo = key_value(lo), vfin = key_value(fin);
  if (lo != hi && fin > lo && isfinite(vlo) && isfinite(vfin) && vfin > vlo) {   // uniform
    // ---- first pass on a score scale from the smallest key to the largest finite one
    const float vscale = (float)kLBins / (vfin - vlo);
    for (int b = tid; b < kLBins; b += NT) sh.hbig[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (valid[i]) atomicAdd(&sh.hbig[value_bin(key[i], vlo, vscale)], 1u);
    __syncthreads();
    if (wave == 0) {   // lane l owns bins 16l .. 16l+15; counts from the top
      uint32_t c[16], local = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) { c[e] = sh.hbig[16 * lane + e]; local += c[e]; }
      uint32_t incl = local;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_down((int)incl, off);
        if (lane + off < 64) incl += y;
      }
      uint32_t run = incl - local;
      for (int e = 15; e >= 0; --e) {
        if (run < (uint32_t)keff && run + c[e] >= (uint32_t)keff) {
          sh.range[0] = 16 * lane + e; sh.range[1] = c[e]; sh.range[2] = run;
        }
        run += c[e];
      }
      if (lane == 0) sh.cnt = 0;
    }
    __syncthreads();
    // ---- exact key range of the chosen bin: every key in it lies in [min, max] of its keys, and
    // (the binning being monotone) every key in that interval is in it; keys above are `above`
    const uint32_t bsel = sh.range[0];
    const int mbin = (int)sh.range[1];
    above = sh.range[2];
    if (mbin <= kBinKeys) {   // uniform: the bin's keys to LDS, then the (keff - above)-th of them
      uint32_t* bk = sh.bkeys;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const bool inb = valid[i] && value_bin(key[i], vlo, vscale) == bsel;
        const unsigned long long bm = __ballot(inb);
        if (bm != 0ull) {   // wave-uniform
          int base = 0;
          if (lane == 0) base = atomicAdd(&sh.cnt, __popcll(bm));
          base = __builtin_amdgcn_readfirstlane(base);
          const int at = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
          if (inb && at < kBinKeys) bk[at] = key[i];   // at < mbin: the histogram's own bin test
        }
      }
      __syncthreads();
      // T is the bin key x with (keys > x) < r <= (keys >= x), r = keff - above (1 <= r <= mbin)
      const int r = keff - (int)above;
      for (int t = tid; t < mbin; t += NT) {
        const uint32_t x = bk[t];
        int gt = 0, ge = 0;
        for (int u = 0; u < mbin; ++u) {   // the same address across the wave: broadcast reads
          const uint32_t y = bk[u];
          gt += y > x;
          ge += y >= x;
        }
        if (gt < r && r <= ge) { sh.range[0] = x; sh.range[2] = above + (uint32_t)gt; }   // equal writes
      }
      __syncthreads();
      lo = hi = sh.range[0];
      above = sh.range[2];
      done = true;
    } else {   // the exact key range of the bin, refined below
      uint32_t bmx = 0u, bmn = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (valid[i] && value_bin(key[i], vlo, vscale) == bsel) { bmx = max(bmx, key[i]); bmn = min(bmn, key[i]); }
      bmx = wave_max_u32(bmx);
      bmn = wave_min_u32(bmn);
      if (lane == 0) { sh.red[wave] = bmx; sh.red[kW + wave] = bmn; }
      __syncthreads();
      lo = 0xffffffffu; hi = 0u;
#pragma unroll
      for (int w = 0; w < kW; ++w) { hi = max(hi, sh.red[w]); lo = min(lo, sh.red[kW + w]); }
    }
  }
  while (!done && lo != hi) {   // uniform
    for (int b = tid; b < kLBins; b += NT) sh.hbig[b] = 0u;
    __syncthreads();
    const unsigned long long span = (unsigned long long)(hi - lo) + 1ull;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (valid[i] && key[i] >= lo && key[i] <= hi)
        atomicAdd(&sh.hbig[(uint32_t)(((unsigned long long)(key[i] - lo) * kLBins) / span)], 1u);
    __syncthreads();
    if (wave == 0) {   // lane l owns bins 16l .. 16l+15; counts from the top
      uint32_t c[16], local = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) { c[e] = sh.hbig[16 * lane + e]; local += c[e]; }
      uint32_t incl = local;  // suffix sum over lanes >= lane
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_down((int)incl, off);
        if (lane + off < 64) incl += y;
      }
      uint32_t run = above + incl - local;   // keys above this lane's bins
      for (int e = 15; e >= 0; --e) {
        if (run < (uint32_t)keff && run + c[e] >= (uint32_t)keff) {
          const unsigned long long bsel = 16ull * lane + e;
          // bin b holds keys lo + [ceil(b*span/1024), ceil((b+1)*span/1024) - 1]
          sh.range[0] = lo + (uint32_t)((bsel * span + kLBins - 1) / kLBins);
          sh.range[1] = lo + (uint32_t)(((bsel + 1) * span + kLBins - 1) / kLBins) - 1u;
          sh.range[2] = run;
        }
        run += c[e];
      }
    }
    __syncthreads();
    lo = sh.range[0]; hi = sh.range[1]; above = sh.range[2];
  }
  const uint32_t T = lo;
  const int need_eq = keff - (int)above;   // >= 1 ties at T are kept, smallest block indices first
  // one ordered prefix of (keys > T, keys == T): a kept key's position is the keys > T before it
  // plus the kept ties before it, min(ties before it, need_eq); a tie is kept while its own rank
  // among the ties is below need_eq
  bool gt[kPer], eq[kPer];
  int rg[kPer], re[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    gt[i] = valid[i] && key[i] > T;
    eq[i] = valid[i] && key[i] == T;
  }
  int pg[kPer];   // decode: the candidates' page ids (ties that stay out included), loaded under the prefix
  if (trow != nullptr) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) pg[i] = gt[i] || eq[i] ? trow[tid + NT * i] : -1;
  }
  ordered_prefix_pair<NT>(gt, eq, rg, re, sh);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (gt[i] || (eq[i] && re[i] < need_eq)) {
      const int pos = rg[i] + min(re[i], need_eq);
      a.idx[(long long)row * a.idx_stride + pos] = tid + NT * i;
      if (trow != nullptr) a.pages[(long long)row * a.k + pos] = page_ok(pg[i], a.num_pages) ? pg[i] : -1;
    }
  }
}

// NT threads: 512 or 1024
template <int NT>
__global__ void __launch_bounds__(NT) k_topk(TopkArgs a) {
  constexpr int kW = NT / 64;
  constexpr int kMaxFast = NT * kPer;
  __shared__ TopkShared sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool prefill = a.lens == nullptr;
  const int len_raw = prefill ? 0 : a.lens[row / a.Hkv];
  float* srow = a.scores + (long long)row * a.row_stride;
  // the row's score loads go first, in flight with the length load: addresses are clamped to the
  // row stride (every row holds row_stride scores), so they wait for nothing; entries past the
  // row's length are masked when used. Page ids (decode) are read later, for kept blocks only:
  // the row's loads are what one CU must pull in before anything else can start.
  float v[kPer];
  const int32_t* trow = a.pages != nullptr ? a.table + (long long)(row / a.Hkv) * a.max_blocks : nullptr;
  const int rs_last = a.row_stride - 1;
  if (rs_last >= 0) {   // uniform
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = srow[min(tid + NT * i, rs_last)];
  }
  const int n = prefill ? a.base_blocks + row / a.Hkv : (clamp_len(len_raw, a.max_len) + kP - 1) / kP;
  const int keff = min(a.k, n);
  const int ngroups = min(n, NT);     // threads holding at least one candidate
  // With one candidate per thread (n <= NT) the group maxima are the candidates and the bound is
  // exact. With several, it prunes well while k_eff is at most a quarter of the groups (a 2048-
  // candidate row on 512 threads with k = 256 ran 53.5 us per 128k-token step through the
  // bound, 40.4 us through the exact select)
  const bool fast = n <= kMaxFast && keff < n && keff <= ngroups && (n <= NT || 4 * keff <= ngroups) &&
                    keff <= kSmallK;   // uniform
  if (!fast) {   // every candidate kept, or the exact path
    if (keff == n) {
      for (int i = tid; i < n; i += NT) emit(a, row, i, i);
    } else if (n <= kMaxFast) {   // large k: exact select on the keys in registers
      uint32_t key[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int j = tid + NT * i;
        key[i] = j < n ? select_key(a, j, n, v[i]) : 0u;
      }
      select_large<NT>(a, row, n, keff, key, trow, sh);
    } else {
      select_fallback<NT>(a, srow, row, n, keff, sh);
    }
    pad<NT>(a, row, keff, n, prefill);
    return;
  }

  // ---- fast path
  uint32_t key[kPer];
  uint32_t cm = 0u;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tid + NT * i;
    key[i] = j < n ? select_key(a, j, n, v[i]) : 0u;
    cm = max(cm, key[i]);
  }
  const bool has = tid < ngroups;
  if (tid == 0) sh.cnt = 0;
  // ---- 1. range of the group maxima: smallest, largest, and largest at or below +inf's key
  const uint32_t wmx = wave_max_u32(has ? cm : 0u), wmn = wave_min_u32(has ? cm : 0xffffffffu);
  const uint32_t wfin = wave_max_u32(has && cm <= kPosInfKey ? cm : 0u);
  if (lane == 0) { sh.red[wave] = wmx; sh.red[kW + wave] = wmn; sh.red[2 * kW + wave] = wfin; }
  if (tid < kBins) sh.hist[tid] = 0u;
  __syncthreads();
  uint32_t mx = 0u, mn = 0xffffffffu, fin = 0u;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    mx = max(mx, sh.red[w]);
    mn = min(mn, sh.red[kW + w]);
    fin = max(fin, sh.red[2 * kW + w]);
  }
  // Binning of the group maxima. Preferred: linear in the score value over [vlo, vfin] (order keys
  // of ordinary scores bunch into a sliver of the key range, so key-linear bins are coarse where
  // the k_eff-th maximum sits). Keys above +inf's (forced blocks, NaN payloads) go to the top bin.
  // Used only when the value range is finite and wide against the values' own magnitude (2^-12),
  // which keeps the float edge below safely under every key of the chosen bin. Otherwise
  // key-linear: bin(d) = min(floor(fl(fl(d) * bscale)), kBins - 1) for d = key - mn.
  const float vlo = key_value(mn), vfin = key_value(fin);
  const bool by_value = fin > mn && isfinite(vlo) && isfinite(vfin) &&
                        (vfin - vlo) > 0x1p-12f * fmaxf(fabsf(vlo), fabsf(vfin));   // uniform
  const float vscale = by_value ? (float)kBins / (vfin - vlo) : 0.f;
  const float bscale = (float)kBins / ((float)(mx - mn) + 1.0f);
  if (has) {
    uint32_t bin;
    if (by_value) {
      const float t = (key_value(cm) - vlo) * vscale;
      bin = cm > kPosInfKey ? (uint32_t)(kBins - 1) : (uint32_t)fminf(fmaxf(t, 0.f), (float)(kBins - 1));
    } else {
      bin = min((uint32_t)((float)(cm - mn) * bscale), (uint32_t)(kBins - 1));
    }
    atomicAdd(&sh.hist[bin], 1u);
  }
  __syncthreads();
  // ---- bin bstar holding the k_eff-th largest group maximum, found by every wave (no barrier):
  // lane l owns bins 4l..4l+3; bin 0 would keep every group maximum, the fallback
  uint32_t bstar;
  {
    const uint4 c4 = reinterpret_cast<const uint4*>(sh.hist)[lane];
    const uint32_t local = c4.x + c4.y + c4.z + c4.w;
    uint32_t incl = local;  // suffix sum over lanes >= lane
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = (uint32_t)__shfl_down((int)incl, off);
      if (lane + off < 64) incl += y;
    }
    uint32_t run = incl - local, mine = 0u;
    const uint32_t cc[4] = {c4.x, c4.y, c4.z, c4.w};
    for (int i = 3; i >= 0; --i) {
      if (run < (uint32_t)keff && run + cc[i] >= (uint32_t)keff) mine = 4 * lane + i;
      run += cc[i];
    }
    bstar = wave_max_u32(mine);
  }
  // ---- T0 = a key at or below every key of bins >= bstar. Those bins hold >= k_eff group maxima,
  // so at least k_eff keys are >= T0.
  //  * value bins: bin(v) >= bstar needs (v - vlo) * vscale >= bstar up to a few float roundings
  //    (relative 2^-22), so v >= vlo + (bstar - 1/2) / vscale with ~half a bin to spare, which
  //    covers the rounding of that edge itself (the range is >= 2^11 ulps of the values);
  //  * key bins: bin(d) >= bstar needs d * bscale * (1 + 2^-24)^2 >= bstar, i.e.
  //    d >= bstar / bscale - 512 (d < 2^32); T0 sits 513 below that.
  uint32_t T0 = mn;
  if (bstar > 0u) {   // uniform
    if (by_value) {
      T0 = max(mn, order_key(vlo + ((float)bstar - 0.5f) / vscale));
    } else {
      const double q = floor((double)bstar / (double)bscale) - 513.0;
      if (q > 0.0) T0 = mn + (uint32_t)q;
    }
  }
  // ---- 2. survivors (keys >= T0) as (key, ~index) composites
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tid + NT * i;
    if (j < n && key[i] >= T0) {
      const int p = atomicAdd(&sh.cnt, 1);
      if (p < kCap) sh.comp[p] = ((unsigned long long)key[i] << 32) | (uint32_t)(~(uint32_t)j);
    }
  }
  __syncthreads();
  const int m = sh.cnt;
  bool done = false;
  if (m >= keff && m <= kCap) {   // uniform; m >= k_eff holds by construction of T0
    // ---- rank of each survivor by (key desc, index asc) = the number of larger composites.
    // Up to kRowRank survivors: 16 lanes (one DPP row) per survivor, each lane counting over
    // every 16th composite, so a row's reads are one contiguous 128 B run; beyond that, one
    // thread per survivor. A kept survivor's page id is read while it is ranked.
    const int part = tid & 15;
    if (m <= kRowRank) {   // uniform
      for (int e = tid >> 4; e < m; e += NT / 16) {   // uniform per 16-lane row
        const unsigned long long ce = sh.comp[e];
        const int je = (int)~(uint32_t)ce;
        const int pge = (trow != nullptr && part == 0) ? trow[je] : -1;
        int c = 0;
        for (int f = part; f < m; f += 16) c += sh.comp[f] > ce;
        const int rank = (int)row16_sum((float)c);   // counts < 2^24: exact
        if (part == 0 && rank < keff) { sh.sel[rank] = je; sh.selpg[rank] = page_ok(pge, a.num_pages) ? pge : -1; }
      }
    } else {
      const int npair = (m + 1) >> 1;
      const ulonglong2* cp = reinterpret_cast<const ulonglong2*>(sh.comp);
      for (int e = tid; e < m; e += NT) {
        const unsigned long long ce = sh.comp[e];
        const int je = (int)~(uint32_t)ce;
        const int pge = trow != nullptr ? trow[je] : -1;
        int rank = 0;
#pragma unroll 4
        for (int f = 0; f < npair; ++f) {
          const ulonglong2 c2 = cp[f];
          rank += (c2.x > ce) + (2 * f + 1 < m && c2.y > ce);   // comp[m] is not a survivor
        }
        if (rank < keff) { sh.sel[rank] = je; sh.selpg[rank] = page_ok(pge, a.num_pages) ? pge : -1; }
      }
    }
    __syncthreads();
    // ---- 3. ascending block order: position = kept blocks with a smaller index (16 lanes each)
    for (int e = tid >> 4; e < keff; e += NT / 16) {   // uniform per 16-lane row
      const int vj = sh.sel[e];
      int c = 0;
      for (int f = part; f < keff; f += 16) c += sh.sel[f] < vj;
      const int pos = (int)row16_sum((float)c);
      if (part == 0) {
        a.idx[(long long)row * a.idx_stride + pos] = vj;
        if (a.pages != nullptr) a.pages[(long long)row * a.k + pos] = sh.selpg[e];
      }
    }
    done = true;
  }
  if (!done) select_large<NT>(a, row, n, keff, key, trow, sh);   // mass ties at T0
  pad<NT>(a, row, keff, n, prefill);
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  // rows of at most 512 * kPer candidates and k <= 512 run on 512 threads (two workgroups fit a
  // CU); longer rows or larger k on 1024
  const bool prefill = a.lens == nullptr;
  const long long n_max = prefill ? (long long)a.base_blocks + (a.rows - 1) / a.Hkv : ((long long)a.max_len + kP - 1) / kP;
  const int nt = n_max <= 512 * kPer && a.k <= 512 ? 512 : kThreads;
  if (log_enabled())
    log_launch("k_topk", dim3(a.rows), nt, 0, "%d threads; k=%d, row length up to %lld%s", nt, a.k, n_max,
               prefill ? ", prefill rows" : "");
  if (nt == 512) k_topk<512><<<a.rows, 512, 0, st>>>(a);
  else k_topk<kThreads><<<a.rows, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
