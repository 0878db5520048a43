// Decode Step 1's TopK and Step 2 in one launch, on the chip's attend workgroups.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 1: TopK keeps
// each group's k best blocks and hands Step 2 a short index list; §1 Step 2: every head of the
// group attends over the real K/V of those blocks only; §3: decode time is bound by the K/V the
// step reads. Readings: order = score descending, then block index ascending (-0 == +0);
// k_eff = min(k, n); the list is ascending and padded with -1.
//
// A top-k of a row on one workgroup is a serial chain of loads and barriers that leaves the
// rest of the chip idle, then hands over to the attend through another launch. Here every
// attend workgroup of a (sequence, group) row finds the row's exact top-k itself, from what the
// scoring launch left: the row's scores and its run maxima (the largest score of each run of
// 8 blocks, kMaxRun; "chunks" below). Grid (split, group, sequence), 256 threads:
//   1. the <= 2048 chunk maxima of the row (8 per thread): a 256-bin histogram of them, linear in
//      score value, gives T0 = the lower edge of the bin where the count from the top reaches
//      k_eff (less half a bin against float rounding). At least k_eff chunk maxima are >= T0, and
//      each is the score of a block, so the k_eff-th largest score is >= T0 and every kept block
//      lies in a chunk whose maximum is >= T0 (a survivor chunk). The sequence's last chunk is
//      always a survivor (with a new token, its last block's score comes from the append and is
//      not in that chunk's recorded maximum);
//   2. the scores of the survivor chunks (typically ~k chunks, 32 B each) that are >= T0 are the
//      candidates (>= k_eff of them, every tie of the k_eff-th score among them); each is ranked
//      exactly by (key desc, index asc) against the others (a quad of lanes per candidate); ranks
//      < k_eff are kept and placed in ascending block order by counting. Forced sink / local
//      blocks (the FORCED instance) take a key above every score, and so does the maximum of each
//      chunk that holds one, so the bound keeps them. A candidate's page id is
//      read in the same round trip as its score, so the attend's K/V loads follow directly;
//   3. the workgroup attends the kept blocks of ranks [split * bps, (split + 1) * bps) with the
//      MFMA attend of attend_mfma.h, and writes the output (one split) or its split partial for
//      k_merge. With those blocks' K/V loads in flight, each kept block's position in ascending
//      order (the number of kept blocks with a smaller index) is counted, and the blocks whose
//      positions fall in the same range are written to the index list: the ordering is off the
//      path to the first load.
// Rows whose survivors or candidates overflow the LDS lists (mass ties, or too few chunks for
// the bound to prune: the host fuses k > 64 only for rows of at least 2k runs) take an exact
// path: a bitwise search for the k_eff-th key over the row's scores, then an ordered compaction.
// Reading the row per workgroup is redundant across a row's splits, but it is ~10 KiB of L2 hits
// per workgroup instead of a launch and a 64 KiB single-CU round trip.
#include "common.h"
#include "kernels.h"
#include "select.h"
#include "attend_mfma.h"

namespace msa {

namespace {

constexpr int kFT = 256;                 // threads per workgroup
constexpr int kFW = kFT / 64;            // waves
constexpr int kMaxFusedRuns = kMaxFusedChunks * kScoreChunk / kMaxRun;   // 2048
constexpr int kFBins = 256;
constexpr int kSurvCap = 1024;           // survivor runs held
static_assert(kFT % kScoreChunk == 0 && kMaxFusedRuns % kFT == 0, "chunks per thread and per round");
// candidates ranked: a row with fewer chunks than k_eff has no chunk-maximum bound, and all its
// n < kMaxRun * k_eff scores are candidates, which this holds for k_eff <= 64; with at least
// 2 k_eff runs the bound leaves ~k_eff .. 2 k_eff candidates; more take the exact path
constexpr int kCandCap = 1024;
constexpr int kRounds = 8;               // survivor-chunk rounds (16 chunks each) with loads in flight

struct SelectShared {
  unsigned long long comp[kCandCap];     // candidates: (key << 32) | ~index, larger = better
  int comppg[kCandCap];                  // ... and their page ids
  alignas(16) int sel[kMaxFusedTopK];    // kept blocks by rank
  int selpg[kMaxFusedTopK];              // ... and their page ids
  int sorted[kMaxFusedTopK];             // kept blocks in ascending order
  int sortedpg[kMaxFusedTopK];           // ... and their page ids
  int surv[kSurvCap];
  alignas(16) uint32_t hist[kFBins];
  uint32_t red[3 * kFW];
  int tmp[kFW];
  int nsurv, ncand;
};

// Inclusive prefix sum over the 64 lanes of a wave (lane 0 first): Hillis-Steele steps on DPP
// row shifts inside each 16-lane row, then the totals of the rows below through readlane.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Exact selection straight from the row's scores (mass ties): T = the k_eff-th largest key by a
// bitwise search, then the keys > T and the first ties == T, in ascending order, into sh.sorted.
template <bool FORCED>
__device__ __forceinline__ void select_exact(const float* srow, const int32_t* trow, int n, int keff, int sink,
                                             int local, SelectShared& sh) {
  auto key_of = [&](int j) { return FORCED ? forced_or_key(j, n, sink, local, srow[j]) : order_key(srow[j]); };
  const int tid = threadIdx.x;
  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
    for (int j = tid; j < n; j += kFT) c += key_of(j) >= cand;
    if (block_sum<kFT>(c, sh.tmp) >= keff) T = cand;
  }
  int gt = 0;
  for (int j = tid; j < n; j += kFT) gt += key_of(j) > T;
  const int need_eq = keff - block_sum<kFT>(gt, sh.tmp);
  int run_eq = 0, run_sel = 0;
  for (int base = 0; base < n; base += kFT) {
    const int j = base + tid;
    const uint32_t key = j < n ? key_of(j) : 0u;
    const bool is_gt = j < n && key > T;
    const bool is_eq = j < n && key == T;
    int tot_eq, tot_sel;
    const int eq_rank = run_eq + block_excl_count<kFT>(is_eq, sh.tmp, &tot_eq);
    const bool take = is_gt || (is_eq && eq_rank < need_eq);
    const int pos = run_sel + block_excl_count<kFT>(take, sh.tmp, &tot_sel);
    if (take) { sh.sorted[pos] = j; sh.sortedpg[pos] = trow[j]; }
    run_eq += tot_eq;
    run_sel += tot_sel;
  }
  __syncthreads();
}

// The row's k_eff kept blocks and their page ids (as the table holds them, unchecked). Returns
// true when they are in sh.sel / sh.selpg by rank (score descending, index ascending; sh.sel is
// padded with INT_MAX up to kMaxFusedTopK), false when they are in sh.sorted / sh.sortedpg in
// ascending order (every block kept, or the exact path). All threads call it; it ends with a
// barrier.
// FORCED: the first `sink` and last `local` blocks of the row are kept whatever their scores.
// RUN: blocks per chunk of the bound, kMaxRun (the recorded runs) or 2 kMaxRun (pairs of them:
// half the maxima to histogram, for k <= 64)
template <bool FORCED, int RUN>
__device__ __forceinline__ bool select_row(const float* srow, const float* crow, const int32_t* trow, int n, int keff,
                                           int sink, int local, SelectShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (keff >= n) {   // every block is kept (uniform)
    for (int e = tid; e < n; e += kFT) { sh.sorted[e] = e; sh.sortedpg[e] = trow[e]; }
    __syncthreads();
    return false;
  }
  static_assert(RUN == kMaxRun || RUN == 2 * kMaxRun, "a chunk is one or two recorded runs");
  constexpr int kCPer = kMaxFusedRuns * kMaxRun / RUN / kFT;   // chunk maxima per thread (8 or 4)
  const int nch = (n + RUN - 1) / RUN;
  uint32_t ck[kCPer];
  bool cv[kCPer];
#pragma unroll
  for (int i = 0; i < kCPer; ++i) {   // loads first, clamped so none is conditional
    const int c = tid + kFT * i;
    cv[i] = c < nch;
    const int cc = min(c, nch - 1);
    if constexpr (RUN == kMaxRun) {
      ck[i] = order_key(crow[cc]);
    } else {   // both runs of the chunk are recorded (-inf for one with no block)
      ck[i] = max(order_key(crow[2 * cc]), order_key(crow[2 * cc + 1]));
    }
    // a chunk holding a forced block has that block's key as its maximum
    if (FORCED && (RUN * c < sink || (local > 0 && RUN * (c + 1) > n - local))) ck[i] = kForcedKey;
  }
  if (tid == 0) { sh.nsurv = 0; sh.ncand = 0; }
  if (tid < kFBins) sh.hist[tid] = 0u;
  // padding read by the guard-free ranking and ordering loops: 0 is below every candidate's
  // composite (key >= order_key(-inf) > 0), INT_MAX above every block index
  for (int i = tid; i < kCandCap / 2; i += kFT)
    reinterpret_cast<ulonglong2*>(sh.comp)[i] = make_ulonglong2(0ull, 0ull);
  if (tid < kMaxFusedTopK) sh.sel[tid] = 0x7fffffff;
  // ---- 1. range of the chunk maxima: smallest, largest, largest at or below +inf's key
  uint32_t mx = 0u, mn = 0xffffffffu, fin = 0u;
#pragma unroll
  for (int i = 0; i < kCPer; ++i) {
    if (cv[i]) {
      mx = max(mx, ck[i]);
      mn = min(mn, ck[i]);
      if (ck[i] <= kPosInfKey) fin = max(fin, ck[i]);
    }
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  fin = wave_max_u32(fin);
  if (lane == 0) { sh.red[wave] = mx; sh.red[kFW + wave] = mn; sh.red[2 * kFW + wave] = fin; }
  __syncthreads();
  mx = 0u; mn = 0xffffffffu; fin = 0u;
#pragma unroll
  for (int w = 0; w < kFW; ++w) {
    mx = max(mx, sh.red[w]);
    mn = min(mn, sh.red[kFW + w]);
    fin = max(fin, sh.red[2 * kFW + w]);
  }
  // value-linear bins where the finite range is usable (as in the top-k kernel), else key-linear
  const float vlo = key_value(mn), vfin = key_value(fin);
  const bool by_value = fin > mn && isfinite(vlo) && isfinite(vfin) &&
                        (vfin - vlo) > 0x1p-12f * fmaxf(fabsf(vlo), fabsf(vfin));   // uniform
  const float vscale = by_value ? (float)kFBins / (vfin - vlo) : 0.f;
  const float bscale = (float)kFBins / ((float)(mx - mn) + 1.0f);
#pragma unroll
  for (int i = 0; i < kCPer; ++i) {
    if (!cv[i]) continue;
    uint32_t bin;
    if (by_value) {
      const float t = (key_value(ck[i]) - vlo) * vscale;
      bin = ck[i] > kPosInfKey ? (uint32_t)(kFBins - 1) : (uint32_t)fminf(fmaxf(t, 0.f), (float)(kFBins - 1));
    } else {
      bin = min((uint32_t)((float)(ck[i] - mn) * bscale), (uint32_t)(kFBins - 1));
    }
    atomicAdd(&sh.hist[bin], 1u);
  }
  __syncthreads();
  // ---- bin holding the k_eff-th largest chunk maximum, read off by every wave (lane: 4 bins)
  uint32_t bstar;
  {   // lane l holds bins 4(63-l) .. 4(63-l)+3, so a prefix over lanes counts from the top bin
    const uint4 c4 = reinterpret_cast<const uint4*>(sh.hist)[63 - lane];
    const uint32_t local = c4.x + c4.y + c4.z + c4.w;
    uint32_t run = wave_incl_scan(local) - local, mine = 0u;   // maxima in the bins above this lane's
    const uint32_t cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (run < (uint32_t)keff && run + cc[i] >= (uint32_t)keff) mine = 4 * (63 - lane) + i;
      run += cc[i];
    }
    bstar = wave_max_u32(mine);
  }
  // T0 at or below every key of the bins >= bstar (the top-k kernel's margins); with fewer chunk
  // maxima than k_eff there is no such bound and every score is a candidate
  uint32_t T0 = mn;
  if (nch < keff) {
    T0 = 0u;
  } else if (bstar > 0u) {
    if (by_value) {
      T0 = max(mn, order_key(vlo + ((float)bstar - 0.5f) / vscale));
    } else {
      const double qd = floor((double)bstar / (double)bscale) - 513.0;
      if (qd > 0.0) T0 = mn + (uint32_t)qd;
    }
  }
  // ---- 2. survivor chunks (any order), then their scores >= T0 as candidates
#pragma unroll
  for (int i = 0; i < kCPer; ++i) {
    const int c = tid + kFT * i;
    if (cv[i] && (ck[i] >= T0 || c == nch - 1)) {
      const int p = atomicAdd(&sh.nsurv, 1);
      if (p < kSurvCap) sh.surv[p] = c;
    }
  }
  __syncthreads();
  const int ns = sh.nsurv;
  bool exact = ns > kSurvCap;   // uniform
  if (!exact) {
    const int sub = tid & (RUN - 1), slot = tid / RUN;   // RUN lanes per chunk: block RUN c + sub
    constexpr int kSlots = kFT / RUN;
    for (int r0 = 0; r0 < ns; r0 += kSlots * kRounds) {
      float v[kRounds];
      int jj[kRounds], pg[kRounds];
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {   // every round's loads in flight before any is used: the
        const int si = r0 + kSlots * r + slot;   // score and, in the same round trip, the block's page id
        const int c = sh.surv[min(si, ns - 1)];
        jj[r] = (si < ns) ? RUN * c + sub : n;
        const int jc = min(RUN * c + sub, n - 1);
        v[r] = srow[jc];
        pg[r] = trow[jc];
      }
      // candidate slots: one LDS atomic per wave for all its rounds, then ballot ranks
      bool take[kRounds];
      unsigned long long bal[kRounds];
      int tot = 0;
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        take[r] = jj[r] < n && (FORCED ? forced_or_key(jj[r], n, sink, local, v[r]) : order_key(v[r])) >= T0;
        bal[r] = __ballot(take[r]);
        tot += __popcll(bal[r]);
      }
      if (tot > 0) {   // wave-uniform
        int b0 = 0;
        if (lane == 0) b0 = atomicAdd(&sh.ncand, tot);
        int run = __builtin_amdgcn_readlane(b0, 0);
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
          const int p = run + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[r] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal[r], 0u));
          if (take[r] && p < kCandCap) {
            const uint32_t key = FORCED ? forced_or_key(jj[r], n, sink, local, v[r]) : order_key(v[r]);
            sh.comp[p] = ((unsigned long long)key << 32) | (uint32_t)(~(uint32_t)jj[r]);
            sh.comppg[p] = pg[r];
          }
          run += __popcll(bal[r]);
        }
      }
    }
    __syncthreads();
    exact = sh.ncand > kCandCap;   // uniform
  }
  if (exact) {
    select_exact<FORCED>(srow, trow, n, keff, sink, local, sh);
    return false;
  }
  const int m = sh.ncand;   // >= keff by the choice of T0
  // ---- rank = number of larger composites: four lanes (a quad) per candidate, each over every
  // fourth pair of the list (broadcast 16 B reads), summed across the quad with DPP
  const ulonglong2* cp = reinterpret_cast<const ulonglong2*>(sh.comp);
  const int npair = (m + 1) >> 1;
  const int qp = tid & 3;
  for (int e0q = 0; e0q < m; e0q += kFT / 4) {   // uniform
    const int e = e0q + (tid >> 2);
    const unsigned long long ce = sh.comp[min(e, m - 1)];
    int c = 0;
#pragma unroll 4
    for (int f = qp; f < npair; f += 4) {   // entries past the list hold 0, below every candidate
      const ulonglong2 c2 = cp[f];
      c += (c2.x > ce) + (c2.y > ce);
    }
    c += __builtin_amdgcn_update_dpp(0, c, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    c += __builtin_amdgcn_update_dpp(0, c, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    if (qp == 0 && e < m && c < keff) { sh.sel[c] = (int)~(uint32_t)ce; sh.selpg[c] = sh.comppg[e]; }
  }
  __syncthreads();
  return true;
}

// Index-list entries [e0, e1) of a row selected by rank (sh.sel, INT_MAX-padded): the kept block
// of rank r goes to position (number of kept blocks with a smaller index); one thread per kept
// block, entries at positions >= k_eff are -1. No barrier: sh.sel is only read.
__device__ __forceinline__ void write_ordered(const SelectShared& sh, int keff, int e0, int e1, int32_t* out) {
  const int tid = threadIdx.x;
  if (tid < keff) {
    const int vj = sh.sel[tid];
    int pos = 0;
    const int4* s4 = reinterpret_cast<const int4*>(sh.sel);
#pragma unroll 4
    for (int f = 0; f < (keff + 3) / 4; ++f) {   // entries past k_eff hold INT_MAX
      const int4 v = s4[f];
      pos += (v.x < vj) + (v.y < vj) + (v.z < vj) + (v.w < vj);
    }
    if (pos >= e0 && pos < e1) out[pos] = vj;
  }
  for (int e = max(e0, keff) + tid; e < e1; e += kFT) out[e] = -1;
}

// G: heads per group; U: blocks whose K/V loads each wave keeps in flight (the launcher uses 2);
// FORCED: forced sink / local blocks (keep_sink or keep_local nonzero)
template <int G, int U, bool FORCED, int RUN>
__global__ void __launch_bounds__(kFT) k_decode_select_attend(FusedArgs f) {
  const AttendArgs& a = f.att;
  __shared__ SelectShared sh;
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
  __shared__ uint16_t s_p[4][G][4][4];
  __shared__ int2 s_list[4][64];
  const SplitRow sr = split_row_of_block();
  const int split = sr.split, g = sr.g, b = sr.b;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int N = clamp_len(a.lens[b], a.max_len);
  const int nb = (N + kP - 1) / kP;
  const int keff = min(a.k, nb);
  const long long rowbg = (long long)b * a.Hkv + g;
  const int e0 = split * a.blocks_per_split;
  const int e1 = min(a.k, e0 + a.blocks_per_split);

  MfmaAttend<G> at;
  at.kpool = reinterpret_cast<const uint16_t*>(a.kpool);
  at.vpool = reinterpret_cast<const uint16_t*>(a.vpool);
  at.page_stride = (long long)a.Hkv * kP * kD;
  at.head_off = (long long)g * kP * kD;
  at.wave = wave; at.lane = lane;
  at.hq = lane & 15; at.c = lane >> 4;
  at.row = lane >> 4; at.d0 = (lane & 15) * 8;
  at.scale_log2 = a.scale_log2;
  {   // the group's queries: in flight during the selection
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((long long)b * a.Hq + g * G + min(at.hq, G - 1)) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * kk + 8 * at.c);
      at.qf[kk] = __builtin_bit_cast(bf16x8_t, at.hq < G ? w : make_uint4(0u, 0u, 0u, 0u));
    }
  }
  at.m_l = -INFINITY; at.l_l = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    at.m_h[h] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) at.acc[h][e] = 0.f;
  }

  const int32_t* trow = a.table + (long long)b * a.max_blocks;
  bool by_rank = false;
  if (keff > 0 && e0 < keff)   // uniform: this split holds kept blocks
    by_rank = select_row<FORCED, RUN>(f.scores + rowbg * f.row_stride, f.cmax + rowbg * f.cstride, trow, nb, keff,
                                 f.keep_sink, f.keep_local, sh);
  // the blocks this split attends: ranks [e0, e1) (by_rank) or positions [e0, e1) of the ascending list
  const int* lst = by_rank ? sh.sel : sh.sorted;
  const int* lstpg = by_rank ? sh.selpg : sh.sortedpg;
  int32_t* idx_row = f.idx_out != nullptr ? f.idx_out + rowbg * a.k : nullptr;
  bool listed = idx_row == nullptr;   // this split's index-list entries written
  if (!by_rank && !listed) {
    for (int e = e0 + tid; e < e1; e += kFT) idx_row[e] = e < keff ? sh.sorted[e] : -1;
    listed = true;
  }
  const int e1k = min(e1, keff);
  for (int base = e0; base < e1k; base += 64) {
    // lane e: page and live token count of kept block base + e (-1: not attended)
    int my_page = -1, my_ntok = 0;
    if (lane < e1k - base) {
      const int j = lst[base + lane];
      const int page = lstpg[base + lane];
      if (page_ok(page, a.num_pages)) {
        my_page = page;
        my_ntok = min(kP, N - j * kP);
      }
    }
    const unsigned long long live = __ballot(my_page >= 0);
    const int cnt = __popcll(live);
    if (cnt == 0) continue;
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(live >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)live, 0u));
    if (my_page >= 0) s_list[wave][rank] = make_int2(my_page, my_ntok);
    __builtin_amdgcn_wave_barrier();
    const int2 ent = s_list[wave][min(lane, cnt - 1)];
    __builtin_amdgcn_wave_barrier();
    for (int t0 = 0; t0 < cnt; t0 += U) {
      KVRegs r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) at.load(r[u], bcast(ent.x, min(t0 + u, cnt - 1)));
      if (!listed) {   // uniform: the index-list entries, while the first K/V loads are in flight
        write_ordered(sh, keff, e0, e1, idx_row);
        listed = true;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u == 0 || t0 + u < cnt) at.step(r[u], bcast(ent.y, min(t0 + u, 63)), s_p[wave]);
    }
  }
  if (!listed) write_ordered(sh, keff, e0, e1, idx_row);   // no live block in this split
  float lsum = at.l_l + __shfl_xor(at.l_l, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) at.acc[h][e] = across_rows_sum(at.acc[h][e]);
    if (lane == h) { s_m[wave][h] = at.m_h[h]; s_l[wave][h] = lsum; }
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][h][at.d0 + e] = at.acc[h][e];
    }
  }
  __syncthreads();
  write_partials<uint16_t, G>(a, s_m, s_l, s_o, b, g, split, tid);
}

template <int G>
hipError_t launch_fused_g(const FusedArgs& f, hipStream_t st) {
  const AttendArgs& a = f.att;
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  // two blocks in flight per wave, looping over the split's blocks: four measured no faster at
  // G <= 5 and, beyond 256 registers per lane at G >= 6 (one workgroup per CU), ~20 % slower
  if (log_enabled()) log_launch("k_decode_select_attend", grid, kFT, 0, "G=%d, blocks in flight %d", G, 2);
  // k <= 64: chunks of 16 blocks (pairs of recorded runs); larger k: the runs of 8 themselves,
  // twice as many maxima for a bound that still prunes at k up to the row's runs / 2
  const bool forced = f.keep_sink > 0 || f.keep_local > 0, fine = a.k > 64;
  if (forced && fine) k_decode_select_attend<G, 2, true, kMaxRun><<<grid, kFT, 0, st>>>(f);
  else if (forced) k_decode_select_attend<G, 2, true, 2 * kMaxRun><<<grid, kFT, 0, st>>>(f);
  else if (fine) k_decode_select_attend<G, 2, false, kMaxRun><<<grid, kFT, 0, st>>>(f);
  else k_decode_select_attend<G, 2, false, 2 * kMaxRun><<<grid, kFT, 0, st>>>(f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_select_attend(const FusedArgs& f, hipStream_t st) {
  const AttendArgs& a = f.att;
  if (a.B == 0) return hipSuccess;
  hipError_t err;
  switch (a.Hq / a.Hkv) {
    case 1: err = launch_fused_g<1>(f, st); break;
    case 2: err = launch_fused_g<2>(f, st); break;
    case 3: err = launch_fused_g<3>(f, st); break;
    case 4: err = launch_fused_g<4>(f, st); break;
    case 5: err = launch_fused_g<5>(f, st); break;
    case 6: err = launch_fused_g<6>(f, st); break;
    case 7: err = launch_fused_g<7>(f, st); break;
    case 8: err = launch_fused_g<8>(f, st); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess || a.nsplit == 1) return err;
  return launch_merge_bf16(a, st);
}

}  // namespace msa
