// Step 1 scoring: one index query per GQA group against every block summary.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 1: each group
// shares one index query, and the scoring pass must be cheap because it touches every block;
// §3: in prefill this pass still scans the whole input. Readings used: the index query is the
// mean of the group's query heads (decode) or of the tile's 64 rows x the group's heads
// (prefill); a block's score is <index query, block summary>, unscaled, in fp32.
//
// Decode is a streaming read of the summary pool (nb x Hkv x 128 fp32 or bf16 per sequence), so
// the kernel is shaped for HBM: a workgroup owns a chunk of 16 logical blocks of one sequence and
// walks (block, group) pairs with 16 B per lane -- 32 lanes per fp32 pair, in passes of 8 blocks,
// or 16 lanes per bf16 pair, in one pass of 16 -- so for Hkv = 8 it reads the chunk's 16 pages
// as 16 contiguous 4 KiB (2 KiB) runs, whatever the page permutation. Each lane reads its pairs' page ids from the table and issues all of its
// summary loads of a pass first, non-temporal (the pool is streamed once per launch); the Hkv index queries are built in LDS while the first pass
// is in flight. The chunk's scores are staged in LDS and leave as one contiguous run per row.
// The number of KV heads is a template parameter for the power-of-two cases, so the pair-index
// arithmetic is shifts, not divisions.
//
// A decode step's new token is appended by the same launch: Hkv more workgroups per sequence
// (dispatched first) each write the token's K/V row of one group, recompute the summary of its
// block from the block's keys, and score that block from the stored summary, while the chunk
// workgroups stream the other summaries and leave that one score alone. Every score the top-k
// kernel then reads describes the cache after the append (§1 Step 1: blocks are scored through
// their summaries).
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

constexpr int kChunk = 16;    // logical blocks per workgroup (decode)
constexpr int kUnroll = 8;    // pairs in flight per 32-lane slot
constexpr int kTailBytes = 1 << 18;   // -inf tail bytes (pad) per writing chunk past a sequence's end

// 8 consecutive elements as floats, in 16 B vector loads
__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
  f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float* f) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}


// The decode step's new token, for sequence b and group g (one 256-thread workgroup): its K/V
// row goes to position N-1 of its block; the block's summary becomes the mean of its older rows
// and the new key (bf16 pools store it rounded); the block's score is <index query, stored
// summary>. Thread -> rows r, r+16, r+32, r+48 (r = tid/16) of the block, 8 dims; its four row
// loads are issued together, and the K/V store goes to a row nothing in this launch reads.
// s_red: 4 x 128 + 2 floats of LDS.
template <typename T, bool SB>
__device__ __forceinline__ void decode_append(const T* __restrict__ q, const T* __restrict__ k_new,
                                              const T* __restrict__ v_new, T* __restrict__ kpool,
                                              T* __restrict__ vpool, void* __restrict__ S,
                                              const int32_t* __restrict__ table, const int32_t* __restrict__ lens,
                                              int num_pages, int max_blocks, int Hq, int Hkv, int max_len,
                                              float* __restrict__ scores, int row_stride, int b, int g,
                                              float* s_red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = clamp_len(lens[b], max_len);
  if (N == 0 || num_pages <= 0) return;   // uniform: no block (an empty pool scores -inf elsewhere)
  const int t = N - 1, jl = t / kP, slot = t % kP;
  const int page = table[(long long)b * max_blocks + jl];
  float* dst = scores + ((long long)b * Hkv + g) * row_stride + jl;
  if (!page_ok(page, num_pages)) {   // uniform: nothing is stored, and the block is never attended
    if (tid == 0) *dst = -INFINITY;
    return;
  }
  const int r0 = tid >> 4, d0 = (tid & 15) * 8;
  const long long head = ((long long)page * Hkv + g) * kP * kD;
  const long long nrow = ((long long)b * Hkv + g) * kD + d0;
  Vec8<T> rows[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // rows past the new one re-read the new key (a valid address; unused)
    const int r = r0 + 16 * i;
    rows[i].load(r < slot ? kpool + head + (long long)r * kD + d0 : k_new + nrow);
  }
  if (r0 == (slot & 15)) {   // the 16 lanes of the new row's thread group
    Vec8<T> kn, vn;
    kn.load(k_new + nrow);
    vn.load(v_new + nrow);
    kn.store(kpool + head + (long long)slot * kD + d0);
    vn.store(vpool + head + (long long)slot * kD + d0);
  }
  const int G = Hq / Hkv;
  float qv[kMaxGroup];
  if (tid < kD) {   // the group's query heads at dim tid
    const T* qb = q + ((long long)b * Hq + g * G) * kD + tid;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if constexpr (sizeof(T) == 2) qv[h] = __uint_as_float((uint32_t)qb[(long long)min(h, G - 1) * kD] << 16);
      else qv[h] = qb[(long long)min(h, G - 1) * kD];
    }
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (r0 + 16 * i <= slot) rows[i].add_to(acc);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = across_rows_sum(acc[e]);   // the wave's four row groups
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_red[wave * kD + d0 + e] = acc[e];
  }
  __syncthreads();
  if (tid < kD) {
    float summary = (s_red[tid] + s_red[kD + tid] + s_red[2 * kD + tid] + s_red[3 * kD + tid]) / (float)(slot + 1);
    const long long si = ((long long)page * Hkv + g) * kD + tid;
    if constexpr (SB) {   // the score uses the value the pool holds
      const uint32_t h = pack_bf16x2(summary, 0.f) & 0xffffu;
      reinterpret_cast<uint16_t*>(S)[si] = (uint16_t)h;
      summary = bf16lo(h);
    } else {
      reinterpret_cast<float*>(S)[si] = summary;
    }
    float qi = 0.f;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
      if (h < G) qi += qv[h];
    const float prod = across_rows_sum(row16_sum((qi / (float)G) * summary));
    if (lane == 0) s_red[4 * kD + wave] = prod;
  }
  __syncthreads();
  if (tid == 0) *dst = s_red[4 * kD] + s_red[4 * kD + 1];
}

// -inf over entries [lo, hi) of every group's score row of sequence b: 16 B stores across the
// workgroup. Kept out of line: inlined into the scoring kernel's exit path it raised the kernel's
// registers past the six-wave step (82 against 78 at 8 groups), and the grid of a batch of mixed
// lengths then ran with fewer slots.
__device__ __attribute__((noinline)) void write_neg_inf_rows(float* __restrict__ scores, int b, int Hkv, int row_stride,
                                                             int lo, int hi) {
  const int tid = threadIdx.x;
  const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  for (int g = 0; g < Hkv && lo < hi; ++g) {
    float* row = scores + ((long long)b * Hkv + g) * row_stride + lo;
    const int n = hi - lo;
    const int head = min(n, (int)(((16u - ((uint32_t)(uintptr_t)row & 15u)) & 15u) / 4u));
    if (tid < head) row[tid] = -INFINITY;
    const int nv = (n - head) / 4;
    float4* r4 = reinterpret_cast<float4*>(row + head);
    for (int i = tid; i < nv; i += 256) r4[i] = ninf;
    const int rem = n - head - 4 * nv;
    if (tid < rem) row[head + 4 * nv + tid] = -INFINITY;
  }
}

// HKV > 0: the number of KV heads as a compile-time constant (so the pair-index divisions are
// shifts); HKV == 0: a runtime count (generic path). SB: the summary pool holds bf16.
// Workgroups x < napp (napp = Hkv with a new token, else 0) append, writing the pool through
// S_app (the same pool as S, which only the scoring workgroups read); the others score chunks.
template <typename TQ, int HKV, bool SB>
__global__ void __launch_bounds__(256) k_score_decode(const TQ* __restrict__ q, const void* __restrict__ S,
                                                      const int32_t* __restrict__ table,
                                                      const int32_t* __restrict__ lens, int num_pages,
                                                      int max_blocks, int Hq, int hkv_arg, int max_len,
                                                      float* __restrict__ scores, int row_stride,
                                                      const TQ* __restrict__ k_new, const TQ* __restrict__ v_new,
                                                      TQ* __restrict__ kpool, TQ* __restrict__ vpool, void* S_app,
                                                      int napp, float* __restrict__ cmax, int cstride, int pad) {
  const int Hkv = HKV > 0 ? HKV : hkv_arg;
  extern __shared__ float s_qidx[];             // [Hkv][128] index queries, then [Hkv][kChunk] scores
  const int b = blockIdx.y;
  if ((int)blockIdx.x < napp) {   // uniform per workgroup
    decode_append<TQ, SB>(q, k_new, v_new, kpool, vpool, S_app, table, lens, num_pages, max_blocks, Hq, Hkv, max_len,
                          scores, row_stride, b, (int)blockIdx.x, s_qidx);
    return;
  }
  const int chunk = (int)blockIdx.x - napp;
  const int j0 = chunk * kChunk;
  const int tid = threadIdx.x;
  const int jend = min(j0 + kChunk, row_stride);
  constexpr int kLanes = SB ? 16 : 32;   // lanes per (block, group) pair, 16 B each
  constexpr int kSlots = 256 / kLanes;   // pairs per load round
  const int slot = tid / kLanes;
  const int lp = tid % kLanes;           // 8 (bf16) or 4 (fp32) dims per lane
  const int npairs = (jend - j0) * Hkv;
  const int32_t* trow = table + (long long)b * max_blocks;
  if (num_pages <= 0) {   // an empty pool: every block of the chunk scores -inf (uniform exit)
    for (int e = tid; e < Hkv * kChunk; e += 256) {
      const int g = e / kChunk, jl = e % kChunk;
      if (j0 + jl < jend) scores[((long long)b * Hkv + g) * row_stride + j0 + jl] = -INFINITY;
    }
    if (cmax != nullptr && tid < 2 * Hkv) cmax[((long long)b * Hkv + tid / 2) * cstride + 2 * chunk + tid % 2] = -INFINITY;
    return;
  }

  // Pass loads: each lane reads the page ids of its own pairs straight from the table (the
  // workgroup's 8 entries share one cache line), then issues every summary load of the pass.
  // Nothing else is on the path from the kernel's start to the summary stream.
  uint4 sv[kUnroll];
  bool live[kUnroll];
  int tp[kUnroll];
  auto table_loads = [&](int p0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) tp[u] = trow[min(j0 + (p0 + u * kSlots + slot) / Hkv, row_stride - 1)];
  };
  auto summary_loads = [&](int p0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {   // branch-free: every load is issued unconditionally
      const int p = p0 + u * kSlots + slot;
      live[u] = (p < npairs) & (tp[u] >= 0) & (tp[u] < num_pages);   // the length is applied later
      const int page = live[u] ? tp[u] : 0;   // page 0: a valid address, result unused
      const long long row = (long long)page * Hkv + p % Hkv;   // 16 B per lane, either pool type
      sv[u] = load_nt(reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(S) + row * kD * (SB ? 2 : 4)) + lp);
    }
  };
  table_loads(0);
  const int nb = (clamp_len(lens[b], max_len) + kP - 1) / kP;   // in flight with the table loads
  if (j0 >= nb) {   // a chunk past the sequence's end (batches of mixed lengths): no summary reads.
    // A caller's score buffer (pad) gets -inf past the sequence's end (every consumer in the
    // library reads a row only up to the sequence's length, run maxima included): the first
    // chunks past the end, one per kTailBytes of the tail (at most all of them), split the tail
    // of every group's row into equal ranges written with 16 B stores; the other chunks exit
    // without a write
    if (!pad) return;
    const int vc = (nb + kChunk - 1) / kChunk;     // chunks holding blocks
    const int wi = chunk - vc;
    const int from0 = vc * kChunk, tn = row_stride - from0;
    const long long tail_bytes = (long long)tn * Hkv * 4;
    const int nw = (int)min((long long)(tn + kChunk - 1) / kChunk,       // past-the-end chunks in the grid
                            max(1ll, (tail_bytes + kTailBytes - 1) / kTailBytes));
    if (wi >= nw) return;
    const int seg = ((tn + nw - 1) / nw + 3) & ~3;                       // nw * seg >= tn
    const int lo = from0 + wi * seg, hi = min(row_stride, lo + seg);
    write_neg_inf_rows(scores, b, Hkv, row_stride, lo, hi);
    return;
  }
  summary_loads(0);
  {  // §1 Step 1 of the page: one index query per group (the mean of its heads), computed while
     // the summaries stream in. Thread -> (group, 8 dims): its G head rows are 16 B vector loads.
    const int G = Hq / Hkv;
    const TQ* qb = q + (long long)b * Hq * kD;
    for (int c0 = 0; c0 < Hkv * (kD / 8); c0 += 256) {
      const int cc = min(c0 + tid, Hkv * (kD / 8) - 1);
      const int g = cc / (kD / 8), d8 = (cc % (kD / 8)) * 8;
      float acc[8];
      if constexpr (sizeof(TQ) == 2) {   // heads kept as packed bf16 while in flight
        uint4 w[kMaxGroup];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
          w[h] = *reinterpret_cast<const uint4*>(qb + (long long)(g * G + min(h, G - 1)) * kD + d8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
            acc[0] += bf16lo(w[h].x); acc[1] += bf16hi(w[h].x); acc[2] += bf16lo(w[h].y); acc[3] += bf16hi(w[h].y);
            acc[4] += bf16lo(w[h].z); acc[5] += bf16hi(w[h].z); acc[6] += bf16lo(w[h].w); acc[7] += bf16hi(w[h].w);
          }
        }
      } else {
        float v[kMaxGroup][8];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) load8(qb + (long long)(g * G + min(h, G - 1)) * kD + d8, v[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[e] = 0.f;
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h)
            if (h < G) acc[e] += v[h][e];
        }
      }
      if (c0 + tid < Hkv * (kD / 8)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_qidx[g * kD + d8 + e] = acc[e] / (float)G;
      }
    }
  }
  __syncthreads();

  float* s_sc = s_qidx + Hkv * kD;
  for (int p0 = 0; p0 < npairs; p0 += kSlots * kUnroll) {
    if (p0 > 0) {
      table_loads(p0);
      summary_loads(p0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u * kSlots + slot;
      if (p >= npairs) continue;   // uniform across the pair's lanes
      const int jl = p / Hkv, g = p % Hkv;
      float part;
      if constexpr (SB) {
        const float4* qp = reinterpret_cast<const float4*>(s_qidx + g * kD + lp * 8);
        const float4 qa = qp[0], qb = qp[1];
        const uint4 w = sv[u];
        part = qa.x * bf16lo(w.x);
        part = fmaf(qa.y, bf16hi(w.x), part);
        part = fmaf(qa.z, bf16lo(w.y), part);
        part = fmaf(qa.w, bf16hi(w.y), part);
        part = fmaf(qb.x, bf16lo(w.z), part);
        part = fmaf(qb.y, bf16hi(w.z), part);
        part = fmaf(qb.z, bf16lo(w.w), part);
        part = fmaf(qb.w, bf16hi(w.w), part);
        part = row16_sum(part);
      } else {
        const float4 qv = *reinterpret_cast<const float4*>(s_qidx + g * kD + lp * 4);
        const float4 f = __builtin_bit_cast(float4, sv[u]);
        part = qv.x * f.x;
        part = fmaf(qv.y, f.y, part);
        part = fmaf(qv.z, f.z, part);
        part = fmaf(qv.w, f.w, part);
        part = row16_sum(part);
        part += __shfl_xor(part, 16);
      }
      if (lp == 0) s_sc[g * kChunk + jl] = (live[u] && j0 + jl < nb) ? part : -INFINITY;
    }
  }
  __syncthreads();
  // each row's chunk of scores leaves as one contiguous run; with a new token, its block's score
  // is the append workgroup's
  // The maxima of the chunk's two 8-block runs per group (for the fused select-and-attend) are
  // taken over the scores written here, in the same pass: the 16 scores of a group are one 16-lane
  // row (kChunk = 16 and every pass covers whole rows), so a reduction over each half-row gives
  // them. The appended block's score is the append workgroup's and is not in them.
  static_assert(kChunk == 16 && 256 % kChunk == 0, "one group's chunk of scores per 16-lane row");
  const int jskip = napp > 0 ? nb - 1 : -1;
  for (int e = tid; e < Hkv * kChunk; e += 256) {
    const int g = e / kChunk, jl = e % kChunk;
    const int j = j0 + jl;
    const float v = s_sc[e];
    if (j < jend && j != jskip) scores[((long long)b * Hkv + g) * row_stride + j] = v;
    if (cmax != nullptr) {   // uniform
      const float mrun = row8_max(j < jend && j < nb && j != jskip ? v : -INFINITY);
      if ((jl & (kMaxRun - 1)) == 0) cmax[((long long)b * Hkv + g) * cstride + 2 * chunk + jl / kMaxRun] = mrun;
    }
  }
}

// prefill scores: a 64-tile x 65-block fp32 product per workgroup, 64 blocks on fp32 MFMA
// (v_mfma_f32_32x32x2_f32: exact fp32 products, fp32 accumulation) and the 65th on the vector
// ALU; tile tau scores the blocks j < past_blocks + tau (its causal candidates), -inf elsewhere
// in the row. 65 rather than 64 blocks per workgroup: a 4096-token chunk on a cache of a multiple
// of 4096 tokens has 64k + 64 candidate blocks, and 65-block groups make that 64k + 64 = 65 m
// groups, 512 workgroups at 8 KV groups, which run in one round at two per CU instead of 520 in
// two.
// Staging: the 64 tile queries and the 64 block summaries (512 B rows) are read coalesced, 32
// lanes per row, all 16 loads of a thread in flight at once, and stored to LDS rows padded to
// 132 floats. Wave w then computes the 32 x 32 output tile (tiles 32*(w/2) .., blocks
// 32*(w%2) ..): MFMA step s contracts dims s and 64 + s, so lane (i = l%32, h = l/32) reads
// dims 64h .. 64h+63 of one tile row (A) and one block row (B) as 16 B LDS reads (row pitch
// 132 floats: the 16 rows a read touches fall on distinct banks).
constexpr int kPT = 64;     // tiles per workgroup
constexpr int kPB = 64;     // blocks per workgroup on MFMA
constexpr int kPBW = kPB + 1;   // blocks per workgroup: the MFMA ones and one on the vector ALU
constexpr int kRowP = 132;  // LDS row pitch (floats)
__device__ __forceinline__ int pgx_of(const int32_t* table, int j, int ncand_max) {
  return table[min(j, max(ncand_max - 1, 0))];
}
typedef float f32x16s __attribute__((ext_vector_type(16)));

template <bool SB>
__global__ void __launch_bounds__(256) k_score_prefill(const float* __restrict__ qtile, const void* __restrict__ S,
                                                       const int32_t* __restrict__ table, int num_pages,
                                                       int past_blocks, int ntiles, int Hkv,
                                                       float* __restrict__ scores, int row_stride) {
  __shared__ __align__(16) float s_a[kPT * kRowP];
  __shared__ __align__(16) float s_b[kPBW * kRowP];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = blockIdx.y;
  const int tz = blockIdx.z * kPT, jz = blockIdx.x * kPBW;
  const int ncand_max = past_blocks + ntiles - 1;      // candidates of the last tile
  {
    // thread -> rows (tid/32) + 8*it, float4 column tid%32; table entries first, then the rows
    const int c4 = tid & 31;
    int pg[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) pg[it] = table[min(jz + (tid >> 5) + 8 * it, max(ncand_max - 1, 0))];
    // the 65th block's row: threads 0..31, one float4 each
    const int pgx = table[min(jz + kPB, max(ncand_max - 1, 0))];
    float4 av[8], bv[8], bx = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = (tid >> 5) + 8 * it;
      av[it] = reinterpret_cast<const float4*>(qtile + ((long long)min(tz + r, ntiles - 1) * Hkv + g) * kD)[c4];
      const int page = page_ok(pg[it], num_pages) ? pg[it] : 0;   // page 0: a valid address
      const long long srow = (long long)page * Hkv + g;
      if constexpr (SB) {   // 4 bf16 values widened exactly to fp32
        const uint2 w = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(S) + srow * kD)[c4];
        bv[it] = make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
      } else {
        bv[it] = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(S) + srow * kD)[c4];
      }
    }
    if (tid < 32) {
      const int page = page_ok(pgx, num_pages) ? pgx : 0;
      const long long srow = (long long)page * Hkv + g;
      if constexpr (SB) {
        const uint2 w = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(S) + srow * kD)[c4];
        bx = make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
      } else {
        bx = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(S) + srow * kD)[c4];
      }
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = (tid >> 5) + 8 * it;
      *reinterpret_cast<float4*>(s_a + r * kRowP + 4 * c4) = av[it];
      *reinterpret_cast<float4*>(s_b + r * kRowP + 4 * c4) = bv[it];
    }
    if (tid < 32) *reinterpret_cast<float4*>(s_b + kPB * kRowP + 4 * c4) = bx;
  }
  __syncthreads();
  const int i = lane & 31, h = lane >> 5;
  const int ta = 32 * (w >> 1), jb = 32 * (w & 1);
  const float* arow = s_a + (ta + i) * kRowP + 64 * h;
  const float* brow = s_b + (jb + i) * kRowP + 64 * h;
  f32x16s acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float4 a4 = *reinterpret_cast<const float4*>(arow + 4 * e);
    const float4 b4 = *reinterpret_cast<const float4*>(brow + 4 * e);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, b4.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, b4.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, b4.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, b4.w, acc, 0, 0, 0);
  }
  {  // the 65th block on the vector ALU: thread -> (tile tid/4, dims 32 (tid%4) ..), fp32 FMAs in
     // dim order, then a sum over the quad
    const int t = tid >> 2, q4 = tid & 3;
    const float* ar = s_a + t * kRowP + 32 * q4;
    const float* br = s_b + kPB * kRowP + 32 * q4;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float4 a4 = *reinterpret_cast<const float4*>(ar + 4 * e);
      const float4 b4 = *reinterpret_cast<const float4*>(br + 4 * e);
      part = fmaf(a4.x, b4.x, part);
      part = fmaf(a4.y, b4.y, part);
      part = fmaf(a4.z, b4.z, part);
      part = fmaf(a4.w, b4.w, part);
    }
    part += dpp_mov<0xB1>(part);   // quad_perm [1,0,3,2]
    part += dpp_mov<0x4E>(part);   // quad_perm [2,3,0,1]
    const int jx = jz + kPB, tau = tz + t;
    if (q4 == 0 && jx < row_stride && tau < ntiles) {
      const bool okx = jx < ncand_max && page_ok(pgx_of(table, jx, ncand_max), num_pages);
      scores[((long long)tau * Hkv + g) * row_stride + jx] = (okx && jx < past_blocks + tau) ? part : -INFINITY;
    }
  }
  // lane l holds block jz + jb + l%32 of tiles tz + ta + 8*(r/4) + 4*(l/32) + r%4
  const int j = jz + jb + i;
  if (j >= row_stride) return;
  const bool ok = j < ncand_max && page_ok(table[min(j, max(ncand_max - 1, 0))], num_pages);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tau = tz + ta + 8 * (r >> 2) + 4 * h + (r & 3);
    if (tau >= ntiles) continue;
    scores[((long long)tau * Hkv + g) * row_stride + j] = (ok && j < past_blocks + tau) ? acc[r] : -INFINITY;
  }
}


template <typename TQ, bool SB>
void launch_score_typed(const TQ* q, const CacheArgs& c, int B, int Hq, int Hkv, int max_len, float* scores,
                        int row_stride, const TQ* k_new, const TQ* v_new, float* cmax, int cstride, int pad,
                        hipStream_t st) {
  static_assert(kChunk == kScoreChunk && kChunk == 2 * kMaxRun, "two run maxima per scoring chunk");
  const int napp = k_new != nullptr ? Hkv : 0;
  const dim3 grid(napp + (row_stride + kChunk - 1) / kChunk, B);
  const int lds_floats = Hkv * (kD + kChunk) > 4 * kD + 2 ? Hkv * (kD + kChunk) : 4 * kD + 2;
  const size_t lds = (size_t)lds_floats * sizeof(float);
  TQ* kp = static_cast<TQ*>(c.k);
  TQ* vp = static_cast<TQ*>(c.v);
  if (log_enabled())
    log_launch("k_score_decode", grid, 256, lds, "%s q, Hkv=%d, %s summaries%s%s", sizeof(TQ) == 2 ? "bf16" : "f32",
               Hkv, SB ? "bf16" : "f32", napp > 0 ? ", with the new token's append" : "",
               cmax != nullptr ? ", run maxima" : "");
#define MSA_SCORE_CASE(H)                                                                                  \
  case H:                                                                                                  \
    k_score_decode<TQ, H, SB><<<grid, 256, lds, st>>>(q, c.S, c.table, c.lens, c.num_pages, c.max_blocks, Hq, \
                                                      Hkv, max_len, scores, row_stride, k_new, v_new, kp, vp, \
                                                      c.S, napp, cmax, cstride, pad);                      \
    break;
  switch (Hkv) {
    MSA_SCORE_CASE(1)
    MSA_SCORE_CASE(2)
    MSA_SCORE_CASE(4)
    MSA_SCORE_CASE(8)
    MSA_SCORE_CASE(16)
    MSA_SCORE_CASE(32)
    MSA_SCORE_CASE(64)
    default:
      k_score_decode<TQ, 0, SB><<<grid, 256, lds, st>>>(q, c.S, c.table, c.lens, c.num_pages, c.max_blocks, Hq,
                                                        Hkv, max_len, scores, row_stride, k_new, v_new, kp, vp, c.S,
                                                        napp, cmax, cstride, pad);
  }
#undef MSA_SCORE_CASE
}

}  // namespace

hipError_t launch_score_decode(bool bf16, const void* q, const CacheArgs& c, int B, int Hq, int Hkv, int max_len,
                               float* scores, int row_stride, const void* k_new, const void* v_new, hipStream_t st,
                               float* cmax, int cstride, bool pad) {
  if (B == 0 || row_stride == 0) return hipSuccess;
#define MSA_SCORE_TYPED(T, SB)                                                                                 \
  launch_score_typed<T, SB>((const T*)q, c, B, Hq, Hkv, max_len, scores, row_stride, (const T*)k_new, (const T*)v_new, \
                            cmax, cstride, pad ? 1 : 0, st)
  if (bf16) {
    if (c.s_bf16) MSA_SCORE_TYPED(uint16_t, true); else MSA_SCORE_TYPED(uint16_t, false);
  } else {
    if (c.s_bf16) MSA_SCORE_TYPED(float, true); else MSA_SCORE_TYPED(float, false);
  }
#undef MSA_SCORE_TYPED
  return hipGetLastError();
}


hipError_t launch_score_prefill(const float* qtile, const CacheArgs& c, int past_blocks, int ntiles, int Hkv,
                                float* scores, int row_stride, hipStream_t st) {
  const dim3 grid((row_stride + kPBW - 1) / kPBW, Hkv, (ntiles + kPT - 1) / kPT);
  if (log_enabled()) log_launch("k_score_prefill", grid, 256, 0, "%s summaries", c.s_bf16 ? "bf16" : "f32");
  if (c.s_bf16)
    k_score_prefill<true><<<grid, 256, 0, st>>>(qtile, c.S, c.table, c.num_pages, past_blocks, ntiles, Hkv, scores,
                                                row_stride);
  else
    k_score_prefill<false><<<grid, 256, 0, st>>>(qtile, c.S, c.table, c.num_pages, past_blocks, ntiles, Hkv, scores,
                                                 row_stride);
  return hipGetLastError();
}

}  // namespace msa
