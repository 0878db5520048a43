// Step 1 scoring: one index query per GQA group against every block summary.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 1: each group
// shares one index query, and the scoring pass must be cheap because it touches every block;
// §3: in prefill this pass still scans the whole input. Readings used: the index query is the
// mean of the group's query heads (decode) or of the tile's 64 rows x the group's heads
// (prefill); a block's score is <index query, block summary>, unscaled, in fp32.
//
// Decode is a streaming read of the summary pool (nb x Hkv x 128 fp32 per sequence), so the
// kernel is shaped for HBM: a workgroup owns a chunk of 32 logical blocks of one sequence,
// stages the chunk's page ids and the Hkv index queries in LDS, and then walks (block, group)
// pairs with 32 lanes per pair and 16 B per lane -- for Hkv = 8 one pass of a wave reads two
// whole 4 KiB pages' worth of contiguous summaries, whatever the page permutation. Eight
// independent 16 B loads per lane are issued before any arithmetic. Each score also bumps a
// coarse per-row histogram of its order key, which lets the top-k kernel find the k-th score's
// neighbourhood in one pass.
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

constexpr int kChunk = 32;    // logical blocks per workgroup (decode)
constexpr int kUnroll = 8;    // pairs in flight per 32-lane slot

template <typename T> __device__ __forceinline__ float ld(const T* p, long long i);
template <> __device__ __forceinline__ float ld<float>(const float* p, long long i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, long long i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

template <typename TQ>
__global__ void __launch_bounds__(256) k_score_decode(const TQ* __restrict__ q, const float* __restrict__ S,
                                                      const int32_t* __restrict__ table,
                                                      const int32_t* __restrict__ lens, int num_pages,
                                                      int max_blocks, int Hq, int Hkv, int max_len,
                                                      float* __restrict__ scores, int row_stride,
                                                      uint32_t* __restrict__ hist) {
  extern __shared__ float s_qidx[];             // [Hkv][128] index queries
  __shared__ int s_page[kChunk];
  const int b = blockIdx.y;
  const int j0 = blockIdx.x * kChunk;
  const int tid = threadIdx.x;
  const int N = clamp_len(lens[b], max_len);
  const int nb = (N + kP - 1) / kP;
  const int jend = min(j0 + kChunk, row_stride);

  if (tid < kChunk) {
    const int j = j0 + tid;
    int page = -1;
    if (j < nb) {
      page = table[(long long)b * max_blocks + j];
      if (!page_ok(page, num_pages)) page = -1;
    }
    s_page[tid] = page;
  }
  if (j0 < nb) {  // [MGS §1 Step 1] one index query per group: mean of the group's heads
    const int G = Hq / Hkv;
    const TQ* qb = q + (long long)b * Hq * kD;
    for (int e = tid; e < Hkv * kD; e += 256) {
      const int g = e / kD, d = e % kD;
      float acc = 0.f;
      for (int h = 0; h < G; ++h) acc += ld(qb, (long long)(g * G + h) * kD + d);
      s_qidx[e] = acc / (float)G;
    }
  }
  __syncthreads();

  const int slot = tid >> 5;    // 8 pair slots per pass
  const int l32 = tid & 31;     // 4 dims per lane
  const int npairs = (jend - j0) * Hkv;
  for (int p0 = 0; p0 < npairs; p0 += 8 * kUnroll) {
    float4 sv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u * 8 + slot;
      const int jl = p / Hkv, g = p % Hkv;
      const int page = (p < npairs) ? s_page[jl] : -1;
      sv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (page >= 0) sv[u] = *reinterpret_cast<const float4*>(S + ((long long)page * Hkv + g) * kD + l32 * 4);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u * 8 + slot;
      if (p >= npairs) continue;   // uniform across the 32-lane slot
      const int jl = p / Hkv, g = p % Hkv;
      const int j = j0 + jl;
      const float4 qv = *reinterpret_cast<const float4*>(s_qidx + g * kD + l32 * 4);
      float part = qv.x * sv[u].x;
      part = fmaf(qv.y, sv[u].y, part);
      part = fmaf(qv.z, sv[u].z, part);
      part = fmaf(qv.w, sv[u].w, part);
      part = row16_sum(part);
      part += __shfl_xor(part, 16);
      if (l32 == 0) {
        const long long row = (long long)b * Hkv + g;
        float s = -INFINITY;
        if (j < nb) {
          if (s_page[jl] >= 0) s = part;
          atomicAdd(&hist[row * kHistBins + (order_key(s) >> (32 - kHistBits))], 1u);
        }
        scores[row * row_stride + j] = s;
      }
    }
  }
}

// tile index query: qtile[tau][g][d] = mean over the tile's rows and the group's heads
template <typename TQ>
__global__ void __launch_bounds__(128) k_tile_query(const TQ* __restrict__ q, int T, int Hq, int Hkv,
                                                    float* __restrict__ qtile) {
  const int tau = blockIdx.x, g = blockIdx.y, d = threadIdx.x;
  const int G = Hq / Hkv;
  const int i0 = tau * kP, i1 = min(T, i0 + kP);
  float acc = 0.f;
  for (int i = i0; i < i1; ++i)
#pragma unroll 4
    for (int h = 0; h < G; ++h) acc += ld(q, ((long long)i * Hq + g * G + h) * kD + d);
  qtile[((long long)tau * Hkv + g) * kD + d] = acc / (float)((i1 - i0) * G);
}

// prefill scores: a 64-tile x 64-block fp32 product per workgroup, from LDS; tile tau scores
// the blocks j < past_blocks + tau (its causal candidates), -inf elsewhere in the row.
// LDS holds both operands transposed ([d][tile], [d][block]) so that the inner loop's reads are
// broadcast or consecutive, with no bank conflicts.
constexpr int kPT = 64;   // tiles per workgroup
constexpr int kPB = 64;   // blocks per workgroup

__global__ void __launch_bounds__(256) k_score_prefill(const float* __restrict__ qtile, const float* __restrict__ S,
                                                       const int32_t* __restrict__ table, int num_pages,
                                                       int past_blocks, int ntiles, int Hkv,
                                                       float* __restrict__ scores, int row_stride,
                                                       uint32_t* __restrict__ hist) {
  __shared__ float s_q[kD][kPT];
  __shared__ float s_s[kD][kPB];
  const int j0 = blockIdx.x * kPB, g = blockIdx.y, t0 = blockIdx.z * kPT;
  const int tid = threadIdx.x;
  const int ncand_max = past_blocks + ntiles - 1;   // candidates of the last tile
  for (int e = tid; e < kPT * (kD / 4); e += 256) {
    const int t = e % kPT, c = e / kPT;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t0 + t < ntiles) v = *reinterpret_cast<const float4*>(qtile + ((long long)(t0 + t) * Hkv + g) * kD + c * 4);
    s_q[c * 4 + 0][t] = v.x; s_q[c * 4 + 1][t] = v.y; s_q[c * 4 + 2][t] = v.z; s_q[c * 4 + 3][t] = v.w;
  }
  for (int e = tid; e < kPB * (kD / 4); e += 256) {
    const int jl = e % kPB, c = e / kPB;
    const int j = j0 + jl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j < ncand_max) {
      const int page = table[j];
      if (page_ok(page, num_pages)) v = *reinterpret_cast<const float4*>(S + ((long long)page * Hkv + g) * kD + c * 4);
    }
    s_s[c * 4 + 0][jl] = v.x; s_s[c * 4 + 1][jl] = v.y; s_s[c * 4 + 2][jl] = v.z; s_s[c * 4 + 3][jl] = v.w;
  }
  __syncthreads();
  // thread owns tiles ty*4 .. +3 and blocks tx + 16*c, c = 0..3
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
  for (int d = 0; d < kD; ++d) {
    float qa[4], sb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) qa[a] = s_q[d][ty * 4 + a];
#pragma unroll
    for (int c = 0; c < 4; ++c) sb[c] = s_s[d][tx + 16 * c];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(qa[a], sb[c], acc[a][c]);
  }
  bool ok[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = j0 + tx + 16 * c;
    ok[c] = j < ncand_max && page_ok(table[j], num_pages);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int tau = t0 + ty * 4 + a;
    if (tau >= ntiles) continue;
    const long long row = (long long)tau * Hkv + g;
    const int ncand = past_blocks + tau;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tx + 16 * c;
      if (j >= row_stride) continue;
      float s = -INFINITY;
      if (j < ncand) {
        if (ok[c]) s = acc[a][c];
        atomicAdd(&hist[row * kHistBins + (order_key(s) >> (32 - kHistBits))], 1u);
      }
      scores[row * row_stride + j] = s;
    }
  }
}

}  // namespace

hipError_t launch_score_decode(bool bf16, const void* q, const CacheArgs& c, int B, int Hq, int Hkv, int max_len,
                               float* scores, int row_stride, uint32_t* hist, hipStream_t st) {
  if (B == 0 || row_stride == 0) return hipSuccess;
  const dim3 grid((row_stride + kChunk - 1) / kChunk, B);
  const size_t lds = (size_t)Hkv * kD * sizeof(float);
  if (bf16)
    k_score_decode<uint16_t><<<grid, 256, lds, st>>>((const uint16_t*)q, c.S, c.table, c.lens, c.num_pages,
                                                     c.max_blocks, Hq, Hkv, max_len, scores, row_stride, hist);
  else
    k_score_decode<float><<<grid, 256, lds, st>>>((const float*)q, c.S, c.table, c.lens, c.num_pages,
                                                  c.max_blocks, Hq, Hkv, max_len, scores, row_stride, hist);
  return hipGetLastError();
}

hipError_t launch_tile_query(bool bf16, const void* q, int T, int Hq, int Hkv, float* qtile, hipStream_t st) {
  const dim3 grid((T + kP - 1) / kP, Hkv);
  if (bf16)
    k_tile_query<uint16_t><<<grid, 128, 0, st>>>((const uint16_t*)q, T, Hq, Hkv, qtile);
  else
    k_tile_query<float><<<grid, 128, 0, st>>>((const float*)q, T, Hq, Hkv, qtile);
  return hipGetLastError();
}

hipError_t launch_score_prefill(const float* qtile, const CacheArgs& c, int past_blocks, int ntiles, int Hkv,
                                float* scores, int row_stride, uint32_t* hist, hipStream_t st) {
  const dim3 grid((row_stride + kPB - 1) / kPB, Hkv, (ntiles + kPT - 1) / kPT);
  k_score_prefill<<<grid, 256, 0, st>>>(qtile, c.S, c.table, c.num_pages, past_blocks, ntiles, Hkv, scores,
                                        row_stride, hist);
  return hipGetLastError();
}

}  // namespace msa
