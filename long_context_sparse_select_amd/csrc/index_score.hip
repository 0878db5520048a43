// Step 1, the index branch as the diagram draws it: token scores through a single-head index
// key, Block Max Pool, then the shared top-k kernel.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 1: each GQA
// group's index query scores the context through one index key shared by all groups; the token
// scores are max-pooled per fixed-size block, and TopK keeps the best blocks. Readings: the
// index keys are paged like K (one head, 128 dims: [num_pages][64][128]); a token's score is
// <q_index[b][g], K_idx[t]>, unscaled; a block's score is the maximum over its valid tokens;
// blocks past a sequence's length, or on a bad page id, score -inf.
//
// HBM-bound streaming of the index keys (64 x 128 elements per block): a workgroup owns 4 blocks
// of one sequence; thread -> (token t = tid/4 of the block, a quarter of its dims), and every
// thread's loads for the 4 blocks are in flight before any arithmetic. Dot products are packed bf16 dot2 (fp32 FMAs for fp32 keys)
// against the Hkv index queries held in LDS, reduced across the 4 lanes of a token with DPP, then
// max-reduced with DPP over each 16-lane row (4 tokens) and through LDS over the block's 16 rows.
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

constexpr int kIB = 4;   // blocks per workgroup

// A lane's quarter of one 128-dim index-key row: 16 B chunks c, c+4, c+8, ... of the row (lane c of
// the token's 4), so the 4 lanes of a token read 64 contiguous bytes per load instruction.
template <typename T> struct RowQuarter;
template <> struct RowQuarter<uint16_t> {
  uint4 w[4];   // 4 chunks of 8 bf16
  __device__ __forceinline__ void load(const uint16_t* row, int c) {
    const uint4* p = reinterpret_cast<const uint4*>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = p[c + 4 * i];
  }
  // q: an index query in storage form (64 words of bf16 pairs) in LDS; the same chunks
  __device__ __forceinline__ float dot(const uint32_t* q, int c) const {
    const uint4* qp = reinterpret_cast<const uint4*>(q);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 qq = qp[c + 4 * i];
      acc = dot2_bf16(w[i].x, qq.x, acc);
      acc = dot2_bf16(w[i].y, qq.y, acc);
      acc = dot2_bf16(w[i].z, qq.z, acc);
      acc = dot2_bf16(w[i].w, qq.w, acc);
    }
    return acc;
  }
};
template <> struct RowQuarter<float> {
  float4 f[8];  // 8 chunks of 4 fp32
  __device__ __forceinline__ void load(const float* row, int c) {
    const float4* p = reinterpret_cast<const float4*>(row);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = p[c + 4 * i];
  }
  __device__ __forceinline__ float dot(const uint32_t* q, int c) const {
    const float4* qp = reinterpret_cast<const float4*>(q);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 qq = qp[c + 4 * i];
      acc = fmaf(f[i].x, qq.x, acc);
      acc = fmaf(f[i].y, qq.y, acc);
      acc = fmaf(f[i].z, qq.z, acc);
      acc = fmaf(f[i].w, qq.w, acc);
    }
    return acc;
  }
};

template <typename T>
__global__ void __launch_bounds__(256) k_score_index(const T* __restrict__ q_index, const T* __restrict__ ikeys,
                                                     const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ lens, int num_pages,
                                                     int max_blocks, int Hkv, int max_len,
                                                     float* __restrict__ scores, int row_stride) {
  // [Hkv][128] index queries in storage form (bf16 pairs or fp32), then [kIB][Hkv][16] row maxima
  extern __shared__ uint32_t s_dyn[];
  constexpr int kQW = kD * sizeof(T) / 4;           // 32-bit words per index query
  uint32_t* s_q = s_dyn;
  float* s_wm = reinterpret_cast<float*>(s_dyn + Hkv * kQW);
  const int b = blockIdx.y, j0 = blockIdx.x * kIB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 3, t = tid >> 2;              // lane of the token's 4, token within the block
  const int32_t* trow = table + (long long)b * max_blocks;
  int pg[kIB];
#pragma unroll
  for (int u = 0; u < kIB; ++u) pg[u] = trow[min(j0 + u, row_stride - 1)];
  const int N = clamp_len(lens[b], max_len);
  const int nb = (N + kP - 1) / kP;
  if (j0 >= nb || num_pages <= 0) {   // uniform: every block of the chunk scores -inf
    for (int e = tid; e < Hkv * kIB; e += 256) {
      const int g = e / kIB, u = e % kIB;
      if (j0 + u < row_stride) scores[((long long)b * Hkv + g) * row_stride + j0 + u] = -INFINITY;
    }
    return;
  }
  RowQuarter<T> kr[kIB];
#pragma unroll
  for (int u = 0; u < kIB; ++u) {     // every load issued before any arithmetic (page 0: valid, unused)
    const int page = page_ok(pg[u], num_pages) ? pg[u] : 0;
    kr[u].load(ikeys + ((long long)page * kP + t) * kD, c);
  }
  {   // one 16 B load per thread for Hkv <= 16 (bf16) / 8 (fp32)
    const uint4* qsrc = reinterpret_cast<const uint4*>(q_index + (long long)b * Hkv * kD);
    for (int e = tid; e < Hkv * kQW / 4; e += 256) reinterpret_cast<uint4*>(s_q)[e] = qsrc[e];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kIB; ++u) {
    const int j = j0 + u;
    const bool live = j < nb && page_ok(pg[u], num_pages) && kP * j + t < N;
    for (int g = 0; g < Hkv; ++g) {
      float s = kr[u].dot(s_q + g * kQW, c);
      s += dpp_mov<0xB1>(s);         // the token's 4 lanes
      s += dpp_mov<0x4E>(s);
      s = row16_max(live ? s : -INFINITY);   // the 4 tokens of each 16-lane row
      if ((lane & 15) == 0) s_wm[(u * Hkv + g) * 16 + wave * 4 + (lane >> 4)] = s;
    }
  }
  __syncthreads();
  for (int e = tid; e < Hkv * kIB; e += 256) {       // g-major: each row's 4 scores are contiguous
    const int g = e / kIB, u = e % kIB, j = j0 + u;
    if (j >= row_stride) continue;
    const float4* w16 = reinterpret_cast<const float4*>(s_wm + (u * Hkv + g) * 16);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fmaxf(w16[i].x, w16[i].y), fmaxf(w16[i].z, w16[i].w)));
    scores[((long long)b * Hkv + g) * row_stride + j] = (j < nb && page_ok(pg[u], num_pages)) ? m : -INFINITY;
  }
}

}  // namespace

hipError_t launch_score_index(bool bf16, const void* q_index, const void* index_keys, const CacheArgs& c, int B,
                              int Hkv, int max_len, float* scores, int row_stride, hipStream_t st) {
  if (B == 0 || row_stride == 0) return hipSuccess;
  const dim3 grid((row_stride + kIB - 1) / kIB, B);
  if (bf16) {
    const size_t lds = (size_t)Hkv * (kD / 2) * 4 + (size_t)kIB * Hkv * 16 * sizeof(float);
    k_score_index<uint16_t><<<grid, 256, lds, st>>>((const uint16_t*)q_index, (const uint16_t*)index_keys, c.table,
                                                    c.lens, c.num_pages, c.max_blocks, Hkv, max_len, scores,
                                                    row_stride);
  } else {
    const size_t lds = (size_t)Hkv * kD * 4 + (size_t)kIB * Hkv * 16 * sizeof(float);
    k_score_index<float><<<grid, 256, lds, st>>>((const float*)q_index, (const float*)index_keys, c.table, c.lens,
                                                 c.num_pages, c.max_blocks, Hkv, max_len, scores, row_stride);
  }
  return hipGetLastError();
}

}  // namespace msa
