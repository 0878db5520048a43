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
// HBM-bound streaming of the index keys (64 x 128 elements per block): a workgroup owns kIB
// blocks of one sequence (one: 16,384 workgroups at 1M tokens; 1, 2, 4 and 8 swept, one was
// fastest); thread -> (tokens t = tid/8 and t + 32 of the block, an eighth of their dims), so
// each load instruction reads whole 128 B lines (index dimension 64 or 128), and every thread's
// loads for its blocks are in flight before any arithmetic. Dot products are packed bf16 dot2 (fp32 FMAs for
// fp32 keys) against the Hkv index queries held in LDS, summed across the 8 lanes of a token
// with DPP, max-reduced with DPP over each 16-lane row (4 tokens) and through LDS over the
// block's 16 rows.
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

constexpr int kIB = 1;   // blocks per workgroup

// One thread's share of a block: two tokens (t and t + 32) of the block, and of each token the
// 16 B chunks c, c + 8, ... (c = lane of the token's 8), so the 8 lanes of a token read one whole
// 128 B line per load instruction. bf16 rows are 16 chunks (2 per lane), fp32 rows 32 (4).
template <typename T, int DI>
struct TokenPair {
  static constexpr int kC = DI * (int)sizeof(T) / 16 / 8;   // chunks per lane per token
  uint4 w[2][kC];
  __device__ __forceinline__ void load(const T* block, int t, int c) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint4* row = reinterpret_cast<const uint4*>(block + (long long)(t + 32 * k) * DI);
#pragma unroll
      for (int i = 0; i < kC; ++i) w[k][i] = load_nt(row + c + 8 * i);
    }
  }
  // token k's partial dot product with an index query held in LDS in storage form
  __device__ __forceinline__ float dot(int k, const uint32_t* q, int c) const {
    const uint4* qp = reinterpret_cast<const uint4*>(q);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      const uint4 qq = qp[c + 8 * i], x = w[k][i];
      if constexpr (sizeof(T) == 2) {
        acc = dot2_bf16(x.x, qq.x, acc);
        acc = dot2_bf16(x.y, qq.y, acc);
        acc = dot2_bf16(x.z, qq.z, acc);
        acc = dot2_bf16(x.w, qq.w, acc);
      } else {
        acc = fmaf(__uint_as_float(x.x), __uint_as_float(qq.x), acc);
        acc = fmaf(__uint_as_float(x.y), __uint_as_float(qq.y), acc);
        acc = fmaf(__uint_as_float(x.z), __uint_as_float(qq.z), acc);
        acc = fmaf(__uint_as_float(x.w), __uint_as_float(qq.w), acc);
      }
    }
    return acc;
  }
};

template <typename T, int DI>
__global__ void __launch_bounds__(256) k_score_index(const T* __restrict__ q_index, const T* __restrict__ ikeys,
                                                     const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ lens, int num_pages,
                                                     int max_blocks, int Hkv, int max_len,
                                                     float* __restrict__ scores, int row_stride) {
  // [Hkv][128] index queries in storage form (bf16 pairs or fp32), then [kIB][Hkv][16] row maxima
  extern __shared__ uint32_t s_dyn[];
  constexpr int kQW = DI * sizeof(T) / 4;           // 32-bit words per index query
  uint32_t* s_q = s_dyn;
  float* s_wm = reinterpret_cast<float*>(s_dyn + Hkv * kQW);
  const int b = blockIdx.y, j0 = blockIdx.x * kIB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 7, t = tid >> 3;              // lane of the token's 8; tokens t and t + 32
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
  TokenPair<T, DI> kr[kIB];
#pragma unroll
  for (int u = 0; u < kIB; ++u) {     // every load issued before any arithmetic (page 0: valid, unused)
    const int page = page_ok(pg[u], num_pages) ? pg[u] : 0;
    kr[u].load(ikeys + (long long)page * kP * DI, t, c);
  }
  {   // one 16 B load per thread for Hkv <= 16 (bf16) / 8 (fp32)
    const uint4* qsrc = reinterpret_cast<const uint4*>(q_index + (long long)b * Hkv * DI);
    for (int e = tid; e < Hkv * kQW / 4; e += 256) reinterpret_cast<uint4*>(s_q)[e] = qsrc[e];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kIB; ++u) {
    const int j = j0 + u;
    const bool blk = j < nb && page_ok(pg[u], num_pages);
    const bool live0 = blk && kP * j + t < N, live1 = blk && kP * j + t + 32 < N;
    for (int g = 0; g < Hkv; ++g) {
      float s0 = kr[u].dot(0, s_q + g * kQW, c), s1 = kr[u].dot(1, s_q + g * kQW, c);
      s0 += dpp_mov<0xB1>(s0);       // the token's 8 lanes: quad sums, then the two quads
      s1 += dpp_mov<0xB1>(s1);
      s0 += dpp_mov<0x4E>(s0);
      s1 += dpp_mov<0x4E>(s1);
      s0 += dpp_mov<0x141>(s0);
      s1 += dpp_mov<0x141>(s1);
      float m = fmaxf(live0 ? s0 : -INFINITY, live1 ? s1 : -INFINITY);
      m = fmaxf(m, dpp_mov<0x140>(m));   // the row's two 8-lane token groups: 4 tokens per row
      if ((lane & 15) == 0) s_wm[(u * Hkv + g) * 16 + wave * 4 + (lane >> 4)] = m;
    }
  }
  __syncthreads();
  for (int e = tid; e < Hkv * kIB; e += 256) {       // g-major: each row's kIB scores are contiguous
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

hipError_t launch_score_index(bool bf16, const void* q_index, const void* index_keys, int index_dim,
                              const CacheArgs& c, int B, int Hkv, int max_len, float* scores, int row_stride,
                              hipStream_t st) {
  if (B == 0 || row_stride == 0) return hipSuccess;
  const dim3 grid((row_stride + kIB - 1) / kIB, B);
  // LDS: the Hkv index queries in storage form, then the [kIB][Hkv][16] row maxima
  const size_t lds = (size_t)Hkv * index_dim * (bf16 ? 2 : 4) + (size_t)kIB * Hkv * 16 * sizeof(float);
  if (log_enabled()) log_launch("k_score_index", grid, 256, lds, "%s, index dim %d", bf16 ? "bf16" : "f32", index_dim);
#define MSA_INDEX(TT, DD)                                                                                 \
  k_score_index<TT, DD><<<grid, 256, lds, st>>>((const TT*)q_index, (const TT*)index_keys, c.table, c.lens, \
                                                c.num_pages, c.max_blocks, Hkv, max_len, scores, row_stride)
  if (bf16) {
    if (index_dim == 64) MSA_INDEX(uint16_t, 64); else MSA_INDEX(uint16_t, 128);
  } else {
    if (index_dim == 64) MSA_INDEX(float, 64); else MSA_INDEX(float, 128);
  }
#undef MSA_INDEX
  return hipGetLastError();
}

}  // namespace msa
