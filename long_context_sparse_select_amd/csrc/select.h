// Wave-level helpers of the Step 1 selection ("MiniMax goes sparse: decoding M3's attention from
// a single diagram", §1 Step 1: TopK over block scores), shared by the top-k kernel and the fused
// select-and-attend decode kernel. Scores are compared as order-preserving 32-bit keys
// (order_key in common.h).
#pragma once

#include "common.h"

namespace msa {
namespace {

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
// wave-uniform max / min: DPP within each 16-lane row, then the four rows through readlane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));
  v = min(v, dpp_u32<0x4E>(v));
  v = min(v, dpp_u32<0x141>(v));
  v = min(v, dpp_u32<0x140>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

// The score an order key came from (keys of NaN payloads give NaN; the forced key is not a score).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
constexpr uint32_t kPosInfKey = 0xff800000u;   // order_key(+inf)
// A forced block's key sits above every order key (even a NaN's), so every selection path keeps
// it; forced blocks tie among themselves and fit in k_eff, so all of them are kept.
constexpr uint32_t kForcedKey = 0xffffffffu;
// the selection key of block j of a row of n blocks: forced (the first `sink` or the last
// `local` blocks) or the order key of its score
__device__ __forceinline__ uint32_t forced_or_key(int j, int n, int sink, int local, float s) {
  return (j < sink || j >= n - local) ? kForcedKey : order_key(s);
}

// block-wide integer sum (all threads get it); s_tmp holds NT/64 ints
template <int NT>
__device__ int block_sum(int v, int* s_tmp) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) total += s_tmp[w];
  __syncthreads();
  return total;
}

// exclusive count of `pred` over threads in index order; *total gets the block's count
template <int NT>
__device__ int block_excl_count(bool pred, int* s_tmp, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long m = __ballot(pred);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_tmp[wave] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int c = s_tmp[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

}  // namespace
}  // namespace msa
