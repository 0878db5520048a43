// Block summaries and KV append.
//
// The index branch scores blocks, not tokens ("MiniMax goes sparse: decoding M3's attention
// from a single diagram", §1 Step 1). Its summary of a block here is the fp32 mean of the
// block's valid keys per KV head (the mean-pooled reading), stored next to the paged cache as
// summaries[page][g][0..127] and recomputed from the tokens whenever a block changes, so it
// always equals its definition.
//
// Work mapping: one wavefront per (block, KV head). A wave reads a 64 x 128 block as 16
// loads of 4 rows; lane l owns dims 8*(l%16) .. +7 of rows l/16, l/16+4, ... so each load
// instruction covers four whole 256 B (bf16) rows. Partial sums are combined across the four
// 16-lane rows with cross-lane moves; lanes 0..15 write 8 dims each.
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

// Reduce the per-lane partial sums over the wave's four rows and write the mean.
__device__ __forceinline__ void write_mean(float* acc, int n, float* dst, int lane) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = across_rows_sum(acc[e]);
  if (lane < 16) {
    const float fn = (float)n;
    float4 lo = make_float4(acc[0] / fn, acc[1] / fn, acc[2] / fn, acc[3] / fn);
    float4 hi = make_float4(acc[4] / fn, acc[5] / fn, acc[6] / fn, acc[7] / fn);
    reinterpret_cast<float4*>(dst + lane * 8)[0] = lo;
    reinterpret_cast<float4*>(dst + lane * 8)[1] = hi;
  }
}

// summaries of every block j < nb_b of every sequence b < B
template <typename T>
__global__ void __launch_bounds__(256) k_build_summaries(const T* __restrict__ kpool, float* __restrict__ S,
                                                         const int32_t* __restrict__ table,
                                                         const int32_t* __restrict__ lens, int num_pages,
                                                         int max_blocks, int B, int Hkv, int max_len, int mb) {
  const int lane = threadIdx.x & 63;
  const long long unit = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= (long long)B * mb * Hkv) return;
  const int g = (int)(unit % Hkv);
  const int j = (int)((unit / Hkv) % mb);
  const int b = (int)(unit / ((long long)Hkv * mb));
  const int N = clamp_len(lens[b], max_len);
  const int n = min(kP, N - j * kP);
  if (n <= 0) return;
  const int page = table[(long long)b * max_blocks + j];
  if (!page_ok(page, num_pages)) return;
  const T* base = kpool + ((long long)page * Hkv + g) * kP * kD + (lane & 15) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  Vec8<T> v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)  // all 16 row loads in flight before the sum (clamped rows)
    v[i].load(base + (long long)min((lane >> 4) + 4 * i, n - 1) * kD);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if ((lane >> 4) + 4 * i < n) v[i].add_to(acc);
  write_mean(acc, n, S + ((long long)page * Hkv + g) * kD, lane);
}

// prefill append: T new tokens after past_len (a multiple of 64) -> whole new blocks
template <typename T>
__global__ void __launch_bounds__(256) k_append_prefill(T* __restrict__ kpool, T* __restrict__ vpool, float* __restrict__ S,
                                                        const int32_t* __restrict__ table, int num_pages,
                                                        const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                        int past_blocks, int T_new, int Hkv) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ntiles = (T_new + kP - 1) / kP;
  if (unit >= ntiles * Hkv) return;
  const int g = unit % Hkv, jn = unit / Hkv;
  const int n = min(kP, T_new - jn * kP);
  const int page = table[past_blocks + jn];
  if (!page_ok(page, num_pages)) return;
  const long long head = ((long long)page * Hkv + g) * kP * kD;
  const int d0 = (lane & 15) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
  for (int r = lane >> 4; r < n; r += 4) {
    const long long src = ((long long)(jn * kP + r) * Hkv + g) * kD + d0;
    Vec8<T> kv, vv;
    kv.load(k_new + src);
    vv.load(v_new + src);
    kv.store(kpool + head + (long long)r * kD + d0);
    vv.store(vpool + head + (long long)r * kD + d0);
    kv.add_to(acc);
  }
  write_mean(acc, n, S + ((long long)page * Hkv + g) * kD, lane);
}

}  // namespace

hipError_t launch_build_summaries(bool bf16, const CacheArgs& c, int B, int Hkv, int max_len, hipStream_t st) {
  const int mb = (max_len + kP - 1) / kP;
  const long long units = (long long)B * mb * Hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 3) / 4));
  if (bf16)
    k_build_summaries<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)c.k, c.S, c.table, c.lens, c.num_pages,
                                                      c.max_blocks, B, Hkv, max_len, mb);
  else
    k_build_summaries<float><<<grid, 256, 0, st>>>((const float*)c.k, c.S, c.table, c.lens, c.num_pages,
                                                   c.max_blocks, B, Hkv, max_len, mb);
  return hipGetLastError();
}

hipError_t launch_append_prefill(bool bf16, const CacheArgs& c, const void* k_new, const void* v_new,
                                 int past_blocks, int T, int Hkv, hipStream_t st) {
  const int units = ((T + kP - 1) / kP) * Hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid((units + 3) / 4);
  if (bf16)
    k_append_prefill<uint16_t><<<grid, 256, 0, st>>>((uint16_t*)c.k, (uint16_t*)c.v, c.S, c.table, c.num_pages,
                                                     (const uint16_t*)k_new, (const uint16_t*)v_new,
                                                     past_blocks, T, Hkv);
  else
    k_append_prefill<float><<<grid, 256, 0, st>>>((float*)c.k, (float*)c.v, c.S, c.table, c.num_pages,
                                                  (const float*)k_new, (const float*)v_new, past_blocks, T, Hkv);
  return hipGetLastError();
}

}  // namespace msa
