// Block summaries and KV append.
//
// The index branch scores blocks, not tokens ("MiniMax goes sparse: decoding M3's attention
// from a single diagram", §1 Step 1). Its summary of a block here is the fp32 mean of the
// block's valid keys per KV head (the mean-pooled reading), stored next to the paged cache as
// summaries[page][g][0..127] and recomputed from the tokens whenever a block changes, so it
// always equals its definition. The pool holds fp32, or bf16 (the fp32 mean rounded to nearest
// even on store), which halves what the decode scoring pass reads.
//
// The prefill chunk's append shares a launch with the tile index queries (k_prefill_prologue):
// the two are independent, so they overlap.
//
// Work mapping: one wavefront per (block, KV head). A wave reads a 64 x 128 block as 16
// loads of 4 rows; lane l owns dims 8*(l%16) .. +7 of rows l/16, l/16+4, ... so each load
// instruction covers four whole 256 B (bf16) rows. Partial sums are combined across the four
// 16-lane rows with cross-lane moves; lanes 0..15 write 8 dims each.
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

// Reduce the per-lane partial sums over the wave's four rows and write the mean (row `row` of
// the summary pool; bf16 pools store it rounded to nearest even).
template <bool SB>
__device__ __forceinline__ void write_mean(float* acc, int n, void* S, long long row, int lane) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = across_rows_sum(acc[e]);
  if (lane < 16) {
    const float fn = (float)n;
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = acc[e] / fn;
    if constexpr (SB) {
      reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(S) + row * kD)[lane] =
          make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]), pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7]));
    } else {
      float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(S) + row * kD + lane * 8);
      dst[0] = make_float4(m[0], m[1], m[2], m[3]);
      dst[1] = make_float4(m[4], m[5], m[6], m[7]);
    }
  }
}

// summaries of every block j < nb_b of every sequence b < B
template <typename T, bool SB>
__global__ void __launch_bounds__(256) k_build_summaries(const T* __restrict__ kpool, void* __restrict__ S,
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
  write_mean<SB>(acc, n, S, (long long)page * Hkv + g, lane);
}

// prefill append, one wave per unit = (new block jn, group g): T new tokens after past_len (a
// multiple of 64) fill whole new blocks; the wave copies the block's rows into its page and
// writes the block's summary
template <typename T, bool SB>
__device__ __forceinline__ void append_unit(T* __restrict__ kpool, T* __restrict__ vpool, void* __restrict__ S,
                                            const int32_t* __restrict__ table, int num_pages,
                                            const T* __restrict__ k_new, const T* __restrict__ v_new,
                                            int past_blocks, int T_new, int Hkv, int unit) {
  const int lane = threadIdx.x & 63;
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
  write_mean<SB>(acc, n, S, (long long)page * Hkv + g, lane);
}

// tile index query (512 threads): qtile[tau][g][d] = mean over the tile's rows and the group's
// heads. Thread (row i = tid/8, 16 dims 16*(tid%8)..) sums its row's G heads (2G 16 B loads in
// flight at once); the 64 rows are then summed per dim through LDS, in row order.
template <typename TQ>
__device__ __forceinline__ void tile_query(const TQ* __restrict__ q, int T, int Hq, int Hkv, float* __restrict__ qtile,
                                           int tau, int g, float (*s_rows)[kD + 1]) {
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int i0 = tau * kP, n = min(T, i0 + kP) - i0;
  const int i = tid >> 3, d0 = (tid & 7) * 16;
  const int row = i0 + min(i, n - 1);
  Vec8<TQ> v[kMaxGroup][2];   // the row's 16 dims of each head: 16 B vector loads, all in flight
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    const TQ* src = q + ((long long)row * Hq + g * G + min(h, G - 1)) * kD + d0;
    v[h][0].load(src);
    v[h][1].load(src + 8);
  }
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      float f[16];
      v[h][0].to_f32(f);
      v[h][1].to_f32(f + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += f[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) s_rows[i][d0 + e] = i < n ? acc[e] : 0.f;
  __syncthreads();
  if (tid < kD) {
    float acc = 0.f;
    for (int r = 0; r < n; ++r) acc += s_rows[r][tid];
    qtile[((long long)tau * Hkv + g) * kD + tid] = acc / (float)(n * G);
  }
}

// The prefill chunk's two independent first steps in one launch: workgroups [0, n_app) append
// (eight (new block, group) units each, one per wave), the others compute one tile index query
// each, so the two overlap instead of running back to back.
template <typename T, bool SB>
__global__ void __launch_bounds__(512) k_prefill_prologue(T* __restrict__ kpool, T* __restrict__ vpool,
                                                          void* __restrict__ S, const int32_t* __restrict__ table,
                                                          int num_pages, const T* __restrict__ k_new,
                                                          const T* __restrict__ v_new, const T* __restrict__ q,
                                                          int past_blocks, int T_new, int Hq, int Hkv, int n_app,
                                                          float* __restrict__ qtile) {
  __shared__ float s_rows[kP][kD + 1];
  if ((int)blockIdx.x < n_app) {   // uniform per workgroup
    append_unit<T, SB>(kpool, vpool, S, table, num_pages, k_new, v_new, past_blocks, T_new, Hkv,
                       (int)blockIdx.x * 8 + (int)(threadIdx.x >> 6));
    return;
  }
  const int e = (int)blockIdx.x - n_app, ntiles = (T_new + kP - 1) / kP;
  tile_query<T>(q, T_new, Hq, Hkv, qtile, e % ntiles, e / ntiles, s_rows);
}

}  // namespace

hipError_t launch_build_summaries(bool bf16, const CacheArgs& c, int B, int Hkv, int max_len, hipStream_t st) {
  const int mb = (max_len + kP - 1) / kP;
  const long long units = (long long)B * mb * Hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 3) / 4));
  if (log_enabled())
    log_launch("k_build_summaries", grid, 256, 0, "%s keys, %s summaries", bf16 ? "bf16" : "f32", c.s_bf16 ? "bf16" : "f32");
#define MSA_BUILD(T, SB)                                                                                       \
  k_build_summaries<T, SB><<<grid, 256, 0, st>>>((const T*)c.k, c.S, c.table, c.lens, c.num_pages, c.max_blocks, \
                                                 B, Hkv, max_len, mb)
  if (bf16) {
    if (c.s_bf16) MSA_BUILD(uint16_t, true); else MSA_BUILD(uint16_t, false);
  } else {
    if (c.s_bf16) MSA_BUILD(float, true); else MSA_BUILD(float, false);
  }
#undef MSA_BUILD
  return hipGetLastError();
}

hipError_t launch_prefill_prologue(bool bf16, const CacheArgs& c, const void* k_new, const void* v_new,
                                   const void* q, int past_blocks, int T, int Hq, int Hkv, float* qtile,
                                   hipStream_t st) {
  const int ntiles = (T + kP - 1) / kP;
  if (ntiles == 0) return hipSuccess;
  const int n_app = (ntiles * Hkv + 7) / 8;
  const dim3 grid(n_app + ntiles * Hkv);
  if (log_enabled())
    log_launch("k_prefill_prologue", grid, 512, 0, "%s, %s summaries, %d append workgroups", bf16 ? "bf16" : "f32",
               c.s_bf16 ? "bf16" : "f32", n_app);
#define MSA_PROLOGUE(TT, SB)                                                                                  \
  k_prefill_prologue<TT, SB><<<grid, 512, 0, st>>>((TT*)c.k, (TT*)c.v, c.S, c.table, c.num_pages, (const TT*)k_new, \
                                                   (const TT*)v_new, (const TT*)q, past_blocks, T, Hq, Hkv, n_app,  \
                                                   qtile)
  if (bf16) {
    if (c.s_bf16) MSA_PROLOGUE(uint16_t, true); else MSA_PROLOGUE(uint16_t, false);
  } else {
    if (c.s_bf16) MSA_PROLOGUE(float, true); else MSA_PROLOGUE(float, false);
  }
#undef MSA_PROLOGUE
  return hipGetLastError();
}

}  // namespace msa
