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
// one workgroup does both jobs of one new block and group, so their loads overlap.
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

// The prefill chunk's first step, one 512-thread workgroup per (tile tau, group g). Each tile is
// one new block (past_len is a multiple of 64), so the workgroup does both of that block's jobs
// for group g, with all of their loads in flight together:
//   * the tile index query: qtile[tau][g][d] = mean over the tile's rows and the group's heads.
//     Thread (row i = tid/8, 16 dims 16*(tid%8)..) sums its row's G heads (2G 16 B loads); the 64
//     rows are then summed per dim through LDS, in row order;
//   * the append: thread (row r = tid/16, 8 dims 8*(tid%16)..) copies rows r and r + 32 of the
//     block's new K and V into its page and sums their keys; the 32 row groups are summed per
//     dim across each wave's four (cross-lane moves), then across the 8 waves through LDS, in
//     wave order, and the mean is written as the block's summary.
// One barrier serves both. A launch of ntiles * Hkv workgroups (512 for a 4096-token chunk with
// 8 groups) fits the chip in one round.
template <typename T, bool SB>
__global__ void __launch_bounds__(512) k_prefill_prologue(T* __restrict__ kpool, T* __restrict__ vpool,
                                                          void* __restrict__ S, const int32_t* __restrict__ table,
                                                          int num_pages, const T* __restrict__ k_new,
                                                          const T* __restrict__ v_new, const T* __restrict__ q,
                                                          int past_blocks, int T_new, int Hq, int Hkv,
                                                          float* __restrict__ qtile) {
  __shared__ float s_rows[kP][kD + 1];
  __shared__ float s_wsum[8][kD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = (T_new + kP - 1) / kP;
  const int tau = (int)blockIdx.x % ntiles, g = (int)blockIdx.x / ntiles;
  const int G = Hq / Hkv;
  const int i0 = tau * kP, n = min(T_new, i0 + kP) - i0;
  // tile query loads: the row's 16 dims of each head
  const int i = tid >> 3, dq = (tid & 7) * 16;
  const int row = i0 + min(i, n - 1);
  Vec8<T> v[kMaxGroup][2];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    const T* src = q + ((long long)row * Hq + g * G + min(h, G - 1)) * kD + dq;
    v[h][0].load(src);
    v[h][1].load(src + 8);
  }
  // append loads: rows r and r + 32 of the block (a row past the chunk re-reads row n - 1; unused)
  const int page = table[past_blocks + tau];
  const bool app = page_ok(page, num_pages);   // uniform
  const int r = tid >> 4, da = (tid & 15) * 8;
  Vec8<T> kv[2], vv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const long long src = ((long long)(i0 + min(r + 32 * u, n - 1)) * Hkv + g) * kD + da;
    kv[u].load(k_new + src);
    vv[u].load(v_new + src);
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (app) {
    const long long head = ((long long)page * Hkv + g) * kP * kD;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (r + 32 * u < n) {
        kv[u].store(kpool + head + (long long)(r + 32 * u) * kD + da);
        vv[u].store(vpool + head + (long long)(r + 32 * u) * kD + da);
        kv[u].add_to(acc);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = across_rows_sum(acc[e]);   // the wave's four row groups
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_wsum[wave][da + e] = acc[e];
    }
  }
  // tile query: the row's sum over the group's heads
  float qs[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) qs[e] = 0.f;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      float f[16];
      v[h][0].to_f32(f);
      v[h][1].to_f32(f + 8);
#pragma unroll
      for (int e = 0; e < 16; ++e) qs[e] += f[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) s_rows[i][dq + e] = i < n ? qs[e] : 0.f;
  __syncthreads();
  if (tid < kD) {
    float t = 0.f;
    for (int rr = 0; rr < n; ++rr) t += s_rows[rr][tid];
    qtile[((long long)tau * Hkv + g) * kD + tid] = t / (float)(n * G);
    if (app) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) sum += s_wsum[w][tid];
      const float m = sum / (float)n;
      const long long si = ((long long)page * Hkv + g) * kD + tid;
      if constexpr (SB) reinterpret_cast<uint16_t*>(S)[si] = (uint16_t)(pack_bf16x2(m, 0.f) & 0xffffu);
      else reinterpret_cast<float*>(S)[si] = m;
    }
  }
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
  const dim3 grid(ntiles * Hkv);
  if (log_enabled())
    log_launch("k_prefill_prologue", grid, 512, 0, "%s, %s summaries", bf16 ? "bf16" : "f32", c.s_bf16 ? "bf16" : "f32");
#define MSA_PROLOGUE(TT, SB)                                                                                  \
  k_prefill_prologue<TT, SB><<<grid, 512, 0, st>>>((TT*)c.k, (TT*)c.v, c.S, c.table, c.num_pages, (const TT*)k_new, \
                                                   (const TT*)v_new, (const TT*)q, past_blocks, T, Hq, Hkv, qtile)
  if (bf16) {
    if (c.s_bf16) MSA_PROLOGUE(uint16_t, true); else MSA_PROLOGUE(uint16_t, false);
  } else {
    if (c.s_bf16) MSA_PROLOGUE(float, true); else MSA_PROLOGUE(float, false);
  }
#undef MSA_PROLOGUE
  return hipGetLastError();
}

}  // namespace msa
