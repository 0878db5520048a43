// Step 2, decode: gather-attend over the selected blocks of a paged KV cache.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 2: every query
// head of a GQA group attends with ordinary softmax attention over the real K/V of the group's
// selected blocks only; §1 (hardware alignment): one query group loads one KV block set;
// §3: decode time is bound by the KV-cache bandwidth, which selection cuts.
//
// The kernels are HBM-bound (about 4 FLOP per KV byte at G = 4), so they are built for streaming:
//   * grid = (split, group, sequence); a workgroup walks `blocks_per_split` entries of the
//     group's index list and reads each selected 64 x 128 K and V block (16 KiB each in bf16)
//     once, for all G heads of the group. The block list (index and page id per entry) is read
//     once, up front, one entry per lane;
//   * bf16 (k_attend_decode_mfma): each of the 4 waves owns 16 keys of a block. q.k runs on
//     MFMA (S^T = K.Q^T, 16 keys x 16 padded head columns, four v_mfma_f32_16x16x32_bf16); the
//     online softmax is per head and wave-local (log2 domain, exp2); P crosses to the P.V layout
//     through a small per-wave LDS patch, and P.V is packed bf16 dot2 on token pairs. A workgroup
//     issues the loads of U blocks (2 or 4) before the first block's arithmetic;
//   * fp32 (k_attend_decode): lane l holds 8 dims (one float4 pair) of rows 4i + l/16; q.k by
//     VALU FMAs and a 16-lane DPP row sum, P.V by FMAs, all in fp32;
//   * each workgroup writes an unnormalised partial (O, m, l) per head; k_merge (one workgroup
//     per (sequence, query head), every partial load in flight at once) combines the splits with
//     a log-sum-exp merge and writes o (bf16 / fp32) and lse (natural log). With one split the
//     workgroup's partial is final and is written directly.
#include "common.h"
#include "kernels.h"
#include "attend_mfma.h"

namespace msa {

namespace {

template <typename T> struct KV8;

template <> struct KV8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { w = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
  }
};

template <> struct KV8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// this lane's 8 dims of the query of one head
template <typename T> struct Q8;

template <> struct Q8<uint16_t> {
  uint4 w;  // bf16 pairs
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float dot(const KV8<uint16_t>& k) const {
    float z = dot2_bf16(k.w.x, w.x, 0.f);
    z = dot2_bf16(k.w.y, w.y, z);
    z = dot2_bf16(k.w.z, w.z, z);
    return dot2_bf16(k.w.w, w.w, z);
  }
};

template <> struct Q8<float> {
  float f[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ float dot(const KV8<float>& k) const {
    float z = f[0] * k.a.x;
    z = fmaf(f[1], k.a.y, z); z = fmaf(f[2], k.a.z, z); z = fmaf(f[3], k.a.w, z);
    z = fmaf(f[4], k.b.x, z); z = fmaf(f[5], k.b.y, z); z = fmaf(f[6], k.b.z, z);
    return fmaf(f[7], k.b.w, z);
  }
};

template <typename T, int G>
__global__ void __launch_bounds__(256) k_attend_decode(AttendArgs a) {
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
  const SplitRow sr = split_row_of_block();
  const int split = sr.split, g = sr.g, b = sr.b;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, row = lane >> 4;
  const int d0 = (lane & 15) * 8;
  const int N = clamp_len(a.lens[b], a.max_len);
  const int nb = (N + kP - 1) / kP;
  const int e0 = split * a.blocks_per_split;
  const int e1 = min(a.k, e0 + a.blocks_per_split);
  const long long rowbg = (long long)b * a.Hkv + g;

  Q8<T> q[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    q[h].load(reinterpret_cast<const T*>(a.q) + ((long long)b * a.Hq + g * G + h) * kD + d0);
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const int32_t* ids = a.idx + rowbg * a.k;
  for (int e = e0; e < e1; ++e) {
    const int j = ids[e];
    if (j < 0 || j >= nb) continue;
    const int page = a.pages != nullptr ? a.pages[rowbg * a.k + e] : a.table[(long long)b * a.max_blocks + j];
    if (!page_ok(page, a.num_pages)) continue;
    const int ntok = min(kP, N - j * kP);
    const long long head = ((long long)page * a.Hkv + g) * kP * kD;
    const T* kb = reinterpret_cast<const T*>(a.kpool) + head + d0;
    const T* vb = reinterpret_cast<const T*>(a.vpool) + head + d0;
    KV8<T> kr[4], vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = wave * 16 + i * 4 + row;
      kr[i].load(kb + (long long)t * kD);
      vr[i].load(vb + (long long)t * kD);
    }
    float z[G][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool live = wave * 16 + i * 4 + row < ntok;
      if (!live) vr[i].zero();  // slots past the length never reach the accumulator
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float zz = row16_sum(q[h].dot(kr[i])) * a.scale_log2;
        z[h][i] = live ? zz : -INFINITY;
      }
    }
    float vf[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i].to_f32(vf[i]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = across_rows_max(fmaxf(fmaxf(z[h][0], z[h][1]), fmaxf(z[h][2], z[h][3])));
      const float mn = fmaxf(m[h], mx);
      if (mn == -INFINITY) continue;  // nothing visible yet for this wave
      const float alpha = rescale(m[h], mn);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(z[h][i] - mn);
      l[h] = l[h] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float o = acc[h][e] * alpha;
        o = fmaf(p[0], vf[0][e], o);
        o = fmaf(p[1], vf[1][e], o);
        o = fmaf(p[2], vf[2][e], o);
        acc[h][e] = fmaf(p[3], vf[3][e], o);
      }
      m[h] = mn;
    }
  }

  // rows of the wave -> one partial per wave; then the 4 waves through LDS
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = across_rows_sum(l[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = across_rows_sum(acc[h][e]);
    if (lane == 0) { s_m[wave][h] = m[h]; s_l[wave][h] = l[h]; }
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][h][d0 + e] = acc[h][e];
    }
  }
  __syncthreads();
  write_partials<T, G>(a, s_m, s_l, s_o, b, g, split, tid);
}


template <int G, int U>
__global__ void __launch_bounds__(256) k_attend_decode_mfma(AttendArgs a) {
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
  __shared__ uint16_t s_p[4][G][4][4];     // per wave: [head][token row r][pair slot i] -> key 4i + r
  __shared__ int2 s_list[4][64];           // per wave: (page, live tokens) of the attended blocks
  const SplitRow sr = split_row_of_block();
  const int split = sr.split, g = sr.g, b = sr.b;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int N = clamp_len(a.lens[b], a.max_len);
  const int nb = (N + kP - 1) / kP;
  const int e0 = split * a.blocks_per_split;
  const int e1 = min(a.k, e0 + a.blocks_per_split);
  const long long rowbg = (long long)b * a.Hkv + g;

  MfmaAttend<G> at;
  at.kpool = reinterpret_cast<const uint16_t*>(a.kpool);
  at.vpool = reinterpret_cast<const uint16_t*>(a.vpool);
  at.page_stride = (long long)a.Hkv * kP * kD;
  at.head_off = (long long)g * kP * kD;
  at.wave = wave; at.lane = lane;
  at.hq = lane & 15; at.c = lane >> 4;
  at.row = lane >> 4; at.d0 = (lane & 15) * 8;
  at.scale_log2 = a.scale_log2;
  {
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

  const int32_t* ids = a.idx + rowbg * a.k;
  const int32_t* pgs = a.pages != nullptr ? a.pages + rowbg * a.k : nullptr;
  for (int base = e0; base < e1; base += 64) {
    // lane e: page and live token count of block base + e, or page -1 when it is not attended.
    // The index and page loads go out together (clamped slot) before either is checked.
    int my_page = -1, my_ntok = 0;
    {
      const int e = base + min(lane, e1 - base - 1);
      const int j = ids[e];
      int page = pgs != nullptr ? pgs[e] : 0;
      if (pgs == nullptr && j >= 0 && j < nb) page = a.table[(long long)b * a.max_blocks + j];
      if (lane < e1 - base && j >= 0 && j < nb && page_ok(page, a.num_pages)) {
        my_page = page;
        my_ntok = min(kP, N - j * kP);
      }
    }
    // compact the attended blocks to the front (wave-private LDS list; LDS is in order per wave)
    const unsigned long long live = __ballot(my_page >= 0);
    const int cnt = __popcll(live);
    if (cnt == 0) continue;
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(live >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)live, 0u));
    if (my_page >= 0) s_list[wave][rank] = make_int2(my_page, my_ntok);
    __builtin_amdgcn_wave_barrier();
    const int2 ent = s_list[wave][min(lane, cnt - 1)];
    __builtin_amdgcn_wave_barrier();
    // U blocks per trip: all U blocks' loads are issued before the first block's arithmetic.
    // Loads never depend on a branch (past the end they re-read the last block, a cache hit);
    // steps past the end are skipped.
    for (int t0 = 0; t0 < cnt; t0 += U) {
      KVRegs r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) at.load(r[u], bcast(ent.x, min(t0 + u, cnt - 1)));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u == 0 || t0 + u < cnt) at.step(r[u], bcast(ent.y, min(t0 + u, 63)), s_p[wave]);
    }
  }
  // head sums over the wave: l of head h lives in lanes h, h+16, h+32, h+48
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

// log-sum-exp merge of the splits of one (sequence, group): G heads x 128 dims
// grid (Hq, B), 256 threads: thread = (float4 column c of the head's 128 dims, split group sg);
// split group sg holds splits sg, sg + 8, ... (NB of them). Every partial load is issued before
// wave 0 reads the splits' (m, l), so the two round trips overlap.
template <typename T, int NB>
__global__ void __launch_bounds__(256) k_merge(AttendArgs a) {
  static_assert(8 * NB <= kMaxSplit, "split count");
  constexpr int kPer = (8 * NB + 63) / 64;
  __shared__ float s_w[8 * NB];
  __shared__ float s_ML[2];
  __shared__ float4 s_red[8][kD / 4];
  // (sequence, head) from the linear id as the attend launches place rows: row r = id % R on XCD
  // r % 8 when R = Hkv * B is a multiple of 8 (see split_row_of_block), its G heads at id / R
  int hq = blockIdx.x, b = blockIdx.y;
  {
    const int G = a.Hq / a.Hkv, R = a.Hkv * (int)gridDim.y;
    if ((R & 7) == 0) {
      const int id = (int)(blockIdx.x + gridDim.x * blockIdx.y), r = id % R;
      b = r / a.Hkv;
      hq = (r % a.Hkv) * G + id / R;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, c = tid & 31, sg = tid >> 5;
  const int ns = a.nsplit;
  const long long unit0 = ((long long)b * a.Hq + hq) * ns;   // split s -> unit0 + s
  const float* po = a.part_o + unit0 * kD + c * 4;
  float4 v[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
    v[i] = *reinterpret_cast<const float4*>(po + (long long)min(sg + 8 * i, ns - 1) * kD);
  if (tid < 64) {
    const float2* ml = reinterpret_cast<const float2*>(a.part_ml + unit0 * 2);
    float2 mlv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) mlv[i] = ml[min(lane + 64 * i, ns - 1)];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + 64 * i < ns) mx = fmaxf(mx, mlv[i].x);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int s2 = lane + 64 * i;
      if (s2 < ns && s2 < 8 * NB) {
        const float w = rescale(mlv[i].x, mx);
        s_w[s2] = w;
        L = fmaf(mlv[i].y, w, L);
      }
    }
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (lane == 0) { s_ML[0] = mx; s_ML[1] = L; }
  }
  __syncthreads();
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int s2 = sg + 8 * i;
    const float w = s2 < ns ? s_w[s2] : 0.f;
    sum.x = fmaf(v[i].x, w, sum.x); sum.y = fmaf(v[i].y, w, sum.y);
    sum.z = fmaf(v[i].z, w, sum.z); sum.w = fmaf(v[i].w, w, sum.w);
  }
  s_red[sg][c] = sum;
  __syncthreads();
  if (tid < kD / 4) {
    float4 t = s_red[0][c];
#pragma unroll
    for (int k2 = 1; k2 < 8; ++k2) {
      const float4 u = s_red[k2][c];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    const float L = s_ML[1];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T* out = reinterpret_cast<T*>(a.out);
    const long long oi = ((long long)b * a.Hq + hq) * kD + c * 4;
    store_out2<T>(out, oi, t.x * inv, t.y * inv);
    store_out2<T>(out, oi + 2, t.z * inv, t.w * inv);
    if (a.lse != nullptr && c == 0)
      a.lse[(long long)b * a.Hq + hq] = L > 0.f ? (s_ML[0] + log2f(L)) * kLn2 : -INFINITY;
  }
}

template <typename T>
hipError_t launch_merge(const AttendArgs& a, hipStream_t st) {
  const dim3 grid(a.Hq, a.B);
  if (log_enabled())
    log_launch("k_merge", grid, 256, 0, "%s, splits/8 = %d", sizeof(T) == 2 ? "bf16" : "f32",
               a.nsplit <= 8 ? 1 : a.nsplit <= 32 ? 4 : kMaxSplit / 8);
  if (a.nsplit <= 8) k_merge<T, 1><<<grid, 256, 0, st>>>(a);
  else if (a.nsplit <= 32) k_merge<T, 4><<<grid, 256, 0, st>>>(a);
  else k_merge<T, kMaxSplit / 8><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int G>
hipError_t launch_attend_g(const AttendArgs& a, hipStream_t st) {
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  if (log_enabled()) {
    if (sizeof(T) == 2) log_launch("k_attend_decode_mfma", grid, 256, 0, "G=%d, blocks in flight %d", G,
                                   a.blocks_per_split >= 4 ? 4 : 2);
    else log_launch("k_attend_decode", grid, 256, 0, "f32, G=%d", G);
  }
  if constexpr (sizeof(T) == 2) {
    if (a.blocks_per_split >= 4) k_attend_decode_mfma<G, 4><<<grid, 256, 0, st>>>(a);
    else k_attend_decode_mfma<G, 2><<<grid, 256, 0, st>>>(a);
  } else {
    k_attend_decode<T, G><<<grid, 256, 0, st>>>(a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nsplit == 1) return err;
  return launch_merge<T>(a, st);
}

template <typename T>
hipError_t launch_attend_typed(const AttendArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_attend_g<T, 1>(a, st);
    case 2: return launch_attend_g<T, 2>(a, st);
    case 3: return launch_attend_g<T, 3>(a, st);
    case 4: return launch_attend_g<T, 4>(a, st);
    case 5: return launch_attend_g<T, 5>(a, st);
    case 6: return launch_attend_g<T, 6>(a, st);
    case 7: return launch_attend_g<T, 7>(a, st);
    case 8: return launch_attend_g<T, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Blocks per workgroup: two when that already gives at most 512 workgroups (one or two per CU at
// small batch), else four (the attend kernel's blocks in flight), doubled while there would be
// more than 512 workgroups (large batches and large k: fewer, longer workgroups, fewer partials
// to merge) or more splits than one merge workgroup takes. With at least 256 (sequence, group)
// rows -- a workgroup per CU without splitting -- each row is one workgroup that writes the final
// output, and the merge launch goes away (batch 32 x 8 groups, k = 64: attend 104.6 -> 99.5 us).
int decode_blocks_per_split(int B, int Hkv, int k) {
  const long long rows = (long long)B * Hkv;
  if (k <= 2 || (rows * ((k + 1) / 2) <= 512 && (k + 1) / 2 <= kMaxSplit)) return 2;
  if (rows >= 256) return k;
  int bps = 4;
  while (bps < k && (rows * ((k + bps - 1) / bps) > 512 || (k + bps - 1) / bps > kMaxSplit)) bps *= 2;
  return bps;
}


hipError_t launch_merge_bf16(const AttendArgs& a, hipStream_t st) { return launch_merge<uint16_t>(a, st); }

hipError_t launch_attend_decode(bool bf16, const AttendArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  return bf16 ? launch_attend_typed<uint16_t>(a, G, st) : launch_attend_typed<float>(a, G, st);
}

}  // namespace msa
