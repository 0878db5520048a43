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

constexpr int kMaxSplit = kMaxDecodeSplit;

template <typename T> __device__ __forceinline__ void store_out2(T* out, long long i, float a, float b);
template <> __device__ __forceinline__ void store_out2<uint16_t>(uint16_t* out, long long i, float a, float b) {
  reinterpret_cast<uint32_t*>(out)[i / 2] = pack_bf16x2(a, b);
}
template <> __device__ __forceinline__ void store_out2<float>(float* out, long long i, float a, float b) {
  reinterpret_cast<float2*>(out)[i / 2] = make_float2(a, b);
}

// A workgroup's (m, l, O) per head over its blocks -> the output (one split) or a partial.
template <typename T, int G>
__device__ __forceinline__ void write_partials(const AttendArgs& a, float (*s_m)[G], float (*s_l)[G],
                                               float (*s_o)[G][kD], int b, int g, int split, int tid) {
  T* out = reinterpret_cast<T*>(a.out);
  if (a.nsplit == 1) {  // the workgroup holds the whole row: normalise and write
    for (int x = 2 * tid; x < G * kD; x += 512) {
      const int h = x / kD, d = x % kD;
      const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
      float O0 = 0.f, O1 = 0.f, L = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = rescale(s_m[w][h], M);
        O0 = fmaf(s_o[w][h][d], sc, O0);
        O1 = fmaf(s_o[w][h][d + 1], sc, O1);
        L = fmaf(s_l[w][h], sc, L);
      }
      const long long oi = ((long long)b * a.Hq + g * G + h) * kD + d;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      store_out2<T>(out, oi, O0 * inv, O1 * inv);
      if (a.lse != nullptr && d == 0)
        a.lse[(long long)b * a.Hq + g * G + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
    return;
  }
  for (int x = tid; x < G * kD; x += 256) {
    const int h = x / kD, d = x % kD;
    const float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) O = fmaf(s_o[w][h][d], rescale(s_m[w][h], M), O);
    const long long unit = ((long long)b * a.Hq + g * G + h) * a.nsplit + split;
    a.part_o[unit * kD + d] = O;
    if (d == 0) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) L = fmaf(s_l[w][h], rescale(s_m[w][h], M), L);
      a.part_ml[unit * 2] = M;
      a.part_ml[unit * 2 + 1] = L;
    }
  }
}

template <typename T, int G>
__global__ void __launch_bounds__(256) k_attend_decode(AttendArgs a) {
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
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

// bf16 decode attend with the q.k contraction on MFMA.
// Wave w owns keys 16w .. 16w+15 of each block. S^T (16 keys x 16 head columns, G real) comes from
// four v_mfma_f32_16x16x32_bf16 (A = the keys' rows, B = the group's queries; lane l holds head
// l%16 and keys 4*(l/16) + j). The wave's softmax state is per head; P goes through a small
// per-wave LDS patch as bf16 pairs along tokens, and P.V runs as packed bf16 dot2 in the layout
// where lane l owns 8 dims of token rows 4i + l/16 (V pairs along tokens built with v_perm_b32).
// A workgroup reads its block list once (lane e holds block e's page), compacts the attended
// blocks, and walks them U at a time with all U blocks' K/V loads in flight together.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct KVRegs { uint4 k[4], v[4]; };

template <int G>
struct MfmaAttend {
  const uint16_t* kpool;
  const uint16_t* vpool;
  long long page_stride, head_off;   // elements per page, offset of KV head g inside a page
  int wave, lane, hq, c, row, d0;
  float scale_log2;
  bf16x8_t qf[4];                    // B operand: head hq, dims 32kk + 8c .. +7 (zero past G)
  float m_l, l_l;                    // QK layout: state of head hq over this lane's keys
  float acc[G][8];                   // PV layout: head h, dims d0 .. d0+7
  float m_h[G];                      // wave-uniform running max per head

  // Issues the block's eight 16-byte loads; the scheduling barrier keeps them ahead of the
  // arithmetic that follows in program order.
  __device__ __forceinline__ void load(KVRegs& r, int page) const {
    const long long base = (long long)page * page_stride + head_off;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)   // A operand: key 16w + hq, dims 32kk + 8c
      r.k[kk] = *reinterpret_cast<const uint4*>(kpool + base + (16 * wave + hq) * kD + 32 * kk + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i)      // PV layout: token 16w + 4i + row, dims d0
      r.v[i] = *reinterpret_cast<const uint4*>(vpool + base + (16 * wave + 4 * i + row) * kD + d0);
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ __forceinline__ void step(KVRegs& r, int ntok, uint16_t (*sp)[4][4]) {
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[kk]), qf[kk], st, 0, 0, 0);
    // logits of head hq for keys 16w + 4c + jj (log2 domain); keys past the length masked
    float z[4];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      z[jj] = 16 * wave + 4 * c + jj < ntok ? st[jj] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, z[jj]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m_l, mx);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha_l = fast_exp2(m_l - mref);   // -inf -> 0
    float p[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) p[jj] = fast_exp2(z[jj] - mref);
    l_l = l_l * alpha_l + ((p[0] + p[1]) + (p[2] + p[3]));
    m_l = mn;
    if (hq < G) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)   // key 4c + jj is token row jj of pair slot c
        sp[hq][jj][c] = (uint16_t)(pack_bf16x2(p[jj], 0.f) & 0xffffu);
    }
    if (ntok < kP) {   // slots past the length never reach the accumulator
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * wave + 4 * i + row >= ntok) r.v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    // V pairs along tokens: (t_0, t_1) and (t_2, t_3) for each 2-dim word
    uint32_t vlo[2][4], vhi[2][4];
    const uint32_t* v32 = reinterpret_cast<const uint32_t*>(r.v);
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const uint32_t x0 = v32[(2 * pr) * 4 + w4], x1 = v32[(2 * pr + 1) * 4 + w4];
        vlo[pr][w4] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        vhi[pr][w4] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's P patch is written
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mn), h));
      const float ah = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha_l), h));
      if (ah != 1.f) {
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) acc[h][e2] *= ah;
      }
      m_h[h] = mh;
      const uint2 pp = *reinterpret_cast<const uint2*>(&sp[h][row][0]);   // (p_i0, p_i1), (p_i2, p_i3)
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        acc[h][2 * w4] = dot2_bf16(pp.x, vlo[0][w4], acc[h][2 * w4]);
        acc[h][2 * w4 + 1] = dot2_bf16(pp.x, vhi[0][w4], acc[h][2 * w4 + 1]);
        acc[h][2 * w4] = dot2_bf16(pp.y, vlo[1][w4], acc[h][2 * w4]);
        acc[h][2 * w4 + 1] = dot2_bf16(pp.y, vhi[1][w4], acc[h][2 * w4 + 1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
};

__device__ __forceinline__ int bcast(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

template <int G, int U>
__global__ void __launch_bounds__(256) k_attend_decode_mfma(AttendArgs a) {
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_o[4][G][kD];
  __shared__ uint16_t s_p[4][G][4][4];     // per wave: [head][token row r][pair slot i] -> key 4i + r
  __shared__ int2 s_list[4][64];           // per wave: (page, live tokens) of the attended blocks
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
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
  const int hq = blockIdx.x, b = blockIdx.y;
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
  if (a.nsplit <= 8) k_merge<T, 1><<<grid, 256, 0, st>>>(a);
  else if (a.nsplit <= 32) k_merge<T, 4><<<grid, 256, 0, st>>>(a);
  else k_merge<T, kMaxSplit / 8><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int G>
hipError_t launch_attend_g(const AttendArgs& a, hipStream_t st) {
  const dim3 grid(a.nsplit, a.Hkv, a.B);
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


hipError_t launch_attend_decode(bool bf16, const AttendArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  return bf16 ? launch_attend_typed<uint16_t>(a, G, st) : launch_attend_typed<float>(a, G, st);
}

}  // namespace msa
