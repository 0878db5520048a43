// Step 2, decode: gather-attend over the selected blocks of a paged KV cache.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 2: every query
// head of a GQA group attends with ordinary softmax attention over the real K/V of the group's
// selected blocks only; §1 (hardware alignment): one query group loads one KV block set;
// §3: decode time is bound by the KV-cache bandwidth, which selection cuts.
//
// The kernel is HBM-bound (about 4 FLOP per KV byte at G = 4), so it is built for streaming:
//   * grid = (split, group, sequence); a workgroup walks `blocks_per_split` entries of the
//     group's index list and reads each selected 64 x 128 K and V block (16 KiB each in bf16)
//     once, for all G heads of the group;
//   * each of the 4 waves owns 16 tokens of a block: lane l holds 8 dims (16 B) of rows
//     4i + l/16, so every load instruction reads four whole 256 B rows; all 8 K/V loads of a
//     block are issued before any arithmetic;
//   * q.k uses packed bf16 dot2 (v_dot2c_f32_bf16) and a 16-lane DPP row sum; the softmax is
//     online and wave-local (running max in the log2 domain, exp2), so no barrier is needed
//     inside the block loop; the 4 waves merge through LDS at the end;
//   * each workgroup writes an unnormalised partial (O, m, l) per head; k_merge (one workgroup
//     per (sequence, group), every partial load in flight at once) combines the splits with a
//     log-sum-exp merge and writes o (bf16 / fp32) and lse (natural log). With one split the
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

constexpr int kMaxSplit = 256;

template <typename T> __device__ __forceinline__ void store_out2(T* out, long long i, float a, float b);
template <> __device__ __forceinline__ void store_out2<uint16_t>(uint16_t* out, long long i, float a, float b) {
  reinterpret_cast<uint32_t*>(out)[i / 2] = pack_bf16x2(a, b);
}
template <> __device__ __forceinline__ void store_out2<float>(float* out, long long i, float a, float b) {
  reinterpret_cast<float2*>(out)[i / 2] = make_float2(a, b);
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

// log-sum-exp merge of the splits of one (sequence, group): G heads x 128 dims
template <typename T, int G>
__global__ void __launch_bounds__(256) k_merge(AttendArgs a) {
  __shared__ float s_w[kMaxSplit * G];
  __shared__ float s_M[G], s_L[G];
  __shared__ float4 s_red[256];
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ns = a.nsplit;
  const long long unit0 = ((long long)b * a.Hq + g * G) * ns;   // head h, split s -> unit0 + h*ns + s
  // thread -> float4 column c of G*128/4 and split group sg; its first batch of partial outputs
  // is requested before the (m, l) phase so that both round trips overlap
  constexpr int kCols = G * (kD / 4);
  constexpr int kGroups = 256 / kCols > 0 ? 256 / kCols : 1;
  constexpr int kBatch = 32;
  const int c = tid % kCols, sg = tid / kCols;
  const int hc = c / (kD / 4), c4 = c % (kD / 4);
  const float* po = a.part_o + (unit0 + hc * ns) * kD + c4 * 4;
  float4 v[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i)
    v[i] = *reinterpret_cast<const float4*>(po + (long long)min(sg + kGroups * i, ns - 1) * kD);
  // per-head max and weights: wave w handles heads w, w+4, ...
  for (int h = wave; h < G; h += 4) {
    const float* ml = a.part_ml + (unit0 + h * ns) * 2;
    float mv[kMaxSplit / 64], lv[kMaxSplit / 64];
#pragma unroll
    for (int i = 0; i < kMaxSplit / 64; ++i) {   // all loads first, from clamped addresses
      const int s2 = min(lane + 64 * i, ns - 1);
      mv[i] = ml[2 * s2];
      lv[i] = ml[2 * s2 + 1];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxSplit / 64; ++i)
      if (lane + 64 * i < ns) mx = fmaxf(mx, mv[i]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxSplit / 64; ++i) {
      const int s2 = lane + 64 * i;
      if (s2 < ns) {
        const float w = rescale(mv[i], mx);
        s_w[s2 * G + h] = w;
        L = fmaf(lv[i], w, L);
      }
    }
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (lane == 0) { s_M[h] = mx; s_L[h] = L; }
  }
  __syncthreads();
  // weighted sum of the partial outputs
  const int h = hc;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  if (sg < kGroups) {
    for (int s0 = sg; s0 < ns; s0 += kGroups * kBatch) {
      if (s0 != sg) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          v[i] = *reinterpret_cast<const float4*>(po + (long long)min(s0 + kGroups * i, ns - 1) * kD);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int s2 = s0 + kGroups * i;
        const float w = s2 < ns ? s_w[s2 * G + h] : 0.f;
        sum.x = fmaf(v[i].x, w, sum.x); sum.y = fmaf(v[i].y, w, sum.y);
        sum.z = fmaf(v[i].z, w, sum.z); sum.w = fmaf(v[i].w, w, sum.w);
      }
    }
    s_red[sg * kCols + c] = sum;   // kGroups * kCols <= 256
  }
  __syncthreads();
  if (sg == 0) {
    float4 t = s_red[c];
    for (int k2 = 1; k2 < kGroups; ++k2) {
      const float4 u = s_red[k2 * kCols + c];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    const float L = s_L[h];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T* out = reinterpret_cast<T*>(a.out);
    const long long oi = ((long long)b * a.Hq + g * G + h) * kD + c4 * 4;
    store_out2<T>(out, oi, t.x * inv, t.y * inv);
    store_out2<T>(out, oi + 2, t.z * inv, t.w * inv);
    if (a.lse != nullptr && c4 == 0)
      a.lse[(long long)b * a.Hq + g * G + h] = L > 0.f ? (s_M[h] + log2f(L)) * kLn2 : -INFINITY;
  }
}

template <typename T, int G>
hipError_t launch_attend_g(const AttendArgs& a, hipStream_t st) {
  k_attend_decode<T, G><<<dim3(a.nsplit, a.Hkv, a.B), 256, 0, st>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nsplit == 1) return err;
  k_merge<T, G><<<dim3(a.Hkv, a.B), 256, 0, st>>>(a);
  return hipGetLastError();
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

int decode_blocks_per_split(int B, int Hkv, int k) {
  const long long rows = (long long)B * Hkv;
  int bps = 1;
  while (bps < k && (rows * ((k + bps - 1) / bps) > 2048 || (k + bps - 1) / bps > kMaxSplit)) bps *= 2;
  return bps;
}


hipError_t launch_attend_decode(bool bf16, const AttendArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  return bf16 ? launch_attend_typed<uint16_t>(a, G, st) : launch_attend_typed<float>(a, G, st);
}

}  // namespace msa
