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
//   * each workgroup writes an unnormalised partial (O, m, l) per head; k_merge combines the
//     splits with a log-sum-exp merge and writes o (bf16 / fp32) and lse (natural log).
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

  const int32_t* ids = a.idx + ((long long)b * a.Hkv + g) * a.k;
  for (int e = e0; e < e1; ++e) {
    const int j = ids[e];
    if (j < 0 || j >= nb) continue;
    const int page = a.table[(long long)b * a.max_blocks + j];
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

// log-sum-exp merge of the splits: one wave per (sequence, head), 2 dims per lane
template <typename TO>
__global__ void __launch_bounds__(256) k_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                               int nsplit, int units, TO* __restrict__ out, float* __restrict__ lse) {
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= units) return;
  const float* ml = part_ml + (long long)unit * nsplit * 2;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  const float* po = part_o + (long long)unit * nsplit * kD + 2 * lane;
  for (int s = 0; s < nsplit; ++s) {
    const float w = rescale(ml[2 * s], M);
    L = fmaf(ml[2 * s + 1], w, L);
    const float2 v = *reinterpret_cast<const float2*>(po + (long long)s * kD);
    o0 = fmaf(v.x, w, o0);
    o1 = fmaf(v.y, w, o1);
  }
  float lv = -INFINITY;
  if (L > 0.f) {
    o0 /= L;
    o1 /= L;
    lv = (M + log2f(L)) * kLn2;
  } else {
    o0 = o1 = 0.f;
  }
  if constexpr (sizeof(TO) == 2) {
    reinterpret_cast<uint32_t*>(out)[(long long)unit * (kD / 2) + lane] = f32_to_bf16_bits(o0) | (f32_to_bf16_bits(o1) << 16);
  } else {
    reinterpret_cast<float2*>(out)[(long long)unit * (kD / 2) + lane] = make_float2(o0, o1);
  }
  if (lse != nullptr && lane == 0) lse[unit] = lv;
}

template <typename T>
hipError_t launch_attend_typed(const AttendArgs& a, int G, hipStream_t st) {
  const dim3 grid(a.nsplit, a.Hkv, a.B);
  switch (G) {
    case 1: k_attend_decode<T, 1><<<grid, 256, 0, st>>>(a); break;
    case 2: k_attend_decode<T, 2><<<grid, 256, 0, st>>>(a); break;
    case 3: k_attend_decode<T, 3><<<grid, 256, 0, st>>>(a); break;
    case 4: k_attend_decode<T, 4><<<grid, 256, 0, st>>>(a); break;
    case 5: k_attend_decode<T, 5><<<grid, 256, 0, st>>>(a); break;
    case 6: k_attend_decode<T, 6><<<grid, 256, 0, st>>>(a); break;
    case 7: k_attend_decode<T, 7><<<grid, 256, 0, st>>>(a); break;
    case 8: k_attend_decode<T, 8><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int units = a.B * a.Hq;
  const dim3 mgrid((units + 3) / 4);
  k_merge<T><<<mgrid, 256, 0, st>>>(a.part_o, a.part_ml, a.nsplit, units, reinterpret_cast<T*>(a.out), a.lse);
  return hipGetLastError();
}

}  // namespace

int decode_blocks_per_split(int B, int Hkv, int k) {
  const long long rows = (long long)B * Hkv;
  int bps = 1;
  while (bps < k && rows * ((k + bps - 1) / bps) > 2048) bps *= 2;
  return bps;
}

hipError_t launch_attend_decode(bool bf16, const AttendArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  return bf16 ? launch_attend_typed<uint16_t>(a, G, st) : launch_attend_typed<float>(a, G, st);
}

}  // namespace msa
