// Device helpers shared by the gfx950 kernels of libmsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kD = 128;        // head_dim
constexpr int kP = 64;         // tokens per block (== page)
constexpr int kMaxGroup = 8;   // query heads per KV head
constexpr int kHistBits = 12;  // coarse score histogram: top 12 bits of the order key
constexpr int kHistBins = 1 << kHistBits;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- 8 consecutive elements
// One lane's 16 B (bf16) or 32 B (fp32) slice of a 128-dim row, as a unit of load / store / sum.
template <typename T> struct Vec8;

template <> struct Vec8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = w; }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
  }
  __device__ __forceinline__ void add_to(float* acc) const {
    acc[0] += bf16lo(w.x); acc[1] += bf16hi(w.x); acc[2] += bf16lo(w.y); acc[3] += bf16hi(w.y);
    acc[4] += bf16lo(w.z); acc[5] += bf16hi(w.z); acc[6] += bf16lo(w.w); acc[7] += bf16hi(w.w);
  }
};

template <> struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ __forceinline__ void to_f32(float* f) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ void add_to(float* acc) const {
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
};

// ---------------------------------------------------------------- order-preserving key
// Larger float -> larger unsigned key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- cross-lane sums
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes; every lane of the row gets the row's sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// Maximum over each half (8 lanes) of a 16-lane row; every lane of the half gets it.
__device__ __forceinline__ float row8_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x141>(x));   // row_half_mirror
  return x;
}

// Combine the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float across_rows_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float across_rows_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte load marked non-temporal (the "nt" bit): for data read once per launch (block
// summaries, the selected K/V, index keys), so the stream does not displace reused lines.
typedef unsigned int u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 2^(a-b) for a <= b, with a = -inf giving 0 and a = b = -inf giving 0 (no NaN).
__device__ __forceinline__ float rescale(float a, float b) {
  return (a == -INFINITY) ? 0.0f : fast_exp2(a - b);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Visible length of a sequence, clamped so that no access leaves the block table.
__device__ __forceinline__ int clamp_len(int n, int max_len) {
  return n < 0 ? 0 : (n > max_len ? max_len : n);
}

__device__ __forceinline__ bool page_ok(int page, int num_pages) {
  return page >= 0 && page < num_pages;
}

}  // namespace msa
