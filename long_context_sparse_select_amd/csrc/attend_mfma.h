// Building blocks of the bf16 decode attend shared by the attend kernels of libmsa: the
// per-wave MFMA attend over one selected 64-token block, and the end of a workgroup (its
// per-head (m, l, O) combined over its four waves into the output or a split partial).
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 2: every query
// head of a GQA group attends with ordinary softmax attention over the real K/V of the group's
// selected blocks; one query group loads one KV block set.
#pragma once

#include "common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kMaxSplit = kMaxDecodeSplit;

// Workgroup -> (split, group, sequence) for a grid (nsplit, Hkv, B). Workgroups go to the 8 XCDs
// round-robin by linear id, so when the row count R = Hkv * B is a multiple of 8, taking
// row = id % R and split = id / R puts every split of a row on XCD row % 8, the XCD whose L2 then
// holds the row's partials for k_merge (which maps its workgroups the same way). Any mapping is
// correct; this one only places work.
struct SplitRow { int split, g, b; };
__device__ __forceinline__ SplitRow split_row_of_block() {
  const int R = (int)(gridDim.y * gridDim.z);
  if ((R & 7) != 0) return {(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
  const int id = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  const int row = id % R;
  return {id / R, row % (int)gridDim.y, row / (int)gridDim.y};
}

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

  // Issues the block's eight 16-byte loads, non-temporal (a selected block is read once per
  // launch); the scheduling barrier keeps them ahead of the arithmetic that follows in program order.
  __device__ __forceinline__ void load(KVRegs& r, int page) const {
    const long long base = (long long)page * page_stride + head_off;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)   // A operand: key 16w + hq, dims 32kk + 8c
      r.k[kk] = load_nt(kpool + base + (16 * wave + hq) * kD + 32 * kk + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i)      // PV layout: token 16w + 4i + row, dims d0
      r.v[i] = load_nt(vpool + base + (16 * wave + 4 * i + row) * kD + d0);
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

}  // namespace
}  // namespace msa
