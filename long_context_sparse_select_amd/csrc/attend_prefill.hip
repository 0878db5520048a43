// Step 2, prefill: MFMA attention of 64-query tiles over their selected blocks.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 2 and the
// hardware-alignment note: every head of a GQA group shares the group's selection, so one
// query group loads one KV block set and runs a dense attention over it; §3: in prefill the
// savings fall on this main attention. Readings: selection per 64-query tile and group; the
// tile's diagonal block is always attended, causally (key position <= query position).
//
// One workgroup per (tile, KV group): rows = 64 tokens x G heads (256 for G = 4), 2G waves of
// 32 rows (wave w -> head w/2, tokens 32*(w%2) .. +31). For each selected block (64 keys):
//   * K (row-major, padded) and V (transposed, [dim][key], padded) are staged in LDS by the
//     whole workgroup; the next block's K/V are already in flight into registers while the
//     current one is computed;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (2 key tiles x 8 k-steps). Each lane owns one
//     query row (its C column), so the softmax row max needs one exchange with lane ^ 32;
//   * keys are fed to the A operand in an order with bits 2 and 3 of the key index swapped,
//     which makes the S^T accumulator registers of a lane, converted to bf16, exactly the
//     P^T B operand of O^T = V^T P^T (8 consecutive keys per lane and k-step): no LDS round
//     trip for P;
//   * online softmax in the log2 domain, fp32 statistics, fp32 accumulation in the MFMA.
#include "common.h"
#include "kernels.h"

namespace msa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKPitch = 136;  // K rows in LDS: 128 dims + 8 pad (bf16 elements)
constexpr int kVPitch = 72;   // V^T rows in LDS: 64 keys + 8 pad

__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }


template <int G>
struct PrefillBlockLoader {
  static constexpr int NT = 128 * G;                  // threads
  static constexpr int KI = (1024 + NT - 1) / NT;     // 16 B K chunks per thread
  static constexpr int VI = (512 + NT - 1) / NT;      // V key pairs per thread
  uint4 kreg[KI];
  uint4 vreg[VI][2];

  __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb, int tid) {
#pragma unroll
    for (int it = 0; it < KI; ++it) {
      const int q = tid + NT * it;
      if (q < 1024) kreg[it] = *reinterpret_cast<const uint4*>(kb + (q >> 4) * kD + (q & 15) * 8);
    }
#pragma unroll
    for (int it = 0; it < VI; ++it) {
      const int q = tid + NT * it;
      if (q < 512) {
        const int w = q >> 6, l = q & 63;
        const int tp = (l & 15) + 16 * (w & 1), dc = 4 * (w >> 1) + (l >> 4);
        vreg[it][0] = *reinterpret_cast<const uint4*>(vb + (2 * tp) * kD + dc * 8);
        vreg[it][1] = *reinterpret_cast<const uint4*>(vb + (2 * tp + 1) * kD + dc * 8);
      }
    }
  }

  // keys >= nvalid are stored as zeros (they are masked, and 0 * garbage must not reach P.V)
  __device__ __forceinline__ void store(uint16_t* sK, uint16_t* sV, int tid, int nvalid) {
#pragma unroll
    for (int it = 0; it < KI; ++it) {
      const int q = tid + NT * it;
      if (q < 1024) {
        const int t = q >> 4;
        const uint4 v = t < nvalid ? kreg[it] : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(sK + t * kKPitch + (q & 15) * 8) = v;
      }
    }
#pragma unroll
    for (int it = 0; it < VI; ++it) {
      const int q = tid + NT * it;
      if (q < 512) {
        const int w = q >> 6, l = q & 63;
        const int tp = (l & 15) + 16 * (w & 1), dc = 4 * (w >> 1) + (l >> 4);
        const uint4 a = 2 * tp < nvalid ? vreg[it][0] : make_uint4(0u, 0u, 0u, 0u);
        const uint4 b = 2 * tp + 1 < nvalid ? vreg[it][1] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
        uint32_t* dst = reinterpret_cast<uint32_t*>(sV + (dc * 8) * kVPitch + 2 * tp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // dims 8dc + 2e (low halves) and 8dc + 2e + 1 (high halves) of keys 2tp, 2tp+1
          dst[(2 * e) * (kVPitch / 2)] = (av[e] & 0xffffu) | (bv[e] << 16);
          dst[(2 * e + 1) * (kVPitch / 2)] = (av[e] >> 16) | (bv[e] & 0xffff0000u);
        }
      }
    }
  }
};

template <int G>
__global__ void __launch_bounds__(128 * G) k_attend_prefill(PrefillArgs a) {
  __shared__ __align__(16) uint16_t sK[kP * kKPitch];
  __shared__ __align__(16) uint16_t sV[kD * kVPitch];
  const int tau = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = lane & 31, c = lane >> 5;
  const int h = w >> 1;
  const int il = (w & 1) * 32 + n;                 // token within the tile
  const int i0 = tau * kP;
  const int rows_valid = min(kP, a.T - i0);
  const int diag = a.past_len / kP + tau;
  const bool row_ok = il < rows_valid;
  const int qhead = g * G + h;

  // Q^T fragments: lane (n, c) holds dims 16kk + 8c .. +7 of its query row
  bf16x8 qf[8];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((long long)(i0 + il) * a.Hq + qhead) * kD;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = as_bf16x8(row_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * c) : make_uint4(0u, 0u, 0u, 0u));
  }

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int32_t* ids = a.idx + ((long long)tau * a.Hkv + g) * (a.k + 1);
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(a.kpool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(a.vpool);
  auto valid_page = [&](int e, int* page) -> bool {
    const int j = ids[e];
    if (j < 0 || j > diag) return false;
    const int p = a.table[j];
    *page = p;
    return page_ok(p, a.num_pages);
  };
  auto next_valid = [&](int e, int* page) -> int {
    while (e <= a.k && !valid_page(e, page)) ++e;
    return e;
  };

  PrefillBlockLoader<G> ld;
  int page = -1;
  int e = next_valid(0, &page);
  if (e <= a.k) {
    const long long head = ((long long)page * a.Hkv + g) * kP * kD;
    ld.load(kpool + head, vpool + head, tid);
  }
  while (e <= a.k) {
    const int j = ids[e];
    const bool is_diag = j == diag;
    const int nvalid = is_diag ? rows_valid : kP;
    __syncthreads();                               // the previous block's LDS reads are done
    ld.store(sK, sV, tid, nvalid);
    __syncthreads();
    int page2 = -1;
    const int e2 = next_valid(e + 1, &page2);
    if (e2 <= a.k) {                               // next block in flight during this one
      const long long head = ((long long)page2 * a.Hkv + g) * kP * kD;
      ld.load(kpool + head, vpool + head, tid);
    }

    // ---- S^T = K Q^T: tile t holds keys swap23(32t + row)
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
      const uint16_t* krow = sK + swap_bits23(32 * t + n) * kKPitch + 8 * c;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(krow + 16 * kk));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], s[t], 0, 0, 0);
      }
    }
    // ---- online softmax (log2 domain): max on raw scores, p = exp2(s * scale - m)
    if (is_diag) {  // causal mask inside the diagonal block only
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // C row of register i in lane group c -> S^T row -> key index within the block
          const int key = swap_bits23(32 * t + 8 * (i >> 2) + 4 * c + (i & 3));
          if (key > il) s[t][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
    const float mn = fmaxf(m, mx);
    const float mref = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(m - mref);        // m = -inf -> 0
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[t][i], a.scale_log2, -mref));
        s[t][i] = p;
        psum += p;
      }
    l = l * alpha + psum;
    m = mn;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    // ---- P^T operands straight from the accumulators: k-step ks uses registers 8(ks%2) .. +7
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int t = ks >> 1, b = (ks & 1) * 8;
      pf[ks] = as_bf16x8(make_uint4(pack_bf16x2(s[t][b + 0], s[t][b + 1]), pack_bf16x2(s[t][b + 2], s[t][b + 3]),
                                    pack_bf16x2(s[t][b + 4], s[t][b + 5]), pack_bf16x2(s[t][b + 6], s[t][b + 7])));
    }
    // ---- O^T += V^T P^T: dim tile dt, keys 16ks + 8c .. +7
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t* vrow = sV + (32 * dt + n) * kVPitch + 8 * c;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 16 * ks));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[ks], o[dt], 0, 0, 0);
      }
    }
    e = e2;
  }

  // ---- normalise and write: lane (n, c) holds dims 32dt + 8(i/4) + 4c + (i%4) of its row
  const float ltot = l + __shfl_xor(l, 32);
  if (!row_ok) return;
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((long long)(i0 + il) * a.Hq + qhead) * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint2 pk;
      pk.x = pack_bf16x2(o[dt][4 * i4 + 0] * inv, o[dt][4 * i4 + 1] * inv);
      pk.y = pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * i4 + 4 * c) = pk;
    }
  if (a.lse != nullptr && c == 0)
    a.lse[(long long)(i0 + il) * a.Hq + qhead] = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_attend_prefill(const PrefillArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid((a.T + kP - 1) / kP, a.Hkv);
  switch (G) {
    case 1: k_attend_prefill<1><<<grid, 128, 0, st>>>(a); break;
    case 2: k_attend_prefill<2><<<grid, 256, 0, st>>>(a); break;
    case 3: k_attend_prefill<3><<<grid, 384, 0, st>>>(a); break;
    case 4: k_attend_prefill<4><<<grid, 512, 0, st>>>(a); break;
    case 5: k_attend_prefill<5><<<grid, 640, 0, st>>>(a); break;
    case 6: k_attend_prefill<6><<<grid, 768, 0, st>>>(a); break;
    case 7: k_attend_prefill<7><<<grid, 896, 0, st>>>(a); break;
    case 8: k_attend_prefill<8><<<grid, 1024, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
