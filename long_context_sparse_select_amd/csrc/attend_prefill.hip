// Step 2, prefill: MFMA attention of 64-query tiles over their selected blocks.
//
// "MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 2 and the
// hardware-alignment note: every head of a GQA group shares the group's selection, so one
// query group loads one KV block set and runs a dense attention over it; §3: in prefill the
// savings fall on this main attention. Readings: selection per 64-query tile and group; the
// tile's diagonal block is always attended, causally (key position <= query position).
//
// One workgroup per (tile, KV group): rows = 64 tokens x G heads (256 for G = 4), 2G waves of
// 32 rows (wave w -> head w/2, tokens 32*(w%2) .. +31). A group of more than 4 heads is split
// over two workgroups of ceil(G/2) heads each, which stage the same blocks: one workgroup of
// 2G > 8 waves would need more registers per lane than a CU holds for them. A short chunk also
// splits each tile's list over several workgroups (too few (tile, group) pairs to fill the chip),
// which write partial softmax states that k_merge_prefill combines. The diagonal block is
// attended first, then the selected blocks in list order (the online softmax does not depend on
// the order).
// For each block (64 keys):
//   * K (row-major, padded) and V (transposed, [dim][key], padded) are staged in LDS by the
//     whole workgroup into one of two buffers while the other is read; the loads of the block
//     after next are already in flight into registers; one barrier per block;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (2 key tiles x 8 k-steps). Each lane owns one
//     query row (its C column), so the softmax row max needs one exchange with lane ^ 32;
//   * keys are fed to the A operand in an order with bits 2 and 3 of the key index swapped,
//     which makes the S^T accumulator registers of a lane, converted to bf16, exactly the
//     P^T B operand of O^T = V^T P^T (8 consecutive keys per lane and k-step): no LDS round
//     trip for P;
//   * online softmax in the log2 domain, fp32 statistics, fp32 accumulation in the MFMA; the
//     reference max moves only when a row's max outgrows it by 2^8, so the O rescale is rare;
//     the causal mask is a branch taken on the diagonal block only.
// At the roofline the kernel is bound by HBM: at k = 32 each (tile, group) streams 33 blocks of
// K and V for ~250 FLOP per byte, under the chip's ridge. It runs well below that floor, limited
// on chip: each 32-row wave reads the whole K and V^T block from LDS (1 KiB per 32 KFLOP of
// MFMA), and the two waves of a SIMD meet the same barrier, so MFMA, LDS and softmax phases add
// up. The fragment reads are issued four MFMAs ahead, and the first V^T fragments are requested
// before the softmax.
#include <algorithm>

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

// Online-softmax state of one wave (32 query rows; lane (n, c) holds row n's statistics).
// The running max used for P moves only when a row's max grows by more than kLazy (log2 units):
// P = exp2(s * scale - m) then stays <= 2^kLazy and the O/l rescale is skipped for most blocks.
// The algebra is exact for any reference max; only rounding differs.
constexpr float kLazy = 8.f;

template <int G>
struct PrefillWave {
  bf16x8 qf[8];       // Q^T fragments: lane (n, c) holds dims 16kk + 8c .. +7 of its query row
  f32x16 o[4];        // O^T accumulators: dim tile dt, rows = the wave's 32 queries
  float m, l;         // reference max (log2 domain) and running sum of this lane's 32 keys
  int n, c, il;
  float scale_log2;

  __device__ __forceinline__ void step(const uint16_t* sK, const uint16_t* sV, bool diag_block) {
    // ---- S^T = K Q^T: tile t holds keys swap23(32t + row). Fragment f = (t = f/8, kk = f%8),
    // read from LDS four fragments ahead of its MFMA.
    constexpr int kAhead = 4;
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;
    const uint16_t* krow0 = sK + swap_bits23(n) * kKPitch + 8 * c;
    const uint16_t* krow1 = sK + swap_bits23(32 + n) * kKPitch + 8 * c;
    uint4 kf[kAhead];
#pragma unroll
    for (int f = 0; f < kAhead; ++f) kf[f] = *reinterpret_cast<const uint4*>((f < 8 ? krow0 : krow1) + 16 * (f % 8));
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      const bf16x8 af = as_bf16x8(kf[f % kAhead]);
      if (f + kAhead < 16) {
        const int g2 = f + kAhead;
        kf[f % kAhead] = *reinterpret_cast<const uint4*>((g2 < 8 ? krow0 : krow1) + 16 * (g2 % 8));
      }
      s[f / 8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[f % 8], s[f / 8], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // first V^T fragments requested before the softmax: fragment f = (dt = f/4, ks = f%4)
    const uint16_t* vbase = sV + n * kVPitch + 8 * c;
    uint4 vf[kAhead];
#pragma unroll
    for (int f = 0; f < kAhead; ++f) vf[f] = *reinterpret_cast<const uint4*>(vbase + (32 * (f / 4)) * kVPitch + 16 * (f % 4));
    if (diag_block) {  // causal mask: key position within the block <= query position
      __builtin_amdgcn_sched_barrier(0);   // keeps the mask a branch, not selects on every block
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
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
    // move the reference only when the row's max outgrows it by more than kLazy
    const bool grow = mx > m + kLazy || (m == -INFINITY && mx != -INFINITY);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform
      const float mn = grow ? mx : m;
      const float alpha = fast_exp2(m - mn);        // 1 for rows that keep m; m = -inf -> 0
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      m = mn;
    }
    const float mref = m == -INFINITY ? 0.f : m;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[t][i], scale_log2, -mref));
        s[t][i] = p;
        psum += p;
      }
    l += psum;
    // ---- P^T operands straight from the accumulators: k-step ks uses registers 8(ks%2) .. +7
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int t = ks >> 1, b = (ks & 1) * 8;
      pf[ks] = as_bf16x8(make_uint4(pack_bf16x2(s[t][b + 0], s[t][b + 1]), pack_bf16x2(s[t][b + 2], s[t][b + 3]),
                                    pack_bf16x2(s[t][b + 4], s[t][b + 5]), pack_bf16x2(s[t][b + 6], s[t][b + 7])));
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T P^T: dim tile dt, keys 16ks + 8c .. +7; fragments four ahead
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      const bf16x8 af = as_bf16x8(vf[f % kAhead]);
      if (f + kAhead < 16) {
        const int g2 = f + kAhead;
        vf[f % kAhead] = *reinterpret_cast<const uint4*>(vbase + (32 * (g2 / 4)) * kVPitch + 16 * (g2 % 4));
      }
      o[f / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[f % 4], o[f / 4], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

constexpr int kKBuf = kP * kKPitch;    // bf16 elements of one staged K block
constexpr int kVBuf = kD * kVPitch;    // bf16 elements of one staged V^T block

// G = 2 (four waves) is held to 256 registers per lane so that two workgroups share a CU, two
// waves per SIMD (unbounded, the compiler took 312 and one workgroup per CU ran 40 % slower);
// G = 3 at three waves per SIMD would spill, and G = 4 runs two per SIMD within its own bound
template <int G>
__global__ void __launch_bounds__(128 * G, G == 2 ? 2 : 1) k_attend_prefill(PrefillArgs a) {
  // G here is the heads of one workgroup; a group of more heads is split over hsplit workgroups
  // of G heads (the last may hold fewer: its other waves stage and wait only); with a.nsplit > 1
  // the tile's list is split too (gridDim.z = hsplit * a.nsplit)
  // two staging buffers: block i is read from buffer i%2 while block i+1 is written to the other,
  // so one barrier per block separates the two
  __shared__ __align__(16) uint16_t sK[2 * kKBuf];
  __shared__ __align__(16) uint16_t sV[2 * kVBuf];
  const int tau = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int h = w >> 1;
  const int i0 = tau * kP;
  const int rows_valid = min(kP, a.T - i0);
  const int diag = a.past_len / kP + tau;
  const int group = a.Hq / a.Hkv;
  const int hsplit = (group + G - 1) / G;
  const int hs = (int)blockIdx.z % hsplit, ks = (int)blockIdx.z / hsplit;
  const int h0 = hs * G;
  const bool head_ok = h0 + h < group;                  // uniform per wave
  const int qhead = g * group + min(h0 + h, group - 1);

  PrefillWave<G> wv;
  PrefillBlockLoader<G> ld;
  wv.n = lane & 31;
  wv.c = lane >> 5;
  wv.il = (w & 1) * 32 + wv.n;                     // token within the tile
  wv.scale_log2 = a.scale_log2;
  const bool row_ok = wv.il < rows_valid;
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((long long)(i0 + wv.il) * a.Hq + qhead) * kD;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      wv.qf[kk] = as_bf16x8(row_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * kk + 8 * wv.c)
                                   : make_uint4(0u, 0u, 0u, 0u));
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) wv.o[dt][i] = 0.f;
  wv.m = -INFINITY;
  wv.l = 0.f;

  const int32_t* ids = a.idx + ((long long)tau * a.Hkv + g) * (a.k + 1);
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(a.kpool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(a.vpool);
  auto block_head = [&](int page) { return ((long long)page * a.Hkv + g) * kP * kD; };
  // Split ks of a.nsplit attends the list slots [e_lo, e_hi) and, the first one, the diagonal
  // block. Selected entries: indices below the diagonal with a valid page (the list also holds the
  // diagonal itself and -1 padding, both skipped here)
  const int per = (a.k + a.nsplit) / a.nsplit;    // ceil((k + 1) / nsplit)
  const int e_lo = min(a.k + 1, ks * per), e_hi = min(a.k + 1, e_lo + per);
  auto next_valid = [&](int e, int* page) -> int {
    for (; e < e_hi; ++e) {
      const int j = ids[e];
      if (j < 0 || j >= diag) continue;
      const int p = a.table[j];
      if (page_ok(p, a.num_pages)) { *page = p; return e; }
    }
    return e;
  };

  // Order: the diagonal block first (causal), then the selected blocks; the online softmax does
  // not depend on the order. The loop stages block i+1 into one LDS buffer while block i is read
  // from the other, with the loads of block i+2 in flight: one barrier per block.
  const int pdiag = a.table[diag];
  const bool with_diag = ks == 0 && page_ok(pdiag, a.num_pages);
  int pe = -1;
  int e;                                           // list position of the staged block; e_lo - 1 = diagonal
  if (with_diag) { e = e_lo - 1; pe = pdiag; }
  else e = next_valid(e_lo, &pe);
  if (e < e_hi) {
    ld.load(kpool + block_head(pe), vpool + block_head(pe), tid);
    ld.store(sK, sV, tid, with_diag ? rows_valid : kP);
    int pe2 = -1;
    int e2 = next_valid(e + 1, &pe2);
    if (e2 < e_hi) ld.load(kpool + block_head(pe2), vpool + block_head(pe2), tid);
    __syncthreads();
    int buf = 0;
    bool diag_block = with_diag;
    for (;;) {
      if (head_ok) wv.step(sK + buf * kKBuf, sV + buf * kVBuf, diag_block);
      if (e2 >= e_hi) break;
      ld.store(sK + (buf ^ 1) * kKBuf, sV + (buf ^ 1) * kVBuf, tid, kP);
      int pe3 = -1;
      const int e3 = next_valid(e2 + 1, &pe3);
      if (e3 < e_hi) ld.load(kpool + block_head(pe3), vpool + block_head(pe3), tid);
      e2 = e3;
      buf ^= 1;
      diag_block = false;
      __syncthreads();                             // the staged block is complete; the old one is free
    }
  }

  // ---- normalise and write: lane (n, c) holds dims 32dt + 8(i/4) + 4c + (i%4) of its row
  const float ltot = wv.l + __shfl_xor(wv.l, 32);
  if (!row_ok || !head_ok) return;
  const long long orow_i = (long long)(i0 + wv.il) * a.Hq + qhead;
  if (a.nsplit > 1) {   // split-K partial: O and l relative to the reference max m (log2 domain)
    const long long unit = orow_i * a.nsplit + ks;
    float* po = a.part_o + unit * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(po + 32 * dt + 8 * i4 + 4 * wv.c) =
            make_float4(wv.o[dt][4 * i4 + 0], wv.o[dt][4 * i4 + 1], wv.o[dt][4 * i4 + 2], wv.o[dt][4 * i4 + 3]);
    if (wv.c == 0) {
      a.part_ml[unit * 2] = wv.m;
      a.part_ml[unit * 2 + 1] = ltot;
    }
    return;
  }
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + orow_i * kD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint2 pk;
      pk.x = pack_bf16x2(wv.o[dt][4 * i4 + 0] * inv, wv.o[dt][4 * i4 + 1] * inv);
      pk.y = pack_bf16x2(wv.o[dt][4 * i4 + 2] * inv, wv.o[dt][4 * i4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * i4 + 4 * wv.c) = pk;
    }
  if (a.lse != nullptr && wv.c == 0)
    a.lse[orow_i] = ltot > 0.f ? (wv.m + log2f(ltot)) * kLn2 : -INFINITY;
}

// Log-sum-exp merge of the list splits of every (token, head) row of a split prefill chunk:
// 32 lanes per row (4 of its 128 dims each), 8 rows per workgroup. Split s of a row holds O_s and
// l_s relative to its own reference m_s (m_s = -inf: the split attended nothing); with
// M = max_s m_s, the row's O = sum_s 2^(m_s - M) O_s, l = sum_s 2^(m_s - M) l_s, out = O / l and
// lse = (M + log2 l) ln 2.
__global__ void __launch_bounds__(256) k_merge_prefill(const float* __restrict__ part_o,
                                                       const float* __restrict__ part_ml, int rows, int ns,
                                                       uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int l32 = threadIdx.x & 31;
  const long long row = (long long)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + row * ns;
  const float4* po = reinterpret_cast<const float4*>(part_o + row * ns * kD) + l32;   // split s at + 32 s
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[s].x);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const float2 v = ml[s];
    const float4 o = po[32 * s];
    const float wgt = rescale(v.x, M);   // 0 for a split that attended nothing
    L = fmaf(v.y, wgt, L);
    acc.x = fmaf(o.x, wgt, acc.x); acc.y = fmaf(o.y, wgt, acc.y);
    acc.z = fmaf(o.z, wgt, acc.z); acc.w = fmaf(o.w, wgt, acc.w);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<uint2*>(out + row * kD + 4 * l32) =
      make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
  if (lse != nullptr && l32 == 0) lse[row] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

int prefill_splits(int T, int Hq, int Hkv, int k) {
  const int hsplit = Hq / Hkv > 4 ? 2 : 1;
  const long long units = (long long)((T + kP - 1) / kP) * Hkv * hsplit;
  if (units >= kPrefillSplitTarget) return 1;
  const int s = (int)((kPrefillSplitTarget + units - 1) / units);
  return std::max(1, std::min({s, (k + 1) / 2, kMaxDecodeSplit}));
}

hipError_t launch_merge_prefill(const PrefillArgs& a, hipStream_t st) {
  const int rows = a.T * a.Hq;
  const dim3 grid((rows + 7) / 8);
  if (log_enabled()) log_launch("k_merge_prefill", grid, 256, 0, "%d rows x %d splits", rows, a.nsplit);
  k_merge_prefill<<<grid, 256, 0, st>>>(a.part_o, a.part_ml, rows, a.nsplit, reinterpret_cast<uint16_t*>(a.out),
                                        a.lse);
  return hipGetLastError();
}

hipError_t launch_attend_prefill(const PrefillArgs& a, hipStream_t st) {
  // groups of up to 4 heads take one workgroup; wider groups are split over two workgroups of
  // ceil(G / 2) heads, so that no instance needs more than 512 threads (and their registers);
  // a.nsplit > 1 splits every tile's list over that many workgroups as well
  const int G = a.Hq / a.Hkv;
  const int hsplit = G > 4 ? 2 : 1;
  const int hw = (G + hsplit - 1) / hsplit;
  if (a.nsplit < 1 || (a.nsplit > 1 && (a.part_o == nullptr || a.part_ml == nullptr))) return hipErrorInvalidValue;
  const dim3 grid((a.T + kP - 1) / kP, a.Hkv, hsplit * a.nsplit);
  if (log_enabled())
    log_launch("k_attend_prefill", grid, 128 * hw, 0, "G=%d, heads per workgroup=%d, list splits=%d, k=%d", G, hw,
               a.nsplit, a.k);
  switch (hw) {
    case 1: k_attend_prefill<1><<<grid, 128, 0, st>>>(a); break;
    case 2: k_attend_prefill<2><<<grid, 256, 0, st>>>(a); break;
    case 3: k_attend_prefill<3><<<grid, 384, 0, st>>>(a); break;
    case 4: k_attend_prefill<4><<<grid, 512, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nsplit == 1) return err;
  return launch_merge_prefill(a, st);
}

}  // namespace msa
