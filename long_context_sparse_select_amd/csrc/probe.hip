// Measurement probes of the GPU itself (declared in msa_probe.h): a streaming HBM read and a bf16
// MFMA chain. They give the rooflines of the method's kernels a denominator measured on the GPU
// at hand beside the published one.
#include "common.h"
#include "kernels.h"
#include "msa_probe.h"

namespace msa {

namespace {

constexpr int kReadBlocks = 2048;   // workgroups of the read probe (eight per CU; swept: 1024-4096)
constexpr int kReadUnroll = 8;      // 16 B loads in flight per thread

__global__ void __launch_bounds__(256) k_probe_read(const uint4* __restrict__ p, long long n16,
                                                    float* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * 256 * kReadUnroll;
  uint32_t acc = 0u;
  for (long long base = (long long)blockIdx.x * 256 * kReadUnroll + threadIdx.x; base < n16; base += stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const long long i = base + (long long)u * 256;
      v[u] = i < n16 ? p[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // every thread's fold is stored, so no load can be dropped (2 MiB of writes against the read)
  sink[(long long)blockIdx.x * 256 + threadIdx.x] = (float)(acc & 0xffffu);
}

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) k_probe_mfma(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16x8_p a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)((float)((lane + e) & 7) * 0.125f);
    b[e] = (__bf16)((float)((lane * 3 + e) & 7) * -0.0625f);
  }
  f32x16_p c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  if (lane == 0) sink[blockIdx.x * 4 + wave] = s;   // every wave's result is used
}

}  // namespace

}  // namespace msa

extern "C" {

msa_status msa_probe_hbm_read(const void* buf, size_t bytes, float* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0) return MSA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return MSA_ERR_INVALID_ARG;
  if (msa::log_enabled()) msa::log_launch("k_probe_read", dim3(msa::kReadBlocks), 256, 0, "%zu B", bytes);
  msa::k_probe_read<<<msa::kReadBlocks, 256, 0, (hipStream_t)stream>>>(
      static_cast<const uint4*>(buf), (long long)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

msa_status msa_probe_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, void* stream) {
  if (sink == nullptr || workgroups < 1 || workgroups > 65535 || iters < 1) return MSA_ERR_INVALID_ARG;
  if (msa::log_enabled()) msa::log_launch("k_probe_mfma", dim3(workgroups), 256, 0, "%d rounds", iters);
  msa::k_probe_mfma<<<workgroups, 256, 0, (hipStream_t)stream>>>(sink, iters);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

}  // extern "C"
