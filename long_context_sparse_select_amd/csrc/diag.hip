// Diagnostics of libmsa: launch logging and device-side checks of the caller's index data.
//
// With MSA_LOG set to a non-empty value other than "0" in the environment (read once, at the
// first launch or entry-point call), every entry point prints one line with its arguments and the
// layout it chose, and every kernel launch one line with the kernel, its template parameters,
// grid, threads per workgroup and dynamic LDS bytes, on stderr. Off by default; when off, the
// cost is one test of a cached flag per launch.
//
// With MSA_DEVICE_CHECKS set the same way, every entry point that reads a paged cache first checks,
// on the device, what the kernels otherwise tolerate silently: a seq_lens value outside
// [0, min(max_seq_len, max_blocks * 64)] (the kernels clamp it), a page id outside [0, num_pages)
// for a visible block (its block scores -inf and is never attended), and, for msa_attend, a valid
// block index listed twice in one row (the one case the contract leaves undefined). The first
// violation found is printed on stderr and the call returns MSA_ERR_INVALID_ARG with nothing else
// enqueued. The check synchronises the stream, so it is a debugging mode: it is skipped while the
// stream is being captured into a graph. Its result word is a file-scope device array, so the mode
// allocates nothing (msa_decode_step_noalloc included).
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace msa {

namespace {
std::mutex g_log_mutex;

// result of the last check on this GPU: {code, sequence, position, value}; code 0 = no violation
__device__ int32_t check_word[4];

__device__ void report(int32_t* w, int code, int b, int pos, int value) {
  if (atomicCAS(&w[0], 0, code) == 0) {
    w[1] = b;
    w[2] = pos;
    w[3] = value;
  }
}

__global__ void k_check_clear(int32_t* w) {
  if (threadIdx.x < 4) w[threadIdx.x] = 0;
}

// grid (ceil(max_blocks / 256), B): thread (b, j) checks sequence b's length (j = 0) and, when the
// length is in range, the page id of its block j when j is visible (a length out of range is
// reported alone, not with the table padding it would reach)
__global__ void __launch_bounds__(256) k_check_cache(const int32_t* __restrict__ table,
                                                     const int32_t* __restrict__ lens, int fixed_len,
                                                     int max_blocks, int max_len, int num_pages, int32_t* w) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int lim = (long long)max_blocks * 64 < max_len ? max_blocks * 64 : max_len;
  const int n = lens != nullptr ? lens[b] : fixed_len;
  if (n < 0 || n > lim) {   // uniform per sequence
    if (j == 0) report(w, 1, b, 0, n);
    return;
  }
  const int nb = (n + 63) / 64;
  if (j < nb) {
    const int p = table[(long long)b * max_blocks + j];
    if (p < 0 || p >= num_pages) report(w, 2, b, j, p);
  }
}

// one workgroup per (sequence, group) row of an attend list: a valid entry (0 <= e < nb_b) seen
// twice (either occurrence may be the one reported); a bitmap of the row's blocks in dynamic LDS
// (nbits bits, a multiple of 32)
__global__ void __launch_bounds__(256) k_check_repeats(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ lens, int max_len, int k,
                                                       int Hkv, int nbits, int32_t* w) {
  extern __shared__ uint32_t bits[];
  const int row = blockIdx.x, b = row / Hkv;
  for (int i = threadIdx.x; i < nbits / 32; i += 256) bits[i] = 0u;
  __syncthreads();
  int n = lens[b];
  n = n < 0 ? 0 : (n > max_len ? max_len : n);
  const int nb = (n + 63) / 64;
  for (int i = threadIdx.x; i < k; i += 256) {
    const int e = idx[(long long)row * k + i];
    if (e >= 0 && e < nb && e < nbits) {
      const uint32_t m = 1u << (e & 31);
      if (atomicOr(&bits[e >> 5], m) & m) report(w, 3, b, (row % Hkv) * k + i, e);
    }
  }
}

int32_t* check_word_of_current_device() {
  static std::mutex mu;
  static int32_t* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_word)) != hipSuccess) return nullptr;
    ptrs[dev] = static_cast<int32_t*>(p);
  }
  return ptrs[dev];
}
}  // namespace

bool checks_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("MSA_DEVICE_CHECKS");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

int device_check(const char* entry, const CheckArgs& a, hipStream_t st) {
  if (!checks_enabled()) return 0;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess) return -1;
  if (cap != hipStreamCaptureStatusNone) return 0;   // a check must synchronise: not under capture
  int32_t* w = check_word_of_current_device();
  if (w == nullptr) return -1;
  k_check_clear<<<1, 64, 0, st>>>(w);
  if (a.B > 0 && a.max_blocks > 0) {
    const dim3 grid((a.max_blocks + 255) / 256, a.B);
    k_check_cache<<<grid, 256, 0, st>>>(a.table, a.lens, a.fixed_len, a.max_blocks, a.max_len, a.num_pages, w);
  }
  if (a.idx != nullptr && a.B > 0 && a.k > 0) {
    const long long mb = ((long long)a.max_len + 63) / 64;
    const int nbits = (int)((mb < kCheckMaxBits ? mb : kCheckMaxBits) + 31) / 32 * 32;
    if (nbits > 0)
      k_check_repeats<<<a.B * a.Hkv, 256, (size_t)nbits / 8, st>>>(a.idx, a.lens, a.max_len, a.k, a.Hkv, nbits, w);
  }
  int32_t h[4] = {0, 0, 0, 0};
  if (hipGetLastError() != hipSuccess) return -1;
  if (hipMemcpyAsync(h, w, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess) return -1;
  if (hipStreamSynchronize(st) != hipSuccess) return -1;
  if (h[0] == 0) return 0;
  char msg[256];
  if (h[0] == 1)
    std::snprintf(msg, sizeof(msg), "seq_lens[%d] = %d is outside [0, min(max_seq_len, max_blocks * 64)]", h[1], h[3]);
  else if (h[0] == 2)
    std::snprintf(msg, sizeof(msg), "block_table[%d][%d] = %d is not a page id in [0, num_pages)", h[1], h[2], h[3]);
  else
    std::snprintf(msg, sizeof(msg), "idx[%d][%d][%d] = %d repeats a block already listed in its row", h[1],
                  h[2] / a.k, h[2] % a.k, h[3]);
  std::lock_guard<std::mutex> lock(g_log_mutex);
  std::fprintf(stderr, "[msa] MSA_DEVICE_CHECKS: %s: %s\n", entry, msg);
  return 1;
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("MSA_LOG");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void log_call(const char* fmt, ...) {
  if (!log_enabled()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::lock_guard<std::mutex> lock(g_log_mutex);
  std::fprintf(stderr, "[msa] %s\n", buf);
}

void log_launch(const char* kernel, dim3 grid, int threads, size_t lds_bytes, const char* fmt, ...) {
  if (!log_enabled()) return;
  char detail[256] = "";
  if (fmt != nullptr) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(detail, sizeof(detail), fmt, ap);
    va_end(ap);
  }
  std::lock_guard<std::mutex> lock(g_log_mutex);
  std::fprintf(stderr, "[msa]   launch %s<%s> grid %u x %u x %u, %d threads, %zu B dynamic LDS\n", kernel, detail,
               grid.x, grid.y, grid.z, threads, lds_bytes);
}

}  // namespace msa
