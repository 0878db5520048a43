/* Test program (not part of the library): plain C use of libmsa's C ABI (include/msa.h). One fp32
 * decode step of a small seeded case (2 sequences of 1000 and 300 tokens, 8 query / 2 KV heads,
 * top-4, permuted pages, two planted blocks per sequence and group) through msa_workspace_size,
 * msa_build_summaries and msa_decode_step, checked against the fp64 oracle (orc_decode in
 * liboracle.so): index lists equal, outputs and lse within 1e-5 + 1e-5 |ref| (the fp32
 * tolerance). Device memory comes from the HIP runtime's C API; nothing else is needed.
 * Exit status 0 on success. Inputs come from splitmix64, a counter-based generator that holds
 * none of the method's arithmetic and serves both sides. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "msa.h"

/* the oracle's decode step (oracle.c): fp64, threaded over (sequence, group) units */
int orc_decode(int B, int Hq, int Hkv, int D, int P, int top_k, int keep_sink, int keep_local,
               int summary_bf16, double scale, int dtype, const void* q, const void* k_pool, const void* v_pool,
               int num_pages, const int32_t* block_table, int max_blocks, const int32_t* seq_lens,
               const double* summaries, const int32_t* idx_in, double* scores_out, int32_t* idx_out,
               double* o_out, double* lse_out, double* w_out, int nthreads);

static uint64_t g_ctr = 0x5eedull;
static double urand(void) {   /* splitmix64 -> uniform in [-1, 1) */
  uint64_t z = (g_ctr += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

#define HIP_OK(x)                                                                   \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                \
      return 2;                                                                     \
    }                                                                               \
  } while (0)
#define MSA_OK_(x)                                                                  \
  do {                                                                              \
    msa_status s_ = (x);                                                            \
    if (s_ != MSA_OK) {                                                             \
      fprintf(stderr, "%s failed: %s\n", #x, msa_status_string(s_));                \
      return 3;                                                                     \
    }                                                                               \
  } while (0)

enum { B = 2, HQ = 8, HKV = 2, D = 128, P = 64, K = 4, MAXB = 16, NPAGES = 21 };

int main(void) {
  const int lens[B] = {1000, 300};
  const int max_len = 1000;
  const double scale = 1.0 / sqrt((double)D);
  static float q[B * HQ * D], k[NPAGES * HKV * P * D], v[NPAGES * HKV * P * D];
  static int32_t table[B * MAXB];
  /* pages: sequence 0 takes 16 pages, sequence 1 the next 5, in a fixed permutation */
  for (int i = 0; i < B * MAXB; ++i) table[i] = -1;
  for (int j = 0; j < 16; ++j) table[j] = (7 * j + 3) % 16;
  for (int j = 0; j < 5; ++j) table[MAXB + j] = 16 + (3 * j + 1) % 5;
  for (int i = 0; i < B * HQ * D; ++i) q[i] = (float)(0.5 + 0.25 * urand());
  for (int i = 0; i < NPAGES * HKV * P * D; ++i) {
    k[i] = (float)(0.3 * urand());
    v[i] = (float)urand();
  }
  /* planted: logical blocks 2 and 11 of sequence 0, 1 and 4 of sequence 1, every group */
  const int planted[B][2] = {{2, 11}, {1, 4}};
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < 2; ++t) {
      const int page = table[b * MAXB + planted[b][t]];
      for (int g = 0; g < HKV; ++g)
        for (int r = 0; r < P; ++r)
          for (int d = 0; d < D; ++d) k[(((size_t)page * HKV + g) * P + r) * D + d] += 0.5f;
    }

  /* the GPU path through the C ABI */
  float *dq, *dk, *dv, *ds, *dout, *dlse, *dscores;
  int32_t *dtable, *dlens, *didx;
  void* dws;
  HIP_OK(hipMalloc((void**)&dq, sizeof q));
  HIP_OK(hipMalloc((void**)&dk, sizeof k));
  HIP_OK(hipMalloc((void**)&dv, sizeof v));
  HIP_OK(hipMalloc((void**)&ds, sizeof(float) * NPAGES * HKV * D));
  HIP_OK(hipMalloc((void**)&dout, sizeof(float) * B * HQ * D));
  HIP_OK(hipMalloc((void**)&dlse, sizeof(float) * B * HQ));
  HIP_OK(hipMalloc((void**)&dscores, sizeof(float) * B * HKV * MAXB));
  HIP_OK(hipMalloc((void**)&dtable, sizeof table));
  HIP_OK(hipMalloc((void**)&dlens, sizeof lens));
  HIP_OK(hipMalloc((void**)&didx, sizeof(int32_t) * B * HKV * K));
  HIP_OK(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, k, sizeof k, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dtable, table, sizeof table, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, lens, sizeof lens, hipMemcpyHostToDevice));

  msa_config cfg = {0};
  cfg.num_q_heads = HQ;
  cfg.num_kv_heads = HKV;
  cfg.head_dim = D;
  cfg.block_size = P;
  cfg.top_k = K;
  cfg.softmax_scale = (float)scale;
  cfg.q_dtype = cfg.kv_dtype = cfg.out_dtype = MSA_F32;
  cfg.score_mode = MSA_SCORE_MEAN_KEY;
  cfg.q_tile = 64;
  cfg.summary_dtype = MSA_F32;
  msa_kv_cache cache = {dk, dv, ds, dtable, dlens, NPAGES, MAXB};
  size_t ws_bytes = 0;
  MSA_OK_(msa_workspace_size(&cfg, MSA_OP_DECODE, B, max_len, 0, &ws_bytes));
  HIP_OK(hipMalloc(&dws, ws_bytes));
  MSA_OK_(msa_build_summaries(&cfg, &cache, B, max_len, NULL));
  MSA_OK_(msa_decode_step(&cfg, dq, &cache, B, max_len, NULL, NULL, didx, dscores, dout, dlse, dws, ws_bytes, NULL));
  /* an invalid call is refused before anything is enqueued */
  if (msa_decode_step(&cfg, dq, &cache, B, max_len, NULL, NULL, didx, dscores, dout, dlse, dws, ws_bytes - 1, NULL) !=
      MSA_ERR_WORKSPACE) {
    fprintf(stderr, "a short workspace was not refused\n");
    return 4;
  }
  HIP_OK(hipDeviceSynchronize());
  static float out[B * HQ * D], lse[B * HQ];
  static int32_t idx[B * HKV * K];
  HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, dlse, sizeof lse, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(idx, didx, sizeof idx, hipMemcpyDeviceToHost));

  /* the oracle on the same inputs */
  static double o_ref[B * HQ * D], lse_ref[B * HQ];
  static int32_t idx_ref[B * HKV * K];
  const int rc = orc_decode(B, HQ, HKV, D, P, K, 0, 0, 0, scale, 0, q, k, v, NPAGES, table, MAXB, lens, NULL, NULL,
                            NULL, idx_ref, o_ref, lse_ref, NULL, 1);
  if (rc != 0) {
    fprintf(stderr, "orc_decode failed (%d)\n", rc);
    return 5;
  }
  int bad = 0;
  for (int i = 0; i < B * HKV * K; ++i)
    if (idx[i] != idx_ref[i]) {
      fprintf(stderr, "idx[%d] = %d, oracle %d\n", i, idx[i], idx_ref[i]);
      ++bad;
    }
  double worst = 0.0;
  for (int i = 0; i < B * HQ * D; ++i) {
    const double err = fabs((double)out[i] - o_ref[i]), lim = 1e-5 + 1e-5 * fabs(o_ref[i]);
    if (err / lim > worst) worst = err / lim;
    if (err > lim && bad++ < 8) fprintf(stderr, "o[%d] = %.9g, oracle %.9g\n", i, out[i], o_ref[i]);
  }
  for (int i = 0; i < B * HQ; ++i) {
    const double err = fabs((double)lse[i] - lse_ref[i]), lim = 1e-5 + 1e-5 * fabs(lse_ref[i]);
    if (err / lim > worst) worst = err / lim;
    if (err > lim && bad++ < 16) fprintf(stderr, "lse[%d] = %.9g, oracle %.9g\n", i, lse[i], lse_ref[i]);
  }
  printf("C ABI decode step: lists %s, worst error / tolerance %.3f, %s\n", bad ? "checked" : "equal", worst,
         bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
