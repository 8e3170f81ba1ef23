/*
 * c_abi_step.c -- the shard step driven from plain C through the library's
 * C ABI (include/zero_shard.h) and the HIP runtime API, with no Python and
 * no PyTorch in the process.  Used by tests/test_gpu_c_abi.py.
 *
 * Usage: c_abi_step IN OUT [graph]
 * With "graph" the step is captured once into a HIP graph and replayed at
 * every step: the allocation-free norm pass (zero_shard_gnorm_noalloc, no
 * spill) and zero_shard_step_dev, which re-reads the contributions and takes
 * lr, lr*wd and the bias corrections from a device array the program
 * refreshes (zero_shard_step_consts) before each replay, outside the graph.
 * IN (little-endian, packed):
 *   int64 n; int32 n_d; int32 quant_block; int32 steps;
 *   float lr, weight_decay, max_norm;
 *   float master[n], m[n], v[n];
 *   uint16 rows[steps][n_d][n]      bf16 contributions of each step
 * OUT:
 *   float master[n], m[n], v[n]; uint16 p[n];
 *   int8 codes[n]; float scales[ceil(n / quant_block)]  (if quant_block > 0)
 *   double sumsq[steps]             (if max_norm > 0: each step's S)
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_shard.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));            \
      return 1;                                                             \
    }                                                                       \
  } while (0)

#define ZS_OK_(call)                                                        \
  do {                                                                      \
    int z_ = (call);                                                        \
    if (z_ != ZS_OK) {                                                      \
      fprintf(stderr, "%s: %s\n", #call, zero_shard_strerror(z_));          \
      return 1;                                                             \
    }                                                                       \
  } while (0)

static int read_all(FILE *f, void *p, size_t bytes) {
  return fread(p, 1, bytes, f) == bytes ? 0 : 1;
}

int main(int argc, char **argv) {
  if (argc != 3 && !(argc == 4 && strcmp(argv[3], "graph") == 0)) {
    fprintf(stderr, "usage: %s IN OUT [graph]\n", argv[0]);
    return 2;
  }
  const int graph = argc == 4;
  FILE *in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int64_t n;
  int32_t nd, qb, steps;
  float lr, wd, max_norm;
  if (read_all(in, &n, 8) || read_all(in, &nd, 4) || read_all(in, &qb, 4) ||
      read_all(in, &steps, 4) || read_all(in, &lr, 4) || read_all(in, &wd, 4) ||
      read_all(in, &max_norm, 4)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  if (n < 1 || nd < 1 || nd > ZS_MAX_ND || steps < 1 || qb < 0) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  const int64_t nb = qb ? (n + qb - 1) / qb : 0;
  const size_t f32 = (size_t)n * 4, b16 = (size_t)n * 2;
  float *h_state = (float *)malloc(3 * f32);
  uint16_t *h_rows = (uint16_t *)malloc((size_t)steps * nd * b16);
  if (!h_state || !h_rows) return 1;
  if (read_all(in, h_state, 3 * f32) || read_all(in, h_rows, (size_t)steps * nd * b16)) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  fclose(in);

  float *master, *m, *v, *gbar = NULL, *scales = NULL;
  uint16_t *p;
  int8_t *codes = NULL;
  double *sumsq;
  HIP_OK(hipMalloc((void **)&master, f32));
  HIP_OK(hipMalloc((void **)&m, f32));
  HIP_OK(hipMalloc((void **)&v, f32));
  HIP_OK(hipMalloc((void **)&p, b16));
  HIP_OK(hipMalloc((void **)&sumsq, 8 * (size_t)steps));
  if (max_norm > 0.0f) HIP_OK(hipMalloc((void **)&gbar, f32));
  if (qb) {
    HIP_OK(hipMalloc((void **)&codes, (size_t)n));
    HIP_OK(hipMalloc((void **)&scales, (size_t)nb * 4));
  }
  zs_bf16 *rows[ZS_MAX_ND];
  for (int k = 0; k < nd; ++k) HIP_OK(hipMalloc((void **)&rows[k], b16));
  HIP_OK(hipMemcpy(master, h_state, f32, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(m, h_state + n, f32, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, h_state + 2 * n, f32, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  zs_desc d;
  memset(&d, 0, sizeof d);
  d.phi = n;
  d.n_d = nd;
  d.r = 0;
  d.shard_len = n;
  d.beta1 = 0.9f;
  d.beta2 = 0.999f;
  d.eps = 1e-8f;
  d.weight_decay = wd;
  d.bias_correction = 1;
  d.max_norm = max_norm;
  d.quant_block = qb;
  d.master = master;
  d.m = m;
  d.v = v;
  d.param_out = p;
  d.q_codes = codes;
  d.q_scales = scales;
  d.gbar_ws = gbar;
  d.stream = stream;
  if (graph) d.gbar_ws = NULL;  /* the captured step re-reads the contributions */
  zs_handle *h = NULL;
  ZS_OK_(zero_shard_init(&d, &h));
  const zs_bf16 *const *c = (const zs_bf16 *const *)rows;
  if (!graph) {
    for (int32_t s = 0; s < steps; ++s) {
      for (int k = 0; k < nd; ++k)
        HIP_OK(hipMemcpyAsync(rows[k], h_rows + ((size_t)s * nd + k) * n, b16,
                              hipMemcpyHostToDevice, stream));
      if (max_norm > 0.0f) {
        ZS_OK_(zero_shard_gnorm(h, c, sumsq + s));
        ZS_OK_(zero_shard_step(h, NULL, lr, s + 1, sumsq + s));  /* reads the spill */
      } else {
        ZS_OK_(zero_shard_step(h, c, lr, s + 1, NULL));
      }
    }
  } else {
    double *consts_dev, *ssq;
    double *consts_host = (double *)malloc((size_t)steps * 4 * sizeof(double));
    if (!consts_host) return 1;
    HIP_OK(hipMalloc((void **)&consts_dev, 4 * sizeof(double)));
    HIP_OK(hipMalloc((void **)&ssq, sizeof(double)));
    for (int32_t s = 0; s < steps; ++s)
      ZS_OK_(zero_shard_step_consts(&d, lr, s + 1, consts_host + 4 * (size_t)s));
    hipGraph_t g;
    hipGraphExec_t exec;
    HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
    if (max_norm > 0.0f) ZS_OK_(zero_shard_gnorm_noalloc(&d, c, ssq));
    ZS_OK_(zero_shard_step_dev(h, c, consts_dev, max_norm > 0.0f ? ssq : NULL));
    HIP_OK(hipStreamEndCapture(stream, &g));
    HIP_OK(hipGraphInstantiate(&exec, g, NULL, NULL, 0));
    for (int32_t s = 0; s < steps; ++s) {
      for (int k = 0; k < nd; ++k)
        HIP_OK(hipMemcpyAsync(rows[k], h_rows + ((size_t)s * nd + k) * n, b16,
                              hipMemcpyHostToDevice, stream));
      HIP_OK(hipMemcpyAsync(consts_dev, consts_host + 4 * (size_t)s, 4 * sizeof(double),
                            hipMemcpyHostToDevice, stream));
      HIP_OK(hipGraphLaunch(exec, stream));
      if (max_norm > 0.0f)
        HIP_OK(hipMemcpyAsync(sumsq + s, ssq, sizeof(double), hipMemcpyDeviceToDevice,
                              stream));
    }
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipGraphExecDestroy(exec));
    HIP_OK(hipGraphDestroy(g));
    HIP_OK(hipFree(consts_dev));
    HIP_OK(hipFree(ssq));
    free(consts_host);
  }
  HIP_OK(hipStreamSynchronize(stream));

  FILE *out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 1;
  }
  void *buf = malloc(f32 > (size_t)steps * 8 ? f32 : (size_t)steps * 8);
  if (!buf) return 1;
  float *arrs[3] = {master, m, v};
  for (int i = 0; i < 3; ++i) {
    HIP_OK(hipMemcpy(buf, arrs[i], f32, hipMemcpyDeviceToHost));
    fwrite(buf, 1, f32, out);
  }
  HIP_OK(hipMemcpy(buf, p, b16, hipMemcpyDeviceToHost));
  fwrite(buf, 1, b16, out);
  if (qb) {
    HIP_OK(hipMemcpy(buf, codes, (size_t)n, hipMemcpyDeviceToHost));
    fwrite(buf, 1, (size_t)n, out);
    HIP_OK(hipMemcpy(buf, scales, (size_t)nb * 4, hipMemcpyDeviceToHost));
    fwrite(buf, 1, (size_t)nb * 4, out);
  }
  if (max_norm > 0.0f) {
    HIP_OK(hipMemcpy(buf, sumsq, 8 * (size_t)steps, hipMemcpyDeviceToHost));
    fwrite(buf, 1, 8 * (size_t)steps, out);
  }
  if (fclose(out) != 0) return 1;
  ZS_OK_(zero_shard_free(h));
  HIP_OK(hipStreamDestroy(stream));
  free(buf);
  free(h_state);
  free(h_rows);
  return 0;
}
