// hbm_probe.hip -- HBM bandwidth ceiling of MI355X for read/write mixes.
//
// Measures streaming kernels with R read streams and W write streams of
// 16-byte vectors (each wave sweeps U consecutive 1 KiB runs of every
// stream per iteration, as the shard-step kernels do), so that a kernel's
// achieved GB/s can be set against what the memory system sustains for the
// same mix on the same box.  Two launch shapes: a fixed grid striding over
// the streams, and a one-shot grid (one sweep per wave) laid out as F
// separated fronts, as the norm pass is.  Stream i starts i * 1280 bytes
// past a 2 MiB boundary, so that the streams do not all hit the same HBM
// channel at the same offset (the shard-step rows are staggered the same
// way).  Mixes, per 8 shard elements:
//   R1W0   pure read                    R0W1   pure write
//   R1W1   copy
//   R16W2  norm pass at N_d = 16: 16 bf16 rows in, fp32 spill out
//   R8W8   clipped update: spill + fp32 state in, state + bf16 + int8 out
//   R64W0  the rows of the N_d = 64 update (plus its small state stream)
// Every access is in bounds: the sweep stops at the last whole chunk.
// Build and run:  hipcc --offload-arch=gfx950 -O3 hbm_probe.hip -o hbm_probe
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
constexpr int kMaxIn = 64, kMaxOut = 8;
struct Streams {
  const u32x4 *in[kMaxIn];
  u32x4 *out[kMaxOut];
};

// F = 0: fixed grid, grid-stride loop.  F > 0: one sweep per wave, block b
// in front b mod F (the grid is a multiple of F).
template <int R, int W, int U, int F>
__global__ void __launch_bounds__(256) probe(const Streams S, long n, unsigned *sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long span = 64L * U;
  long first = ((long)blockIdx.x * 4 + wave) * span, stride = (long)gridDim.x * 4 * span;
  if (F > 0) {
    const long per_front = (long)gridDim.x / (F > 0 ? F : 1);
    const long slot = (long)(blockIdx.x % (F > 0 ? F : 1)) * per_front + blockIdx.x / (F > 0 ? F : 1);
    first = (slot * 4 + wave) * span;
    stride = n;  // one sweep
  }
  unsigned acc = 0;
  for (long wb = first; wb + span <= n; wb += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = (u32x4){0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] += __builtin_nontemporal_load(S.in[r] + wb + 64 * u + lane);
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int u = 0; u < U; ++u) S.out[w][wb + 64 * u + lane] = v[u] + (unsigned)w;
#pragma unroll
    for (int u = 0; u < U; ++u) acc += v[u].x ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the reads alive
}

static void check(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

template <int R, int W, int U, int F = 0>
static double run(const Streams &S, long n, int grid, unsigned *sink) {
  if (F > 0) {  // one-shot: one block per 4 * 64 * U vectors, a multiple of F
    const long blocks = n / (4L * 64 * U);
    grid = int((blocks + F - 1) / F * F);
  }
  hipEvent_t a, b;
  check(hipEventCreate(&a), "event");
  check(hipEventCreate(&b), "event");
  hipLaunchKernelGGL((probe<R, W, U, F>), dim3(grid), dim3(256), 0, 0, S, n, sink);
  check(hipEventRecord(a), "record");
  const int iters = 4;
  for (int it = 0; it < iters; ++it)
    hipLaunchKernelGGL((probe<R, W, U, F>), dim3(grid), dim3(256), 0, 0, S, n, sink);
  check(hipEventRecord(b), "record");
  check(hipEventSynchronize(b), "sync");
  float ms = 0;
  check(hipEventElapsedTime(&ms, a, b), "elapsed");
  return double(R + W) * n * 16.0 * iters / (ms * 1e-3) / 1e9;
}

template <int R, int W>
static void mix(const char *name, const Streams &S, long n, unsigned *sink) {
  const int grids[] = {2048, 16384, 65536};
  double best = 0;
  std::printf("%-6s", name);
  for (int g : grids) {
    const double a = run<R, W, 1>(S, n, g, sink), b = run<R, W, 4>(S, n, g, sink);
    std::printf("  g%-5d U1 %6.0f U4 %6.0f", g, a, b);
    best = a > best ? a : best;
    best = b > best ? b : best;
  }
  const double o14 = run<R, W, 4, 1>(S, n, 0, sink), o24 = run<R, W, 4, 2>(S, n, 0, sink),
               o28 = run<R, W, 8, 2>(S, n, 0, sink);
  std::printf("  one-shot F1 U4 %6.0f F2 U4 %6.0f F2 U8 %6.0f", o14, o24, o28);
  for (double x : {o14, o24, o28}) best = x > best ? x : best;
  std::printf("  | best %6.0f GB/s\n", best);
  std::fflush(stdout);
}

int main() {
  // 64 input streams of 512 MiB (32 GiB), 8 output streams of 512 MiB (each
  // larger than the 256 MB last-level cache);
  // n vectors per stream, a multiple of every sweep span.
  const long n = (512L << 20) / 16;
  Streams S;
  const long stagger = 1280 / 16;  // vectors
  for (int i = 0; i < kMaxIn; ++i) {
    u32x4 *p;
    check(hipMalloc(&p, (n + kMaxIn * stagger) * 16), "malloc");
    check(hipMemset(p, i, (n + kMaxIn * stagger) * 16), "memset");
    S.in[i] = p + i * stagger;
  }
  for (int i = 0; i < kMaxOut; ++i) {
    u32x4 *p;
    check(hipMalloc(&p, (n + (kMaxIn + kMaxOut) * stagger) * 16), "malloc");
    S.out[i] = p + (kMaxIn + i) * stagger;
  }
  unsigned *sink;
  check(hipMalloc(&sink, 64), "malloc");
  hipDeviceProp_t prop;
  check(hipGetDeviceProperties(&prop, 0), "props");
  std::printf("device %s, %d CUs; GB/s per mix (grid, lane-vectors per wave sweep)\n",
              prop.gcnArchName, prop.multiProcessorCount);
  mix<1, 0>("R1W0", S, n, sink);
  mix<0, 1>("R0W1", S, n, sink);
  mix<1, 1>("R1W1", S, n, sink);
  mix<16, 2>("R16W2", S, n, sink);
  mix<8, 8>("R8W8", S, n, sink);
  mix<64, 0>("R64W0", S, n, sink);
  return 0;
}
