// zero_shard_offload.cpp -- the ZeRO-Offload pipeline of one rank's shard
// (declared in include/zero_shard.h: zero_shard_offload_*).
//
// ZeRO-Offload keeps the optimizer states and their update on the host and
// hides the update behind the GPU's next step with a one-step delayed
// update ("ZeRO (딥 러닝)", follow-ups table "후속 기법").  Per step s:
//
//   GPU, caller's stream   norm pass of step s (averaged gradient -> the
//                          device spill, S_local -> a device scalar)
//   download stream        S_local, then the spill in chunks of 2^24
//                          elements -> pinned host slot s mod 2, an event
//                          after each chunk
//   host worker thread     a3-a5 over the host-resident fp32 state (the
//                          update of zero_shard_host_step) into pinned bf16
//                          slot s mod 2, each chunk as soon as its download
//                          has landed; each chunk's bf16 uploaded (upload
//                          stream) into device parameter buffer s mod 2 as
//                          soon as it is written
//
// The chunks stream the download, the update and the upload through one
// another: the update of step s starts when the first chunk of its gradient
// has arrived instead of the whole spill, and its parameters are on the
// device a chunk after the update ends.
//
// The call for step s returns once the GPU work is queued and the host
// update of step s-1 has finished; the host update of step s then runs
// while the caller's stream goes on (the next forward and backward), and
// the caller's stream is ordered after the upload of step s-1, so the next
// forward reads parameters one step old -- the delayed update.  Parameter
// buffers, gradient slots and bf16 slots are double-buffered so that no
// transfer overwrites data still in use.
//
// Host code only: the HIP runtime API for pinned memory, streams, events
// and copies (all streams at default priority).

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <thread>
#include <unordered_set>

#include "zero_shard.h"
#include "zs_args.h"
#include "zs_host.h"

struct zs_offload {
  uint32_t magic;
  int device;
  zs_handle *dev;        // norm-only device handle over the spill
  zs_desc host;          // host state; param_out is replaced per slot
  int32_t threads;
  int64_t n;
  hipStream_t compute;   // the caller's stream
  hipStream_t down, up;  // downloads and uploads, so that both directions overlap
  float *gbar_ws;        // device spill (library-owned)
  double *sumsq_dev;     // device S_local (library-owned)
  zs_bf16 *param_dev[2]; // device bf16 parameters, double-buffered (caller's)
  float *gbar_host[2];   // pinned
  double *s_host[2];     // pinned
  zs_bf16 *p_host[2];    // pinned
  hipEvent_t normed;     // the norm pass of the current step is done
  hipEvent_t copied[2], uploaded[2];
  hipEvent_t s_copied[2];     // S_local of slot k is in host memory
  hipEvent_t *chunk_copied[2]; // spill chunk h of slot k is in host memory
  int64_t nio;                 // spill chunks of kIoChunk elements
  std::thread worker;
  int worker_rc;
  int64_t steps;         // steps queued so far
  int ready;             // parameter buffer holding the newest uploaded step, or -1
};

namespace {

constexpr uint32_t kOffloadMagic = 0x5a534f31u;
// Elements per streamed chunk of the download and the upload (64 MiB of the
// fp32 spill, about a millisecond of PCIe): a multiple of the host update's
// work unit.
constexpr int64_t kIoChunk = int64_t(1) << 24;

std::mutex g_mu;
std::unordered_set<zs_offload *> g_live;

bool live(zs_offload *o) {
  std::lock_guard<std::mutex> lk(g_mu);
  return o && g_live.count(o) && o->magic == kOffloadMagic;
}

int join_worker(zs_offload *o) {
  if (o->worker.joinable()) o->worker.join();
  const int rc = o->worker_rc;
  o->worker_rc = ZS_OK;
  return rc;
}

void release(zs_offload *o) {
  for (int k = 0; k < 2; ++k) {
    if (o->gbar_host[k]) (void)hipHostFree(o->gbar_host[k]);
    if (o->s_host[k]) (void)hipHostFree(o->s_host[k]);
    if (o->p_host[k]) (void)hipHostFree(o->p_host[k]);
    if (o->copied[k]) (void)hipEventDestroy(o->copied[k]);
    if (o->uploaded[k]) (void)hipEventDestroy(o->uploaded[k]);
    if (o->s_copied[k]) (void)hipEventDestroy(o->s_copied[k]);
    if (o->chunk_copied[k]) {
      for (int64_t h = 0; h < o->nio; ++h)
        if (o->chunk_copied[k][h]) (void)hipEventDestroy(o->chunk_copied[k][h]);
      delete[] o->chunk_copied[k];
    }
  }
  if (o->normed) (void)hipEventDestroy(o->normed);
  if (o->dev) (void)zero_shard_free(o->dev);
  if (o->down) (void)hipStreamDestroy(o->down);
  if (o->up) (void)hipStreamDestroy(o->up);
  if (o->gbar_ws) (void)hipFree(o->gbar_ws);
  if (o->sumsq_dev) (void)hipFree(o->sumsq_dev);
}

struct Slot {
  zs_offload *o;
  int k;
};

int64_t io_len(const zs_offload *o, int64_t h) {
  const int64_t lo = h * kIoChunk;
  return o->n - lo < kIoChunk ? o->n - lo : kIoChunk;
}

// Hooks of the host update (called from its threads): wait for spill chunk
// h of the slot to land; queue the upload of the slot's bf16 chunk h.
int chunk_ready(void *ctx, int64_t h) {
  const Slot *s = static_cast<const Slot *>(ctx);
  return hipSetDevice(s->o->device) != hipSuccess ||
         hipEventSynchronize(s->o->chunk_copied[s->k][h]) != hipSuccess;
}

int chunk_done(void *ctx, int64_t h) {
  const Slot *s = static_cast<const Slot *>(ctx);
  const int64_t lo = h * kIoChunk;
  return hipSetDevice(s->o->device) != hipSuccess ||
         hipMemcpyAsync(s->o->param_dev[s->k] + lo, s->o->p_host[s->k] + lo,
                        size_t(io_len(s->o, h)) * 2, hipMemcpyHostToDevice,
                        s->o->up) != hipSuccess;
}

// The host half of step t from slot k: run on the worker thread.
void host_half(zs_offload *o, int k, float lr, int64_t t, double s_other) {
  int rc = ZS_OK;
  // S_local has landed, and the upload that last read bf16 slot k is done
  if (hipSetDevice(o->device) != hipSuccess || hipEventSynchronize(o->s_copied[k]) != hipSuccess ||
      hipEventSynchronize(o->uploaded[k]) != hipSuccess) {
    o->worker_rc = ZS_EHIP;
    return;
  }
  zs_desc h = o->host;
  h.param_out = o->p_host[k];
  Slot slot{o, k};
  const zs_host::Hooks hooks{kIoChunk, &slot, chunk_ready, chunk_done};
  rc = zs_host::step(&h, o->gbar_host[k], lr, t, *o->s_host[k] + s_other, o->threads,
                     o->n > 0 ? &hooks : nullptr);
  // every chunk's upload is queued: the event marks the last of them
  if (rc == ZS_OK && o->n > 0 && hipEventRecord(o->uploaded[k], o->up) != hipSuccess)
    rc = ZS_EHIP;
  o->worker_rc = rc;
}

}  // namespace

extern "C" {

int zero_shard_offload_init(const zs_desc *host, zs_bf16 *param_dev0, zs_bf16 *param_dev1,
                            void *stream, int32_t threads, zs_offload **out) {
  if (!host || !out || threads < 1) return ZS_EINVAL;
  *out = nullptr;
  const int64_t n = host->shard_len;
  // everything the host update will check, before anything is allocated
  if (!zs_args::geometry_ok(*host) || !zs_args::hyper_ok(*host)) return ZS_EINVAL;
  if (n > 0 && (!host->master || !host->m || !host->v || !param_dev0 || !param_dev1))
    return ZS_EINVAL;
  if (n > 0 && host->quant_block && (!host->q_codes || !host->q_scales)) return ZS_EINVAL;
  if ((reinterpret_cast<uintptr_t>(param_dev0) | reinterpret_cast<uintptr_t>(param_dev1)) % 16)
    return ZS_EALIGN;
  zs_offload *o = new (std::nothrow) zs_offload();
  if (!o) return ZS_ENOMEM;
  o->host = *host;
  o->host.param_out = nullptr;
  o->host.gbar_ws = nullptr;
  o->host.stream = nullptr;
  o->threads = threads;
  o->n = n;
  o->compute = static_cast<hipStream_t>(stream);
  o->param_dev[0] = param_dev0;
  o->param_dev[1] = param_dev1;
  o->worker_rc = ZS_OK;
  o->ready = -1;
  int rc = ZS_OK;
  const size_t nb = size_t(n > 0 ? n : 1);
  if (hipGetDevice(&o->device) != hipSuccess) rc = ZS_EHIP;
  if (!rc && (hipStreamCreateWithFlags(&o->down, hipStreamNonBlocking) != hipSuccess ||
              hipStreamCreateWithFlags(&o->up, hipStreamNonBlocking) != hipSuccess))
    rc = ZS_EHIP;
  if (!rc && hipEventCreateWithFlags(&o->normed, hipEventDisableTiming) != hipSuccess) rc = ZS_EHIP;
  if (!rc && (hipMalloc(&o->gbar_ws, nb * 4) != hipSuccess ||
              hipMalloc(&o->sumsq_dev, 8) != hipSuccess))
    rc = ZS_ENOMEM;
  for (int k = 0; !rc && k < 2; ++k) {
    if (hipHostMalloc(&o->gbar_host[k], nb * 4, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc(&o->s_host[k], 8, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc(&o->p_host[k], nb * 2, hipHostMallocDefault) != hipSuccess)
      rc = ZS_ENOMEM;
    else if (hipEventCreateWithFlags(&o->copied[k], hipEventDisableTiming) != hipSuccess ||
             hipEventCreateWithFlags(&o->uploaded[k], hipEventDisableTiming) != hipSuccess ||
             hipEventCreateWithFlags(&o->s_copied[k], hipEventDisableTiming) != hipSuccess)
      rc = ZS_EHIP;
  }
  o->nio = n > 0 ? (n + kIoChunk - 1) / kIoChunk : 0;
  for (int k = 0; !rc && k < 2; ++k) {
    o->chunk_copied[k] = new (std::nothrow) hipEvent_t[o->nio > 0 ? o->nio : 1]();
    if (!o->chunk_copied[k]) {
      rc = ZS_ENOMEM;
      break;
    }
    for (int64_t h = 0; !rc && h < o->nio; ++h)
      if (hipEventCreateWithFlags(&o->chunk_copied[k][h], hipEventDisableTiming) != hipSuccess)
        rc = ZS_EHIP;
  }
  if (!rc) {
    // the device side: a norm-only handle (no state on the GPU) over the spill
    zs_desc d = *host;
    d.master = d.m = d.v = nullptr;
    d.param_out = nullptr;
    d.quant_block = 0;  // the device side only runs the norm pass
    d.q_codes = nullptr;
    d.q_scales = nullptr;
    d.gbar_ws = o->gbar_ws;
    d.stream = stream;
    rc = zero_shard_init(&d, &o->dev);
  }
  if (rc) {
    release(o);
    delete o;
    return rc;
  }
  o->magic = kOffloadMagic;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(o);
  }
  *out = o;
  return ZS_OK;
}

int zero_shard_offload_step(zs_offload *o, const zs_bf16 *const *contrib, float lr, int64_t t,
                            double s_other) {
  if (!live(o)) return ZS_ESTATE;
  // everything the host update will check, before anything is queued
  if (!zs_args::step_ok(lr, t) || !(s_other >= 0.0) || !std::isfinite(s_other)) return ZS_EINVAL;
  const int k = int(o->steps & 1), prev = k ^ 1;
  // the spill of the previous step has left the device before it is rewritten
  if (hipStreamWaitEvent(o->compute, o->copied[prev], 0) != hipSuccess) return ZS_EHIP;
  int rc = zero_shard_gnorm(o->dev, contrib, o->sumsq_dev);
  if (rc) return rc;
  if (hipEventRecord(o->normed, o->compute) != hipSuccess ||
      hipStreamWaitEvent(o->down, o->normed, 0) != hipSuccess)
    return ZS_EHIP;
  // S_local first (the update needs it before any chunk), then the spill
  // chunk by chunk, an event after each
  if (hipMemcpyAsync(o->s_host[k], o->sumsq_dev, 8, hipMemcpyDeviceToHost, o->down) != hipSuccess ||
      hipEventRecord(o->s_copied[k], o->down) != hipSuccess)
    return ZS_EHIP;
  for (int64_t h = 0; h < o->nio; ++h) {
    const int64_t lo = h * kIoChunk;
    if (hipMemcpyAsync(o->gbar_host[k] + lo, o->gbar_ws + lo, size_t(io_len(o, h)) * 4,
                       hipMemcpyDeviceToHost, o->down) != hipSuccess ||
        hipEventRecord(o->chunk_copied[k][h], o->down) != hipSuccess)
      return ZS_EHIP;
  }
  if (hipEventRecord(o->copied[k], o->down) != hipSuccess) return ZS_EHIP;
  // the host update of the previous step has finished (its state is the
  // input of this one) and its upload is queued: the caller's stream reads
  // those parameters from here on
  if ((rc = join_worker(o))) return rc;
  if (o->steps > 0) {
    if (hipStreamWaitEvent(o->compute, o->uploaded[prev], 0) != hipSuccess) return ZS_EHIP;
    o->ready = prev;
  }
  try {
    o->worker = std::thread(host_half, o, k, lr, t, s_other);
  } catch (...) {
    return ZS_ENOMEM;
  }
  ++o->steps;
  return ZS_OK;
}

zs_bf16 *zero_shard_offload_params(zs_offload *o) {
  if (!live(o) || o->ready < 0) return nullptr;
  return o->param_dev[o->ready];
}

int zero_shard_offload_wait(zs_offload *o) {
  if (!live(o)) return ZS_ESTATE;
  int rc = join_worker(o);
  for (int k = 0; k < 2; ++k)
    if (hipEventSynchronize(o->uploaded[k]) != hipSuccess) rc = rc ? rc : ZS_EHIP;
  if (o->steps > 0) {
    if (hipStreamWaitEvent(o->compute, o->uploaded[(o->steps - 1) & 1], 0) != hipSuccess)
      rc = rc ? rc : ZS_EHIP;
    else if (!rc)
      o->ready = int((o->steps - 1) & 1);
  }
  return rc;
}

int zero_shard_offload_free(zs_offload *o) {
  if (!o) return ZS_OK;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_live.count(o)) return ZS_ESTATE;
    g_live.erase(o);
  }
  int rc = join_worker(o);
  if (hipStreamSynchronize(o->down) != hipSuccess || hipStreamSynchronize(o->up) != hipSuccess)
    rc = rc ? rc : ZS_EHIP;
  if (o->compute && hipStreamSynchronize(o->compute) != hipSuccess) rc = rc ? rc : ZS_EHIP;
  o->magic = 0;
  release(o);
  delete o;
  return rc;
}

}  // extern "C"
