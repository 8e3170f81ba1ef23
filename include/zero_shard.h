/*
 * zero_shard.h -- C ABI of the MI355X (gfx950) ZeRO-1/2 shard optimizer step.
 *
 * One data-parallel rank owns partition r of the flat parameter vector
 * theta = [theta_1 .. theta_N] and keeps the fp32 optimizer state for that
 * partition only ("Data parallelism and ZeRO optimization", sections
 * "ZeRO-1: Optimizer State Partitioning" and "ZeRO-2: Gradient
 * Partitioning"; "ZeRO (딥 러닝)", stage table of "ZeRO-DP의 세 단계").
 * Between the reduce-scatter of the gradients and the all-gather of the
 * updated weights ("ZeRO (딥 러닝)", "왜 통신량이 늘지 않는가") the rank:
 *
 *   a1  sums the N_d incoming bf16 gradient contributions for its slice in
 *       rank order and averages them ("大模型并行技术", "优化状态与梯度分割",
 *       step 2; "How Standard Data Parallelism Works": the average);
 *   a2  optionally clips by the global L2 norm of the averaged gradient
 *       ("ZeRO (딥 러닝)", "DeepSpeed에서 쓰기": gradient_clipping);
 *   a3  runs mixed-precision AdamW on its fp32 master weights, momentum and
 *       variance ("Memory Consumption Analysis"; "精度混合训练");
 *   a4  writes the bf16 copy of the updated master weights, the buffer the
 *       all-gather sends;
 *   a5  optionally block-quantizes that copy to int8 codes plus one fp32
 *       scale per block (ZeRO++ qwZ, "ZeRO (딥 러닝)", follow-ups table
 *       "후속 기법").
 *
 * Arithmetic (what every call computes, element i of the shard):
 *   s_i    = sum_{k=0}^{n_d-1} bf16(contrib[k][i])   binary64, k ascending
 *   gbar_i = binary32(s_i / n_d)                      one rounding
 *   g_i    = coef * gbar_i                            binary64; coef = 1
 *            unless clipping: coef = min(1, max_norm / (sqrt(S) + 1e-6)),
 *            S = global sum of gbar^2 handed to zero_shard_step
 *   m'     = b1 m + (1-b1) g        v' = b2 v + (1-b2) (g g)
 *   theta' = theta - (lr wd) theta - lr (m'/bc1) / (sqrt(v'/bc2) + eps)
 *            bc = 1 - beta^t with bias correction, else 1; all binary64
 *            from the binary32 state, each result rounded once to binary32
 *   p_i    = bf16(theta'_i), round to nearest even
 *   int8:  block b = elements [b*B, b*B+B) of the shard (last one partial);
 *          a = max |p|, scale = binary32(a / 127), code = round-half-even(
 *          binary32(p / scale)) clamped to +-127; scale 0 => codes 0;
 *          a non-finite quotient gives code 0.
 * With int8 contributions (the _q8 calls) element i of row k stands for
 * code_k[i] * scale_k[i / block], an exact binary64 product, and s_i sums
 * those products in the same k order.
 * Non-finite inputs propagate per IEEE; no step is skipped.
 *
 * Memory: every pointer in zs_desc and every contribution pointer is a
 * device pointer (HBM of the current device), allocated and owned by the
 * caller, and must stay valid until the work queued on the stream is done.
 * Layouts are flat, contiguous, element i at offset i.  fp32 and bf16
 * arrays and every contribution row must be 16-byte aligned; q_codes 8-byte
 * aligned.  The library owns only the handle and a small device scratch
 * (one fp64 partial of the norm per 16384 shard elements, or per 4096 with
 * int8 contributions), allocated at init; the bucketed calls add worker
 * streams and per-bucket scratch on first use.
 *
 * Errors: every call returns ZS_OK (0) or a negative zs_status.  Arguments
 * are validated before anything is queued: on an error nothing is launched
 * and no output is touched.  Launch failures are reported as ZS_EHIP;
 * faults inside a kernel surface at the caller's next synchronisation.
 * Calls are asynchronous on the handle's stream; a handle is used by one
 * host thread at a time.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zs_handle zs_handle; /* opaque */
typedef uint16_t zs_bf16;           /* bf16 bit pattern */

typedef enum zs_status {
  ZS_OK = 0,
  ZS_EINVAL = -1,  /* bad size, index, hyper-parameter or missing pointer */
  ZS_EALIGN = -2,  /* a pointer is not aligned as required                */
  ZS_ENOMEM = -3,  /* the library's own scratch could not be allocated     */
  ZS_EHIP = -4,    /* a HIP runtime call or kernel launch failed           */
  ZS_EDEVICE = -5, /* the current device is not gfx950                     */
  ZS_ESTATE = -6,  /* call out of order (step reading a gradient spill
                      that no norm pass has written) or a dead handle      */
  ZS_ETOOBIG = -7  /* shard longer than zero_shard_gnorm_noalloc's static
                      scratch allows                                       */
} zs_status;

#define ZS_MAX_ND 64 /* most contributions one call can average */

/* How the work of a call is split into kernel launches (on the call's
 * stream, in order; the split changes no result).  The norm pass over n
 * elements (the shard, or one bucket) queues ceil(n / ZS_NORM_LAUNCH_LEN)
 * partial-sum launches and one final reduction.  An update that reads the
 * contribution rows (no spill) runs in its wide form, as
 * ceil(n / ZS_WIDE_LAUNCH_LEN) launches, from ZS_WIDE_MIN_ROWS bf16 rows
 * (ZS_WIDE_MIN_ROWS_QUANT when it also writes int8) or ZS_WIDE_MIN_ROWS_Q8
 * int8 rows; any other update is one launch. */
#define ZS_NORM_LAUNCH_LEN (INT64_C(1) << 26)
#define ZS_WIDE_LAUNCH_LEN (INT64_C(1) << 25)
#define ZS_WIDE_MIN_ROWS 18
#define ZS_WIDE_MIN_ROWS_QUANT 32
#define ZS_WIDE_MIN_ROWS_Q8 16

typedef struct zs_desc {
  /* partition geometry */
  int64_t phi;       /* parameters in the whole flat buffer, >= 0           */
  int32_t n_d;       /* data-parallel degree, 1..ZS_MAX_ND                  */
  int32_t r;         /* partition index, 0 <= r < n_d                       */
  int64_t shard_len; /* elements of partition r: min(ceil(phi/n_d),
                        phi - r*ceil(phi/n_d)) clamped at 0; or phi with
                        r == 0 for the unpartitioned (stage 0) update        */
  /* optimizer: binary32 values, used widened to binary64 */
  float beta1, beta2; /* in [0, 1)                                          */
  float eps;          /* > 0                                                */
  float weight_decay; /* >= 0, decoupled; 0 = plain Adam                    */
  int32_t bias_correction; /* 1: divide by 1 - beta^t; 0: do not          */
  float max_norm;     /* > 0: clip by the global norm; <= 0: no clipping   */
  int32_t quant_block; /* 0: no int8; else 32, 64, 128, 256 or 512: the
                          step also writes codes and scales (fused)        */
  /* state and outputs (device pointers, caller-owned) */
  float *master, *m, *v; /* fp32[shard_len], updated in place; these four  */
  zs_bf16 *param_out;    /* bf16[shard_len]  may all be NULL for a norm-only
                            handle (state offloaded to the host, see
                            zero_shard_host_step), which needs gbar_ws and
                            refuses zero_shard_step / zero_shard_quant     */
  int8_t *q_codes;       /* int8[shard_len]; needed iff quant_block > 0 or
                            zero_shard_quant is called                     */
  float *q_scales;       /* fp32[ceil(shard_len / block)], same condition  */
  float *gbar_ws;        /* optional fp32[shard_len] workspace; with
                            clipping, zero_shard_gnorm stores the averaged
                            gradient there and zero_shard_step reads it
                            instead of re-reading the contributions        */
  void *stream;          /* hipStream_t for every call; NULL = null stream */
} zs_desc;

/* Validate d, check that the current device is gfx950, allocate the norm
 * scratch, and return a handle in *out.  The descriptor is copied.
 * Errors: ZS_EINVAL, ZS_EALIGN, ZS_EDEVICE, ZS_ENOMEM, ZS_EHIP. */
int zero_shard_init(const zs_desc *d, zs_handle **out);

/* a2, first sweep: this shard's sum of squares of the averaged gradient,
 * S_local = sum_i gbar_i^2 (binary64), reduced over a grid fixed by the
 * shard length, in a fixed order, with no atomics (same inputs => same
 * bits).  contrib is a HOST array of n_d device pointers, contrib[k] =
 * rank k's bf16 gradient for this shard (shard-local index).  Writes
 * S_local to *sumsq_dev (device, one double).  With gbar_ws set, also
 * stores gbar there for the next step.
 * Summing S_local over the shards (one scalar all-reduce across ranks) gives
 * the S that zero_shard_step takes.  Errors: ZS_EINVAL, ZS_EALIGN, ZS_EHIP,
 * ZS_ESTATE. */
int zero_shard_gnorm(zs_handle *h, const zs_bf16 *const *contrib, double *sumsq_dev);

/* zero_shard_gnorm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same sum of squares S_local and the same spill (when
 * d->gbar_ws is set), bit for bit, without a handle.  Takes the descriptor
 * itself (d->n_d, d->shard_len, d->gbar_ws and d->stream are used; the
 * state pointers and hyper-parameters are ignored), contrib and sumsq_dev as
 * for zero_shard_gnorm.  It allocates nothing: the block partials live in a
 * static device array of the library (512 KiB on each GPU the library runs
 * on, kept until the process ends), which bounds the shard at one partial
 * per 16384 elements, 65536 partials: shard_len <= 2^30 (ZS_ETOOBIG
 * beyond).  Every call on one GPU uses that GPU's one array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller; the partials need no clearing (each call writes
 * all it reads).  Queues ceil(shard_len / ZS_NORM_LAUNCH_LEN) + 1 kernel
 * launches (at least two) on d->stream and nothing else.
 * Errors: ZS_EINVAL, ZS_EALIGN, ZS_ETOOBIG, ZS_EDEVICE, ZS_EHIP. */
int zero_shard_gnorm_noalloc(const zs_desc *d, const zs_bf16 *const *contrib,
                             double *sumsq_dev);

/* a1 + a3 + a4 (+ a5 when quant_block > 0): one optimizer step at 1-based
 * step counter t with learning rate lr >= 0.  contrib as for gnorm; it may
 * be NULL when clipping with gbar_ws (the spill written by the preceding
 * zero_shard_gnorm is read instead).  global_sumsq_dev (device, one double)
 * is S and is required iff max_norm > 0; it is read on the device, so no
 * host synchronisation is needed between gnorm and step.  gnorm and step
 * queue kernel launches only (no allocation, no memset), so they can be
 * captured in a HIP graph on the handle's stream; t and lr are then fixed
 * in the captured launches (zero_shard_step_dev reads them from device
 * memory instead).
 * Errors: ZS_EINVAL, ZS_EALIGN, ZS_ESTATE, ZS_EHIP. */
int zero_shard_step(zs_handle *h, const zs_bf16 *const *contrib, float lr, int64_t t,
                    const double *global_sumsq_dev);

/* The constants of step t at learning rate lr as the library computes them
 * on the host for zero_shard_step: out[0] = lr, out[1] = lr * weight_decay,
 * out[2] = bc1 = 1 - beta1^t, out[3] = bc2 = 1 - beta2^t (1 and 1 without
 * bias correction), binary64 from d's binary32 values (pow of the C
 * library).  out is a HOST array of 4 doubles; only d's hyper-parameters are
 * read.  Errors: ZS_EINVAL (bad d, lr or t). */
int zero_shard_step_consts(const zs_desc *d, float lr, int64_t t, double *out);

/* zero_shard_step with the step's constants read on the device, when the
 * kernel runs, from consts_dev (device, 4 doubles, 8-byte aligned, laid out
 * as zero_shard_step_consts writes them) instead of fixed at the call.  A
 * step captured in a HIP graph then serves every step: before each replay
 * the caller writes that step's constants to consts_dev (outside the graph,
 * e.g. an asynchronous copy on the same stream).  With the constants of
 * (lr, t) the results are zero_shard_step's at (lr, t), bit for bit.  The
 * constants are trusted as given.  Errors: ZS_EINVAL, ZS_EALIGN, ZS_ESTATE,
 * ZS_EHIP. */
int zero_shard_step_dev(zs_handle *h, const zs_bf16 *const *contrib, const double *consts_dev,
                        const double *global_sumsq_dev);

/* a1 with int8 contributions: ZeRO++ qgZ ("ZeRO (딥 러닝)", follow-ups table
 * "후속 기법": gradients are quantized and averaged after an all-to-all).
 * Row k is codes[k], int8[shard_len] (8-byte aligned), with one fp32 scale
 * per `block` contiguous shard elements starting at element 0, scales[k],
 * fp32[ceil(shard_len / block)] (4-byte aligned); codes and scales are HOST
 * arrays of n_d device pointers; block is 32, 64, 128, 256 or 512.
 * Otherwise exactly zero_shard_gnorm and zero_shard_step (codes and scales
 * may be NULL when the step reads the gradient spill).  Errors: as there. */
int zero_shard_gnorm_q8(zs_handle *h, const int8_t *const *codes, const float *const *scales,
                        int32_t block, double *sumsq_dev);
int zero_shard_step_q8(zs_handle *h, const int8_t *const *codes, const float *const *scales,
                       int32_t block, float lr, int64_t t, const double *global_sumsq_dev);

/* Bucketed step ("ZeRO (딥 러닝)", "DeepSpeed에서 쓰기": overlap_comm,
 * contiguous_gradients, reduce_bucket_size in the configuration example;
 * "ZeRO-R: 잔여 메모리 최적화": gradient communication through buffers of a
 * fixed size, independent of the model).  Gradients reach the owner rank
 * bucket by bucket, so the shard's elements [0, shard_len) are processed in
 * buckets of bucket_len elements (bucket j: [j*bucket_len, ...), the last
 * one shorter), each as soon as its slice of the contributions is in place,
 * overlapping the arrival of later buckets.
 *
 * contrib is a HOST array of n_d device pointers to the whole shard's rows,
 * as for zero_shard_gnorm (contiguous gradients: bucket j of row k starts at
 * contrib[k] + j*bucket_len).  bucket_len > 0 is a multiple of 512 (every
 * bucket starts on a vector and a quantizer-block boundary).  ready is NULL
 * (everything in place) or a HOST array of ceil(shard_len / bucket_len)
 * hipEvent_t, entries may be NULL: bucket j's work waits for ready[j],
 * which the caller has recorded (e.g. on its communication stream after
 * bucket j's reduce-scatter) before this call.  Buckets are distributed
 * round-robin over `streams` (1..4) worker streams that the handle creates
 * on first use (default priority) and that start after the work already
 * queued on the handle's stream; the handle's stream waits for all of them
 * before the call returns, so later calls on it are ordered after every
 * bucket.  The first call, or one with more buckets than before, allocates
 * the per-bucket scratch.
 *
 * zero_shard_gnorm_bucketed: a2's first sweep per bucket (spilling gbar as
 * zero_shard_gnorm does), then S_local = the per-bucket sums added in
 * bucket order, to *sumsq_dev.  Same result as zero_shard_gnorm up to the
 * association of the binary64 sum.
 * zero_shard_step_bucketed: the fused step (a1, a3, a4, a5) per bucket;
 * each element's result is bit-identical to zero_shard_step's.  With
 * clipping and gbar_ws it reads the spill and contrib may be NULL.
 * Errors: as zero_shard_gnorm / zero_shard_step; ZS_EINVAL also for a bad
 * bucket_len or streams; ZS_ENOMEM. */
int zero_shard_gnorm_bucketed(zs_handle *h, const zs_bf16 *const *contrib, int64_t bucket_len,
                              int32_t streams, const void *const *ready, double *sumsq_dev);
int zero_shard_step_bucketed(zs_handle *h, const zs_bf16 *const *contrib, int64_t bucket_len,
                             int32_t streams, const void *const *ready, float lr, int64_t t,
                             const double *global_sumsq_dev);

/* The bucketed calls with int8 contributions (qgZ, as the _q8 calls above):
 * codes[k] / scales[k] are rank k's whole-shard rows; bucket j of row k
 * starts at codes[k] + j*bucket_len and scales[k] + j*bucket_len/block
 * (bucket_len is a multiple of 512, so of every block).  Errors: as the
 * bucketed calls and the _q8 calls. */
int zero_shard_gnorm_bucketed_q8(zs_handle *h, const int8_t *const *codes,
                                 const float *const *scales, int32_t block, int64_t bucket_len,
                                 int32_t streams, const void *const *ready, double *sumsq_dev);
int zero_shard_step_bucketed_q8(zs_handle *h, const int8_t *const *codes,
                                const float *const *scales, int32_t block, int64_t bucket_len,
                                int32_t streams, const void *const *ready, float lr, int64_t t,
                                const double *global_sumsq_dev);

/* a5 as a separate pass: quantize param_out into q_codes / q_scales with
 * the given block (32, 64, 128, 256 or 512); q_scales must hold
 * ceil(shard_len / block) floats.  Errors: ZS_EINVAL, ZS_EHIP. */
int zero_shard_quant(zs_handle *h, int32_t block);

/* qwZ receive side (ZeRO++, "ZeRO (딥 러닝)" follow-ups table "후속 기법"):
 * after the all-gather of the n_d int8 shards, rebuild the whole bf16
 * parameter vector.  Shard r holds flat elements [r*ceil(phi/n_d), ...) of
 * length zero_shard_len(phi, n_d, r); codes[r] is its int8[len] (8-byte
 * aligned) and scales[r] its fp32[ceil(len / block)] (4-byte aligned), one
 * scale per `block` elements counted from the shard's own element 0, as
 * zero_shard_step writes them.  codes and scales are HOST arrays of n_d
 * device pointers (entries of empty shards may be NULL).  Writes
 * param_out[i] = bf16(binary32(code * scale)) (nearest even) for all phi
 * elements of param_out (device, 16-byte aligned).  No handle: it reads
 * every rank's shard.  Asynchronous on `stream` (hipStream_t, NULL = null
 * stream).  Errors: ZS_EINVAL, ZS_EALIGN, ZS_EDEVICE, ZS_EHIP. */
int zero_shard_dequant(const int8_t *const *codes, const float *const *scales, int32_t n_d,
                       int64_t phi, int32_t block, zs_bf16 *param_out, void *stream);

/* ZeRO-Offload host step ("ZeRO (딥 러닝)", follow-ups table "후속 기법":
 * optimizer states and the update in CPU memory, an optimized CPU Adam, a
 * one-step delayed update).  a3 + a4 (+ a5) on the CPU for the shard
 * described by d, whose master/m/v/param_out/q_codes/q_scales are HOST
 * pointers here (d->stream and d->gbar_ws are ignored); gbar is the host
 * fp32[shard_len] averaged gradient, e.g. the device spill that
 * zero_shard_gnorm wrote, copied to the host.  global_sumsq is S, used iff
 * d->max_norm > 0.  The arithmetic is the device step's, so the result is
 * bit-identical to zero_shard_step on the same inputs.  Synchronous; runs
 * on `threads` host threads (>= 1), which take contiguous 2^18-element,
 * block-aligned pieces of the shard in turn (the split changes no bit).
 * Errors: ZS_EINVAL. */
int zero_shard_host_step(const zs_desc *d, const float *gbar, float lr, int64_t t,
                         double global_sumsq, int32_t threads);

/* ZeRO-Offload pipeline for one rank's shard ("ZeRO (딥 러닝)", follow-ups
 * table "후속 기법": optimizer states and their update on the CPU, the
 * update hidden behind the GPU's next step by a one-step delayed update).
 *
 * zero_shard_offload_init: `host` describes the shard with HOST pointers
 * for master/m/v (and q_codes/q_scales when quant_block > 0), as for
 * zero_shard_host_step; its param_out, gbar_ws and stream are ignored.
 * param_dev0/param_dev1 are two device bf16[shard_len] buffers (16-byte
 * aligned) that the updated parameters are uploaded into, alternately;
 * `stream` is the caller's compute stream; `threads` (>= 1) host threads
 * run the update.  The library allocates a device spill and S scalar, two
 * pinned gradient slots and two pinned bf16 slots, a download and an
 * upload stream, and one event per 2^24-element chunk of each gradient slot.
 *
 * zero_shard_offload_step: step t.  Queues on `stream` the norm pass over
 * contrib (a HOST array of n_d device pointers, as for zero_shard_gnorm),
 * then copies S_local and the averaged gradient to pinned memory (the
 * gradient in chunks of 2^24 elements), waits for the host update of the
 * previous step to finish, orders `stream` after that step's upload, starts
 * this step's host update (a3-a5 with S = S_local + s_other, s_other >= 0
 * being the other shards' sum) on a host thread, and returns.  The host
 * update takes each chunk as soon as its copy has landed and uploads each
 * chunk of its bf16 parameters into buffer (call index mod 2) as soon as
 * it is written.  Work queued on `stream` after the call
 * sees the parameters of the previous step: zero_shard_offload_params
 * names that buffer (NULL before any update has been uploaded).
 * zero_shard_offload_wait: finish the running host update and order
 * `stream` after its upload; zero_shard_offload_params then names the
 * newest parameters.  zero_shard_offload_init rejects a descriptor the host
 * update would reject (geometry, beta, eps, weight decay, max_norm, block)
 * before it allocates anything, and zero_shard_offload_step rejects a bad
 * lr, t or s_other (negative or non-finite) before it queues anything; an
 * error inside a running host update is returned by the next step or wait
 * call.  zero_shard_offload_free waits and releases.
 * The results are those of zero_shard_step on the same inputs, bit for bit.
 * Errors: ZS_EINVAL, ZS_EALIGN, ZS_ENOMEM, ZS_EHIP, ZS_ESTATE. */
typedef struct zs_offload zs_offload;
int zero_shard_offload_init(const zs_desc *host, zs_bf16 *param_dev0, zs_bf16 *param_dev1,
                            void *stream, int32_t threads, zs_offload **out);
int zero_shard_offload_step(zs_offload *o, const zs_bf16 *const *contrib, float lr, int64_t t,
                            double s_other);
zs_bf16 *zero_shard_offload_params(zs_offload *o);
int zero_shard_offload_wait(zs_offload *o);
int zero_shard_offload_free(zs_offload *o);

/* Wait for the handle's stream, release its scratch and the handle.
 * Passing NULL is a no-op returning ZS_OK. */
int zero_shard_free(zs_handle *h);

/* Static description of a status code (never NULL). */
const char *zero_shard_strerror(int code);

/* Length of partition r of phi parameters over n_d ranks (the geometry
 * zero_shard_init checks), or -1 for invalid arguments. */
int64_t zero_shard_len(int64_t phi, int32_t n_d, int32_t r);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_SHARD_H */
