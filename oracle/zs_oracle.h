/*
 * zs_oracle.h -- CPU oracle for one data-parallel rank's ZeRO-1/2 shard
 * optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code with the HIP
 * library: no headers, kernels, helpers or constants.
 *
 * Plain, slow, fp64.  Every routine is the definition of what it computes,
 * written out elementwise in index order.  Sources (the web pages the method
 * is described on):
 *   [DP]   "Data parallelism and ZeRO optimization -- Hinglish notes"
 *          (brentwoodlivery 6.1.8): "How Standard Data Parallelism Works",
 *          "Memory Consumption Analysis", "ZeRO-1", "ZeRO-2".
 *   [BIMU] "大模型并行技术" (bimu.site): sections "精度混合训练",
 *          "优化状态与梯度分割".
 *   [WIKI] "ZeRO (딥 러닝)" (itwiki.kr): memory table, stage table
 *          ("ZeRO-DP의 세 단계"), follow-ups table ("후속 기법", ZeRO++ qwZ),
 *          "DeepSpeed에서 쓰기" (gradient_clipping), "FSDP와의 관계"
 *          (reduce_dtype float32).
 * Where the pages leave a step open, the reading taken is stated at the
 * routine.  Three such conventions are pinned only to the reading, not to
 * anything the pages fix (parity unpinned by the pages): where eps enters
 * Adam (after bias correction: the tests pin the closed forms of that
 * reading), the clip constant 1e-6 with min(1, .) in orc_clip_coef, and the
 * int8 scale convention (symmetric, absmax / 127, round half to even) of
 * orc_quant_int8 and orc_dequant_bf16.
 */
#ifndef ZS_ORACLE_H
#define ZS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Hyper-parameters of one step.  Floating values are the binary32 values the
 * caller uses, widened to binary64. */
typedef struct orc_hyper {
  double lr, beta1, beta2, eps, weight_decay;
  int32_t bias_correction; /* 1: divide m, v by 1-beta^t                    */
  int32_t quant_block;     /* 0: no int8 output; else elements per block    */
  int64_t t;               /* 1-based step counter                          */
  double max_norm;         /* > 0: clip by the global L2 norm               */
  double s_other;          /* other shards' sum of squares (0 on one rank)  */
} orc_hyper;

/* Model-state bytes per GPU for stage 0..3 (WIKI stage table). */
double orc_model_state_bytes(double n_params, double n_gpus, int32_t stage,
                             double k_optimizer);

/* bf16 <-> binary32 (bf16 = upper 16 bits of binary32). */
float orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float x);
void orc_cast_bf16(const float *x, int64_t n, uint16_t *out);

/* a1: fp64 sum of the n_d contributions in rank order (exact for these
 * inputs) -> sums; average rounded once to binary32 -> gbar. */
void orc_reduce_sum(const uint16_t *const *rows, int32_t n_d, int64_t n,
                    double *sums);
void orc_reduce_average(const uint16_t *const *rows, int32_t n_d, int64_t n,
                        float *gbar);

/* a1 with int8 contributions (ZeRO++ qgZ): row k is codes[k] (int8) with
 * one fp32 scale per `block` elements, scales[k][i / block]; element i of
 * row k stands for code * scale.  Same rank-order binary64 sum, same single
 * rounding of the average. */
void orc_reduce_sum_q8(const int8_t *const *codes, const float *const *scales, int32_t n_d,
                       int64_t n, int32_t block, double *sums);
void orc_reduce_average_q8(const int8_t *const *codes, const float *const *scales,
                           int32_t n_d, int64_t n, int32_t block, float *gbar);

/* a2: sum of squares of gbar (fp64, index order). */
double orc_sumsq(const float *gbar, int64_t n);
double orc_clip_coef(double sumsq, double max_norm);

/* a3: AdamW on binary32 state, arithmetic in binary64, gradient coef*gbar. */
void orc_adam(float *master, float *m, float *v, const float *gbar,
              double coef, int64_t n, const orc_hyper *h);

/* a5: int8 block quantization of a bf16 vector. */
void orc_quant_int8(const uint16_t *p, int64_t n, int32_t block,
                    int8_t *codes, float *scales);

/* qwZ receive side: the all-gathered int8 shards back to the full bf16
 * parameter vector.  Shard r (r = 0..n_d-1) holds elements
 * [r*ceil(phi/n_d), ...) of the flat vector, codes[r] with one fp32 scale
 * per `block` elements of the shard (blocks start at the shard's element
 * 0), scales[r].  out[i] = bf16(binary32(code * scale)). */
void orc_dequant_bf16(const int8_t *const *codes, const float *const *scales, int32_t n_d,
                      int64_t phi, int32_t block, uint16_t *out);

/* The whole step a1..a5 over one shard.  Chunked over `threads` host
 * threads; chunk partial sums are combined in chunk order, so the result
 * does not depend on the thread count.  sumsq_out (may be NULL) receives
 * this shard's sum of squares when clipping.  Returns 0, or -1 on bad
 * arguments. */
int orc_step(const uint16_t *const *rows, int32_t n_d, int64_t n,
             float *master, float *m, float *v, uint16_t *p_out,
             int8_t *codes, float *scales, const orc_hyper *h,
             double *sumsq_out, int32_t threads);

/* Averaged gradient and its sum of squares for a chunk, multithreaded the
 * same way (for callers that stream a large shard through in pieces). */
double orc_gbar_sumsq(const uint16_t *const *rows, int32_t n_d, int64_t n,
                      float *gbar, int32_t threads);
double orc_gbar_sumsq_q8(const int8_t *const *codes, const float *const *scales, int32_t n_d,
                         int64_t n, int32_t block, float *gbar, int32_t threads);

/* The whole step with int8 contributions (qgZ front end, then a2..a5 as in
 * orc_step).  `block` must divide 2^20 (the chunk) so that blocks never
 * straddle chunks. */
int orc_step_q8(const int8_t *const *codes, const float *const *scales, int32_t n_d,
                int64_t n, int32_t block, float *master, float *m, float *v,
                uint16_t *p_out, int8_t *q_codes, float *q_scales, const orc_hyper *h,
                double *sumsq_out, int32_t threads);

#ifdef __cplusplus
}
#endif
#endif
