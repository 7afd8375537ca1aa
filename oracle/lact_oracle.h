/*
 * lact_oracle.h -- entry points of the CPU oracle (lact_oracle.c).
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU baseline
 * use it; the GPU library never includes or links it.
 */
#ifndef LACT_ORACLE_H
#define LACT_ORACLE_H

#include <stdint.h>

/* codecs */
double lacto_bf16_value(uint16_t code);
uint16_t lacto_bf16_encode(float x);
void lacto_bf16_encode_array(const float* x, uint16_t* out, int64_t n);
double lacto_e4m3_value(uint8_t code);
uint8_t lacto_e4m3_encode(float x);
void lacto_quant_e4m3_rows(const float* x, int64_t rows, int32_t D, uint8_t* codes, float* scales);
void lacto_e4m3_dequant_f32(const uint8_t* codes, const float* scales, int64_t rows, int32_t D,
                            float* out);

/* ConvKV compression of one group of r frames */
void lacto_compress_chain_f32(const float* x, int32_t r, int64_t TC, int32_t C, const float* w,
                              const float* b, float* out);
void lacto_compress_exact(const float* x, int32_t r, int64_t TC, int32_t C, const float* w,
                          const float* b, double* out);

/* RoPE with reset positions, in place */
void lacto_rope_rotate(double* x, int64_t n, int32_t H, int32_t D, const int32_t* t,
                       const int32_t* u, int32_t mode, const int32_t* split, int32_t T,
                       int32_t grid_w, double theta);

/* attention over [history | current] with the block-wise causal mask */
typedef struct {
  int32_t H, D;
  int64_t Lq, Lhist;
  const float *q, *q_scale;            /* [Lq][H][D], [Lq][H] or NULL                     */
  const float *k_hist, *k_hist_scale;  /* [Lhist][H][D], [Lhist][H] or NULL               */
  const float *v_hist, *v_hist_scale;
  const float *k_cur, *k_cur_scale;    /* [Lq][H][D]                                      */
  const float *v_cur, *v_cur_scale;
  const int32_t *hist_t, *hist_u;      /* positions of the history tokens                 */
  const int32_t *cur_t, *cur_u;        /* positions of the current tokens (q and k)       */
  int32_t rope_mode, rope_split[3], T, grid_w;
  double rope_theta;
  int32_t n_blocks;
  const int64_t* block_start;          /* [n_blocks + 1] query-token offsets, 0 .. Lq     */
  int64_t n_sel;
  const int32_t* sel_head;             /* selected (head, row) outputs, sorted by head    */
  const int64_t* sel_row;
  int32_t form;                        /* 0 explicit mask matrix, 1 segments             */
  int32_t threads;
  double* out;                         /* [n_sel][D]                                      */
  double* lse;                         /* [n_sel]                                         */
  double* rms;                         /* [n_sel] or NULL: sqrt(sum_j w_j^2 |v_j|^2), w the
                                          softmax weights -- the size of the weighted
                                          terms a rounding of each weight perturbs O by    */
} lacto_attn_args;

/* Returns 0 on success, 1 on bad arguments, 2 if form 0's mask matrix would be too big. */
int lacto_attention(const lacto_attn_args* a);

#endif /* LACT_ORACLE_H */
