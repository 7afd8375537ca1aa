/*
 * lact_oracle.c -- plain, slow CPU oracle of the ConvKV-memory block-causal attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library.  It shares no source with the GPU library and
 * never touches HIP.  Floating point is double unless a function says otherwise; the
 * compressor's f32 fma chain and the codecs are the storage definitions that let the GPU
 * match bit for bit.
 *
 * Sources (the pages this follows):
 *   [W]  walkthrough "SoulX-LiveAct" (gongshangzheng.github.io/paper-liveact.html):
 *        sections "ConvKV Memory", "Streaming Pipeline", "Neighbor Forcing" (block-wise
 *        causal mask of block size m), "system-level optimisation" (FP8).
 *   [PR] press release, digi.china.com (2026-04-21), technical-principle paragraph:
 *        exact recent window + rolling compression at a fixed ratio into a fixed-length
 *        representation, and RoPE Reset.
 *   [NS] news summary "SoulX-LiveAct - Soul App ..." (aiboss88.com), section "technical
 *        principle", ConvKV Memory bullet: 1D convolution at 5:1, RoPE reset.
 *   [MC] model card "SoulX-LiveAct: Towards Hour-Scale Real-Time Human Animation ..."
 *        (hf.xjtesla.cn/Soul-AILab/LiveAct), section "Command Line Arguments":
 *        --fp8_kv_cache stores the KV cache in FP8 and dequantises on use.
 *
 * Readings where the pages are silent (the plainest ones the rest of the pages support):
 *   conv: depthwise over time per (token, channel), kernel = stride = r, bias, no padding,
 *   tap k on frame r*g + k; RoPE: interleaved pairs, angle pos * theta^(-2i/d_part),
 *   3D split (t, h, w); positions reset to ranks [reference | memory | window | current];
 *   e4m3 = OCP E4M3FN, one f32 scale per (token, head) = amax / 448.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py against closed
 * forms, brute force or special cases.  The FP8 attention is the oracle's attention over
 * the stored (quantised) values; what a kernel's own extra rounding adds is held to the
 * FP8 bar, not pinned to a value.
 */
#include "lact_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ===================================================================================== */
/* bf16: the upper 16 bits of an IEEE binary32.                                          */
/* ===================================================================================== */

static float f32_of_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}
static uint32_t bits_of_f32(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* Exact value of a bf16 code. */
double lacto_bf16_value(uint16_t code) { return (double)f32_of_bits((uint32_t)code << 16); }

/* Round a float to the nearest bf16; on a tie take the code whose last mantissa bit is 0
 * (round-to-nearest-even).  Past the largest finite value the neighbour above is +-inf,
 * treated as 2^128 for the distance, as IEEE rounding does.  NaN -> quiet NaN, same sign. */
uint16_t lacto_bf16_encode(float x) {
  uint32_t b = bits_of_f32(x);
  if (isnan(x)) return (uint16_t)((b >> 16) | 0x0040u);
  uint32_t lo = b & 0xFFFF0000u; /* same sign, magnitude truncated: |lo| <= |x| */
  if (lo == b) return (uint16_t)(b >> 16);
  uint32_t hi = lo + 0x10000u;   /* next magnitude up */
  double xd = (double)x;
  double vlo = (double)f32_of_bits(lo);
  double vhi = ((hi & 0x7FFFFFFFu) == 0x7F800000u) ? copysign(ldexp(1.0, 128), xd)
                                                   : (double)f32_of_bits(hi);
  double dlo = fabs(xd - vlo), dhi = fabs(vhi - xd);
  if (dlo < dhi) return (uint16_t)(lo >> 16);
  if (dhi < dlo) return (uint16_t)(hi >> 16);
  return (uint16_t)((((lo >> 16) & 1u) != 0u) ? (hi >> 16) : (lo >> 16));
}

void lacto_bf16_encode_array(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = lacto_bf16_encode(x[i]);
}

/* ===================================================================================== */
/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;         */
/* S.1111.111 is NaN; largest finite 448; subnormals m/8 * 2^-6 (smallest 2^-9).          */
/* The FP8 KV cache of [MC] ("store in FP8, dequantise on use").                          */
/* ===================================================================================== */

double lacto_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* The magnitudes of codes 0x00..0x7E, lacto_e4m3_value of each, computed once. */
static double e4m3_mag[127];
static pthread_once_t e4m3_mag_once = PTHREAD_ONCE_INIT;
static void e4m3_mag_init(void) {
  for (int c = 0; c < 127; ++c) e4m3_mag[c] = lacto_e4m3_value((uint8_t)c);
}

/* Nearest finite e4m3 value to x (sign kept, so -0 -> 0x80); a tie goes to the code with
 * an even mantissa; |x| >= 448 saturates to +-448; NaN -> 0x7F / 0xFF.  The magnitudes of
 * codes 0x00..0x7E increase with the code, so a bisection finds the two neighbours. */
uint8_t lacto_e4m3_encode(float x) {
  pthread_once(&e4m3_mag_once, e4m3_mag_init);
  if (isnan(x)) return signbit(x) ? 0xFF : 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  int lo = 0, hi = 126; /* largest code c with value(c) <= a */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (e4m3_mag[mid] <= a)
      lo = mid;
    else
      hi = mid - 1;
  }
  int c = lo;
  double d0 = a - e4m3_mag[c];
  double d1 = e4m3_mag[c + 1] - a;
  if (d0 < d1) return (uint8_t)(sign | c);
  if (d1 < d0) return (uint8_t)(sign | (c + 1));
  return (uint8_t)(sign | ((c & 1) ? c + 1 : c));
}

/* Per-row (one row = the D channels of one (token, head)) quantiser of the FP8 KV cache:
 * amax = max |x|; scale = amax / 448 and y = x * (448 / amax), both in f32 (one rounding
 * each); code = e4m3(y).  amax = 0 gives scale 1 and y = x.  The stored value of element
 * d is e4m3_value(code) * scale. */
void lacto_quant_e4m3_rows(const float* x, int64_t rows, int32_t D, uint8_t* codes,
                           float* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * D;
    float amax = 0.0f;
    for (int32_t d = 0; d < D; ++d) {
      float a = fabsf(xr[d]);
      if (a > amax) amax = a;
    }
    float scale = 1.0f, inv = 1.0f;
    if (amax > 0.0f) {
      scale = amax / 448.0f;
      inv = 448.0f / amax;
    }
    for (int32_t d = 0; d < D; ++d) {
      float y = xr[d] * inv;
      codes[r * D + d] = lacto_e4m3_encode(y);
    }
    scales[r] = scale;
  }
}

/* Dequantise to f32 (one f32 multiply of the exact code value by the row scale). */
void lacto_e4m3_dequant_f32(const uint8_t* codes, const float* scales, int64_t rows, int32_t D,
                            float* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t d = 0; d < D; ++d)
      out[r * D + d] = (float)lacto_e4m3_value(codes[r * D + d]) * scales[r];
}

/* ===================================================================================== */
/* ConvKV compression ([NS] ConvKV Memory bullet: 1D convolution at 5:1 into a fixed-    */
/* length memory; [PR]: rolling compression at a fixed ratio; [W] "ConvKV Memory").      */
/* One memory slot from r consecutive evicted frames, per token u and channel c:         */
/*   m[u][c] = b[c] + sum_k w[c][k] * x_{k}[u][c]                                         */
/* ===================================================================================== */

/* The storage definition: an f32 fma chain in tap order, acc = b; acc = fmaf(w_k, x_k, acc).
 * x: [r][TC] (frame-major, token-major inside: element e -> channel e mod C); w: [C][r];
 * b: [C]; out: [TC]. */
void lacto_compress_chain_f32(const float* x, int32_t r, int64_t TC, int32_t C, const float* w,
                              const float* b, float* out) {
  for (int64_t e = 0; e < TC; ++e) {
    int64_t c = e % C;
    float acc = b[c];
    for (int32_t k = 0; k < r; ++k) acc = fmaf(w[c * r + k], x[(int64_t)k * TC + e], acc);
    out[e] = acc;
  }
}

/* The same sum in double (reference for the chain's rounding error). */
void lacto_compress_exact(const float* x, int32_t r, int64_t TC, int32_t C, const float* w,
                          const float* b, double* out) {
  for (int64_t e = 0; e < TC; ++e) {
    int64_t c = e % C;
    double acc = (double)b[c];
    for (int32_t k = 0; k < r; ++k) acc += (double)w[c * r + k] * (double)x[(int64_t)k * TC + e];
    out[e] = acc;
  }
}

/* ===================================================================================== */
/* RoPE with reset positions ([PR] RoPE Reset; [NS]).  Interleaved channel pairs          */
/* (2i, 2i+1) of each part; angle = pos * theta^(-2i / d_part);                           */
/* (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).                                        */
/*   mode 1: one part of D channels, pos = t*T + u.                                       */
/*   mode 3: parts (d_t, d_h, d_w) at channel offsets 0, d_t, d_t + d_h, with positions   */
/*           (t, u / grid_w, u mod grid_w).                                               */
/* ===================================================================================== */

typedef struct {
  int32_t mode, split[3], T, grid_w;
  double theta;
} rope_params;

/* cos and sin of every pair of one token: cs[2*i] = cos, cs[2*i+1] = sin, i < D/2. */
static void rope_token_angles(const rope_params* rp, int32_t D, int32_t t, int32_t u, double* cs) {
  if (rp->mode == 1) {
    double pos = (double)t * (double)rp->T + (double)u;
    for (int32_t i = 0; i < D / 2; ++i) {
      double ang = pos * pow(rp->theta, -2.0 * (double)i / (double)D);
      cs[2 * i] = cos(ang);
      cs[2 * i + 1] = sin(ang);
    }
    return;
  }
  double pos[3] = {(double)t, (double)(u / rp->grid_w), (double)(u % rp->grid_w)};
  int32_t pair = 0;
  for (int part = 0; part < 3; ++part) {
    int32_t dp = rp->split[part];
    for (int32_t i = 0; i < dp / 2; ++i, ++pair) {
      double ang = pos[part] * pow(rp->theta, -2.0 * (double)i / (double)dp);
      cs[2 * pair] = cos(ang);
      cs[2 * pair + 1] = sin(ang);
    }
  }
}

static void rope_apply_row(const double* cs, int32_t D, const double* x, double* y) {
  for (int32_t i = 0; i < D / 2; ++i) {
    double c = cs[2 * i], s = cs[2 * i + 1];
    double x0 = x[2 * i], x1 = x[2 * i + 1];
    y[2 * i] = x0 * c - x1 * s;
    y[2 * i + 1] = x0 * s + x1 * c;
  }
}

/* In place on x [n][H][D] (double), token i at positions (t[i], u[i]). */
void lacto_rope_rotate(double* x, int64_t n, int32_t H, int32_t D, const int32_t* t,
                       const int32_t* u, int32_t mode, const int32_t* split, int32_t T,
                       int32_t grid_w, double theta) {
  rope_params rp = {mode, {split[0], split[1], split[2]}, T, grid_w, theta};
  double* cs = (double*)malloc(sizeof(double) * (size_t)D);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
  for (int64_t i = 0; i < n; ++i) {
    rope_token_angles(&rp, D, t[i], u[i], cs);
    for (int32_t h = 0; h < H; ++h) {
      double* row = x + (i * H + h) * D;
      rope_apply_row(cs, D, row, tmp);
      memcpy(row, tmp, sizeof(double) * (size_t)D);
    }
  }
  free(cs);
  free(tmp);
}

/* ===================================================================================== */
/* Attention over [history | current] with the block-wise causal mask ([W] "Neighbor     */
/* Forcing": mask of block size m; "ConvKV Memory": context = memory, window, current).   */
/*   s_j = (rot(q_i) . rot(k_j)) / sqrt(D);  O_i = sum_j softmax(s)_j v_j;               */
/*   LSE_i = max + log sum exp.  History keys are visible to every query; current key j   */
/*   is visible to query i iff block(j) <= block(i).                                      */
/* Two independent forms: form 0 builds the explicit Lq x Lk 0/-inf mask matrix and       */
/* softmaxes over every key; form 1 walks the visible segments only.                      */
/* ===================================================================================== */

typedef struct {
  const lacto_attn_args* a;
  const double* hist_cs; /* [Lhist][D] cos/sin pairs */
  const double* cur_cs;  /* [Lq][D] */
  const double* mask;    /* [Lq][Lk] for form 0 */
  int64_t sel_lo, sel_hi;
} attn_job;

static double value_at(const float* x, const float* scale, int64_t tok, int32_t h, int32_t H,
                       int32_t D, int32_t d) {
  double v = (double)x[(tok * H + h) * D + d];
  if (scale) v *= (double)scale[tok * H + h];
  return v;
}

static int32_t block_of(const lacto_attn_args* a, int64_t i) {
  for (int32_t b = 0; b < a->n_blocks; ++b)
    if (i < a->block_start[b + 1]) return b;
  return a->n_blocks - 1;
}

static void* attn_worker(void* p) {
  attn_job* job = (attn_job*)p;
  const lacto_attn_args* a = job->a;
  const int32_t H = a->H, D = a->D;
  const int64_t Lk = a->Lhist + a->Lq;
  double* krot = (double*)malloc(sizeof(double) * (size_t)(Lk * D));
  double* vals = (double*)malloc(sizeof(double) * (size_t)(Lk * D));
  double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
  double* raw = (double*)malloc(sizeof(double) * (size_t)D);
  double* qh = (double*)malloc(sizeof(double) * (size_t)D);
  double* vn2 = (double*)malloc(sizeof(double) * (size_t)Lk); /* |v_j|^2 of head cur_head */
  int32_t cur_head = -1;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  for (int64_t n = job->sel_lo; n < job->sel_hi; ++n) {
    int32_t h = a->sel_head[n];
    int64_t i = a->sel_row[n];
    if (h != cur_head) { /* rotated keys and values of head h, key order [history | current] */
      for (int64_t j = 0; j < Lk; ++j) {
        int hist = j < a->Lhist;
        int64_t tok = hist ? j : j - a->Lhist;
        const double* cs = hist ? job->hist_cs + tok * D : job->cur_cs + tok * D;
        vn2[j] = 0.0;
        for (int32_t d = 0; d < D; ++d) {
          raw[d] = hist ? value_at(a->k_hist, a->k_hist_scale, tok, h, H, D, d)
                        : value_at(a->k_cur, a->k_cur_scale, tok, h, H, D, d);
          vals[j * D + d] = hist ? value_at(a->v_hist, a->v_hist_scale, tok, h, H, D, d)
                                 : value_at(a->v_cur, a->v_cur_scale, tok, h, H, D, d);
          vn2[j] += vals[j * D + d] * vals[j * D + d];
        }
        rope_apply_row(cs, D, raw, krot + j * D);
      }
      cur_head = h;
    }
    for (int32_t d = 0; d < D; ++d) raw[d] = value_at(a->q, a->q_scale, i, h, H, D, d);
    rope_apply_row(job->cur_cs + i * D, D, raw, qh);

    /* visible key set */
    int64_t n_vis = 0;
    double mx = -INFINITY;
    if (a->form == 0) {
      for (int64_t j = 0; j < Lk; ++j) {
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += qh[d] * krot[j * D + d];
        s[j] = dot * inv_sqrt_d + job->mask[i * Lk + j];
        if (s[j] > mx) mx = s[j];
      }
      n_vis = Lk;
    } else {
      int32_t bi = block_of(a, i);
      int64_t end = a->Lhist + a->block_start[bi + 1]; /* history, then current blocks <= bi */
      for (int64_t j = 0; j < end; ++j) {
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += qh[d] * krot[j * D + d];
        s[j] = dot * inv_sqrt_d;
        if (s[j] > mx) mx = s[j];
      }
      n_vis = end;
    }
    double l = 0.0, q2 = 0.0;
    double* o = a->out + n * D;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
      double pj = exp(s[j] - mx);
      if (pj == 0.0) continue;
      l += pj;
      q2 += pj * pj * vn2[j];
      for (int32_t d = 0; d < D; ++d) o[d] += pj * vals[j * D + d];
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= l;
    a->lse[n] = mx + log(l);
    if (a->rms) a->rms[n] = sqrt(q2) / l;
  }
  free(krot);
  free(vals);
  free(s);
  free(raw);
  free(qh);
  free(vn2);
  return NULL;
}

/* Returns 0 on success, 1 on bad arguments, 2 if form 0's mask matrix would be too big. */
int lacto_attention(const lacto_attn_args* a) {
  if (!a || a->H < 1 || a->D < 2 || (a->D & 1) || a->Lq < 1 || a->Lhist < 0 || a->n_blocks < 1)
    return 1;
  if (a->block_start[0] != 0 || a->block_start[a->n_blocks] != a->Lq) return 1;
  const int32_t D = a->D;
  const int64_t Lk = a->Lhist + a->Lq;
  rope_params rp = {a->rope_mode, {a->rope_split[0], a->rope_split[1], a->rope_split[2]}, a->T,
                    a->grid_w, a->rope_theta};
  double* hist_cs = (double*)malloc(sizeof(double) * (size_t)((a->Lhist > 0 ? a->Lhist : 1) * D));
  double* cur_cs = (double*)malloc(sizeof(double) * (size_t)(a->Lq * D));
  for (int64_t j = 0; j < a->Lhist; ++j)
    rope_token_angles(&rp, D, a->hist_t[j], a->hist_u[j], hist_cs + j * D);
  for (int64_t i = 0; i < a->Lq; ++i)
    rope_token_angles(&rp, D, a->cur_t[i], a->cur_u[i], cur_cs + i * D);

  double* mask = NULL;
  if (a->form == 0) {
    if (a->Lq * Lk > (int64_t)64 * 1024 * 1024) {
      free(hist_cs);
      free(cur_cs);
      return 2;
    }
    mask = (double*)malloc(sizeof(double) * (size_t)(a->Lq * Lk));
    for (int64_t i = 0; i < a->Lq; ++i) {
      int32_t bi = block_of(a, i);
      for (int64_t j = 0; j < Lk; ++j) {
        int visible = 1;
        if (j >= a->Lhist) visible = block_of(a, j - a->Lhist) <= bi;
        mask[i * Lk + j] = visible ? 0.0 : -INFINITY;
      }
    }
  }

  int32_t threads = a->threads < 1 ? 1 : (a->threads > 256 ? 256 : a->threads);
  if (threads > a->n_sel) threads = (int32_t)(a->n_sel > 0 ? a->n_sel : 1);
  attn_job* jobs = (attn_job*)calloc((size_t)threads, sizeof(attn_job));
  pthread_t* tid = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
  int* created = (int*)calloc((size_t)threads, sizeof(int));
  int64_t per = (a->n_sel + threads - 1) / threads;
  for (int32_t t = 0; t < threads; ++t) {
    jobs[t].a = a;
    jobs[t].hist_cs = hist_cs;
    jobs[t].cur_cs = cur_cs;
    jobs[t].mask = mask;
    jobs[t].sel_lo = t * per < a->n_sel ? t * per : a->n_sel;
    jobs[t].sel_hi = (t + 1) * per < a->n_sel ? (t + 1) * per : a->n_sel;
  }
  for (int32_t t = 1; t < threads; ++t)
    created[t] = pthread_create(&tid[t], NULL, attn_worker, &jobs[t]) == 0;
  attn_worker(&jobs[0]);
  for (int32_t t = 1; t < threads; ++t) {
    if (created[t])
      pthread_join(tid[t], NULL);
    else
      attn_worker(&jobs[t]);
  }
  free(jobs);
  free(tid);
  free(created);
  free(mask);
  free(hist_cs);
  free(cur_cs);
  return 0;
}
