/* Drives every entry of the CPU oracle (oracle/lact_oracle.c) and the input generator
 * (synth/synth.c) on small inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Exit status 0 = every call ran
 * and its results are finite where they must be; the sanitizers abort on any invalid
 * access or undefined operation. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lact_oracle.h"

/* the input generator's entry points (synth/synth.c) */
void synth_normal(uint64_t seed, uint32_t tensor, uint64_t frame, uint64_t first, uint64_t count,
                  double stddev, float* out, int threads);
void synth_outliers(uint64_t seed, uint32_t tensor, uint64_t frame, uint64_t first,
                    uint64_t count, double prob, float factor, float* x, int threads);
void synth_uniform(uint64_t seed, uint32_t tensor, uint64_t frame, uint64_t first, uint64_t count,
                   float* out, int threads);
uint64_t synth_stream_key(uint64_t seed, uint32_t tensor, uint64_t frame);

static int fails = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "line %d: %s\n", __LINE__, #c);         \
      ++fails;                                                \
    }                                                         \
  } while (0)

static float* fbuf(size_t n) { return (float*)calloc(n, sizeof(float)); }

int main(void) {
  /* codecs over every code and a spread of values */
  for (int c = 0; c < 65536; ++c) {
    double v = lacto_bf16_value((uint16_t)c);
    if (isfinite(v)) CHECK(lacto_bf16_encode((float)v) == (uint16_t)c || v == 0.0);
  }
  for (int c = 0; c < 256; ++c) {
    double v = lacto_e4m3_value((uint8_t)c);
    if (!isnan(v)) CHECK(lacto_e4m3_encode((float)v) == (uint8_t)c);
  }
  const int D = 64, H = 2, T = 6, gw = 3, nh = 3, nc = 2;
  const int64_t Lh = (int64_t)nh * T, Lq = (int64_t)nc * T;
  float* x = fbuf((size_t)(Lh + Lq) * H * D);
  synth_normal(0, 2, 0, 0, (uint64_t)(Lh + Lq) * H * D, 1.0, x, 3);
  synth_outliers(0, 2, 0, 0, (uint64_t)(Lh + Lq) * H * D, 0.01, 8.0f, x, 3);
  float* un = fbuf(100);
  synth_uniform(0, 8, 0, 0, 100, un, 2);
  for (int i = 0; i < 100; ++i) CHECK(un[i] > 0.0f && un[i] <= 1.0f);
  CHECK(synth_stream_key(1, 2, 3) != synth_stream_key(1, 2, 4));
  uint16_t* b16 = (uint16_t*)calloc((size_t)(Lh + Lq) * H * D, 2);
  lacto_bf16_encode_array(x, b16, (Lh + Lq) * H * D);

  /* FP8 rows, dequantised */
  const int64_t rows = (Lh + Lq) * H;
  uint8_t* codes = (uint8_t*)calloc((size_t)rows * D, 1);
  float* scales = fbuf((size_t)rows);
  float* deq = fbuf((size_t)rows * D);
  lacto_quant_e4m3_rows(x, rows, D, codes, scales);
  lacto_e4m3_dequant_f32(codes, scales, rows, D, deq);
  for (int64_t i = 0; i < rows * D; ++i) CHECK(isfinite(deq[i]));

  /* compression of 5 frames of T tokens x C channels */
  const int r = 5, C = H * D;
  const int64_t TC = (int64_t)T * C;
  float* fr = fbuf((size_t)r * TC);
  synth_normal(0, 3, 1, 0, (uint64_t)r * TC, 1.0, fr, 1);
  float* w = fbuf((size_t)C * r);
  float* b = fbuf((size_t)C);
  synth_normal(0, 4, 0, 0, (uint64_t)C * r, 0.2, w, 1);
  float* m32 = fbuf((size_t)TC);
  double* m64 = (double*)calloc((size_t)TC, sizeof(double));
  lacto_compress_chain_f32(fr, r, TC, C, w, b, m32);
  lacto_compress_exact(fr, r, TC, C, w, b, m64);
  for (int64_t i = 0; i < TC; ++i) CHECK(fabs((double)m32[i] - m64[i]) < 1e-4);

  /* RoPE, 1D and 3D */
  int32_t* tt = (int32_t*)calloc((size_t)(Lh + Lq), 4);
  int32_t* uu = (int32_t*)calloc((size_t)(Lh + Lq), 4);
  for (int64_t i = 0; i < Lh + Lq; ++i) {
    tt[i] = (int32_t)(i / T);
    uu[i] = (int32_t)(i % T);
  }
  double* xr = (double*)calloc((size_t)(Lh + Lq) * H * D, sizeof(double));
  for (int64_t i = 0; i < (Lh + Lq) * H * D; ++i) xr[i] = x[i];
  const int32_t s1[3] = {64, 0, 0}, s3[3] = {22, 22, 20};
  lacto_rope_rotate(xr, Lh + Lq, H, D, tt, uu, 1, s1, T, gw, 10000.0);
  lacto_rope_rotate(xr, Lh + Lq, H, D, tt, uu, 3, s3, T, gw, 10000.0);

  /* attention: both forms, two query blocks, scales on every tensor, all rows and a
   * subset, one to four threads */
  const int64_t bs[3] = {0, T, Lq};
  float* ones = fbuf((size_t)rows);
  for (int64_t i = 0; i < rows; ++i) ones[i] = 0.5f + (float)(i % 3);
  const int64_t nsel = H * Lq;
  int32_t* sh = (int32_t*)calloc((size_t)nsel, 4);
  int64_t* sr = (int64_t*)calloc((size_t)nsel, 8);
  for (int64_t i = 0; i < nsel; ++i) {
    sh[i] = (int32_t)(i / Lq);
    sr[i] = i % Lq;
  }
  double* out = (double*)calloc((size_t)nsel * D, sizeof(double));
  double* lse = (double*)calloc((size_t)nsel, sizeof(double));
  double* rms = (double*)calloc((size_t)nsel, sizeof(double));
  for (int form = 0; form < 2; ++form) {
    for (int threads = 1; threads <= 4; threads += 3) {
      for (int scaled = 0; scaled < 2; ++scaled) {
        lacto_attn_args a;
        memset(&a, 0, sizeof(a));
        a.H = H;
        a.D = D;
        a.Lq = Lq;
        a.Lhist = Lh;
        const float* base = scaled ? deq : x;
        a.k_hist = base;
        a.v_hist = base + Lh * H * D / 2;
        a.q = base + Lh * H * D;
        a.k_cur = base + Lh * H * D;
        a.v_cur = base + Lh * H * D;
        if (scaled) {
          a.q_scale = ones;
          a.k_hist_scale = ones;
          a.v_hist_scale = ones + 1;
          a.k_cur_scale = ones;
          a.v_cur_scale = ones + 2;
        }
        a.hist_t = tt;
        a.hist_u = uu;
        a.cur_t = tt + Lh;
        a.cur_u = uu + Lh;
        a.rope_mode = 3;
        memcpy(a.rope_split, s3, sizeof(s3));
        a.T = T;
        a.grid_w = gw;
        a.rope_theta = 10000.0;
        a.n_blocks = 2;
        a.block_start = bs;
        a.n_sel = scaled ? nsel / 3 : nsel;
        a.sel_head = sh;
        a.sel_row = sr;
        a.form = form;
        a.threads = threads;
        a.out = out;
        a.lse = lse;
        a.rms = scaled ? rms : NULL;
        CHECK(lacto_attention(&a) == 0);
        for (int64_t i = 0; i < a.n_sel; ++i) CHECK(isfinite(lse[i]));
      }
    }
  }
  free(x); free(un); free(b16); free(codes); free(scales); free(deq); free(fr); free(w); free(b);
  free(m32); free(m64); free(tt); free(uu); free(xr); free(ones); free(sh); free(sr); free(out);
  free(lse); free(rms);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  return fails ? 1 : 0;
}
