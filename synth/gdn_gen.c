/*
 * Seeded synthetic verify-step state buffers for the state reader.
 *
 * Each (sequence, selected layer, head) pair gets its own counter-based random
 * stream and runs the fp32 gated delta rule from a zero state,
 *
 *   S_i = alpha_i S_{i-1} + beta_i (v_i - alpha_i S_{i-1} k_i) k_i^T,
 *
 * which is the expanded form of S_i = S_{i-1} alpha_i (I - beta_i k_i k_i^T)
 * + beta_i v_i k_i^T (ReaDy arXiv text, Appendix D.1, Eqs. D.2-D.3; rainbus
 * summary, 前置知识 "Gated DeltaNet 循环状态"), with unit-norm Gaussian keys,
 * standard normal values, alpha ~ U(alpha_lo, 1) and beta ~ U(0, 1).  Buffer
 * position p receives S_{t+p}: the committed state after the root token and p
 * drafts of an 8-position verify block.
 *
 * This file is an input generator: it holds none of the reader's arithmetic.
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), written from its published round
 * function.  Key = the 64-bit seed; counter = (block, step, stream low,
 * stream high | domain).  Uniforms take the top 24 bits, offset by half a unit
 * so they lie strictly inside (0, 1); normals come from the Box-Muller
 * transform in single precision (libm logf, sincosf).  Every pair's stream depends only on
 * (seed, pair index), so the result does not depend on the thread count.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
  uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
  uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n1 = lo1;
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  uint32_t n3 = lo0;
  c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    philox_round(c, k);
    if (r < 9) { k[0] += PHILOX_W0; k[1] += PHILOX_W1; }
  }
  memcpy(out, c, sizeof(c));
}

enum { DOM_KEY = 0, DOM_VALUE = 1, DOM_GATE = 2 };

static inline double unit_open(uint32_t x) {  /* (0, 1) */
  return ((double)(x >> 8) + 0.5) * (1.0 / 16777216.0);
}

/* n normals for (stream, step, domain) into out[0..n). */
static void normals(uint64_t seed, uint64_t stream, uint32_t step, uint32_t dom,
                    int n, float* out) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  const float two_pi = 6.28318530717958647692f;
  for (int blk = 0; 4 * blk < n; ++blk) {
    uint32_t ctr[4] = {(uint32_t)blk, step, (uint32_t)stream,
                       (uint32_t)(stream >> 32) ^ (dom << 28)};
    uint32_t r[4];
    synth_philox4x32_10(ctr, key, r);
    for (int h = 0; h < 2; ++h) {
      float u1 = (float)unit_open(r[2 * h]), u2 = (float)unit_open(r[2 * h + 1]);
      float rad = sqrtf(-2.0f * logf(u1));
      float sn, cs;
      sincosf(two_pi * u2, &sn, &cs);
      int i0 = 4 * blk + 2 * h;
      if (i0 < n) out[i0] = rad * cs;
      if (i0 + 1 < n) out[i0 + 1] = rad * sn;
    }
  }
}

static void gates(uint64_t seed, uint64_t stream, uint32_t step, float alpha_lo,
                  float* alpha, float* beta) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {0u, step, (uint32_t)stream, (uint32_t)(stream >> 32) ^ ((uint32_t)DOM_GATE << 28)};
  uint32_t r[4];
  synth_philox4x32_10(ctr, key, r);
  *alpha = (float)(alpha_lo + (1.0 - alpha_lo) * unit_open(r[0]));
  *beta = (float)unit_open(r[1]);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Draw the step's key (normalised), value and gates; gates may be forced. */
static void draw_step(uint64_t seed, uint64_t stream, uint32_t step, int dk, int dv,
                      float alpha_lo, float alpha_fixed, float beta_fixed,
                      float* k, float* v, float* alpha, float* beta) {
  normals(seed, stream, step, DOM_KEY, dk, k);
  normals(seed, stream, step, DOM_VALUE, dv, v);
  double ss = 0.0;
  for (int i = 0; i < dk; ++i) ss += (double)k[i] * k[i];
  float inv = (float)(1.0 / sqrt(ss));
  for (int i = 0; i < dk; ++i) k[i] *= inv;
  gates(seed, stream, step, alpha_lo, alpha, beta);
  if (alpha_fixed >= 0.0f) *alpha = alpha_fixed;
  if (beta_fixed >= 0.0f) *beta = beta_fixed;
}

/*
 * buf: [B][P][L_tot][H][d_v][d_k] (strides in elements for the four outer
 * axes, tile contiguous), fp32 (out_bf16 = 0) or bf16 bit patterns.
 * layer_slots[l] (l < L_sel): slot on the layer axis that receives selected
 * layer l.  Pair stream index = (b * L_sel + l) * H + a.
 * coef_out (nullable): [npairs][t + P - 1][d_k + d_v + 2] = (k, v, alpha, beta)
 * of steps 1 .. t+P-1.
 * alpha_fixed / beta_fixed >= 0 override the drawn gates (tests).
 * Returns 0, or -1 on a bad argument.
 */
int synth_gdn_states(void* buf, int out_bf16, int64_t stride_b, int64_t stride_p,
                     int64_t stride_l, int64_t stride_h, int B, int P, int L_sel,
                     const int32_t* layer_slots, int H, int d_k, int d_v, int t,
                     float alpha_lo, float alpha_fixed, float beta_fixed, uint64_t seed,
                     float* coef_out, int nthreads) {
  if (!buf || B < 0 || P < 1 || L_sel < 1 || H < 1 || d_k < 1 || d_v < 1 || t < 0 || !layer_slots)
    return -1;
  const int64_t npairs = (int64_t)B * L_sel * H;
  const int steps = t + P - 1;
  const int coef_w = d_k + d_v + 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int failed = 0;
#pragma omp parallel
  {
    float* S = (float*)malloc(sizeof(float) * (size_t)d_v * d_k);
    float* y = (float*)malloc(sizeof(float) * (size_t)d_v);      /* S_{i-1} k_i */
    float* k = (float*)malloc(sizeof(float) * (size_t)d_k);
    float* v = (float*)malloc(sizeof(float) * (size_t)d_v);
    float* kn = (float*)malloc(sizeof(float) * (size_t)d_k);
    float* vn = (float*)malloc(sizeof(float) * (size_t)d_v);
    if (!S || !y || !k || !v || !kn || !vn) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t s = 0; s < npairs; ++s) {
        const int b = (int)(s / ((int64_t)L_sel * H));
        const int l = (int)((s / H) % L_sel);
        const int a = (int)(s % H);
        const uint64_t stream = (uint64_t)s;
        float alpha = 0.f, beta = 0.f, alpha_n = 0.f, beta_n = 0.f;
        memset(S, 0, sizeof(float) * (size_t)d_v * d_k);
        memset(y, 0, sizeof(float) * (size_t)d_v);
        memset(kn, 0, sizeof(float) * (size_t)d_k);
        if (steps >= 1)
          draw_step(seed, stream, 1u, d_k, d_v, alpha_lo, alpha_fixed, beta_fixed, k, v, &alpha, &beta);
        for (int i = 0; i <= steps; ++i) {
          if (i >= 1) {
            /* coefficients of step i are in (k, v, alpha, beta); y = S_{i-1} k */
            if (coef_out) {
              float* c = coef_out + ((size_t)s * steps + (size_t)(i - 1)) * coef_w;
              memcpy(c, k, sizeof(float) * d_k);
              memcpy(c + d_k, v, sizeof(float) * d_v);
              c[d_k + d_v] = alpha;
              c[d_k + d_v + 1] = beta;
            }
            const int have_next = (i + 1 <= steps);
            if (have_next)
              draw_step(seed, stream, (uint32_t)(i + 1), d_k, d_v, alpha_lo, alpha_fixed,
                        beta_fixed, kn, vn, &alpha_n, &beta_n);
            for (int r = 0; r < d_v; ++r) {
              const float w = beta * (v[r] - alpha * y[r]);
              float* row = S + (size_t)r * d_k;
              float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
              int c0 = 0;
              for (; c0 + 8 <= d_k; c0 += 8) {
                for (int j = 0; j < 8; ++j) {
                  float nv = alpha * row[c0 + j] + w * k[c0 + j];
                  row[c0 + j] = nv;
                  acc[j] += nv * kn[c0 + j];
                }
              }
              for (; c0 < d_k; ++c0) {
                float nv = alpha * row[c0] + w * k[c0];
                row[c0] = nv;
                acc[0] += nv * kn[c0];
              }
              y[r] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
            }
            if (have_next) {
              float* tp;
              tp = k; k = kn; kn = tp;
              tp = v; v = vn; vn = tp;
              alpha = alpha_n;
              beta = beta_n;
            }
          }
          if (i >= t) {
            const int p = i - t;
            const int64_t off = (int64_t)b * stride_b + (int64_t)p * stride_p +
                                (int64_t)layer_slots[l] * stride_l + (int64_t)a * stride_h;
            const size_t ne = (size_t)d_v * d_k;
            if (out_bf16) {
              uint16_t* dst = (uint16_t*)buf + off;
              for (size_t e = 0; e < ne; ++e) dst[e] = f32_to_bf16_rne(S[e]);
            } else {
              memcpy((float*)buf + off, S, sizeof(float) * ne);
            }
          }
        }
      }
    }
    free(S); free(y); free(k); free(v); free(kn); free(vn);
  }
  return failed ? -1 : 0;
}

/* fp32 -> bf16 bit patterns, round to nearest even (inputs of bf16 configs). */
void synth_to_bf16(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(x[i]);
}
