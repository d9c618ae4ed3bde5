/*
 * oracle.c -- plain, slow CPU reference for the ternary selective-SSM mixer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; neither includes
 * the other.
 *
 * Sources (cited by page title and section):
 *  [TriSSM]   "Associative Recall Under Ternary Quantization ... at 5M Parameters",
 *             repository README: intro paragraph and the BitSSM mixer paragraph
 *             (Delta, B, C are BitNet b1.58 BitLinear layers with ternary weights
 *             and int8 activations; an RMSNorm precedes each ternary projection;
 *             the recurrence is evaluated with a parallel associative scan).
 *  [TMamba]   "Ternary Mamba: Grouped Quantization-Aware Training of W1.58A16
 *             State Space Models", abstract (grouped ternary scales, W1.58A16,
 *             the zero ratio of the ternary codes, error accumulation through
 *             the recurrence).
 *  [TSSM]     "Ternary State-Space Models: Hardware-Efficient Language Modeling
 *             with -1, 0, +1 Weights", Key Points and Abstract (weights in
 *             {-1,0,+1}; multiply-free add/subtract/skip inference; SSM parallel scan).
 *  [Builds-on] works cited by title in "Baseline Shape Decides the Verdict ...",
 *             section "Builds on": BitNet b1.58 ("The Era of 1-bit LLMs": absmean
 *             ternary weights, absmax int8 activations), Mamba ("Linear-Time
 *             Sequence Modeling with Selective State Spaces": softplus Delta,
 *             exp(Delta A) discretisation, selective recurrence); and in
 *             "SSDi8 ...", section "Builds on": "Transformers are SSMs" (state
 *             space duality, scalar A per head) and S4 (convolution mode).
 *  [Shape]    "Baseline Shape Decides the Verdict: A Controlled Re-Examination of
 *             Ternary Language Models at 60K Parameters", abstract, finding (ii):
 *             a plain gated diagonal-SSM block is the strongest block measured.
 *
 * Precision: every floating-point result is computed in fp64, except the steps
 * whose float value decides an integer (the absmean scale feeding the ternary
 * codes, the RMSNorm scale and the absmax scale feeding the int8 codes).  Those
 * follow one fixed fp32 order so that the integer codes are unique; the order is
 * written out where it is used.  Build with -ffp-contract=off and no fast-math.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------------------- */
/* storage rounding                                                          */
/* ------------------------------------------------------------------------- */

/* fp32 -> bf16 -> fp32, round to nearest, ties to even (finite inputs). */
float orc_round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u = u + 0x7FFFu + lsb;
  u &= 0xFFFF0000u;
  float r;
  memcpy(&r, &u, 4);
  return r;
}

/* Value as it is stored in an activation tensor of the given dtype. */
static double store_as(double v, int dtype) {
  float f = (float)v;
  if (dtype == ORC_BF16) f = orc_round_bf16(f);
  return (double)f;
}

void orc_round_array(const double* in, float* out, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)store_as(in[i], dtype);
}

/* ------------------------------------------------------------------------- */
/* O0: absmean ternary weights ([Builds-on] BitNet b1.58; [TMamba] grouped)   */
/* ------------------------------------------------------------------------- */

/*
 * gamma = mean |W| over the whole tensor (group == 0) or over each run of
 * `group` consecutive weights of a row (group > 0, k % group == 0).
 * Fixed order: each row (or row-group) is summed in fp64 from 0.0 in
 * ascending k; a per-tensor mean adds the row sums in ascending row order;
 * gamma = (float)(sum / count).
 */
void orc_absmean(const float* w, int64_t n, int64_t k, int64_t group, float* scale) {
  if (group == 0) {
    double total = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      double row = 0.0;
      for (int64_t j = 0; j < k; ++j) row += fabs((double)w[i * k + j]);
      total += row;
    }
    scale[0] = (float)(total / (double)(n * k));
  } else {
    int64_t ng = k / group;
    for (int64_t i = 0; i < n; ++i)
      for (int64_t g = 0; g < ng; ++g) {
        double s = 0.0;
        for (int64_t j = 0; j < group; ++j) s += fabs((double)w[i * k + g * group + j]);
        scale[i * ng + g] = (float)(s / (double)group);
      }
  }
}

/*
 * Ternary code of each weight: q = clamp(round(w / g), -1, +1) with
 * g = max(gamma, 1e-5), an IEEE fp32 division and round-half-to-even.
 * Returns the number of zero codes (the zero ratio numerator, [TMamba]).
 */
int64_t orc_ternarize(const float* w, int64_t n, int64_t k, int64_t group, const float* scale,
                      int8_t* codes) {
  int64_t zeros = 0;
  int64_t ng = group ? k / group : 1;
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      float gamma = group ? scale[i * ng + j / group] : scale[0];
      float g = fmaxf(gamma, 1e-5f);
      float r = rintf(w[i * k + j] / g);
      int8_t q = (int8_t)(r > 1.0f ? 1 : (r < -1.0f ? -1 : (int)r));
      codes[i * k + j] = q;
      zeros += (q == 0);
    }
  return zeros;
}

/*
 * Packed format (2 bits per weight).  A row of k weights occupies
 * 4 * ceil(k / 16) bytes: little-endian 32-bit words, each holding 16
 * consecutive weights.  Weight i of a word (i = 4 j + p, 0 <= j, p < 4) lives
 * in byte p at bits 2j..2j+1.  Code 0b00 = 0, 0b01 = +1, 0b11 = -1; 0b10 is
 * never written.  Weights past k in the last word are 0.
 */
int64_t orc_packed_row_bytes(int64_t k) { return ((k + 15) / 16) * 4; }

void orc_pack(const int8_t* codes, int64_t n, int64_t k, uint8_t* packed) {
  int64_t rb = orc_packed_row_bytes(k);
  memset(packed, 0, (size_t)(n * rb));
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      int q = codes[r * k + c];
      unsigned code = q == 0 ? 0u : (q == 1 ? 1u : 3u);
      int64_t word = c / 16;
      int i = (int)(c % 16);
      int j = i / 4, p = i % 4;
      packed[r * rb + word * 4 + p] |= (uint8_t)(code << (2 * j));
    }
}

/* Inverse of orc_pack.  Returns the number of invalid (0b10) codes seen. */
int64_t orc_unpack(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes) {
  int64_t rb = orc_packed_row_bytes(k), bad = 0;
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c) {
      int64_t word = c / 16;
      int i = (int)(c % 16);
      int j = i / 4, p = i % 4;
      unsigned code = (packed[r * rb + word * 4 + p] >> (2 * j)) & 3u;
      bad += (code == 2u);
      codes[r * k + c] = (int8_t)(code == 0u ? 0 : (code == 1u ? 1 : -1));
    }
  return bad;
}

/* ------------------------------------------------------------------------- */
/* O1 / O2: RMSNorm and absmax int8 ([TriSSM]; [Builds-on] BitNet b1.58)      */
/* ------------------------------------------------------------------------- */

/*
 * 1 / sqrt(mean(v^2) + eps) in fp32, in this fixed order: 64 partial sums,
 * partial j accumulating v[k]^2 for k = j, j+64, j+128, ... in ascending k with
 * a fused multiply-add from 0; then six halving rounds with distance 32, 16, 8,
 * 4, 2, 1 in which every partial j becomes s[j] + s[j ^ distance]; the mean is
 * s / k (fp32 division), then sqrt and a division into 1.
 */
float orc_rms_scale(const float* v, int64_t k, float eps) {
  float s[64];
  for (int j = 0; j < 64; ++j) s[j] = 0.0f;
  for (int64_t i = 0; i < k; ++i) s[i % 64] = fmaf(v[i], v[i], s[i % 64]);
  for (int d = 32; d >= 1; d /= 2) {
    float t[64];
    for (int j = 0; j < 64; ++j) t[j] = s[j] + s[j ^ d];
    memcpy(s, t, sizeof s);
  }
  float ms = s[0] / (float)k;
  return 1.0f / sqrtf(ms + eps);
}

/*
 * Normalised row xh[k] = (v[k] * r) * g[k] (g == NULL: unit gains, xh = v * r),
 * all fp32.  For A8 also: m = max |xh|, sigma = 127 / max(m, 1e-5) and
 * q = clamp(round_half_even(xh * sigma), -128, 127).
 */
void orc_norm_row(const float* v, int64_t k, const float* g, float eps, float* xh) {
  float r = orc_rms_scale(v, k, eps);
  for (int64_t i = 0; i < k; ++i) {
    float t = v[i] * r;
    xh[i] = g ? t * g[i] : t;
  }
}

float orc_quant_row(const float* xh, int64_t k, int8_t* q) {
  float m = 0.0f;
  for (int64_t i = 0; i < k; ++i) m = fmaxf(m, fabsf(xh[i]));
  float sigma = 127.0f / fmaxf(m, 1e-5f);
  for (int64_t i = 0; i < k; ++i) {
    float r = rintf(xh[i] * sigma);
    q[i] = (int8_t)(r > 127.0f ? 127 : (r < -128.0f ? -128 : (int)r));
  }
  return m;
}

/* ------------------------------------------------------------------------- */
/* O3 / O4: BitLinear forward ([TriSSM] BitLinear; [TSSM] multiply-free)       */
/* ------------------------------------------------------------------------- */

/*
 * y[m, n] for rows x[m, 0:k] (row stride ldx, values as float; bf16 inputs are
 * passed already widened).
 *  act_bits 8 : acc = sum_k q[k] * w[n, k] (exact integer); y = acc * s_w *
 *               max(m, 1e-5) / 127 (+ bias), fp64.  s_w is the tensor scale
 *               (group 0) or, for group > 0, each group's partial is scaled:
 *               y = max(m,1e-5)/127 * sum_g s[n,g] * acc_g.
 *  act_bits 16: y = sum_g s[n,g] * sum_{k in g} xh[k] * w[n,k] (+ bias), fp64,
 *               xh the fp32 RMSNorm output (no activation quantisation).
 * Optional stage outputs: xq [m,k], absmax [m], acc [m,n] (int32; A8 only).
 * Returns 0, or -1 if an accumulator does not fit int32.
 */
int orc_bitlinear(const float* x, int64_t m, int64_t k, int64_t ldx, const float* norm_w, float eps,
                  int act_bits, const int8_t* codes, const float* w_scale, int64_t n, int64_t group,
                  const float* bias, double* y, int8_t* xq, float* absmax, int32_t* acc_out) {
  int overflow = 0;
  int64_t ng = group ? k / group : 1;
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t r = 0; r < m; ++r) {
    float* xh = (float*)malloc(sizeof(float) * (size_t)k);
    int8_t* q = (int8_t*)malloc((size_t)k);
    orc_norm_row(x + r * ldx, k, norm_w, eps, xh);
    if (act_bits == 8) {
      float am = orc_quant_row(xh, k, q);
      if (xq) memcpy(xq + r * k, q, (size_t)k);
      if (absmax) absmax[r] = am;
      double deq = (double)fmaxf(am, 1e-5f) / 127.0;
      for (int64_t c = 0; c < n; ++c) {
        int64_t total = 0;
        double yv = 0.0;
        for (int64_t g = 0; g < ng; ++g) {
          int64_t k0 = group ? g * group : 0, k1 = group ? k0 + group : k;
          int64_t a = 0;
          for (int64_t i = k0; i < k1; ++i) a += (int64_t)q[i] * (int64_t)codes[c * k + i];
          total += a;
          yv += (double)(group ? w_scale[c * ng + g] : w_scale[0]) * (double)a;
        }
        if (total > INT32_MAX || total < INT32_MIN) overflow = 1;
        if (acc_out) acc_out[r * n + c] = (int32_t)total;
        yv *= deq;
        if (bias) yv += (double)bias[c];
        y[r * n + c] = yv;
      }
    } else {
      for (int64_t c = 0; c < n; ++c) {
        double yv = 0.0;
        for (int64_t g = 0; g < ng; ++g) {
          int64_t k0 = group ? g * group : 0, k1 = group ? k0 + group : k;
          double a = 0.0;
          for (int64_t i = k0; i < k1; ++i) a += (double)xh[i] * (double)codes[c * k + i];
          yv += (double)(group ? w_scale[c * ng + g] : w_scale[0]) * a;
        }
        if (bias) yv += (double)bias[c];
        y[r * n + c] = yv;
      }
    }
    free(xh);
    free(q);
  }
  return overflow ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* O5 / O6: selective scan ([Builds-on] Mamba, Transformers are SSMs)          */
/* ------------------------------------------------------------------------- */

double orc_softplus(double v) { return v > 20.0 ? v : log1p(exp(v)); }

/*
 * Sequential recurrence, fp64.  Layout (dense, token-major):
 *   x  [B, L, H*P]    delta [B, L, H] (pre-activation)    Bm, Cm [B, L, N]
 *   A  [H, N] (a_per_state = 1, Mamba-1, P = 1) or [H] (a_per_state = 0, SSD)
 *   D  [H] or NULL    h0, h_last [B, H, P, N] or NULL     y [B, L, H*P]
 * For each (b, h, p, n):  dt = softplus(delta + bias) (or delta + bias),
 *   h = exp(dt * A) * h + (dt * x) * Bm;   y += Cm * h;   then y += D * x.
 * B and C are shared by every channel / head (one group).
 */
void orc_selective_scan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int a_per_state,
                        const float* x, const float* delta, const float* delta_bias, int softplus,
                        const float* A, const float* Bm, const float* Cm, const float* D,
                        const float* h0, double* y, double* h_last) {
  int64_t HP = H * P;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t hd = 0; hd < H; ++hd) {
      double* h = (double*)malloc(sizeof(double) * (size_t)(P * N));
      for (int64_t i = 0; i < P * N; ++i) h[i] = h0 ? (double)h0[(b * H + hd) * P * N + i] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        int64_t tok = b * L + t;
        double dt = (double)delta[tok * H + hd] + (delta_bias ? (double)delta_bias[hd] : 0.0);
        if (softplus) dt = orc_softplus(dt);
        for (int64_t p = 0; p < P; ++p) {
          double xv = (double)x[tok * HP + hd * P + p];
          double acc = 0.0;
          for (int64_t s = 0; s < N; ++s) {
            double a = a_per_state ? (double)A[hd * N + s] : (double)A[hd];
            double hv = h[p * N + s];
            hv = exp(dt * a) * hv + (dt * xv) * (double)Bm[tok * N + s];
            h[p * N + s] = hv;
            acc += (double)Cm[tok * N + s] * hv;
          }
          y[tok * HP + hd * P + p] = acc + (D ? (double)D[hd] * xv : 0.0);
        }
      }
      if (h_last)
        for (int64_t i = 0; i < P * N; ++i) h_last[(b * H + hd) * P * N + i] = h[i];
      free(h);
    }
}

/*
 * O7: an independent evaluation of the same recurrence as a parallel
 * associative scan ([TriSSM]; [TSSM] "SSM parallel scan").  For one sequence
 * the step pairs e_t = (a_t, b_t) = (exp(dt_t A), dt_t x_t B_t) compose as
 * (a1, b1) o (a2, b2) = (a2 a1, a2 b1 + b2).  The textbook work-efficient
 * up-sweep / down-sweep over a power-of-two array gives the exclusive prefix
 * compositions; h_t = prefix_t o e_t applied to h0.
 */
static void compose(double a1, double b1, double a2, double b2, double* ao, double* bo) {
  *ao = a2 * a1;
  *bo = a2 * b1 + b2;
}

static void blelloch_exclusive(double* a, double* b, int64_t n2) {
  /* up-sweep */
  for (int64_t d = 1; d < n2; d *= 2)
    for (int64_t i = 2 * d - 1; i < n2; i += 2 * d) {
      double ao, bo;
      compose(a[i - d], b[i - d], a[i], b[i], &ao, &bo);
      a[i] = ao;
      b[i] = bo;
    }
  /* down-sweep with the identity (1, 0) */
  a[n2 - 1] = 1.0;
  b[n2 - 1] = 0.0;
  for (int64_t d = n2 / 2; d >= 1; d /= 2)
    for (int64_t i = 2 * d - 1; i < n2; i += 2 * d) {
      double la = a[i - d], lb = b[i - d];
      a[i - d] = a[i];
      b[i - d] = b[i];
      double ao, bo;
      compose(a[i], b[i], la, lb, &ao, &bo); /* prefix(left) then left block */
      a[i] = ao;
      b[i] = bo;
    }
}

void orc_selective_scan_blelloch(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                 int a_per_state, const float* x, const float* delta,
                                 const float* delta_bias, int softplus, const float* A,
                                 const float* Bm, const float* Cm, const float* D, const float* h0,
                                 double* y, double* h_last) {
  int64_t HP = H * P, n2 = 1;
  while (n2 < L) n2 *= 2;
  double* ea = (double*)malloc(sizeof(double) * (size_t)n2);
  double* eb = (double*)malloc(sizeof(double) * (size_t)n2);
  double* pa = (double*)malloc(sizeof(double) * (size_t)n2);
  double* pb = (double*)malloc(sizeof(double) * (size_t)n2);
  for (int64_t i = 0; i < batch * L * HP; ++i) y[i] = 0.0;
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t hd = 0; hd < H; ++hd)
      for (int64_t p = 0; p < P; ++p)
        for (int64_t s = 0; s < N; ++s) {
          double a_c = a_per_state ? (double)A[hd * N + s] : (double)A[hd];
          for (int64_t t = 0; t < n2; ++t) {
            if (t < L) {
              int64_t tok = b * L + t;
              double dt = (double)delta[tok * H + hd] + (delta_bias ? (double)delta_bias[hd] : 0.0);
              if (softplus) dt = orc_softplus(dt);
              ea[t] = exp(dt * a_c);
              eb[t] = dt * (double)x[tok * HP + hd * P + p] * (double)Bm[tok * N + s];
            } else {
              ea[t] = 1.0;
              eb[t] = 0.0;
            }
            pa[t] = ea[t];
            pb[t] = eb[t];
          }
          blelloch_exclusive(pa, pb, n2);
          double hin = h0 ? (double)h0[((b * H + hd) * P + p) * N + s] : 0.0;
          double hv = hin;
          for (int64_t t = 0; t < L; ++t) {
            double ia, ib;
            compose(pa[t], pb[t], ea[t], eb[t], &ia, &ib); /* inclusive prefix */
            hv = ia * hin + ib;
            y[(b * L + t) * HP + hd * P + p] += (double)Cm[(b * L + t) * N + s] * hv;
          }
          if (h_last) h_last[((b * H + hd) * P + p) * N + s] = hv;
        }
  if (D)
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t t = 0; t < L; ++t)
        for (int64_t hd = 0; hd < H; ++hd)
          for (int64_t p = 0; p < P; ++p) {
            int64_t i = (b * L + t) * HP + hd * P + p;
            y[i] += (double)D[hd] * (double)x[i];
          }
  free(ea);
  free(eb);
  free(pa);
  free(pb);
}

/*
 * Quadratic ("attention") form of the same map with h0 = 0, from state space
 * duality ("Transformers are SSMs"): y_t = sum_{s<=t} sum_n C_t[n] B_s[n]
 * exp(A_n * sum_{r=s+1..t} dt_r) dt_s x_s + D x_t.  O(L^2 N); small inputs only.
 */
void orc_selective_scan_quadratic(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                  int a_per_state, const float* x, const float* delta,
                                  const float* delta_bias, int softplus, const float* A,
                                  const float* Bm, const float* Cm, const float* D, double* y) {
  int64_t HP = H * P;
  double* dt = (double*)malloc(sizeof(double) * (size_t)L);
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t hd = 0; hd < H; ++hd) {
      for (int64_t t = 0; t < L; ++t) {
        double v = (double)delta[(b * L + t) * H + hd] + (delta_bias ? (double)delta_bias[hd] : 0.0);
        dt[t] = softplus ? orc_softplus(v) : v;
      }
      for (int64_t p = 0; p < P; ++p)
        for (int64_t t = 0; t < L; ++t) {
          double acc = 0.0;
          for (int64_t s = 0; s <= t; ++s) {
            double seg = 0.0;
            for (int64_t r = s + 1; r <= t; ++r) seg += dt[r];
            for (int64_t n = 0; n < N; ++n) {
              double a_c = a_per_state ? (double)A[hd * N + n] : (double)A[hd];
              acc += (double)Cm[(b * L + t) * N + n] * (double)Bm[(b * L + s) * N + n] *
                     exp(a_c * seg) * dt[s] * (double)x[(b * L + s) * HP + hd * P + p];
            }
          }
          int64_t i = (b * L + t) * HP + hd * P + p;
          y[i] = acc + (D ? (double)D[hd] * (double)x[i] : 0.0);
        }
    }
  free(dt);
}

/* ------------------------------------------------------------------------- */
/* O9: full-precision projections ([TriSSM]: the model keeps its in and out    */
/* projections in full precision, only Delta, B, C are ternary; its fp_ssm      */
/* baseline has no ternary projection)                                          */
/* ------------------------------------------------------------------------- */

/*
 * y[m, n] = sum_k x[m, k] * W[n, k], fp64, for a full-precision linear layer: no
 * RMSNorm, no quantisation, no bias.  x [m, ldx] (first k columns), W [n, k].
 */
void orc_dense(const float* x, int64_t m, int64_t k, int64_t ldx, const float* W, int64_t n, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i)
    for (int64_t j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int64_t c = 0; c < k; ++c) acc += (double)x[i * ldx + c] * (double)W[j * k + c];
      y[i * n + j] = acc;
    }
}

/* ------------------------------------------------------------------------- */
/* O8: the gated block around the mixer ([Builds-on] Mamba: the block's short   */
/* causal depthwise convolution with SiLU on the SSM input, and the SiLU gate   */
/* from the second in_proj branch; [Shape]: the gated diagonal-SSM block)      */
/* ------------------------------------------------------------------------- */

/* SiLU (x times the logistic sigmoid of x), fp64. */
double orc_silu(double a) { return a / (1.0 + exp(-a)); }

/*
 * Causal depthwise convolution of width K along time, then SiLU, per channel:
 *   a[b, t, c] = bias[c] + sum_{j=0..K-1} w[c, j] * x[b, t - (K - 1) + j, c]
 *   out[b, t, c] = silu(a), fp64, rounded to act_dtype.
 * x[b, t, c] at t < 0 is state[b, t + K - 1, c] when state is given, else 0.
 * Layout: x [B, L, ldx] (channels 0..C-1 used), w [C, K], bias [C] or NULL,
 * state [B, K - 1, C] or NULL, out [B, L, C].  state_out (nullable) [B, K - 1, C]
 * receives the last K - 1 inputs (from state and x), i.e. the state after the sequence.
 */
void orc_conv_silu(int64_t batch, int64_t L, int64_t C, int64_t K, const float* x, int64_t ldx,
                   const float* w, const float* bias, const float* state, int act_dtype, float* out,
                   float* state_out) {
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t c = 0; c < C; ++c) {
      for (int64_t t = 0; t < L; ++t) {
        double a = bias ? (double)bias[c] : 0.0;
        for (int64_t j = 0; j < K; ++j) {
          int64_t ts = t - (K - 1) + j;
          double xv = 0.0;
          if (ts >= 0) xv = (double)x[(b * L + ts) * ldx + c];
          else if (state) xv = (double)state[(b * (K - 1) + (ts + K - 1)) * C + c];
          a += (double)w[c * K + j] * xv;
        }
        out[(b * L + t) * C + c] = (float)store_as(orc_silu(a), act_dtype);
      }
      if (state_out)
        for (int64_t i = 0; i < K - 1; ++i) {
          int64_t ts = L - (K - 1) + i;  /* input time held in slot i */
          float v = 0.0f;
          if (ts >= 0) v = x[(b * L + ts) * ldx + c];
          else if (state) v = state[(b * (K - 1) + (ts + K - 1)) * C + c];
          state_out[(b * (K - 1) + i) * C + c] = v;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* O5 / O6: the mixer ([TriSSM] BitSSM mixer; [TMamba] W1.58A16 SSD shape)     */
/* ------------------------------------------------------------------------- */

/*
 * Ternary weights of one mixer layer, as codes + scales (from orc_absmean and
 * orc_ternarize).  Mamba-1 kind uses all four projections; the SSD kind uses
 * w_in and w_out only.
 */
typedef struct {
  const int8_t *c_in, *c_x, *c_dt, *c_out;
  const float *s_in, *s_x, *s_dt, *s_out;
  const float *g_in, *g_x, *g_dt, *g_out; /* RMSNorm gains or NULL */
  const float *dt_bias, *A, *D;
  const float *conv_w, *conv_b; /* gated block only: [Cc, d_conv], [Cc] or NULL */
  const float *f_in, *f_x, *f_dt, *f_out; /* full-precision weights [n_out, k] (O9) or NULL */
} orc_mixer_weights;

/*
 * Mamba-1 kind (a_per_state = 1):
 *   x = BL(u; W_in) [M, Di];  p = BL(x; W_x) = [delta_r | B | C] [M, R + 2N];
 *   z = BL(delta_r; W_dt) [M, Di] (kept unrounded: it is consumed inside the scan);
 *   y = scan(x, softplus(z + dt_bias), A, B, C, D);  out = BL(y; W_out) (+ u).
 * SSD kind (a_per_state = 0, act_bits 16, per-group scales):
 *   v = BL(u; W_in) = [x (H P) | B (N) | C (N) | dt (H)] [M, H P + 2N + H];
 *   y = scan(x, softplus(dt + dt_bias), A[H], B, C, D);  out = BL(y; W_out) (+ u).
 * Every stored activation (x, p, v, y, out) is rounded to act_dtype, as a
 * kernel that stores it must.
 * Gated block (gated != 0, O8): in_proj gains Di output rows for the gate branch
 * zg, placed after the others ([x | zg] for Mamba-1, [x | B | C | dt | zg] for
 * SSD); the SSM input channels (x for Mamba-1, x, B and C for SSD; Cc of them)
 * go through orc_conv_silu of width d_conv before anything reads them, and the
 * scan output becomes y * silu(zg) (fp64, rounded to act_dtype) before out_proj.
 * fp_proj (O9): 0 every projection ternary; 1 in_proj and out_proj full precision
 * (orc_dense with f_in / f_out; the TriSSM model); 2 every projection full precision
 * (the fp_ssm baseline; the Mamba-1 dt projection output is then stored in act_dtype
 * before the scan reads it, like every other stored activation).
 */
int orc_mixer(int kind, int64_t d_model, int64_t d_inner, int64_t d_state, int64_t dt_rank,
              int64_t nheads, int64_t headdim, int64_t group, int act_bits, int act_dtype,
              float eps, const orc_mixer_weights* w, const float* u, int64_t batch, int64_t L,
              int residual, int gated, int64_t d_conv, int fp_proj, double* out) {
  int64_t M = batch * L, Dm = d_model, Di = d_inner, N = d_state, R = dt_rank;
  int rc = 0;
  float* y32 = (float*)malloc(sizeof(float) * (size_t)(M * Di));
  double* yd = (double*)malloc(sizeof(double) * (size_t)(M * Di));
  float* zg = gated ? (float*)malloc(sizeof(float) * (size_t)(M * Di)) : NULL;
  if (kind == 0) {
    int64_t PW = R + 2 * N, XW = gated ? 2 * Di : Di;
    double* xd = (double*)malloc(sizeof(double) * (size_t)(M * XW));
    float* xz = (float*)malloc(sizeof(float) * (size_t)(M * XW));
    float* x32 = (float*)malloc(sizeof(float) * (size_t)(M * Di));
    double* pd = (double*)malloc(sizeof(double) * (size_t)(M * PW));
    float* p32 = (float*)malloc(sizeof(float) * (size_t)(M * PW));
    double* zd = (double*)malloc(sizeof(double) * (size_t)(M * Di));
    float* z32 = (float*)malloc(sizeof(float) * (size_t)(M * Di));
    float* B32 = (float*)malloc(sizeof(float) * (size_t)(M * N));
    float* C32 = (float*)malloc(sizeof(float) * (size_t)(M * N));
    if (fp_proj >= 1) orc_dense(u, M, Dm, Dm, w->f_in, XW, xd);
    else rc |= orc_bitlinear(u, M, Dm, Dm, w->g_in, eps, act_bits, w->c_in, w->s_in, XW, group, NULL,
                             xd, NULL, NULL, NULL);
    orc_round_array(xd, xz, M * XW, act_dtype);
    if (gated) {
      orc_conv_silu(batch, L, Di, d_conv, xz, XW, w->conv_w, w->conv_b, NULL, act_dtype, x32, NULL);
      for (int64_t i = 0; i < M; ++i)
        for (int64_t c = 0; c < Di; ++c) zg[i * Di + c] = xz[i * XW + Di + c];
    } else {
      memcpy(x32, xz, sizeof(float) * (size_t)(M * Di));
    }
    if (fp_proj >= 2) orc_dense(x32, M, Di, Di, w->f_x, PW, pd);
    else rc |= orc_bitlinear(x32, M, Di, Di, w->g_x, eps, act_bits, w->c_x, w->s_x, PW, group, NULL, pd,
                             NULL, NULL, NULL);
    orc_round_array(pd, p32, M * PW, act_dtype);
    /* dt projection reads the first R columns of p (row stride PW) */
    if (fp_proj >= 2) {
      orc_dense(p32, M, R, PW, w->f_dt, Di, zd);
      orc_round_array(zd, z32, M * Di, act_dtype); /* stored, then read by the scan */
    } else {
      rc |= orc_bitlinear(p32, M, R, PW, w->g_dt, eps, act_bits, w->c_dt, w->s_dt, Di, group, NULL,
                          zd, NULL, NULL, NULL);
      /* z is not stored: pass it to the scan at fp32 width (the scan's input type) */
      for (int64_t i = 0; i < M * Di; ++i) z32[i] = (float)zd[i];
    }
    for (int64_t i = 0; i < M; ++i)
      for (int64_t s = 0; s < N; ++s) {
        B32[i * N + s] = p32[i * PW + R + s];
        C32[i * N + s] = p32[i * PW + R + N + s];
      }
    orc_selective_scan(batch, L, Di, 1, N, 1, x32, z32, w->dt_bias, 1, w->A, B32, C32, w->D, NULL,
                       yd, NULL);
    free(xd); free(xz); free(x32); free(pd); free(p32); free(zd); free(z32); free(B32); free(C32);
  } else {
    int64_t H = nheads, P = headdim, VW0 = H * P + 2 * N + H, VW = gated ? VW0 + Di : VW0;
    int64_t Cc = H * P + 2 * N;
    double* vd = (double*)malloc(sizeof(double) * (size_t)(M * VW));
    float* v32 = (float*)malloc(sizeof(float) * (size_t)(M * VW));
    float* xbc = (float*)malloc(sizeof(float) * (size_t)(M * Cc));
    float* xs = (float*)malloc(sizeof(float) * (size_t)(M * H * P));
    float* B32 = (float*)malloc(sizeof(float) * (size_t)(M * N));
    float* C32 = (float*)malloc(sizeof(float) * (size_t)(M * N));
    float* dt32 = (float*)malloc(sizeof(float) * (size_t)(M * H));
    if (fp_proj >= 1) orc_dense(u, M, Dm, Dm, w->f_in, VW, vd);
    else rc |= orc_bitlinear(u, M, Dm, Dm, w->g_in, eps, act_bits, w->c_in, w->s_in, VW, group, NULL, vd,
                             NULL, NULL, NULL);
    orc_round_array(vd, v32, M * VW, act_dtype);
    if (gated) {
      orc_conv_silu(batch, L, Cc, d_conv, v32, VW, w->conv_w, w->conv_b, NULL, act_dtype, xbc, NULL);
    } else {
      for (int64_t i = 0; i < M; ++i)
        for (int64_t c = 0; c < Cc; ++c) xbc[i * Cc + c] = v32[i * VW + c];
    }
    for (int64_t i = 0; i < M; ++i) {
      for (int64_t c = 0; c < H * P; ++c) xs[i * H * P + c] = xbc[i * Cc + c];
      for (int64_t s = 0; s < N; ++s) {
        B32[i * N + s] = xbc[i * Cc + H * P + s];
        C32[i * N + s] = xbc[i * Cc + H * P + N + s];
      }
      for (int64_t hd = 0; hd < H; ++hd) dt32[i * H + hd] = v32[i * VW + H * P + 2 * N + hd];
      if (gated)
        for (int64_t c = 0; c < Di; ++c) zg[i * Di + c] = v32[i * VW + VW0 + c];
    }
    orc_selective_scan(batch, L, H, P, N, 0, xs, dt32, w->dt_bias, 1, w->A, B32, C32, w->D, NULL,
                       yd, NULL);
    free(vd); free(v32); free(xbc); free(xs); free(B32); free(C32); free(dt32);
  }
  if (gated)
    for (int64_t i = 0; i < M * Di; ++i) yd[i] = yd[i] * orc_silu((double)zg[i]);
  free(zg);
  orc_round_array(yd, y32, M * Di, act_dtype);
  if (fp_proj >= 1) orc_dense(y32, M, Di, Di, w->f_out, Dm, out);
  else rc |= orc_bitlinear(y32, M, Di, Di, w->g_out, eps, act_bits, w->c_out, w->s_out, Dm, group, NULL,
                           out, NULL, NULL, NULL);
  if (residual)
    for (int64_t i = 0; i < M * Dm; ++i) out[i] += (double)u[i];
  for (int64_t i = 0; i < M * Dm; ++i) out[i] = store_as(out[i], act_dtype);
  free(y32);
  free(yd);
  return rc;
}

/* Thread count of the parallel loops above (the timed CPU baseline runs single-threaded and
 * on every core); the arithmetic and its order per output do not depend on it. */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }
