/*
 * psi_oracle.c -- plain, slow, dense CPU oracle for the paged BF16 block
 * operator of Precision-Preserving Subtensor Inference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * with the HIP library: it is an independent statement of what the paged
 * operator must compute.
 *
 * Source cited throughout as [PSI]: the paper "Precision-Preserving Subtensor
 * Inference for a 22B Joint Audio-Video Generator under a Fixed GPU Working
 * Set" (Shen and Liao, arXiv 2611.08023v1).
 *
 * What it computes: the DENSE construction.  The paged operator partitions
 * output columns, hidden channels, head groups and key tiles; [PSI] sec. II-B
 * shows these partitions preserve the dense real-arithmetic result, so the
 * oracle is that dense result written out plainly, with the BF16 write
 * boundaries that [PSI] sec. III-A declares.
 *
 * Numeric conventions (plain readings of the pages; each is listed as a
 * reading in the design notes):
 *   B(v)   round to bfloat16, round-to-nearest ties-to-even ([PSI] eq. (5)
 *          uses exactly this rounding); NaN -> 0x7FC0.
 *   f(u)   widen a bfloat16 bit pattern to float (exact).
 *   fp32 accumulation is a sequential chain, index ascending, starting at
 *   +0.0f; every product and sum is one IEEE binary32 operation.  Build with
 *   -ffp-contract=off (no fused multiply-add) and without -ffast-math.
 *   The tanh-GELU is evaluated in double and rounded once to bfloat16.
 *
 * Parallelism: OpenMP only across independent output rows, so results do not
 * depend on the thread count.
 *
 * Every matrix is row-major.  Weights use the [out, in] "Linear" layout, so
 * y = x W^T + b.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the OpenMP loops below will use (reported with timings). */
int orc_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------ */
/* BF16 rounding, [PSI] sec. II-C eq. (5)                               */
/* ------------------------------------------------------------------ */

float orc_f(uint16_t u) {
  uint32_t w = ((uint32_t)u) << 16;
  float v;
  memcpy(&v, &w, sizeof v);
  return v;
}

/* B(v) for a binary32 value: keep the top 16 bits, rounding the dropped 16
 * bits to nearest with ties to the even kept pattern. */
uint16_t orc_bf16_from_float(float v) {
  uint32_t w;
  memcpy(&w, &v, sizeof w);
  if ((w & 0x7F800000u) == 0x7F800000u && (w & 0x007FFFFFu) != 0u)
    return (uint16_t)0x7FC0u; /* NaN */
  uint32_t kept = w >> 16;
  uint32_t dropped = w & 0xFFFFu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
    kept += 1u; /* carries into the exponent correctly, up to infinity */
  return (uint16_t)kept;
}

/* B(v) for a double, rounded ONCE (no intermediate binary32 step).
 * bfloat16 has 8 significant bits, exponent range of binary32, and
 * subnormals spaced 2^-133 apart. */
uint16_t orc_bf16_from_double(double v) {
  if (isnan(v)) return (uint16_t)0x7FC0u;
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  int e;
  (void)frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1 */
  /* quantum (spacing) of bf16 numbers at this magnitude */
  int q = e - 8;
  if (q < -133) q = -133; /* subnormal range: fixed spacing */
  double scaled = ldexp(a, -q);          /* exact: power-of-two scale */
  double r = nearbyint(scaled);          /* default mode: ties to even */
  double rounded = ldexp(r, q);          /* exact: r has <= 9 bits */
  if (rounded > 3.3895313892515355e38) /* above largest finite bf16 */
    return (uint16_t)(sign | 0x7F80u);
  float rf = (float)rounded; /* exact: rounded is a bf16 value */
  uint32_t w;
  memcpy(&w, &rf, sizeof w);
  return (uint16_t)(sign | ((w >> 16) & 0x7FFFu));
}

/* ------------------------------------------------------------------ */
/* Linear, [PSI] sec. III-A (bias handling) and sec. IV-B              */
/* ------------------------------------------------------------------ */

/* The fp32 accumulation of one dot product: sequential over k ascending,
 * starting from `init` (+0.0f for a fresh output; a carried value when the
 * caller continues a chain). */
static float dot_chain(float init, const uint16_t* x, const uint16_t* w, int K) {
  float acc = init;
  for (int k = 0; k < K; ++k) {
    float p = orc_f(x[k]) * orc_f(w[k]); /* exact for normal bf16 operands */
    acc = acc + p;
  }
  return acc;
}

/* y[M,N] = x[M,K] W[N,K]^T (+ b), bf16 in, fp32 accumulate.
 *   acc_in   nullable [M,N] fp32: initial accumulator (continues a chain)
 *   acc_out  nullable [M,N] fp32: the accumulator before the bias epilogue
 *   b        nullable [N]
 *   variant  0 = modified: y = B(acc + f(b))     (bias in fp32, one write)
 *            1 = baseline: y = B(f(B(acc)) + f(b)) (product rounded first)
 *   y        nullable [M,N] bf16 output
 * [PSI] sec. III-A: modified PSI adds the bias in FP32 before the BF16
 * write; baseline PSI rounds the matrix product to BF16 first. */
void orc_linear(const uint16_t* x, int M, int K, const uint16_t* W, int N,
                const uint16_t* b, int variant, const float* acc_in,
                float* acc_out, uint16_t* y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int m = 0; m < M; ++m) {
    for (int n = 0; n < N; ++n) {
      float init = acc_in ? acc_in[(size_t)m * N + n] : 0.0f;
      float acc = dot_chain(init, x + (size_t)m * K, W + (size_t)n * K, K);
      if (acc_out) acc_out[(size_t)m * N + n] = acc;
      if (y) {
        float out;
        if (b == NULL)
          out = acc;
        else if (variant == 1)
          out = orc_f(orc_bf16_from_float(acc)) + orc_f(b[n]);
        else
          out = acc + orc_f(b[n]);
        y[(size_t)m * N + n] = orc_bf16_from_float(out);
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* tanh-GELU, [PSI] sec. II-B eq. (2): "coordinatewise tanh-GELU"      */
/* ------------------------------------------------------------------ */

/* phi(v) = v/2 * (1 + tanh(z)),  z = sqrt(2/pi) * (v + 0.044715 v^3), in
 * double.  The factor 1 + tanh(z) is evaluated through the identity
 * 1 + tanh(z) = 2 / (1 + e^(-2z)) = 2 e^(2z) / (1 + e^(2z)) (second form for
 * z < 0): written literally, 1 + tanh(z) cancels for z below about -19 (tanh
 * rounds to -1) and the real value of phi, a tiny negative number, would be
 * lost. */
double orc_gelu_tanh_double(double v) {
  const double c = sqrt(2.0 / M_PI);
  const double z = c * (v + 0.044715 * v * v * v);
  if (z >= 0.0) return v / (1.0 + exp(-2.0 * z));
  const double e = exp(2.0 * z);
  return v * e / (1.0 + e);
}

/* H = B(phi(f(u))) for each element, rounded once from double. */
void orc_gelu_bf16(const uint16_t* u, size_t n, uint16_t* h) {
#pragma omp parallel for schedule(static)
  for (size_t i = 0; i < n; ++i) h[i] = orc_bf16_from_double(orc_gelu_tanh_double((double)orc_f(u[i])));
}

/* ------------------------------------------------------------------ */
/* FFN, [PSI] sec. II-B eq. (2) and sec. III-A                         */
/* ------------------------------------------------------------------ */

/* F(X) = phi(X U^T + a) V^T + b, dense.
 *   x [M,d], U [h,d], a [h], V [r,h], b [r]  (r output width; r = d for a
 *   transformer FFN but any r is allowed)
 * Declared BF16 boundaries ([PSI] sec. III-A):
 *   pre = B(acc_up + f(a))  (modified; baseline rounds acc_up first)
 *   H   = B(phi(f(pre)))
 *   y   = B(ACC + f(b)),  ACC = sum over hidden channel c ascending,
 *         one sequential fp32 chain per output (the page order of the
 *         hidden-channel partition, channels ascending within a page).
 *   residual != 0: y = B(f(x) + f(y_sub)) (requires r == d).
 *   H_out   nullable [M,h] bf16: the hidden activations (a journaled stage)
 *   acc_out nullable [M,r] fp32: ACC before the output bias
 * Scratch: allocates M*h bf16 for H when H_out is NULL. */
int orc_ffn(const uint16_t* x, int M, int d, const uint16_t* U, int h,
            const uint16_t* a, const uint16_t* V, int r, const uint16_t* b,
            int variant, int residual, uint16_t* H_out, float* acc_out,
            uint16_t* y) {
  if (residual && r != d) return -1;
  uint16_t* pre = (uint16_t*)malloc((size_t)M * h * sizeof(uint16_t));
  uint16_t* H = H_out ? H_out : (uint16_t*)malloc((size_t)M * h * sizeof(uint16_t));
  uint16_t* ysub = (uint16_t*)malloc((size_t)M * r * sizeof(uint16_t));
  if (!pre || !H || !ysub) {
    free(pre);
    if (!H_out) free(H);
    free(ysub);
    return -2;
  }
  orc_linear(x, M, d, U, h, a, variant, NULL, NULL, pre);
  orc_gelu_bf16(pre, (size_t)M * h, H);
  orc_linear(H, M, h, V, r, b, 0, NULL, acc_out, ysub);
  for (size_t i = 0; i < (size_t)M * r; ++i)
    y[i] = residual ? orc_bf16_from_float(orc_f(x[i]) + orc_f(ysub[i])) : ysub[i];
  free(pre);
  if (!H_out) free(H);
  free(ysub);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Attention, [PSI] sec. II-B eqs. (3)-(4) and sec. III-A              */
/* ------------------------------------------------------------------ */

/* Dense softmax attention for every head, i.e. eq. (3) with the processed
 * key set A = all keys (the online tiling of eq. (4) reaches the same value
 * in exact arithmetic for any complete key partition).
 *   q [Mq, ldq], k [Mk, ldk], v [Mk, ldv] bf16; head hd uses columns
 *   hd*dh .. hd*dh+dh-1 of each.  o [Mq, ldo] bf16 (same column blocks).
 * For query i of one head:
 *   alpha = fl32(1/sqrt(dh))
 *   s_j   = fl32(alpha * dot32(q_i, k_j))      (dot32: sequential fp32)
 *   m     = max_j s_j
 *   p_j   = (float) exp( (double) fl32(s_j - m) )
 *   l     = sum_j p_j                           (fp32, j ascending)
 *   z     = sum_j fl32(p_j * f(v_j))            (fp32, j ascending)
 *   o_i   = B(fl32(z / l))
 * The weights p_j stay fp32 (the FP32 accumulation of modified PSI, sec.
 * III-A); unmasked, noncausal, dropout-free, Mk >= 1. */
int orc_attention(const uint16_t* q, int Mq, int ldq, const uint16_t* k,
                  const uint16_t* v, int Mk, int ldk, int ldv, int heads,
                  int dh, uint16_t* o, int ldo) {
  if (Mk < 1 || dh < 1 || heads < 1) return -1;
  const float alpha = (float)(1.0 / sqrt((double)dh));
  int err = 0;
#pragma omp parallel
  {
    float* s = (float*)malloc((size_t)Mk * sizeof(float));
    float* z = (float*)malloc((size_t)dh * sizeof(float));
    if (!s || !z) {
#pragma omp atomic write
      err = -2;
    } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
      for (int hd = 0; hd < heads; ++hd) {
        for (int i = 0; i < Mq; ++i) {
          const uint16_t* qi = q + (size_t)i * ldq + (size_t)hd * dh;
          float m = -INFINITY;
          for (int j = 0; j < Mk; ++j) {
            const uint16_t* kj = k + (size_t)j * ldk + (size_t)hd * dh;
            float dot = dot_chain(0.0f, qi, kj, dh);
            s[j] = alpha * dot;
            if (s[j] > m) m = s[j];
          }
          float l = 0.0f;
          for (int c = 0; c < dh; ++c) z[c] = 0.0f;
          for (int j = 0; j < Mk; ++j) {
            float diff = s[j] - m;
            float p = (float)exp((double)diff);
            l = l + p;
            const uint16_t* vj = v + (size_t)j * ldv + (size_t)hd * dh;
            for (int c = 0; c < dh; ++c) z[c] = z[c] + p * orc_f(vj[c]);
          }
          uint16_t* oi = o + (size_t)i * ldo + (size_t)hd * dh;
          for (int c = 0; c < dh; ++c) oi[c] = orc_bf16_from_float(z[c] / l);
        }
      }
    }
    free(s);
    free(z);
  }
  return err;
}

/* Attention with the BF16-numerator choice of the baseline/modified
 * comparison ([PSI] sec. III-A, sec. IV-B).  bf16_p == 0 is orc_attention.
 * bf16_p != 0 (baseline PSI): the weights multiplying V are rounded to
 * BF16, z = sum_j fl32(f(B(p_j)) * f(v_j)); the normaliser l keeps the fp32
 * weights, as in orc_attention. */
int orc_attention_ex(const uint16_t* q, int Mq, int ldq, const uint16_t* k,
                     const uint16_t* v, int Mk, int ldk, int ldv, int heads,
                     int dh, int bf16_p, uint16_t* o, int ldo) {
  if (!bf16_p) return orc_attention(q, Mq, ldq, k, v, Mk, ldk, ldv, heads, dh, o, ldo);
  if (Mk < 1 || dh < 1 || heads < 1) return -1;
  const float alpha = (float)(1.0 / sqrt((double)dh));
  int err = 0;
#pragma omp parallel
  {
    float* s = (float*)malloc((size_t)Mk * sizeof(float));
    float* z = (float*)malloc((size_t)dh * sizeof(float));
    if (!s || !z) {
#pragma omp atomic write
      err = -2;
    } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
      for (int hd = 0; hd < heads; ++hd) {
        for (int i = 0; i < Mq; ++i) {
          const uint16_t* qi = q + (size_t)i * ldq + (size_t)hd * dh;
          float m = -INFINITY;
          for (int j = 0; j < Mk; ++j) {
            const uint16_t* kj = k + (size_t)j * ldk + (size_t)hd * dh;
            s[j] = alpha * dot_chain(0.0f, qi, kj, dh);
            if (s[j] > m) m = s[j];
          }
          float l = 0.0f;
          for (int c = 0; c < dh; ++c) z[c] = 0.0f;
          for (int j = 0; j < Mk; ++j) {
            float p = (float)exp((double)(s[j] - m));
            l = l + p;
            float pb = orc_f(orc_bf16_from_float(p));
            const uint16_t* vj = v + (size_t)j * ldv + (size_t)hd * dh;
            for (int c = 0; c < dh; ++c) z[c] = z[c] + pb * orc_f(vj[c]);
          }
          uint16_t* oi = o + (size_t)i * ldo + (size_t)hd * dh;
          for (int c = 0; c < dh; ++c) oi[c] = orc_bf16_from_float(z[c] / l);
        }
      }
    }
    free(s);
    free(z);
  }
  return err;
}

/* Full-row RMS normalisation with a tile-partitioned sum of squares
 * ([PSI] sec. II-B): for each row, s = sum over column tiles J (ascending)
 * of s_J = sum_{i in J} f(x_i)^2, then y_i = B(f(g_i) f(x_i) / sqrt(s/d +
 * eps)): one denominator for every tile of the row.  Evaluated in double
 * and rounded once per output.  tile <= 0 means one tile of width d.
 * x and y may alias. */
void orc_rmsnorm(const uint16_t* x, int M, int d, int ldx, const uint16_t* g,
                 double eps, int tile, uint16_t* y, int ldy) {
  if (tile <= 0 || tile > d) tile = d;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < M; ++r) {
    const uint16_t* xr = x + (size_t)r * ldx;
    double s = 0.0;
    for (int j0 = 0; j0 < d; j0 += tile) {
      const int j1 = j0 + tile < d ? j0 + tile : d;
      double sj = 0.0;
      for (int i = j0; i < j1; ++i) sj += (double)orc_f(xr[i]) * (double)orc_f(xr[i]);
      s += sj;
    }
    const double den = sqrt(s / d + eps);
    uint16_t* yr = y + (size_t)r * ldy;
    for (int i = 0; i < d; ++i) yr[i] = orc_bf16_from_double((double)orc_f(g[i]) * (double)orc_f(xr[i]) / den);
  }
}

/* Split rotary embedding ([PSI] sec. II-B): inside each head of width dh,
 * the pair (a, b) = (x_j, x_{j+dh/2}), j < dh/2, becomes
 * (c a - s b, s a + c b) with c = cos[t][j], s = sin[t][j] from the
 * caller's fp32 tables [M, dh/2] (row t = token); evaluated in double,
 * rounded once per output; in place allowed (x == y). */
void orc_rope_split(const uint16_t* x, int M, int heads, int dh, int ldx,
                    const float* cs, const float* sn, uint16_t* y, int ldy) {
  const int hh = dh / 2;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < M; ++t) {
    for (int h = 0; h < heads; ++h) {
      const uint16_t* xr = x + (size_t)t * ldx + (size_t)h * dh;
      uint16_t* yr = y + (size_t)t * ldy + (size_t)h * dh;
      for (int j = 0; j < hh; ++j) {
        const double a = orc_f(xr[j]), b = orc_f(xr[j + hh]);
        const double c = cs[(size_t)t * hh + j], sv = sn[(size_t)t * hh + j];
        const uint16_t u = orc_bf16_from_double(c * a - sv * b);
        const uint16_t w = orc_bf16_from_double(sv * a + c * b);
        yr[j] = u;
        yr[j + hh] = w;
      }
    }
  }
}

/* Attention sub-block with q/k normalisation and rotary positions, each a
 * declared BF16 write:
 *   Q = B(x Wq^T + bq); if gq: Q = rmsnorm(Q, gq, eps, norm_tile); if
 *   cos_q: Q = rope(Q, cos_q, sin_q); K likewise from src with gk and
 *   cos_k/sin_k (NULL cos_k: the query tables, self-attention);
 *   V = B(src Wv^T + bv); O = attention (bf16_p as orc_attention_ex);
 *   Y = B(O Wo^T + bo); residual: y = B(f(x) + f(Y)). */
int orc_attn_sublayer_ext(const uint16_t* x, int M, const uint16_t* ctx, int Mc,
                          int d, int heads, int dh, const uint16_t* Wq,
                          const uint16_t* bq, const uint16_t* Wk,
                          const uint16_t* bk, const uint16_t* Wv,
                          const uint16_t* bv, const uint16_t* Wo,
                          const uint16_t* bo, const uint16_t* gq,
                          const uint16_t* gk, double eps, int norm_tile,
                          const float* cos_q, const float* sin_q,
                          const float* cos_k, const float* sin_k, int variant,
                          int bf16_p, int residual, uint16_t* y) {
  if (heads * dh != d || dh % 2) return -1;
  const uint16_t* src = ctx ? ctx : x;
  const int Ms = ctx ? Mc : M;
  if (!cos_k) { cos_k = cos_q; sin_k = sin_q; }
  if (cos_q && cos_k == cos_q && Ms != M) return -1;
  uint16_t* Q = (uint16_t*)malloc((size_t)M * d * 2);
  uint16_t* Kb = (uint16_t*)malloc((size_t)Ms * d * 2);
  uint16_t* Vb = (uint16_t*)malloc((size_t)Ms * d * 2);
  uint16_t* O = (uint16_t*)malloc((size_t)M * d * 2);
  uint16_t* Y = (uint16_t*)malloc((size_t)M * d * 2);
  int rc = 0;
  if (!Q || !Kb || !Vb || !O || !Y) {
    rc = -2;
  } else {
    orc_linear(x, M, d, Wq, d, bq, variant, NULL, NULL, Q);
    orc_linear(src, Ms, d, Wk, d, bk, variant, NULL, NULL, Kb);
    orc_linear(src, Ms, d, Wv, d, bv, variant, NULL, NULL, Vb);
    if (gq) orc_rmsnorm(Q, M, d, d, gq, eps, norm_tile, Q, d);
    if (gk) orc_rmsnorm(Kb, Ms, d, d, gk, eps, norm_tile, Kb, d);
    if (cos_q) {
      orc_rope_split(Q, M, heads, dh, d, cos_q, sin_q, Q, d);
      orc_rope_split(Kb, Ms, heads, dh, d, cos_k, sin_k, Kb, d);
    }
    rc = orc_attention_ex(Q, M, d, Kb, Vb, Ms, d, d, heads, dh, bf16_p, O, d);
    if (rc == 0) {
      orc_linear(O, M, d, Wo, d, bo, variant, NULL, NULL, Y);
      for (size_t i = 0; i < (size_t)M * d; ++i)
        y[i] = residual ? orc_bf16_from_float(orc_f(x[i]) + orc_f(Y[i])) : Y[i];
    }
  }
  free(Q);
  free(Kb);
  free(Vb);
  free(O);
  free(Y);
  return rc;
}

/* Attention sub-block: projections, attention, output projection, residual.
 *   x [M,d]; ctx [Mc,d] or NULL for self-attention (keys/values from x).
 *   Q = x Wq^T + bq, K = src Wk^T + bk, V = src Wv^T + bv   (bf16 writes)
 *   O = attention per head (bf16 write)
 *   Y = B(O Wo^T + bo)  -- the output projection sums over all d input
 *       channels ascending, i.e. heads ascending, one fp32 chain ("output
 *       bias added once", sec. II-B)
 *   residual != 0: y = B(f(x) + f(Y)); else y = Y.
 *   o_out nullable [M,d]: the attention output O (a journaled stage).
 *   acc_out nullable [M,d] fp32: the O-projection accumulator before bias. */
int orc_attn_sublayer(const uint16_t* x, int M, const uint16_t* ctx, int Mc,
                      int d, int heads, int dh, const uint16_t* Wq,
                      const uint16_t* bq, const uint16_t* Wk,
                      const uint16_t* bk, const uint16_t* Wv,
                      const uint16_t* bv, const uint16_t* Wo,
                      const uint16_t* bo, int variant, int residual,
                      uint16_t* o_out, float* acc_out, uint16_t* y) {
  if (heads * dh != d) return -1;
  const uint16_t* src = ctx ? ctx : x;
  int Ms = ctx ? Mc : M;
  uint16_t* Q = (uint16_t*)malloc((size_t)M * d * 2);
  uint16_t* Kb = (uint16_t*)malloc((size_t)Ms * d * 2);
  uint16_t* Vb = (uint16_t*)malloc((size_t)Ms * d * 2);
  uint16_t* O = o_out ? o_out : (uint16_t*)malloc((size_t)M * d * 2);
  uint16_t* Y = (uint16_t*)malloc((size_t)M * d * 2);
  int rc = 0;
  if (!Q || !Kb || !Vb || !O || !Y) {
    rc = -2;
  } else {
    orc_linear(x, M, d, Wq, d, bq, variant, NULL, NULL, Q);
    orc_linear(src, Ms, d, Wk, d, bk, variant, NULL, NULL, Kb);
    orc_linear(src, Ms, d, Wv, d, bv, variant, NULL, NULL, Vb);
    rc = orc_attention(Q, M, d, Kb, Vb, Ms, d, d, heads, dh, O, d);
    if (rc == 0) {
      orc_linear(O, M, d, Wo, d, bo, variant, NULL, acc_out, Y);
      for (size_t i = 0; i < (size_t)M * d; ++i)
        y[i] = residual ? orc_bf16_from_float(orc_f(x[i]) + orc_f(Y[i])) : Y[i];
    }
  }
  free(Q);
  free(Kb);
  free(Vb);
  if (!o_out) free(O);
  free(Y);
  return rc;
}

/* One synthetic transformer block: self-attention sub-block then FFN
 * sub-block, each followed by its residual write.  x is updated in place. */
int orc_block(uint16_t* x, int M, int d, int heads, int dh, int hidden,
              const uint16_t* Wq, const uint16_t* bq, const uint16_t* Wk,
              const uint16_t* bk, const uint16_t* Wv, const uint16_t* bv,
              const uint16_t* Wo, const uint16_t* bo, const uint16_t* U,
              const uint16_t* a, const uint16_t* V, const uint16_t* b,
              int variant) {
  uint16_t* t = (uint16_t*)malloc((size_t)M * d * 2);
  if (!t) return -2;
  int rc = orc_attn_sublayer(x, M, NULL, 0, d, heads, dh, Wq, bq, Wk, bk, Wv,
                             bv, Wo, bo, variant, 1, NULL, NULL, t);
  if (rc == 0)
    rc = orc_ffn(t, M, d, U, hidden, a, V, d, b, variant, 1, NULL, NULL, x);
  free(t);
  return rc;
}

/* Element-wise residual write, [PSI]-consistent boundary: x = B(f(x)+f(y)). */
void orc_residual(uint16_t* x, const uint16_t* y, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = orc_bf16_from_float(orc_f(x[i]) + orc_f(y[i]));
}
