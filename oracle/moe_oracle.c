/*
 * moe_oracle.c -- plain, slow, obviously-correct fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, by the smoke check and by the
 * benchmark's CPU-baseline leg.  The product path never links or calls it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Every stored code is decoded from its bits into an exact double; every
 * accumulation runs in double, one term at a time, in index order.  The only
 * places where fp32 appears are the ones where the method itself stores an
 * fp32 value that then decides an integer code (the FP8 block scales and the
 * quotient that is rounded to E4M3): there the oracle takes the decision in
 * fp32, as the method's kernels do, so that codes can be compared exactly.
 *
 * Source names are explained in moe_oracle.h.  Parity is pinned by the tests
 * under tests/ (closed forms, library decoders, brute force, hand-worked
 * layers).  Readings of what the pages leave open are marked READING.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ codecs */

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double orc_dec_bf16(uint16_t h) {
  int s = h >> 15, e = (h >> 7) & 0xFF, m = h & 0x7F;
  double v;
  if (e == 0xFF)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -133); /* subnormal: m/128 * 2^-126 */
  else
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
  return s ? -v : v;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits.  The 1-bit
 * format's group scale is stored this way (1-Bit Turbo, Q1_0_G128). */
double orc_dec_fp16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0x1F)
    v = m ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)m, -24); /* m/1024 * 2^-14 */
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return s ? -v : v;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 448.  FP8 E4M3 weights, activation blocks
 * and mid (#85 Mod. rows 1, 10, 18). */
double orc_dec_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0xF && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

/* OCP MX E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 (MXFP4 page; MXFP4 routed experts). */
double orc_dec_e2m1(uint8_t nibble) {
  int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
  double v;
  if (e == 0)
    v = 0.5 * m; /* subnormal: m/2 * 2^0 */
  else
    v = ldexp((double)(2 + m), e - 2); /* (1 + m/2) * 2^(e-1) */
  return s ? -v : v;
}

/* OCP MX E8M0 shared scale: 2^(c - 127), 0xFF is NaN. */
double orc_dec_e8m0(uint8_t c) {
  if (c == 0xFF) return NAN;
  return ldexp(1.0, (int)c - 127);
}

/* fp32 -> E4M3FN by search: the nearest of the 127 finite non-negative codes
 * to |v|, an exact tie going to the code whose mantissa LSB is 0, then v's
 * sign bit.  Values past 448 therefore saturate to 448, and a value that
 * rounds to zero keeps its sign (0x80).  NaN maps to 0x7F.
 * READING: round-to-nearest-even, saturating, never NaN for finite input; the
 * pages name FP8 E4M3 quantisation (#85 Mod. rows 1, 10) but no rounding. */
uint8_t orc_enc_e4m3(float v) {
  if (isnan(v)) return 0x7F;
  double a = fabs((double)v);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7E; c++) {
    double d = fabs(orc_dec_e4m3((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      best = c;
      bd = d;
    }
  }
  return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/* double -> bfloat16 with one round-to-nearest-even step (no detour through
 * fp32); overflow goes to infinity as in IEEE. */
uint16_t orc_round_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  double a = fabs(v), r;
  if (a < ldexp(1.0, -126)) {
    r = ldexp(nearbyint(ldexp(a, 133)), -133); /* subnormal spacing 2^-133 */
  } else {
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e): 8 significant bits -> spacing 2^(e-8) */
    r = ldexp(nearbyint(ldexp(a, 8 - e)), e - 8);
  }
  float f = (float)r; /* exact: r is a bfloat16 value or infinity */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t h = (uint16_t)(bits >> 16);
  if (signbit(v)) h |= 0x8000;
  return h;
}

/* Lookup tables filled once by the bit-by-bit decoders above (memoisation
 * only: every entry is the decoder's own result). */
static double lut_e4m3[256], lut_e2m1[16], lut_e8m0[256];
static int lut_ready = 0;
static void orc_init_luts(void) {
  if (lut_ready) return;
  for (int c = 0; c < 256; c++) {
    lut_e4m3[c] = orc_dec_e4m3((uint8_t)c);
    lut_e8m0[c] = orc_dec_e8m0((uint8_t)c);
  }
  for (int c = 0; c < 16; c++) lut_e2m1[c] = orc_dec_e2m1((uint8_t)c);
  lut_ready = 1;
}

/* ------------------------------------------------------------ step pieces */

/* Order of experts in top-8: larger logit first; equal logits (IEEE equality,
 * so -0 == +0) go to the lower expert ID (#85 Mod. row 9 and Motivation:
 * top-8 rounds reduce the expert ID only on exact ties).  READING: a NaN logit
 * ranks below every number, lower ID first among NaNs. */
static int orc_before(double za, int ia, double zb, int ib) {
  int na = isnan(za), nb = isnan(zb);
  if (na || nb) {
    if (na && nb) return ia < ib;
    return nb; /* the number goes first */
  }
  if (za != zb) return za > zb;
  return ia < ib;
}

/* Top-8 selection: eight rounds, each taking the first not-yet-taken expert
 * under orc_before; picks come out in round order (#85 Mod. row 9). */
void orc_top8(const double* z, int n_experts, int32_t ids[8]) {
  char* taken = (char*)calloc((size_t)n_experts, 1);
  for (int j = 0; j < 8; j++) {
    int best = -1;
    for (int e = 0; e < n_experts; e++) {
      if (taken[e]) continue;
      if (best < 0 || orc_before(z[e], e, z[best], best)) best = e;
    }
    ids[j] = best;
    if (best >= 0) taken[best] = 1;
  }
  free(taken);
}

/* Gate weights.  READING: softmax over the eight selected logits, in pick
 * order, no bias, no rescaling; the shared expert's weight is 1.  (#85 Mod.
 * row 10 says the rstd scales "the 8 logits" but names no gate function.) */
void orc_softmax8(const double z_sel[8], double g[8]) {
  double m = z_sel[0];
  for (int j = 1; j < 8; j++)
    if (z_sel[j] > m) m = z_sel[j];
  double sum = 0.0;
  for (int j = 0; j < 8; j++) {
    g[j] = exp(z_sel[j] - m);
    sum += g[j];
  }
  for (int j = 0; j < 8; j++) g[j] /= sum;
}

/* Expert dedup table (#85 Mod. rows 16 and 20).  The picks are scanned slot
 * major (slot j outer, row r inner); the first use of an expert opens a group
 * whose owner is that (slot, row) -- the row whose job of it comes first, the
 * lowest row on a tie.  Each group records the rows that use it (bit mask)
 * and, per row, the slot where that row picked it (0xFF: not used).
 * READING: slot-major scan order.  The shared expert is not in the table. */
int orc_dedup(const int32_t* ids, int rows, int32_t* n_groups, int32_t* grp_expert,
              uint8_t* grp_owner_slot, uint8_t* grp_owner_row, uint8_t* grp_mask,
              uint8_t* grp_slot) {
  if (rows < 1 || rows > 8) return ORC_ERR;
  int d = 0;
  for (int j = 0; j < 8; j++) {
    for (int r = 0; r < rows; r++) {
      int e = ids[r * 8 + j], g;
      for (g = 0; g < d; g++)
        if (grp_expert[g] == e) break;
      if (g == d) {
        d++;
        grp_expert[g] = e;
        grp_owner_slot[g] = (uint8_t)j;
        grp_owner_row[g] = (uint8_t)r;
        grp_mask[g] = 0;
        for (int rr = 0; rr < 8; rr++) grp_slot[g * 8 + rr] = 0xFF;
      }
      grp_mask[g] |= (uint8_t)(1u << r);
      grp_slot[g * 8 + r] = (uint8_t)j;
    }
  }
  *n_groups = d;
  return ORC_OK;
}

/* FP8 block quantiser for activations and mid (#85 Mod. row 1: mid quantised
 * to FP8 per block with one scale; Layout: 128 code bytes plus a 4-byte scale
 * per block; Mod. row 10: FP8 activation blocks).  Per block of 128 values:
 * s = fp32(amax / 448); q = E4M3(fp32(v / s)); a block of zeros gets s = 0 and
 * all codes 0.  READING: scale amax/448 in fp32; round-to-nearest-even. */
void orc_quant_blocks(const float* v, int n, uint8_t* q, float* s) {
  for (int b = 0; b < n / 128; b++) {
    float a = 0.0f;
    for (int i = 0; i < 128; i++) {
      float t = fabsf(v[b * 128 + i]);
      if (t > a) a = t;
    }
    float sc = a / 448.0f;
    s[b] = sc;
    for (int i = 0; i < 128; i++) {
      float x = v[b * 128 + i];
      q[b * 128 + i] = (sc == 0.0f) ? 0 : orc_enc_e4m3(x / sc);
    }
  }
}

/* y[n] = sum_k W[n,k] * h[k] for one stored matrix, W decoded element by
 * element: FP8 code * fp32 block scale (per 128x128), E2M1 * 2^(E8M0-127)
 * (per 32 along K, low nibble = even element), or +-d for 1-bit group-128
 * weights (1-Bit Turbo, Q1_0_G128).  Two optional outputs size
 * rounding bounds and take no part in y: yabs[n] = sum_k |W[n,k] h[k]|, and
 * ygmax[n] = the sum, over the groups of 8 consecutive k (k = 8i .. 8i+7), of
 * the largest |W[n,k] h[k]| in the group. */
static void orc_gemv(int fmt, const orc_mat* w, int n_out, int k_in, const double* h, double* y,
                     double* yabs, double* ygmax, int nthreads) {
  const uint8_t* codes = w->codes;
#pragma omp parallel num_threads(nthreads)
  {
    double* wrow = (double*)malloc(sizeof(double) * k_in); /* row n of W, decoded */
#pragma omp for schedule(static)
    for (int n = 0; n < n_out; n++) {
      if (fmt == ORC_FMT_FP8) {
        const float* sc = (const float*)w->scales;
        for (int k = 0; k < k_in; k++)
          wrow[k] = lut_e4m3[codes[(size_t)n * k_in + k]] *
                    (double)sc[(size_t)(n / 128) * (k_in / 128) + k / 128];
      } else if (fmt == ORC_FMT_MXFP4) {
        const uint8_t* sc = (const uint8_t*)w->scales;
        for (int k = 0; k < k_in; k++) {
          uint8_t byte = codes[(size_t)n * (k_in / 2) + k / 2];
          uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
          wrow[k] = lut_e2m1[nib] * lut_e8m0[sc[(size_t)n * (k_in / 32) + k / 32]];
        }
      } else {
        /* Q1_0_G128: an 18-byte block per 128 along K, fp16 d then 16 bytes
         * of sign bits, bit k%8 of byte (k%128)/8; 1 means -d */
        for (int k = 0; k < k_in; k++) {
          const uint8_t* blk = codes + ((size_t)n * (k_in / 128) + k / 128) * 18;
          const double d = orc_dec_fp16((uint16_t)(blk[0] | (blk[1] << 8)));
          const int bit = (blk[2 + (k % 128) / 8] >> (k % 8)) & 1;
          wrow[k] = bit ? -d : d;
        }
      }
      double acc = 0.0, aabs = 0.0, gsum = 0.0, gmax = 0.0;
      for (int k = 0; k < k_in; k++) {
        const double t = wrow[k] * h[k];
        acc += t;
        aabs += fabs(t);
        if (fabs(t) > gmax) gmax = fabs(t);
        if (k % 8 == 7 || k == k_in - 1) {
          gsum += gmax;
          gmax = 0.0;
        }
      }
      y[n] = acc;
      if (yabs) yabs[n] = aabs;
      if (ygmax) ygmax[n] = gsum;
    }
    free(wrow);
  }
}

static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert applied to one row: up/gate, SiLU*gate, mid re-quantised to FP8
 * per 1x128 block for FP8 experts, then down (#85 Mod. rows 1, 16).
 * READING: mid = silu(gate) * up; MXFP4 experts keep mid unquantised (#85 Mod.
 * row 1: the MXFP4 experts' path is left as it was, and it read mid as f32).
 * READING: 1-bit (Q1_0_G128) routed experts re-quantise mid to FP8 per 1x128
 * block like FP8 experts: the rule stated for the step in general, with no
 * exception on the pages for 1-bit weights. */
static void orc_expert(int fmt, const orc_mat* wg, const orc_mat* wu, const orc_mat* wd, int h_dim,
                       int i_dim, const double* hin, int nthreads, double* mid_out,
                       uint8_t* midq_out, float* midqs_out, double* y, double* gate,
                       double* upv, double* gate_abs, double* up_abs, double* gate_gmax,
                       double* up_gmax) {
  double* mhat = (double*)malloc(sizeof(double) * i_dim);
  orc_gemv(fmt, wg, i_dim, h_dim, hin, gate, gate_abs, gate_gmax, nthreads);
  orc_gemv(fmt, wu, i_dim, h_dim, hin, upv, up_abs, up_gmax, nthreads);
  for (int n = 0; n < i_dim; n++) mid_out[n] = orc_silu(gate[n]) * upv[n];
  if (fmt == ORC_FMT_FP8 || fmt == ORC_FMT_Q1) {
    float* mf = (float*)malloc(sizeof(float) * i_dim);
    for (int n = 0; n < i_dim; n++) mf[n] = (float)mid_out[n];
    orc_quant_blocks(mf, i_dim, midq_out, midqs_out);
    for (int n = 0; n < i_dim; n++) mhat[n] = lut_e4m3[midq_out[n]] * (double)midqs_out[n / 128];
    free(mf);
  } else {
    for (int n = 0; n < i_dim; n++) mhat[n] = mid_out[n];
  }
  orc_gemv(fmt, wd, h_dim, i_dim, mhat, y, NULL, NULL, nthreads);
  free(mhat);
}

/* The down GEMV of one expert applied to a given mid (#85 Mod. row 16: down
 * units take an expert's tile against its rows' mid; Mod. row 1: down reads
 * mid as FP8 codes with one fp32 scale per 1x128 block).  The check of a
 * device's down outputs calls it on that device's own mid, so that the down
 * GEMV is judged apart from the up/gate before it:
 *   y_n = sum_k W[n,k] * mhat_k,
 * mhat_k = dec(midq[k]) * midqs[k/128] for FP8 and 1-bit experts, and
 * mhat_k = mid32[k] (the fp32 value itself) for MXFP4 experts, whose mid is
 * not re-quantised.  W's scales are unused for 1-bit experts (in the blocks).
 * y_abs_n = sum_k |W[n,k] * mhat_k| and y_gmax (the per-group maxima of
 * orc_gemv) size rounding bounds.  W is [h_dim,
 * i_dim] in the expert's format; every sum runs in double in index order. */
int orc_expert_down(int fmt, const orc_mat* wd, int h_dim, int i_dim, const uint8_t* midq,
                    const float* midqs, const float* mid32, int nthreads, double* y,
                    double* y_abs, double* y_gmax) {
  if (h_dim <= 0 || i_dim <= 0 || i_dim % 128 || !wd || !wd->codes || !y) return ORC_ERR;
  if ((fmt == ORC_FMT_FP8 || fmt == ORC_FMT_Q1) && (!midq || !midqs)) return ORC_ERR;
  if (fmt == ORC_FMT_MXFP4 && !mid32) return ORC_ERR;
  if (fmt != ORC_FMT_FP8 && fmt != ORC_FMT_MXFP4 && fmt != ORC_FMT_Q1) return ORC_ERR;
  if (fmt == ORC_FMT_FP8 && h_dim % 128) return ORC_ERR;
  if (fmt != ORC_FMT_Q1 && !wd->scales) return ORC_ERR; /* 1-bit: the scales are in the blocks */
  if (nthreads < 1) nthreads = 1;
  orc_init_luts();
  double* mhat = (double*)malloc(sizeof(double) * i_dim);
  for (int k = 0; k < i_dim; k++)
    mhat[k] = fmt == ORC_FMT_MXFP4 ? (double)mid32[k] : lut_e4m3[midq[k]] * (double)midqs[k / 128];
  orc_gemv(fmt, wd, h_dim, i_dim, mhat, y, y_abs, y_gmax, nthreads);
  free(mhat);
  return ORC_OK;
}

/* RMSNorm folded into the router logits for one row (#85 Mod. row 10: the
 * router stores bf16(a * gamma) with the row's sum of squares; the rstd scales
 * the logits).  u = bf16(x * gamma) (the product is exact in double, then one
 * rounding); rstd = 1/sqrt(sum(x^2)/H + eps); z_e = rstd * sum_k W_r[e,k] u_k.
 * READING: the mean is of x^2 over the hidden size, eps as given in fp32.
 * Returns rstd; writes u (as doubles, and as bf16 codes if ub) and z[E]. */
static double orc_router_row(int H, int E, float eps, const uint16_t* xr, const uint16_t* gamma,
                             const uint16_t* router_w, double* uf, uint16_t* ub, double* z) {
  double ss = 0.0;
  for (int k = 0; k < H; k++) {
    double xv = orc_dec_bf16(xr[k]);
    ss += xv * xv;
  }
  double rstd = 1.0 / sqrt(ss / H + (double)eps);
  for (int k = 0; k < H; k++) {
    uint16_t b = orc_round_bf16(orc_dec_bf16(xr[k]) * orc_dec_bf16(gamma[k]));
    uf[k] = orc_dec_bf16(b);
    if (ub) ub[k] = b;
  }
  for (int e = 0; e < E; e++) {
    double acc = 0.0;
    for (int k = 0; k < H; k++) acc += orc_dec_bf16(router_w[(size_t)e * H + k]) * uf[k];
    z[e] = rstd * acc;
  }
  return rstd;
}

/* Router stage alone for R rows: z [R][E], rstd [R], u [R][H] (bf16 codes). */
int orc_router(int rows, int hidden, int n_experts, float eps, const uint16_t* x,
               const uint16_t* gamma, const uint16_t* router_w, double* z, double* rstd,
               uint16_t* u) {
  if (rows < 1 || hidden <= 0 || n_experts <= 0) return ORC_ERR;
  double* uf = (double*)malloc(sizeof(double) * hidden);
  for (int r = 0; r < rows; r++) {
    double rs = orc_router_row(hidden, n_experts, eps, x + (size_t)r * hidden, gamma, router_w, uf,
                               u ? u + (size_t)r * hidden : NULL, z + (size_t)r * n_experts);
    if (rstd) rstd[r] = rs;
  }
  free(uf);
  return ORC_OK;
}

/* The whole decode step for 1..8 rows.
 *  1. RMSNorm folded into the router (#85 Mod. row 10): u = bf16(x * gamma);
 *     rstd = 1/sqrt(sum(x^2)/H + eps); logit z_e = rstd * (W_r[e] . u).
 *     READING: the mean is of x^2 over the hidden size.
 *  2. Top-8 (orc_top8) on the oracle's own z, or on the caller's fp32 logits
 *     when anchor_z is given (selection judged on the GPU's own logits);
 *     gates = softmax of the oracle's z at the selected experts.
 *  3. Activation: u quantised to FP8 per 1x128 block (orc_quant_blocks); the
 *     expert input is h = dec(q) * s * rstd (#85 Mod. row 10: the rstd scales
 *     the FP8 activation blocks).  READING: FP8 activations.
 *  4. Each row applies its 8 experts and, if present, the shared expert
 *     (orc_expert).
 *  5. Combine (#85 Mod. row 16: the row's sum over its down units keeps the
 *     order a single row would use): out = bf16(sum_j g_j * y_j + y_shared),
 *     j in pick order.
 *     READING: no residual, no routed scaling factor; shared weight 1. */
int orc_moe_step(const orc_cfg* cfg, const uint16_t* x, const uint16_t* gamma,
                 const uint16_t* router_w, const orc_mat* gate, const orc_mat* up,
                 const orc_mat* down, const orc_mat* sh_gate, const orc_mat* sh_up,
                 const orc_mat* sh_down, const float* anchor_z, uint16_t* out,
                 orc_debug* dbg) {
  const int H = cfg->hidden, I = cfg->inter, E = cfg->n_experts, Is = cfg->shared_inter,
            R = cfg->rows;
  const int nt = cfg->nthreads > 0 ? cfg->nthreads : 1;
  const int Imax = Is > I ? Is : I;
  if (R < 1 || R > 8 || H % 128 || I % 128 || Is % 128 || E < 8 || Is < 0) return ORC_ERR;
  if (cfg->routed_fmt != ORC_FMT_FP8 && cfg->routed_fmt != ORC_FMT_MXFP4 &&
      cfg->routed_fmt != ORC_FMT_Q1)
    return ORC_ERR;
  if (cfg->act_fmt != ORC_ACT_FP8 && cfg->act_fmt != ORC_ACT_BF16) return ORC_ERR;
  if (Is > 0 && (!sh_gate || !sh_up || !sh_down)) return ORC_ERR;
  orc_init_luts();
  orc_debug none;
  memset(&none, 0, sizeof(none));
  if (!dbg) dbg = &none;

  double* z = (double*)malloc(sizeof(double) * (size_t)R * E);
  double* hin = (double*)malloc(sizeof(double) * H);
  double* uf = (double*)malloc(sizeof(double) * H);
  float* u32 = (float*)malloc(sizeof(float) * H);
  uint8_t* aq = (uint8_t*)malloc(H);
  float* as = (float*)malloc(sizeof(float) * (H / 128));
  double* ys = (double*)malloc(sizeof(double) * 9 * H);
  double* midv = (double*)malloc(sizeof(double) * Imax);
  double* gv = (double*)malloc(sizeof(double) * Imax);
  double* uv = (double*)malloc(sizeof(double) * Imax);
  double* ga = (double*)malloc(sizeof(double) * Imax);
  double* ua = (double*)malloc(sizeof(double) * Imax);
  double* gg = (double*)malloc(sizeof(double) * Imax);
  double* ug = (double*)malloc(sizeof(double) * Imax);
  uint8_t* mq = (uint8_t*)malloc(Imax);
  float* ms = (float*)malloc(sizeof(float) * (Imax / 128));
  int rc = ORC_OK;

  for (int r = 0; r < R && rc == ORC_OK; r++) {
    const uint16_t* xr = x + (size_t)r * H;
    /* 1. norm fold and router */
    uint16_t* ub = dbg->u ? dbg->u + (size_t)r * H : NULL;
    double rstd = orc_router_row(H, E, cfg->rms_eps, xr, gamma, router_w, uf, ub,
                                 z + (size_t)r * E);
    for (int k = 0; k < H; k++) u32[k] = (float)uf[k];
    /* 2. selection and gates */
    int32_t ids[8];
    if (anchor_z) {
      double* za = (double*)malloc(sizeof(double) * E);
      for (int e = 0; e < E; e++) za[e] = (double)anchor_z[(size_t)r * E + e];
      orc_top8(za, E, ids);
      free(za);
    } else {
      orc_top8(z + (size_t)r * E, E, ids);
    }
    double zs[8], g[8];
    for (int j = 0; j < 8; j++) zs[j] = z[(size_t)r * E + ids[j]];
    orc_softmax8(zs, g);
    /* 3. the experts' input: FP8 activation blocks (dequantised, times rstd),
     * or with ORC_ACT_BF16 u itself times rstd (no codes, scales 0) */
    if (cfg->act_fmt == ORC_ACT_BF16) {
      memset(aq, 0, H);
      for (int b = 0; b < H / 128; b++) as[b] = 0.0f;
      for (int k = 0; k < H; k++) hin[k] = uf[k] * rstd;
    } else {
      orc_quant_blocks(u32, H, aq, as);
      for (int k = 0; k < H; k++) hin[k] = lut_e4m3[aq[k]] * (double)as[k / 128] * rstd;
    }
    /* 4. experts */
    for (int j = 0; j < 9; j++) {
      if (j == 8 && Is == 0) break;
      const int e = j < 8 ? ids[j] : -1;
      const orc_mat *wg, *wu, *wd;
      int fmt, idim;
      if (j < 8) {
        wg = &gate[e];
        wu = &up[e];
        wd = &down[e];
        fmt = cfg->routed_fmt;
        idim = I;
      } else {
        wg = sh_gate;
        wu = sh_up;
        wd = sh_down;
        fmt = ORC_FMT_FP8;
        idim = Is;
      }
      if (!wg->codes || !wu->codes || !wd->codes ||
          (fmt != ORC_FMT_Q1 && (!wg->scales || !wu->scales || !wd->scales))) {
        rc = ORC_ERR;
        break;
      }
      memset(mq, 0, Imax);
      for (int b = 0; b < Imax / 128; b++) ms[b] = 0.0f;
      orc_expert(fmt, wg, wu, wd, H, idim, hin, nt, midv, mq, ms, ys + (size_t)j * H, gv, uv, ga,
                 ua, gg, ug);
      size_t base = ((size_t)r * 9 + j) * Imax;
      for (int n = 0; n < idim; n++) {
        if (dbg->mid) dbg->mid[base + n] = midv[n];
        if (dbg->gate) dbg->gate[base + n] = gv[n];
        if (dbg->up) dbg->up[base + n] = uv[n];
        if (dbg->gate_abs) dbg->gate_abs[base + n] = ga[n];
        if (dbg->up_abs) dbg->up_abs[base + n] = ua[n];
        if (dbg->gate_gmax) dbg->gate_gmax[base + n] = gg[n];
        if (dbg->up_gmax) dbg->up_gmax[base + n] = ug[n];
      }
      if (dbg->midq) memcpy(dbg->midq + base, mq, idim);
      if (dbg->midqs)
        for (int b = 0; b < idim / 128; b++) dbg->midqs[((size_t)r * 9 + j) * (Imax / 128) + b] = ms[b];
    }
    if (rc != ORC_OK) break;
    /* 5. combine in pick order, then the shared expert */
    for (int k = 0; k < H; k++) {
      double acc = 0.0;
      for (int j = 0; j < 8; j++) acc += g[j] * ys[(size_t)j * H + k];
      if (Is > 0) acc += ys[(size_t)8 * H + k];
      if (dbg->out_f64) dbg->out_f64[(size_t)r * H + k] = acc;
      if (out) out[(size_t)r * H + k] = orc_round_bf16(acc);
    }
    if (dbg->z) memcpy(dbg->z + (size_t)r * E, z + (size_t)r * E, sizeof(double) * E);
    if (dbg->rstd) dbg->rstd[r] = rstd;
    if (dbg->ids) memcpy(dbg->ids + (size_t)r * 8, ids, sizeof(ids));
    if (dbg->gates) memcpy(dbg->gates + (size_t)r * 8, g, sizeof(g));
    if (dbg->act_q) memcpy(dbg->act_q + (size_t)r * H, aq, H);
    if (dbg->act_s) memcpy(dbg->act_s + (size_t)r * (H / 128), as, sizeof(float) * (H / 128));
    if (dbg->y) memcpy(dbg->y + (size_t)r * 9 * H, ys, sizeof(double) * 9 * H);
  }
  free(z);
  free(hin);
  free(uf);
  free(u32);
  free(aq);
  free(as);
  free(ys);
  free(midv);
  free(gv);
  free(uv);
  free(ga);
  free(ua);
  free(gg);
  free(ug);
  free(mq);
  free(ms);
  return rc;
}

/* 1-bit group-128 GEMV (1-Bit Turbo, Q1_0_G128: 1-bit weights with one scale
 * per group of 128, 572 MB for 4B parameters, i.e. about 18 bytes a group).
 * READING: a group is 18 bytes, an fp16 scale d (little-endian) followed by
 * 16 bytes of bits; bit i of byte b is element 8b+i; bit 1 means -d, bit 0
 * means +d.  y_n = bf16(sum_g d_{n,g} * sum_{k in g} sign * x_k), x used as
 * bf16 values directly, accumulated in double. */
int orc_lowbit_gemv_q1(const uint8_t* blocks, const uint16_t* x, int n, int k, int nthreads,
                       uint16_t* y, double* y_f64) {
  if (n < 0 || k <= 0 || k % 128) return ORC_ERR;
  const int groups = k / 128;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int row = 0; row < n; row++) {
    double acc = 0.0;
    for (int g = 0; g < groups; g++) {
      const uint8_t* blk = blocks + ((size_t)row * groups + g) * 18;
      double d = orc_dec_fp16((uint16_t)(blk[0] | (blk[1] << 8)));
      double s = 0.0;
      for (int i = 0; i < 128; i++) {
        int bit = (blk[2 + i / 8] >> (i % 8)) & 1;
        double xv = orc_dec_bf16(x[g * 128 + i]);
        s += bit ? -xv : xv;
      }
      acc += d * s;
    }
    if (y_f64) y_f64[row] = acc;
    if (y) y[row] = orc_round_bf16(acc);
  }
  return ORC_OK;
}

/* Dense decode GEMV over FP8 weights, for the tail after the last layer (the
 * LM-head GEMV of the #85 page's tail launch, Mod. row 24; the page names
 * no weight format for it, and FP8 E4M3 with one fp32 scale per 128x128
 * block is the format of every other weight stream on the path).  READING:
 * the inputs are bf16 rows used as they are, no activation quantisation.
 *   y[r][n] = sum_k dec(W[n][k]) * s[n/128][k/128] * x[r][k]
 * accumulated in double (each product is exact in double); y16 = bf16 RNE of
 * y.  W: codes [n][k]; s: [n/128][k/128]; x: [rows][k]. */
int orc_gemv_fp8(const uint8_t* codes, const float* scales, const uint16_t* x, int rows, int n,
                 int k, int nthreads, uint16_t* y16, double* y) {
  if (rows < 0 || n < 0 || k <= 0 || n % 128 || k % 128) return ORC_ERR;
  const int kb_n = k / 128;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int row = 0; row < n; row++) {
    for (int r = 0; r < rows; r++) {
      double acc = 0.0;
      for (int kk = 0; kk < k; kk++) {
        const double w = orc_dec_e4m3(codes[(size_t)row * k + kk]);
        const double s = (double)scales[(size_t)(row / 128) * kb_n + kk / 128];
        acc += w * s * orc_dec_bf16(x[(size_t)r * k + kk]);
      }
      if (y) y[(size_t)r * n + row] = acc;
      if (y16) y16[(size_t)r * n + row] = orc_round_bf16(acc);
    }
  }
  return ORC_OK;
}

/* The same tail GEMV over bf16 weights (READING: the #85 page's tail names no
 * weight format; an LM head kept in bf16 beside FP8 experts is the other
 * plain reading).  Inputs are bf16 rows used as they are.
 *   y[r][n] = sum_k dec(W[n][k]) * x[r][k]
 * accumulated in double (each product of two bf16 is exact in double); y16 =
 * bf16 RNE of y.  W: [n][k] bf16 bits; x: [rows][k] bf16 bits.  No grid is
 * imposed on n and k here; the device form has its own. */
int orc_gemv_bf16(const uint16_t* w, const uint16_t* x, int rows, int n, int k, int nthreads,
                  uint16_t* y16, double* y) {
  if (rows < 0 || n < 0 || k <= 0) return ORC_ERR;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int row = 0; row < n; row++) {
    for (int r = 0; r < rows; r++) {
      double acc = 0.0;
      for (int kk = 0; kk < k; kk++)
        acc += orc_dec_bf16(w[(size_t)row * k + kk]) * orc_dec_bf16(x[(size_t)r * k + kk]);
      if (y) y[(size_t)r * n + row] = acc;
      if (y16) y16[(size_t)r * n + row] = orc_round_bf16(acc);
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------- array forms for the tests */

void orc_dec_e4m3_n(const uint8_t* c, int n, double* v) {
  for (int i = 0; i < n; i++) v[i] = orc_dec_e4m3(c[i]);
}
void orc_dec_bf16_n(const uint16_t* c, int n, double* v) {
  for (int i = 0; i < n; i++) v[i] = orc_dec_bf16(c[i]);
}
void orc_dec_fp16_n(const uint16_t* c, int n, double* v) {
  for (int i = 0; i < n; i++) v[i] = orc_dec_fp16(c[i]);
}
void orc_enc_e4m3_n(const float* v, int n, uint8_t* c) {
  for (int i = 0; i < n; i++) c[i] = orc_enc_e4m3(v[i]);
}
void orc_round_bf16_n(const double* v, int n, uint16_t* h) {
  for (int i = 0; i < n; i++) h[i] = orc_round_bf16(v[i]);
}
