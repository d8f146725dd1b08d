/*
 * moe_oracle.h -- plain, slow fp64 CPU oracle for the small-row MoE decode step
 * and the 1-bit group-128 GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code with the HIP library.
 *
 * Sources (cited in every function of moe_oracle.c):
 *   "#85"        the body of sgl-amd-mono PR #85 ("...MoE expert dedup and weight
 *                loads, kernarg reload, LM-head loads"), quoted on the GitHub page
 *                of sglang PR #47324; "Mod. row N" is row N of its Modifications
 *                table.
 *   "1-Bit Turbo" the README page "SGLang 1-Bit Turbo", section "PrismML 1-Bit
 *                GGUF Model Support (Q1_0_G128)".
 *   "MXFP4 page" the GitHub page of sglang PR #31683, "[ROCm][MI35X] Enable
 *                GLM-5.2-MXFP4 MTP speculative decoding".
 *   Code-point values follow the OCP 8-bit floating point (E4M3FN) and OCP MX
 *   v1.0 (E2M1, E8M0) definitions, IEEE 754 binary16, and bfloat16.
 *
 * Where the pages leave a step open, the reading taken is stated beside the
 * function that implements it.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_ERR 1

#define ORC_FMT_FP8 1   /* E4M3FN codes, one fp32 scale per 128x128 block  */
#define ORC_FMT_MXFP4 2 /* E2M1 codes, 2 per byte (low nibble first), E8M0 per 32 along K */
#define ORC_FMT_Q1 3    /* 1-bit group-128: [N][K/128] blocks of 18 bytes, fp16 d + 16 sign bytes */
/* Expert inputs: FP8 E4M3 per 1x128 block of u (#85 Mod. row 10, the default),
 * or u itself (bf16) -- an option for comparing what the FP8 blocks cost. */
#define ORC_ACT_FP8 0
#define ORC_ACT_BF16 1

/* ---- scalar codecs ---- */
double orc_dec_bf16(uint16_t h);
double orc_dec_fp16(uint16_t h);
double orc_dec_e4m3(uint8_t c);
double orc_dec_e2m1(uint8_t nibble);
double orc_dec_e8m0(uint8_t c);
uint8_t orc_enc_e4m3(float v);
uint16_t orc_round_bf16(double v);

/* ---- step pieces ---- */
void orc_top8(const double* z, int n_experts, int32_t ids[8]);
void orc_softmax8(const double z_sel[8], double g[8]);
int orc_dedup(const int32_t* ids, int rows, int32_t* n_groups, int32_t* grp_expert,
              uint8_t* grp_owner_slot, uint8_t* grp_owner_row, uint8_t* grp_mask,
              uint8_t* grp_slot);
void orc_quant_blocks(const float* v, int n, uint8_t* q, float* s);

int orc_router(int rows, int hidden, int n_experts, float eps, const uint16_t* x,
               const uint16_t* gamma, const uint16_t* router_w, double* z, double* rstd,
               uint16_t* u);

/* One weight matrix [N, K] in a low-bit format. */
typedef struct {
  const uint8_t* codes; /* FP8: [N][K];  MXFP4: [N][K/2];  Q1: [N][K/128][18] */
  const void* scales;   /* FP8: float [N/128][K/128];  MXFP4: uint8 E8M0 [N][K/32];  Q1: unused */
} orc_mat;

typedef struct {
  int32_t hidden, inter, n_experts, shared_inter, rows;
  float rms_eps;
  int32_t routed_fmt; /* ORC_FMT_FP8, ORC_FMT_MXFP4 or ORC_FMT_Q1; the shared expert is FP8 */
  int32_t nthreads;
  int32_t act_fmt;    /* ORC_ACT_FP8 or ORC_ACT_BF16 */
} orc_cfg;

/* Debug outputs of one step; any pointer may be NULL.  "slot" 0..7 is the
 * row's pick in top-8 order, slot 8 is the shared expert; Imax = max(I, Is). */
typedef struct {
  double* z;        /* [R][E]   router logits rstd * (W_r . u) */
  double* rstd;     /* [R] */
  uint16_t* u;      /* [R][H]   bf16(x * gamma) */
  int32_t* ids;     /* [R][8] */
  double* gates;    /* [R][8] */
  uint8_t* act_q;   /* [R][H] */
  float* act_s;     /* [R][H/128] */
  double* mid;      /* [R][9][Imax] pre-quantisation mid */
  uint8_t* midq;    /* [R][9][Imax] (FP8 experts only) */
  float* midqs;     /* [R][9][Imax/128] */
  double* y;        /* [R][9][H] per-slot down outputs */
  double* out_f64;  /* [R][H] combine before the bf16 rounding */
  double* gate;     /* [R][9][Imax] gate = W_gate . h (h includes rstd) */
  double* up;       /* [R][9][Imax] */
  double* gate_abs; /* [R][9][Imax] sum_k |W_gate[n,k] h_k|: sizes rounding bounds */
  double* up_abs;   /* [R][9][Imax] */
  double* gate_gmax; /* [R][9][Imax] sum over groups of 8 consecutive k of max |W_gate h|:
                        sizes the bounds of dot products summed in groups of 8 */
  double* up_gmax;  /* [R][9][Imax] */
} orc_debug;

int orc_moe_step(const orc_cfg* cfg, const uint16_t* x, const uint16_t* gamma,
                 const uint16_t* router_w, const orc_mat* gate, const orc_mat* up,
                 const orc_mat* down, const orc_mat* sh_gate, const orc_mat* sh_up,
                 const orc_mat* sh_down, const float* anchor_z, uint16_t* out,
                 orc_debug* dbg);

/* The down GEMV of one expert on a given mid: FP8 and 1-bit experts take midq
 * codes [i_dim] with midqs scales [i_dim/128]; MXFP4 experts take mid32. */
int orc_expert_down(int fmt, const orc_mat* wd, int h_dim, int i_dim, const uint8_t* midq,
                    const float* midqs, const float* mid32, int nthreads, double* y,
                    double* y_abs, double* y_gmax);

/* array forms, used by the tests */
void orc_dec_e4m3_n(const uint8_t* c, int n, double* v);
void orc_dec_bf16_n(const uint16_t* c, int n, double* v);
void orc_dec_fp16_n(const uint16_t* c, int n, double* v);
void orc_enc_e4m3_n(const float* v, int n, uint8_t* c);
void orc_round_bf16_n(const double* v, int n, uint16_t* h);

int orc_lowbit_gemv_q1(const uint8_t* blocks, const uint16_t* x, int n, int k, int nthreads,
                       uint16_t* y, double* y_f64);

/* FP8 E4M3 weights with one fp32 scale per 128x128 block, bf16 input rows */
int orc_gemv_fp8(const uint8_t* codes, const float* scales, const uint16_t* x, int rows, int n,
                 int k, int nthreads, uint16_t* y16, double* y);

/* bf16 weights [n][k], bf16 input rows */
int orc_gemv_bf16(const uint16_t* w, const uint16_t* x, int rows, int n, int k, int nthreads,
                  uint16_t* y16, double* y);

#ifdef __cplusplus
}
#endif
#endif
