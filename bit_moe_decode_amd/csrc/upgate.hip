// upgate.hip -- up/gate GEMV of the shared expert and of every distinct
// routed expert, with SiLU * gate; mid is written in fp32 and quantised by
// moe_midq_kernel (midq.hip).
//
// #85 Mod. row 16: up/gate jobs are tiles of the shared expert and of each
// distinct expert, with every row that uses the expert as an MFMA column, so
// an expert's weights stream once however many rows picked it.  Mod. rows 18
// and 21: weights load 16 bytes a lane and, being read once, nontemporal.
//
// Block = 4 waves = NT tiles of 16 intermediate rows x KS parts of K.  For
// each 128-wide K block a wave loads its 16 weight rows of gate and of up
// row-contiguously (8 lanes read one row's 128-byte line: whole lines per
// instruction stream fastest), re-lays them through LDS into MFMA operand
// order, and runs one 16x16x128 FP8 MFMA for gate and one for up whose 16
// columns are the group's using rows.  Each K block's fp32 result is scaled by
// weight scale x activation scale; parts of K are added in part order through
// LDS; then mid = silu(gate * rstd) * (up * rstd).  No block waits for another.
//
// Grid: Is/BR blocks for the shared expert, then I/BR blocks for each of the
// step's possible routed groups; blocks of groups past the step's D exit.
#include "device_common.h"

namespace moe {

template <int KS>
struct UgSmem {
  uint8_t tile[4][2][kTileBytes];  // per wave: gate and up weight tiles
  float red[KS > 1 ? KS - 1 : 1][4 / KS][kWave][8];
};

// One K block of one wave: gate and up weight rows (row-contiguous), the
// using rows' activation codes in operand order and the three scales.  Every
// lane loads (columns past the group's rows read row 0; their results are
// never stored), so the ring below carries no per-lane condition.
struct UgStage {
  u32x4 g0, g1, u0, u1, a0, a1;
  float sg, su, sa;
};

template <int KS, int RFMT, int P>
__global__ __launch_bounds__(256) void moe_upgate_kernel(Weights w, Ws ws, Dims d) {
  constexpr int NT = 4 / KS;  // 16-row tiles per block
  constexpr int BR = 16 * NT;  // intermediate rows per block
  __shared__ UgSmem<KS> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tw = wv % NT, kp = wv / NT;
  const int H = d.H, nkbh = H / 128;

  // ---- which expert slot and tile this block owns
  const int nb_sh = d.Is / BR;
  int b = blockIdx.x, slot, g = -1, nrows, t, I;
  const uint8_t *cg, *cu;
  const float *sg, *su;
  if (b < nb_sh) {
    slot = 0;
    t = b;
    I = d.Is;
    nrows = d.rows;
    cg = w.sg_c;
    cu = w.su_c;
    sg = w.sg_s;
    su = w.su_s;
  } else {
    b -= nb_sh;
    const int per = d.I / BR;
    g = b / per;
    if (g >= *ws.n_groups) return;
    t = b - g * per;
    slot = 1 + g;
    I = d.I;
    nrows = ws.grp_nrows[g];
    const size_t e = (size_t)ws.grp_expert[g];
    cg = w.gate_c + e * (size_t)I * H;
    cu = w.up_c + e * (size_t)I * H;
    sg = reinterpret_cast<const float*>(w.gate_s) + e * (size_t)(I / 128) * nkbh;
    su = reinterpret_cast<const float*>(w.up_s) + e * (size_t)(I / 128) * nkbh;
  }
  (void)I;
  const int n0 = t * BR + tw * 16;
  const int col = lane & 15;
  const bool live = col < nrows;
  const int row = live ? (g < 0 ? col : (int)ws.grp_rows[g * 8 + col]) : 0;
  const int nk = nkbh / KS;  // K blocks of this wave, a multiple of P
  const int kb0 = kp * nk;
  uint8_t* tg = sm.tile[wv][0];
  uint8_t* tu = sm.tile[wv][1];

  float accg[4] = {0.f, 0.f, 0.f, 0.f}, accu[4] = {0.f, 0.f, 0.f, 0.f};
  if (RFMT == kFmtFp8 || g < 0) {
    // lane l loads rows n0 + l/8 and n0 + 8 + l/8, 16-byte chunk l%8
    const size_t roff = (size_t)(n0 + (lane >> 3)) * H + (lane & 7) * 16 + (size_t)kb0 * 128;
    const size_t r8 = (size_t)8 * H;
    const uint8_t* pg = cg + roff;
    const uint8_t* pu = cu + roff;
    const uint8_t* pa = ws.act_q + (size_t)row * H + (lane >> 4) * 32 + (size_t)kb0 * 128;
    const float* psg = sg + (size_t)(n0 / 128) * nkbh + kb0;
    const float* psu = su + (size_t)(n0 / 128) * nkbh + kb0;
    const float* psa = ws.act_s + (size_t)row * nkbh + kb0;
    UgStage st[P];
#define UG_ISSUE(S, K)                            \
  do {                                            \
    (S).g0 = ld_nt16(pg + (K) * 128);             \
    (S).g1 = ld_nt16(pg + r8 + (K) * 128);        \
    (S).u0 = ld_nt16(pu + (K) * 128);             \
    (S).u1 = ld_nt16(pu + r8 + (K) * 128);        \
    (S).a0 = ld16(pa + (K) * 128);                \
    (S).a1 = ld16(pa + (K) * 128 + 16);           \
    (S).sg = psg[K];                              \
    (S).su = psu[K];                              \
    (S).sa = psa[K];                              \
  } while (0)
#define UG_CONSUME(S)                                                       \
  do {                                                                      \
    tile_put(tg, lane, (S).g0, (S).g1);                                     \
    tile_put(tu, lane, (S).u0, (S).u1);                                     \
    asm volatile("" ::: "memory");                                          \
    const v8i bv = cat8((S).a0, (S).a1);                                    \
    const v4f cgv = mfma_fp8(tile_get(tg, lane), bv);                       \
    const v4f cuv = mfma_fp8(tile_get(tu, lane), bv);                       \
    asm volatile("" ::: "memory");                                          \
    const float fg = (S).sg * (S).sa, fu = (S).su * (S).sa;                 \
    _Pragma("unroll") for (int v = 0; v < 4; v++) {                         \
      accg[v] = fmaf(cgv[v], fg, accg[v]);                                  \
      accu[v] = fmaf(cuv[v], fu, accu[v]);                                  \
    }                                                                       \
  } while (0)
#pragma unroll
    for (int p = 0; p < P; p++) UG_ISSUE(st[p], p);
    for (int k = 0; k < nk - P; k += P) {
#pragma unroll
      for (int p = 0; p < P; p++) {
        UG_CONSUME(st[p]);
        UG_ISSUE(st[p], k + P + p);
      }
    }
#pragma unroll
    for (int p = 0; p < P; p++) UG_CONSUME(st[p]);
#undef UG_ISSUE
#undef UG_CONSUME
  }
  pin4(accg);  // the MFMAs run with every lane, before any divergent use
  pin4(accu);

  // ---- add the K parts in part order
  if (KS > 1) {
    if (kp > 0) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        sm.red[kp - 1][tw][lane][v] = accg[v];
        sm.red[kp - 1][tw][lane][4 + v] = accu[v];
      }
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
      for (int q = 0; q < KS - 1; q++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          accg[v] += sm.red[q][tw][lane][v];
          accu[v] += sm.red[q][tw][lane][4 + v];
        }
    }
  }

  // ---- mid = silu(gate) * up, fp32
  if (kp == 0 && live) {
    const float rs = ws.rstd[row];
    v4f m;
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const float gt = accg[v] * rs, up = accu[v] * rs;
      m[v] = gt / (1.0f + expf(-gt)) * up;
    }
    const size_t mrow = ((size_t)slot * d.max_rows + row) * d.imax;
    *reinterpret_cast<v4f*>(ws.mid + mrow + n0 + 4 * (lane >> 4)) = m;
  }
}

// Rows of intermediate a block covers for a K split of ks.
int upgate_block_rows(int ks) { return 16 * (4 / ks); }

// K blocks in flight per wave: the largest of 4, 2, 1 dividing the wave's K blocks.
static int ring_depth(int nk) { return nk % 4 == 0 ? 4 : (nk % 2 == 0 ? 2 : 1); }

template <int KS>
static void launch_ks(int p, dim3 grid, const Weights& w, const Ws& ws, const Dims& d,
                      hipStream_t stream) {
  switch (p) {
    case 4: hipLaunchKernelGGL((moe_upgate_kernel<KS, kFmtFp8, 4>), grid, dim3(256), 0, stream, w, ws, d); break;
    case 2: hipLaunchKernelGGL((moe_upgate_kernel<KS, kFmtFp8, 2>), grid, dim3(256), 0, stream, w, ws, d); break;
    default: hipLaunchKernelGGL((moe_upgate_kernel<KS, kFmtFp8, 1>), grid, dim3(256), 0, stream, w, ws, d); break;
  }
}

hipError_t launch_upgate(int ks, int rfmt, int max_groups, const Weights& w, const Ws& ws,
                         const Dims& d, hipStream_t stream) {
  const int br = upgate_block_rows(ks);
  dim3 grid(d.Is / br + max_groups * (d.I / br));
  if (rfmt != kFmtFp8) return hipErrorInvalidValue;
  const int p = ring_depth(d.H / 128 / ks);
  switch (ks) {
    case 1: launch_ks<1>(p, grid, w, ws, d, stream); break;
    case 2: launch_ks<2>(p, grid, w, ws, d, stream); break;
    case 4: launch_ks<4>(p, grid, w, ws, d, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
