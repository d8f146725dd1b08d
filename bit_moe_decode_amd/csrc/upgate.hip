// upgate.hip -- up/gate GEMV of the shared expert and of every distinct
// routed expert, SiLU * gate, and mid re-quantised to FP8 per 1x128 block.
//
// #85 Mod. row 16: up/gate jobs are tiles of the shared expert and of each
// distinct expert, with every row that uses the expert as an MFMA column, so
// an expert's weights stream once however many rows picked it.  Mod. row 1:
// mid is quantised to FP8 once, per block, with its scale, and the down GEMV
// reads those bytes.  Mod. rows 18 and 21: weights load 16 bytes a lane and,
// being read once, nontemporal.
//
// Block = 4 waves = NT tiles of 16 intermediate rows x KS parts of K.  Wave
// (tile, part) runs one 16x16x128 FP8 MFMA per 128-wide K block for gate and
// one for up; the 16 columns are the group's using rows (unused columns are
// zero).  Each K block's fp32 result is scaled by weight scale x activation
// scale; parts of K are added in part order through LDS.  The block then
// writes mid = silu(gate * rstd) * (up * rstd) in fp32.  The blocks covering
// one 128-row block of mid count their arrivals; the last one quantises that
// block for every using row: s = amax/448, codes = e4m3(mid/s).
//
// Grid: Is/BR blocks for the shared expert, then I/BR blocks for each of the
// max_groups routed groups; blocks of groups past the step's D exit at once.
#include "device_common.h"

namespace moe {

template <int KS>
struct UgSmem {
  float red[KS > 1 ? KS - 1 : 1][4 / KS][kWave][8];
  int last;
};

template <int KS, int RFMT>
__global__ __launch_bounds__(256) void moe_upgate_kernel(Weights w, Ws ws, Dims d) {
  constexpr int NT = 4 / KS;  // 16-row tiles per block
  constexpr int BR = 16 * NT;  // intermediate rows per block
  constexpr int P = 4;         // K blocks in flight per wave
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
  const int kb0 = kp * (nkbh / KS), kb1 = kb0 + nkbh / KS;

  float accg[4] = {0.f, 0.f, 0.f, 0.f}, accu[4] = {0.f, 0.f, 0.f, 0.f};
  if (RFMT == kFmtFp8 || g < 0) {
    const size_t roff = (size_t)(n0 + col) * H + (lane >> 4) * 32;
    const uint8_t* pg = cg + roff;
    const uint8_t* pu = cu + roff;
    const uint8_t* pa = ws.act_q + (size_t)row * H + (lane >> 4) * 32;
    const float* psg = sg + (size_t)(n0 / 128) * nkbh;
    const float* psu = su + (size_t)(n0 / 128) * nkbh;
    const float* psa = ws.act_s + (size_t)row * nkbh;
    struct Stage {
      u32x4 g0, g1, u0, u1, a0, a1;
      float sg, su, sa;
    } st[P];
    auto issue = [&](Stage& s, int kb) {
      s.g0 = ld_nt16(pg + kb * 128);
      s.g1 = ld_nt16(pg + kb * 128 + 16);
      s.u0 = ld_nt16(pu + kb * 128);
      s.u1 = ld_nt16(pu + kb * 128 + 16);
      if (live) {
        s.a0 = ld16(pa + kb * 128);
        s.a1 = ld16(pa + kb * 128 + 16);
        s.sa = psa[kb];
      } else {
        s.a0 = u32x4{0u, 0u, 0u, 0u};
        s.a1 = s.a0;
        s.sa = 0.f;
      }
      s.sg = psg[kb];
      s.su = psu[kb];
    };
#pragma unroll
    for (int p = 0; p < P; p++)
      if (kb0 + p < kb1) issue(st[p], kb0 + p);
    for (int kb = kb0; kb < kb1; kb += P) {
#pragma unroll
      for (int p = 0; p < P; p++) {
        const int k = kb + p;
        if (k < kb1) {
          const v8i bv = cat8(st[p].a0, st[p].a1);
          const v4f cgv = mfma_fp8(cat8(st[p].g0, st[p].g1), bv);
          const v4f cuv = mfma_fp8(cat8(st[p].u0, st[p].u1), bv);
          const float fg = st[p].sg * st[p].sa, fu = st[p].su * st[p].sa;
#pragma unroll
          for (int v = 0; v < 4; v++) {
            accg[v] = fmaf(cgv[v], fg, accg[v]);
            accu[v] = fmaf(cuv[v], fu, accu[v]);
          }
          if (k + P < kb1) issue(st[p], k + P);
        }
      }
    }
  }

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
  const size_t mrow = ((size_t)slot * d.max_rows + row) * d.imax;
  if (kp == 0 && live) {
    const float rs = ws.rstd[row];
    v4f m;
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const float gt = accg[v] * rs, up = accu[v] * rs;
      m[v] = gt / (1.0f + expf(-gt)) * up;
    }
    *reinterpret_cast<v4f*>(ws.mid + mrow + n0 + 4 * (lane >> 4)) = m;
  }
  if (RFMT == kFmtMxfp4 && g >= 0) return;  // MXFP4 experts keep mid in fp32

  // ---- arrival per 128-row mid block; the last block quantises it
  __threadfence();
  __syncthreads();
  const int nb = (t * BR) / 128;
  uint32_t* cnt = ws.ctrl_upgate + (size_t)slot * (d.imax / 128) + nb;
  if (tid == 0) sm.last = (atomicAdd(cnt, 1u) == (uint32_t)(128 / BR - 1));
  __syncthreads();
  if (!sm.last) return;
  __threadfence();
  for (int c2 = wv; c2 < nrows; c2 += 4) {
    const int r2 = g < 0 ? c2 : (int)ws.grp_rows[g * 8 + c2];
    const size_t base = ((size_t)slot * d.max_rows + r2) * d.imax + nb * 128;
    const float v0 = ws.mid[base + 2 * lane], v1 = ws.mid[base + 2 * lane + 1];
    const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float s = amax / 448.0f;
    const uint32_t q = (s > 0.f) ? f32x2_to_e4m3(v0 / s, v1 / s) : 0u;
    *reinterpret_cast<uint16_t*>(ws.midq + base + 2 * lane) = (uint16_t)q;
    if (lane == 0) ws.midqs[((size_t)slot * d.max_rows + r2) * (d.imax / 128) + nb] = s;
  }
  if (tid == 0) *cnt = 0u;
}

template __global__ void moe_upgate_kernel<1, kFmtFp8>(Weights, Ws, Dims);
template __global__ void moe_upgate_kernel<2, kFmtFp8>(Weights, Ws, Dims);
template __global__ void moe_upgate_kernel<4, kFmtFp8>(Weights, Ws, Dims);

}  // namespace moe

namespace moe {
// Rows of intermediate a block covers for a K split of ks.
int upgate_block_rows(int ks) { return 16 * (4 / ks); }

hipError_t launch_upgate(int ks, int rfmt, int max_groups, const Weights& w, const Ws& ws,
                         const Dims& d, hipStream_t stream) {
  const int br = upgate_block_rows(ks);
  dim3 grid(d.Is / br + max_groups * (d.I / br));
  if (rfmt != kFmtFp8) return hipErrorInvalidValue;
  switch (ks) {
    case 1: hipLaunchKernelGGL((moe_upgate_kernel<1, kFmtFp8>), grid, dim3(256), 0, stream, w, ws, d); break;
    case 2: hipLaunchKernelGGL((moe_upgate_kernel<2, kFmtFp8>), grid, dim3(256), 0, stream, w, ws, d); break;
    case 4: hipLaunchKernelGGL((moe_upgate_kernel<4, kFmtFp8>), grid, dim3(256), 0, stream, w, ws, d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace moe
