// upgate.hip -- up/gate GEMV of the shared expert and of every distinct
// routed expert, as K-part sums; moe_midq_kernel (midq.hip) adds the parts,
// applies SiLU * up and quantises mid.
//
// #85 Mod. row 16: up/gate jobs are tiles of the shared expert and of each
// distinct expert, with every row that uses the expert as an MFMA column, so
// an expert's weights stream once however many rows picked it.  Mod. rows 18
// and 21: weights load 16 bytes a lane and, being read once, nontemporal.
//
// Block = 4 waves = 4/ks slabs of 16 intermediate rows x ks parts of K; the
// grid lists the shared expert's slabs, then I/16 slabs for each of the step's
// possible routed groups (blocks of groups past the step's D exit at once).
// Many small blocks let the hardware dispatcher even out the load per CU.
// Per K block a wave loads its 16 weight rows of gate and of up
// row-contiguously (8 lanes read one row's 128-byte line), re-lays them through
// LDS into MFMA operand order and runs one 16x16x128 FP8 MFMA for each, whose
// 16 columns are the expert's using rows; the result is scaled by weight scale
// x activation scale and accumulated in fp32.  The wave then stores its K-part
// sums per (row, pick).  No block waits for another, and no wave for another.
#include "device_common.h"

namespace moe {

// One K block of one wave: gate and up weight rows (row-contiguous), the
// using rows' activation codes in operand order and the three scales.  Every
// lane loads (columns past the expert's rows read row 0; their results are
// never stored), so the ring carries no per-lane condition.
struct UgStage {
  u32x4 g0, g1, u0, u1, a0, a1;
  float sg, su, sa;
};

template <int P>
__global__ __launch_bounds__(256) void moe_upgate_kernel(Weights w, Ws ws, Dims d) {
  __shared__ uint8_t s_tile[4][2][kTileBytes];  // per wave: gate and up weight tiles
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = d.H, nkbh = H / 128, KS = d.ks, nk = nkbh / KS;
  const int spb = 4 / KS;  // slabs per block
  const int col = lane & 15;

  // ---- the block's expert and slab
  const int nb_sh = d.Is / (16 * spb);
  int b = blockIdx.x, g = -1, nrows, row, e;
  uint64_t picks8 = 0;  // pick of each row in the group (routed)
  if (b < nb_sh) {
    nrows = d.rows;
    row = col < nrows ? col : 0;
    e = -1;
  } else {
    b -= nb_sh;
    const int per = d.I / (16 * spb);
    g = b / per;
    b -= g * per;
    // one round of independent loads; the table of a group past D is stale
    // but in bounds, and unused
    const int D = *ws.n_groups;
    e = ws.grp_expert[g];
    nrows = ws.grp_nrows[g];
    const uint64_t rows8 = *reinterpret_cast<const uint64_t*>(ws.grp_rows + g * 8);
    picks8 = *reinterpret_cast<const uint64_t*>(ws.grp_slot + g * 8);
    if (g >= D) return;
    row = col < nrows ? (int)((rows8 >> (8 * (col & 7))) & 0xFF) : 0;
  }
  const int slab = b * spb + wv / KS, kp = wv % KS;
  const int n0 = slab * 16, kb0 = kp * nk;
  const size_t ebytes = (size_t)d.I * H;
  const size_t escl = (size_t)(d.I / 128) * nkbh;  // scales per routed expert
  const uint8_t* bg = e < 0 ? w.sg_c : w.gate_c + (size_t)e * ebytes;
  const uint8_t* bu = e < 0 ? w.su_c : w.up_c + (size_t)e * ebytes;
  const float* sg = e < 0 ? w.sg_s : reinterpret_cast<const float*>(w.gate_s) + (size_t)e * escl;
  const float* su = e < 0 ? w.su_s : reinterpret_cast<const float*>(w.up_s) + (size_t)e * escl;
  // lane l loads rows n0 + l/8 and n0 + 8 + l/8, 16-byte chunk l%8
  const uint8_t* pg = bg + (size_t)(n0 + (lane >> 3)) * H + (lane & 7) * 16 + (size_t)kb0 * 128;
  const uint8_t* pu = bu + (pg - bg);
  const size_t r8 = (size_t)8 * H;
  const uint8_t* pa = ws.act_q + (size_t)row * H + (lane >> 4) * 32 + (size_t)kb0 * 128;
  const float* psg = sg + (size_t)(n0 / 128) * nkbh + kb0;
  const float* psu = su + (size_t)(n0 / 128) * nkbh + kb0;
  const float* psa = ws.act_s + (size_t)row * nkbh + kb0;
  uint8_t* tg = s_tile[wv][0];
  uint8_t* tu = s_tile[wv][1];

  auto issue = [&](UgStage& st, int k) {
    const size_t o = (size_t)k * 128;
    st.g0 = ld_nt16(pg + o);
    st.g1 = ld_nt16(pg + r8 + o);
    st.u0 = ld_nt16(pu + o);
    st.u1 = ld_nt16(pu + r8 + o);
    st.a0 = ld16(pa + o);
    st.a1 = ld16(pa + o + 16);
    st.sg = psg[k];
    st.su = psu[k];
    st.sa = psa[k];
  };
  float accg[4] = {0.f, 0.f, 0.f, 0.f}, accu[4] = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](UgStage& st) {
    tile_put(tg, lane, st.g0, st.g1);
    tile_put(tu, lane, st.u0, st.u1);
    asm volatile("" ::: "memory");
    const v8i bv = cat8(st.a0, st.a1);
    const v4f cgv = mfma_fp8(tile_get(tg, lane), bv);
    const v4f cuv = mfma_fp8(tile_get(tu, lane), bv);
    asm volatile("" ::: "memory");
    const float fg = st.sg * st.sa, fu = st.su * st.sa;
#pragma unroll
    for (int v = 0; v < 4; v++) {
      accg[v] = fmaf(cgv[v], fg, accg[v]);
      accu[v] = fmaf(cuv[v], fu, accu[v]);
    }
  };
  // ring of P K blocks (P divides nk): every issued load is used
  UgStage st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  for (int k0 = 0; k0 < nk - P; k0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p]);
      issue(st[p], k0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p]);
  pin4(accg);  // the MFMAs run with every lane, before the divergent store
  pin4(accu);
  if (col < nrows) {
    const int pick = g < 0 ? 8 : (int)((picks8 >> (8 * row)) & 0xFF);
    const size_t o = ((size_t)(row * 9 + pick) * KS + kp) * d.imax + n0 + 4 * (lane >> 4);
    *reinterpret_cast<v4f*>(ws.gpart + o) = v4f{accg[0], accg[1], accg[2], accg[3]};
    *reinterpret_cast<v4f*>(ws.upart + o) = v4f{accu[0], accu[1], accu[2], accu[3]};
  }
}

// K blocks in flight per wave: the largest of 4, 2, 1 dividing the wave's
// K blocks.
static int ring_depth(int nk) { return nk % 4 == 0 ? 4 : (nk % 2 == 0 ? 2 : 1); }

// K parts of the up/gate slabs: the largest of 4, 2, 1 dividing H/128.
int upgate_k_parts(int hidden, int inter) {
  (void)inter;
  const int nkb = hidden / 128;
  return nkb % 4 == 0 ? 4 : (nkb % 2 == 0 ? 2 : 1);
}

hipError_t launch_upgate(int rfmt, int max_groups, const Weights& w, const Ws& ws,
                         const Dims& d, hipStream_t stream) {
  if (rfmt != kFmtFp8) return hipErrorInvalidValue;
  const int br = 16 * (4 / d.ks);
  const dim3 grid(d.Is / br + max_groups * (d.I / br));
  switch (ring_depth(d.H / 128 / d.ks)) {
    case 4: hipLaunchKernelGGL((moe_upgate_kernel<4>), grid, dim3(256), 0, stream, w, ws, d); break;
    case 2: hipLaunchKernelGGL((moe_upgate_kernel<2>), grid, dim3(256), 0, stream, w, ws, d); break;
    default: hipLaunchKernelGGL((moe_upgate_kernel<1>), grid, dim3(256), 0, stream, w, ws, d); break;
  }
  return hipGetLastError();
}

}  // namespace moe
