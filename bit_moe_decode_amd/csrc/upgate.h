// upgate.h -- up/gate GEMV of the shared expert and of every distinct routed
// expert, and mid = silu(gate) * up from it: the device code of one up/gate
// block, launched by moe_upgate_kernel (upgate.hip) and, beside the routing,
// by moe_route_kernel (route.hip).
//
// #85 Mod. row 16: up/gate jobs are tiles of the shared expert and of each
// distinct expert, with every row that uses the expert as an MFMA column, so
// an expert's weights stream once however many rows picked it.  Mod. rows 18
// and 21: weights load 16 bytes a lane and, being read once, nontemporal.
// Mod. row 1 and the MXFP4 page: routed experts may instead hold MXFP4
// weights (E2M1 pairs, one E8M0 exponent per 32 inputs); the shared expert
// stays FP8.
//
// Block = 4 waves = 4/ks slabs of 16 intermediate rows x ks parts of K; the
// blocks are numbered over the shared expert's slabs, then I/16 slabs for each
// of the step's possible routed groups (blocks of groups past the step's D
// exit at once).  In moe_route_kernel all of them run beside the routing
// block: the shared expert's at once, a routed one once the routing block has
// published its record (below); in moe_upgate_kernel they read the published
// table after a launch boundary.
// Many small blocks let the hardware dispatcher even out the load per CU.
// A wave loads its 16 weight rows of gate and of up row-contiguously (8 lanes
// read one row's 128-byte line), re-lays them through LDS into MFMA operand
// order and runs 16x16x128 MFMAs whose 16 columns are the expert's using rows;
// the fp32 results are scaled and accumulated.  The block then adds its K-part
// sums in part order, through LDS, and stores
//   mid = silu(gate * rstd) * (up * rstd)          (fp32)
// per (row, pick) of its slabs.  No block waits for another, except a routed
// block for its record in moe_route_kernel.  The FP8 re-quantisation of mid
// is done by the down kernel, which reads it.
//
//  FP8 item = one 128-wide K block: one FP8 x FP8 MFMA per matrix, scaled by
//    weight block scale x activation block scale.
//  FP8 item with bf16 activations (MOE_ACT_BF16, u itself as the input): the
//    K block's codes converted to bf16 exactly, four 16x16x32 bf16 MFMAs per
//    matrix against u, scaled by the weight block scale.
//  MXFP4 item = two 128-wide K blocks (a 128-byte line per row): per K block
//    one scaled FP4 x FP8 MFMA per matrix, the E8M0 exponents entering as the
//    MFMA's A scales, then the activation block scale.  Operand layout of that
//    MFMA on gfx950 (established by a device probe): A lane l holds row l%16
//    and the 32 inputs 32*(l/16) .. +32 of the K block as 16 bytes, low nibble
//    first, with the E8M0 of those 32 as its scale; B lane l holds column l%16
//    and the FP8 inputs 16*(l/16) .. +16 and 64 + 16*(l/16) .. +16.
#pragma once
#include "route.h"

namespace moe {

// One K item of one wave: gate and up weight rows (row-contiguous), the using
// rows' activation codes in operand order and the scales.  Every lane loads
// (columns past the expert's rows read row 0; their results are never
// stored), so the ring carries no per-lane condition.
struct UgStage {
  u32x4 g0, g1, u0, u1, a0, a1;
  float sg, su, sa;
};
struct UgStage4 {
  u32x4 g0, g1, u0, u1, a0, a1, a2, a3;  // a0,a1: K block 0; a2,a3: K block 1
  uint32_t eg0, eg1, eu0, eu1;           // E8M0 of the lane's row, K blocks 0 and 1
  float sa0, sa1;
};

// Operand of the scaled MFMA for FP4 A: 16 bytes in the low half.
__device__ __forceinline__ v8i fp4_operand(const u32x4& v) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  r[0] = v[0];
  r[1] = v[1];
  r[2] = v[2];
  r[3] = v[3];
  return r;
}
// Row l%16, bytes 64h + 16(l/16) .. +16 of the tile (K block h of the item).
__device__ __forceinline__ u32x4 tile_get_fp4(const uint8_t* tile, int lane, int h) {
  return *reinterpret_cast<const u32x4*>(tile + (lane & 15) * kTileStride + 64 * h +
                                         (lane >> 4) * 16);
}
__device__ __forceinline__ v4f mfma_fp4_fp8(const v8i& a, const v8i& b, int scale_a) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 0, 0, scale_a, 0, 127);
}

struct UgJob {
  int e, row, n0;  // expert (-1: shared), activation row of the lane's column, first row
  bool live;       // the lane's column is one of the expert's using rows
  int nrows;       // the expert's using rows (the block's columns)
  uint64_t rows8;  // their activation rows, one byte each (routed experts)
};

// FP8 weights: K blocks kb0 .. kb0 + nk of the slab.
template <int P>
__device__ __forceinline__ void ug_fp8(const Weights& w, const Ws& ws, const Dims& d, UgJob j,
                                       int kb0, int nk, uint8_t* tg, uint8_t* tu, int lane,
                                       float* accg, float* accu) {
  const int H = d.H, nkbh = H / 128;
  const size_t ebytes = (size_t)d.I * H;
  const size_t escl = (size_t)(d.I / 128) * nkbh;  // scales per routed expert
  const uint8_t* bg = j.e < 0 ? w.sg_c : w.gate_c + (size_t)j.e * ebytes;
  const uint8_t* bu = j.e < 0 ? w.su_c : w.up_c + (size_t)j.e * ebytes;
  const float* sg =
      j.e < 0 ? w.sg_s : reinterpret_cast<const float*>(w.gate_s) + (size_t)j.e * escl;
  const float* su = j.e < 0 ? w.su_s : reinterpret_cast<const float*>(w.up_s) + (size_t)j.e * escl;
  // lane l loads rows n0 + l/8 and n0 + 8 + l/8, 16-byte chunk l%8
  const uint8_t* pg = bg + (size_t)(j.n0 + (lane >> 3)) * H + (lane & 7) * 16 + (size_t)kb0 * 128;
  const uint8_t* pu = bu + (pg - bg);
  const size_t r8 = (size_t)8 * H;
  const uint8_t* pa = ws.act_q + (size_t)j.row * H + (lane >> 4) * 32 + (size_t)kb0 * 128;
  const float* psg = sg + (size_t)(j.n0 / 128) * nkbh + kb0;
  const float* psu = su + (size_t)(j.n0 / 128) * nkbh + kb0;
  const float* psa = ws.act_s + (size_t)j.row * nkbh + kb0;

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
}

// FP8 weights against bf16 activations (u itself): K blocks kb0 .. kb0 + nk
// of the slab.  The weight rows are re-laid through LDS as for FP8; then per
// 32 inputs of the K block, lane l converts the 8 codes of row l%16 at inputs
// 32s + 8(l/16) .. +8 to bf16 (exact: every E4M3 value is a bf16 value; the
// conversion's scale is 1) and runs one 16x16x32 bf16 MFMA per matrix against
// its using row's u at the same inputs; the K block's fp32 result is scaled
// by the weight block scale (rstd comes in the epilogue).
struct UgStageB {
  u32x4 g0, g1, u0, u1, a[4];
  float sg, su;
};
template <int P>
__device__ __forceinline__ void ug_fp8_bf16a(const Weights& w, const Ws& ws, const Dims& d,
                                             UgJob j, int kb0, int nk, uint8_t* tg, uint8_t* tu,
                                             int lane, float* accg, float* accu) {
  const int H = d.H, nkbh = H / 128;
  const size_t ebytes = (size_t)d.I * H;
  const size_t escl = (size_t)(d.I / 128) * nkbh;
  const uint8_t* bg = j.e < 0 ? w.sg_c : w.gate_c + (size_t)j.e * ebytes;
  const uint8_t* bu = j.e < 0 ? w.su_c : w.up_c + (size_t)j.e * ebytes;
  const float* sg =
      j.e < 0 ? w.sg_s : reinterpret_cast<const float*>(w.gate_s) + (size_t)j.e * escl;
  const float* su = j.e < 0 ? w.su_s : reinterpret_cast<const float*>(w.up_s) + (size_t)j.e * escl;
  const uint8_t* pg = bg + (size_t)(j.n0 + (lane >> 3)) * H + (lane & 7) * 16 + (size_t)kb0 * 128;
  const uint8_t* pu = bu + (pg - bg);
  const size_t r8 = (size_t)8 * H;
  // u of the lane's column at inputs 8(l/16) .. +8 of each 32-input step
  const uint16_t* pa = ws.act_u + (size_t)j.row * H + (lane >> 4) * 8 + (size_t)kb0 * 128;
  const float* psg = sg + (size_t)(j.n0 / 128) * nkbh + kb0;
  const float* psu = su + (size_t)(j.n0 / 128) * nkbh + kb0;
  const int col = lane & 15, g = lane >> 4;

  auto issue = [&](UgStageB& st, int k) {
    const size_t o = (size_t)k * 128;
    st.g0 = ld_nt16(pg + o);
    st.g1 = ld_nt16(pg + r8 + o);
    st.u0 = ld_nt16(pu + o);
    st.u1 = ld_nt16(pu + r8 + o);
#pragma unroll
    for (int s = 0; s < 4; s++) st.a[s] = ld16(pa + o + 32 * s);
    st.sg = psg[k];
    st.su = psu[k];
  };
  auto consume = [&](UgStageB& st) {
    tile_put(tg, lane, st.g0, st.g1);
    tile_put(tu, lane, st.u0, st.u1);
    asm volatile("" ::: "memory");
    v4f cg = {0.f, 0.f, 0.f, 0.f}, cu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const int off = col * kTileStride + 32 * s + 8 * g;
      const v8bf ag = fp8x8_to_bf16(*reinterpret_cast<const uint2*>(tg + off));
      const v8bf au = fp8x8_to_bf16(*reinterpret_cast<const uint2*>(tu + off));
      const v8bf b = __builtin_bit_cast(v8bf, st.a[s]);
      cg = mfma_bf16(ag, b, cg);
      cu = mfma_bf16(au, b, cu);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int v = 0; v < 4; v++) {
      accg[v] = fmaf(cg[v], st.sg, accg[v]);
      accu[v] = fmaf(cu[v], st.su, accu[v]);
    }
  };
  UgStageB st[P];
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
}

// MXFP4 weights: items (pairs of K blocks) it0 .. it0 + ni of the slab.
// E8 (ni <= kUgE8Items): the wave's E8M0 bytes (16 rows x ni x 8 per matrix)
// are loaded once, before its first weight loads, as 8-byte pieces (lane l
// of round r: piece 64r + l, clamped), and kept in its LDS area se8 as
// [matrix][row][item] (measured: the per-item E8M0 loads, four 4-byte loads a
// lane touching 16 rows each, had cost about as much as a tenth of the 8-row
// step); else each item loads its exponents in the ring.
constexpr int kUgE8Items = 8;
template <int P, bool E8>
__device__ __forceinline__ void ug_fp4(const Weights& w, const Ws& ws, const Dims& d, UgJob j,
                                       int it0, int ni, uint8_t* tg, uint8_t* tu, int lane,
                                       float* accg, float* accu, uint8_t* se8) {
  const int H = d.H, nkbh = H / 128;
  const size_t rbytes = H / 2;  // one row of codes
  const size_t ebytes = (size_t)d.I * rbytes, escl = (size_t)d.I * (H / 32);
  const uint8_t* bg = w.gate_c + (size_t)j.e * ebytes;
  const uint8_t* bu = w.up_c + (size_t)j.e * ebytes;
  const uint8_t* eg = reinterpret_cast<const uint8_t*>(w.gate_s) + (size_t)j.e * escl;
  const uint8_t* eu = reinterpret_cast<const uint8_t*>(w.up_s) + (size_t)j.e * escl;
  // lane l loads rows n0 + l/8 and n0 + 8 + l/8, 16-byte chunk l%8 of the
  // item's 128 bytes, and the E8M0 of its MFMA row n0 + l%16 (4 per K block)
  const uint8_t* pg =
      bg + (size_t)(j.n0 + (lane >> 3)) * rbytes + (lane & 7) * 16 + (size_t)it0 * 128;
  const uint8_t* pu = bu + (pg - bg);
  const size_t r8 = 8 * rbytes;
  const uint8_t* peg = eg + (size_t)(j.n0 + (lane & 15)) * (H / 32) + (size_t)it0 * 8;
  const uint8_t* peu = eu + (peg - eg);
  // activation of K block 2i + h: bytes 16(l/16) .. +16 and 64 + 16(l/16) .. +16
  // of the lane's row (the buffer offsets below)
  const float* psa = ws.act_s + (size_t)j.row * nkbh + 2 * it0;
  const int sh = 8 * (lane >> 4);  // the lane's byte of each E8M0 word

  // E8: the wave's exponents, 4 rounds of 64 pieces of 8 bytes (32 ni pieces)
  constexpr int kRounds = kUgE8Items / 2;
  uint2 ev[E8 ? kRounds : 1];
  const int npc = 32 * ni;
  if constexpr (E8) {
#pragma unroll
    for (int r = 0; r < kRounds; r++) {
      int c = r * kWave + lane;
      c = c < npc ? c : npc - 1;
      const int m = c >= 16 * ni, rem = c - m * 16 * ni, row = rem / ni, k = rem - row * ni;
      ev[r] = *reinterpret_cast<const uint2*>((m ? eu : eg) + (size_t)(j.n0 + row) * (H / 32) +
                                              (size_t)(it0 + k) * 8);
    }
    asm volatile("" ::: "memory");  // keep them ahead of the ring's loads
  }
  const uint8_t* pe = se8 + (size_t)(lane & 15) * ni * 8;  // row l%16 of gate; up at +16 ni * 8
  // activation codes through a buffer resource over the step's rows (gfx9
  // raw buffer: stride 0, range d.rows * H bytes): lanes of columns past the
  // expert's using rows take an offset past that range, so their loads return
  // zeros without touching memory (their MFMA columns are never stored).
  // Measured against every lane loading row 0 there: 8 rows 218.3 -> 213.7,
  // 1 row 50.1 -> 49.1 us a step, outputs bitwise equal.
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(ws.act_q), (short)0, d.rows * H, 0x00020000);
  const uint32_t aoff =
      j.live ? (uint32_t)(j.row * H + (lane >> 4) * 16 + it0 * 256) : 0x80000000u;

  auto issue = [&](UgStage4& st, int k) {
    const size_t o = (size_t)k * 128;
    st.g0 = ld_nt16(pg + o);
    st.g1 = ld_nt16(pg + r8 + o);
    st.u0 = ld_nt16(pu + o);
    st.u1 = ld_nt16(pu + r8 + o);
    const int oa = (int)(aoff + (uint32_t)k * 256);
    st.a0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, oa, 0, 0));
    st.a1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, oa + 64, 0, 0));
    st.a2 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, oa + 128, 0, 0));
    st.a3 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, oa + 192, 0, 0));
    if constexpr (!E8) {
      st.eg0 = *reinterpret_cast<const uint32_t*>(peg + 8 * k);
      st.eg1 = *reinterpret_cast<const uint32_t*>(peg + 8 * k + 4);
      st.eu0 = *reinterpret_cast<const uint32_t*>(peu + 8 * k);
      st.eu1 = *reinterpret_cast<const uint32_t*>(peu + 8 * k + 4);
    }
    st.sa0 = psa[2 * k];
    st.sa1 = psa[2 * k + 1];
  };
  auto consume = [&](UgStage4& st, int k) {
    tile_put(tg, lane, st.g0, st.g1);
    tile_put(tu, lane, st.u0, st.u1);
    asm volatile("" ::: "memory");
    uint32_t eg0 = st.eg0, eg1 = st.eg1, eu0 = st.eu0, eu1 = st.eu1;
    if constexpr (E8) {
      const uint2 vg = *reinterpret_cast<const uint2*>(pe + 8 * k);
      const uint2 vu = *reinterpret_cast<const uint2*>(pe + 16 * ni * 8 + 8 * k);
      eg0 = vg.x;
      eg1 = vg.y;
      eu0 = vu.x;
      eu1 = vu.y;
    }
    const v8i b0 = cat8(st.a0, st.a1), b1 = cat8(st.a2, st.a3);
    const v4f cg0 = mfma_fp4_fp8(fp4_operand(tile_get_fp4(tg, lane, 0)), b0, (eg0 >> sh) & 0xFF);
    const v4f cu0 = mfma_fp4_fp8(fp4_operand(tile_get_fp4(tu, lane, 0)), b0, (eu0 >> sh) & 0xFF);
    const v4f cg1 = mfma_fp4_fp8(fp4_operand(tile_get_fp4(tg, lane, 1)), b1, (eg1 >> sh) & 0xFF);
    const v4f cu1 = mfma_fp4_fp8(fp4_operand(tile_get_fp4(tu, lane, 1)), b1, (eu1 >> sh) & 0xFF);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int v = 0; v < 4; v++) {
      accg[v] = fmaf(cg1[v], st.sa1, fmaf(cg0[v], st.sa0, accg[v]));
      accu[v] = fmaf(cu1[v], st.sa1, fmaf(cu0[v], st.sa0, accu[v]));
    }
  };
  // ring of P items (P divides ni)
  UgStage4 st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  if constexpr (E8) {  // the exponents (loaded before the ring) into the wave's area;
    // unconditional (pieces past 32 ni land in slots nothing reads), so that
    // the compiler keeps the loads ahead of the ring instead of sinking one
    // into a branch with a wait for every load in flight
#pragma unroll
    for (int r = 0; r < kRounds; r++)
      *reinterpret_cast<uint2*>(se8 + (size_t)(r * kWave + lane) * 8) = ev[r];
  }
  for (int k0 = 0; k0 < ni - P; k0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p], k0 + p);
      issue(st[p], k0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p], ni - P + p);
}

// 1-bit weights (Q1_0_G128): groups kb0 .. kb0 + nk of the slab (nk a
// multiple of 4, kb0 even).  An item is 4 groups = 2 chunks of 36 bytes per
// row: lane l loads chunk l%2 of row (l%32)/2 of gate (l < 32) or up, 9
// dwords, row-contiguous and nontemporal, and re-aligns it into the wave's
// LDS area (sign dwords and d by chunk, dword and row); then per group the
// lane reads the sign dword l/16 of its MFMA row l%16 for gate and up, builds
// E4M3 +-1 operands from it and runs one FP8 MFMA per matrix against the
// using rows' activation codes; each row's sum is scaled by its group d and
// the activation block scale and accumulated.
// Per wave: the item's activation codes of up to 8 columns (512 bytes each:
// its 4 groups of act_qp) and their 32 block scales, staged through LDS.
constexpr int kUgQ1Bytes = 8 * 512 + 32 * 4;
template <int NA>
struct UgStageQ1 {
  uint32_t w[9];  // the lane's chunk
  u32x4 a[NA];    // 16 bytes of columns 2i + l/32 of the item (act_qp)
  float s;        // scale of column l/4, group l%4 (l < 32)
};
// 1-bit weights: groups kb0 .. kb0 + nk of the slab, items of 4 groups.  The
// activation operand of a lane is 32 bytes a group of its column; loaded by
// each lane from memory that is 9 loads an item (for 16 columns, most of them
// unused), which kept the texture units busy 85% of the launch.  Instead the
// wave loads only its NA pairs of using columns' 512 bytes an item (one
// 16-byte load a lane each) and one scale a lane, parks them in its LDS area
// `sq`, and each lane reads its operands from there.
template <int P, int NA>
__device__ __forceinline__ void ug_q1(const Weights& w, const Ws& ws, const Dims& d, UgJob j,
                                      int kb0, int nk, uint32_t* lds, uint8_t* sq, int lane,
                                      float* accg, float* accu) {
  const int H = d.H, nkbh = H / 128;
  const size_t rb = (size_t)18 * nkbh;  // bytes per row
  const size_t ebytes = (size_t)d.I * rb;
  const int m = lane >> 5, lrow = (lane & 31) >> 1, lq = lane & 1;
  const int col = lane & 15, g = lane >> 4;
  const uint8_t* base = (m ? w.up_c : w.gate_c) + (size_t)j.e * ebytes;
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(base + (size_t)(j.n0 + lrow) * rb) + 9 * (kb0 / 2 + lq);
  // activation codes and block scales through buffer resources over the
  // step's rows: lanes for columns past the expert's using rows take offsets
  // past the range, so their loads return zeros without a memory access
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(ws.act_qp), (short)0, d.rows * H, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ws.act_s), (short)0, d.rows * nkbh * 4, 0x00020000);
  auto crow = [&](int c) { return (int)((j.rows8 >> (8 * c)) & 0xFF); };
  uint32_t aoff[NA];
#pragma unroll
  for (int i = 0; i < NA; i++) {
    const int c = 2 * i + (lane >> 5);
    aoff[i] = c < j.nrows ? (uint32_t)(crow(c) * H + kb0 * 128 + 16 * (lane & 31)) : 0x80000000u;
  }
  const int sc = lane >> 2;
  const uint32_t soff =
      lane < 32 && sc < j.nrows ? (uint32_t)((crow(sc) * nkbh + kb0 + (lane & 3)) * 4) : 0x80000000u;
  const uint32_t m8 = q1_in_vgpr(0x88888888u), o2 = q1_in_vgpr(0x22222222u);
  // the lane's operand column in the staged area (columns past the rows read
  // column 0; their MFMA columns are never stored)
  const int cq = j.live ? col : 0;
  const uint8_t* pa = sq + cq * 512 + 32 * g;
  const float* ps = reinterpret_cast<const float*>(sq + 8 * 512) + 4 * cq;

  auto issue = [&](UgStageQ1<NA>& st, int it) {
    ld_nt_chunk36(src + 18 * it, st.w);
#pragma unroll
    for (int i = 0; i < NA; i++)
      st.a[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff[i] + 512u * it), 0, 0));
    st.s = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(soff + 16u * it), 0, 0));
  };
  auto consume = [&](UgStageQ1<NA>& st) {
    uint32_t u[8], dd;
    q1_chunk_split(st.w, u, &dd);
    const int area = (m * 2 + lq);
#pragma unroll
    for (int i = 0; i < 8; i++) lds[(area * 8 + i) * 16 + lrow] = u[i];
    lds[512 + area * 16 + lrow] = dd;
#pragma unroll
    for (int i = 0; i < NA; i++)
      *reinterpret_cast<u32x4*>(sq + (2 * i + (lane >> 5)) * 512 + 16 * (lane & 31)) = st.a[i];
    if (lane < 32) reinterpret_cast<float*>(sq + 8 * 512)[lane] = st.s;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const u32x4 dg = *reinterpret_cast<const u32x4*>(lds + 512 + (0 * 2 + q) * 16 + 4 * g);
      const u32x4 du = *reinterpret_cast<const u32x4*>(lds + 512 + (1 * 2 + q) * 16 + 4 * g);
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int gi = 2 * q + h;  // group of the item
        const uint32_t wg = lds[((0 * 2 + q) * 8 + 4 * h + g) * 16 + col];
        const uint32_t wu = lds[((1 * 2 + q) * 8 + 4 * h + g) * 16 + col];
        const v8i bv = cat8(*reinterpret_cast<const u32x4*>(pa + 128 * gi),
                            *reinterpret_cast<const u32x4*>(pa + 128 * gi + 16));
        const float sa = ps[gi];
        const v4f cg = mfma_fp4_fp8(q1_fp4_operand(wg, m8, o2), bv);
        const v4f cu = mfma_fp4_fp8(q1_fp4_operand(wu, m8, o2), bv);
#pragma unroll
        for (int v = 0; v < 4; v++) {
          accg[v] = fmaf(cg[v], q1_d(dg[v], h) * sa, accg[v]);
          accu[v] = fmaf(cu[v], q1_d(du[v], h) * sa, accu[v]);
        }
      }
    }
    asm volatile("" ::: "memory");
  };
  const int ni = nk / 4;
  UgStageQ1<NA> st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  for (int k0 = 0; k0 < ni - P; k0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p]);
      issue(st[p], k0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p]);
}

// 1-bit weights, blocks whose 4 waves split K (KS = 4), hidden % 2048 == 0
// and up to 4 using rows: the block's 16 rows are contiguous, so it loads
// them together, a round at a time: round r is items 4r .. 4r+3 (288 bytes of
// each row of gate and of up), loaded by consecutive lanes in consecutive
// 16-byte units (about 11 lines an instruction, against 32-64 when each lane
// fetches 36 bytes of its own row: the per-wave form kept the texture units'
// data path stalled on the cache) into the block's tile area, and wave w takes
// item 4r + w of every row from there while the next round's loads are in
// flight.  Its activations are staged as in ug_q1 (one item ahead).  Pieces
// of a round sit 304 bytes apart in LDS (16-byte aligned; rows on distinct
// banks).
constexpr int kQ1Piece = 304;
constexpr int kQ1Col = 528;  // staged activation columns of the block form
template <int NA>
__device__ __forceinline__ void ug_q1_blk(const Weights& w, const Ws& ws, const Dims& d, UgJob j,
                                          uint8_t* sw, uint8_t* sq, int wv, int lane,
                                          float* accg, float* accu) {
  const int H = d.H, nkbh = H / 128, tid = threadIdx.x;
  const size_t rb = (size_t)18 * nkbh;  // bytes per row
  const size_t ebytes = (size_t)d.I * rb;
  const int col = lane & 15, g = lane >> 4;
  const int R = H / 2048;  // rounds of 4 items
  const uint8_t* bg = w.gate_c + (size_t)j.e * ebytes + (size_t)j.n0 * rb;
  const uint8_t* bu = w.up_c + (size_t)j.e * ebytes + (size_t)j.n0 * rb;
  // this thread's 16-byte units of a round: u = tid + 256 i, piece u / 18
  // (matrix, row), unit u % 18 of its 288 bytes; units past 576 load unit
  // 575 again and are not stored
  const uint8_t* up[3];
  uint32_t lo[3];
  bool uv[3];
#pragma unroll
  for (int i = 0; i < 3; i++) {
    const int u0 = tid + 256 * i;
    uv[i] = u0 < 576;
    const int u = uv[i] ? u0 : 575, pc = u / 18, k = u - pc * 18;
    up[i] = (pc < 16 ? bg : bu) + (size_t)(pc & 15) * rb + 16 * k;
    lo[i] = (uint32_t)(pc * kQ1Piece + 16 * k);
  }
  // activations of the wave's items (as in ug_q1; item q = 4r + wv)
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(ws.act_qp), (short)0, d.rows * H, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ws.act_s), (short)0, d.rows * nkbh * 4, 0x00020000);
  auto crow = [&](int c) { return (int)((j.rows8 >> (8 * c)) & 0xFF); };
  uint32_t aoff[NA];
#pragma unroll
  for (int i = 0; i < NA; i++) {
    const int c = 2 * i + (lane >> 5);
    aoff[i] = c < j.nrows ? (uint32_t)(crow(c) * H + 16 * (lane & 31)) : 0x80000000u;
  }
  const int sc = lane >> 2;
  const uint32_t soff =
      lane < 32 && sc < j.nrows ? (uint32_t)((crow(sc) * nkbh + (lane & 3)) * 4) : 0x80000000u;
  const uint32_t m8 = q1_in_vgpr(0x88888888u), o2 = q1_in_vgpr(0x22222222u);
  // the wave's area: up to 4 staged columns 528 bytes apart (distinct banks
  // for the lanes of different columns), their 32 scales, then the d table of
  // the wave's item: entry (group gi, matrix m, row n) at float 32 gi + 16 m + n
  const int cq = j.live ? col : 0;
  const uint8_t* pa = sq + cq * kQ1Col + 32 * g;
  float* sst = reinterpret_cast<float*>(sq + 4 * kQ1Col);
  const float* ps = sst + 4 * cq;
  float* dt = sst + 32;

  u32x4 wr[3];
  u32x4 av[NA];
  float sv;
  auto issue = [&](int r) {
#pragma unroll
    for (int i = 0; i < 3; i++) wr[i] = ld_nt16(up[i] + 288 * r);
    const uint32_t q = (uint32_t)(4 * r + wv);  // the wave's item
#pragma unroll
    for (int i = 0; i < NA; i++)
      av[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)(aoff[i] + 512u * q), 0, 0));
    sv = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(soff + 16u * q), 0, 0));
  };
  issue(0);
  for (int r = 0; r < R; r++) {
    if (r > 0) __syncthreads();  // the previous round is consumed
#pragma unroll
    for (int i = 0; i < 3; i++)
      if (uv[i]) *reinterpret_cast<u32x4*>(sw + lo[i]) = wr[i];
#pragma unroll
    for (int i = 0; i < NA; i++)
      *reinterpret_cast<u32x4*>(sq + (2 * i + (lane >> 5)) * kQ1Col + 16 * (lane & 31)) = av[i];
    if (lane < 32) sst[lane] = sv;
    __syncthreads();
    if (r + 1 < R) issue(r + 1);
    // item 4r + wv: 72 bytes at 72 wv of every piece; group gi at 18 gi (its
    // fp16 d, then 16 sign bytes).  The wave's 128 d values first go to its
    // table (two a lane), so a lane reads its 4 output rows' d in one load.
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const int e = lane + 64 * k, gi = e >> 5, pc = e & 31;  // pc = 16 m + n
      dt[e] = q1_d(*reinterpret_cast<const uint16_t*>(sw + pc * kQ1Piece + 72 * wv + 18 * gi), 0);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int gi = 0; gi < 4; gi++) {
      const int go = 72 * wv + 18 * gi;  // even gi: go % 4 == 0, odd: 2
      uint32_t wg, wu;
      {
        const int so = go + 2 + 4 * g;  // sign dword g: % 4 == 2 for even gi
        const uint8_t* pg = sw + col * kQ1Piece;
        const uint8_t* pu = sw + (16 + col) * kQ1Piece;
        if (gi % 2 == 0) {
          wg = __builtin_amdgcn_alignbyte(*reinterpret_cast<const uint32_t*>(pg + so + 2),
                                          *reinterpret_cast<const uint32_t*>(pg + so - 2), 2);
          wu = __builtin_amdgcn_alignbyte(*reinterpret_cast<const uint32_t*>(pu + so + 2),
                                          *reinterpret_cast<const uint32_t*>(pu + so - 2), 2);
        } else {
          wg = *reinterpret_cast<const uint32_t*>(pg + so);
          wu = *reinterpret_cast<const uint32_t*>(pu + so);
        }
      }
      const v8i bv = cat8(*reinterpret_cast<const u32x4*>(pa + 128 * gi),
                          *reinterpret_cast<const u32x4*>(pa + 128 * gi + 16));
      const float sa = ps[gi];
      const v4f cg = mfma_fp4_fp8(q1_fp4_operand(wg, m8, o2), bv);
      const v4f cu = mfma_fp4_fp8(q1_fp4_operand(wu, m8, o2), bv);
      const v4f dg = *reinterpret_cast<const v4f*>(dt + 32 * gi + 4 * g);
      const v4f du = *reinterpret_cast<const v4f*>(dt + 32 * gi + 16 + 4 * g);
#pragma unroll
      for (int v = 0; v < 4; v++) {
        accg[v] = fmaf(cg[v], dg[v] * sa, accg[v]);
        accu[v] = fmaf(cu[v], du[v] * sa, accu[v]);
      }
    }
    asm volatile("" ::: "memory");  // this item's table reads before the next round's writes
  }
  __syncthreads();  // every wave is done with the tile area before the K-part sums
}

typedef uint8_t UgTiles[4][2][kTileBytes];  // per wave: gate and up weight tiles
constexpr int kUgE8Bytes = 32 * kUgE8Items * 8;  // per wave: MXFP4 exponents (ug_fp4, E8)
// LDS of the block's per-wave areas: MXFP4 exponents, 1-bit staged activations
// (4 waves; a token size for FP8)
template <int RF>
constexpr int ug_e8_lds() {
  return RF == kFmtMxfp4 ? 4 * kUgE8Bytes : (RF == kFmtQ1 ? 4 * kUgQ1Bytes : 16);
}

// Items in flight per wave, dividing the wave's items: FP8 K blocks the
// largest of 4, 2, 1 (ring_depth); in MXFP4 and 1-bit layers, where more
// waves a SIMD pay more than deeper rings, at most 2 (launch_upgate).
inline int ring_depth(int nk) { return nk % 4 == 0 ? 4 : (nk % 2 == 0 ? 2 : 1); }
inline int ring_depth2(int ni) { return ni % 2 == 0 ? 2 : 1; }

// Up/gate block `rb` of moe_route_kernel waits for its record: lane 0 of wave
// 0 polls it with relaxed agent-scope loads, a short sleep between them, until
// the routing block has published it (bit 0), clears it for the next launch
// and hands it to the block through LDS.  The wait ends after d.wait_ticks of
// the 100 MHz real-time counter at most: then the block gets 0, and when
// `count` (a routed block, which can do no work without its record) it counts
// itself in ws.wait_timeouts.  Runs with every thread of the block (it ends
// with a barrier).
__device__ __forceinline__ uint64_t await_record(const Ws& ws, const Dims& d, int rb,
                                                 bool count, uint64_t* s_rec) {
  if (threadIdx.x == 0) {
    uint64_t* p = ws.blk_rec + rb;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint64_t rec = 0;
    for (;;) {
      rec = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (rec & 1u) {
        __hip_atomic_store(p, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > d.wait_ticks) {
        if (count)
          __hip_atomic_fetch_add(ws.wait_timeouts, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        rec = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *s_rec = rec;
  }
  __syncthreads();
  return *s_rec;
}

// Up/gate block number `blk` of the numbering above (the shared expert's
// slabs, then those of each routed group), with 256 threads.  WAIT (the
// routing launch): a shared block first waits for the routing block's go
// (its record; past the cap it streams anyway), a routed block takes its
// group from its record; else the routed blocks read the published table.
template <int RF, int P, int P4, bool AB, bool WAIT>
__device__ __forceinline__ void upgate_block(const Weights& w, const Ws& ws, const Dims& d,
                                             int blk, UgTiles& s_tile, uint8_t* s_e8,
                                             uint64_t* s_rec) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int KS = d.ks;
  const int spb = 4 / KS;  // slabs per block
  const int col = lane & 15;

  // ---- the block's expert and slab
  const int nb_sh = d.Is / (16 * spb);
  int b = blk, g = -1, nrows, row, e;
  uint64_t rows8 = 0, picks8 = 0;  // using rows, and the pick of each row (routed)
  if (b < nb_sh) {
    nrows = d.rows;
    row = col < nrows ? col : 0;
    e = -1;
    if constexpr (WAIT) await_record(ws, d, b, false, s_rec);
  } else {
    b -= nb_sh;
    const int per = d.I / (16 * spb);
    g = b / per;
    if constexpr (WAIT) {
      const uint64_t rec = await_record(ws, d, nb_sh + b, true, s_rec);
      nrows = (int)((rec >> 11) & 15u);
      e = (int)((rec >> 1) & 1023u);
      if (nrows == 0 || e >= d.E) return;  // no such group this step, or no record
#pragma unroll
      for (int c = 0; c < 8; c++) {
        rows8 |= ((rec >> (15 + 3 * c)) & 7u) << (8 * c);
        picks8 |= ((rec >> (39 + 3 * c)) & 7u) << (8 * c);
      }
    } else {
      // one round of independent loads; the table of a group past D is stale
      // but in bounds, and unused
      const int D = *ws.n_groups;
      e = ws.grp_expert[g];
      nrows = ws.grp_nrows[g];
      rows8 = *reinterpret_cast<const uint64_t*>(ws.grp_rows + g * 8);
      picks8 = *reinterpret_cast<const uint64_t*>(ws.grp_slot + g * 8);
      if (g >= D) return;
    }
    b -= g * per;
    row = col < nrows ? (int)((rows8 >> (8 * (col & 7))) & 0xFF) : 0;
  }
  const int slab = b * spb + wv / KS, kp = wv % KS;
  const UgJob j{e, row, slab * 16, col < nrows, nrows, rows8};
  float accg[4] = {0.f, 0.f, 0.f, 0.f}, accu[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (AB) {  // bf16 activations (FP8 weights only)
    const int nk = d.H / 128 / KS;
    ug_fp8_bf16a<P>(w, ws, d, j, kp * nk, nk, s_tile[wv][0], s_tile[wv][1], lane, accg, accu);
  } else if (RF == kFmtMxfp4 && e >= 0) {
    const int ni = d.H / 256 / KS;  // items of two K blocks per part
    if (ni <= kUgE8Items)
      ug_fp4<P4, true>(w, ws, d, j, kp * ni, ni, s_tile[wv][0], s_tile[wv][1], lane, accg, accu,
                       s_e8 + wv * kUgE8Bytes);
    else
      ug_fp4<P4, false>(w, ws, d, j, kp * ni, ni, s_tile[wv][0], s_tile[wv][1], lane, accg, accu,
                        s_e8 + wv * kUgE8Bytes);
  } else if (RF == kFmtQ1 && e >= 0) {
    const int nk = d.H / 128 / KS;  // groups per part, a multiple of 4
    uint32_t* tl = reinterpret_cast<uint32_t*>(s_tile[wv][0]);
    uint8_t* sq = s_e8 + wv * kUgQ1Bytes;
    if (KS == 4 && d.H % 2048 == 0 && nrows <= 4) {  // block-uniform
      uint8_t* sw = &s_tile[0][0][0];
      if (nrows <= 2)
        ug_q1_blk<1>(w, ws, d, j, sw, sq, wv, lane, accg, accu);
      else
        ug_q1_blk<2>(w, ws, d, j, sw, sq, wv, lane, accg, accu);
    } else if (nrows <= 2)
      ug_q1<P4, 1>(w, ws, d, j, kp * nk, nk, tl, sq, lane, accg, accu);
    else if (nrows <= 4)
      ug_q1<P4, 2>(w, ws, d, j, kp * nk, nk, tl, sq, lane, accg, accu);
    else  // 5 to 8 using rows (rare): one item in flight
      ug_q1<1, 4>(w, ws, d, j, kp * nk, nk, tl, sq, lane, accg, accu);
  } else {
    const int nk = d.H / 128 / KS;
    ug_fp8<P>(w, ws, d, j, kp * nk, nk, s_tile[wv][0], s_tile[wv][1], lane, accg, accu);
  }
  pin4(accg);  // the MFMAs run with every lane, before any divergent use
  pin4(accu);

  // ---- K parts -> mid.  Each wave parks its 16 x 16 sums of gate and of up
  // in its own (finished) tile, column-major: element (n, c) at c*16 + n.
  float* part = reinterpret_cast<float*>(s_tile[wv][0]);
  *reinterpret_cast<v4f*>(part + col * 16 + 4 * (lane >> 4)) = v4f{accg[0], accg[1], accg[2], accg[3]};
  *reinterpret_cast<v4f*>(part + 256 + col * 16 + 4 * (lane >> 4)) =
      v4f{accu[0], accu[1], accu[2], accu[3]};
  __syncthreads();
  // thread t: element n = t%16 of column c = t/16, for each slab of the block
  const int c = tid >> 4, n = tid & 15;
  if (c >= nrows) return;
  const int r = g < 0 ? c : (int)((rows8 >> (8 * c)) & 0xFF);
  const int pick = g < 0 ? 8 : (int)((picks8 >> (8 * r)) & 0xFF);
  const float rs = ws.rstd[r];
  float* mrow = ws.mid + (size_t)(r * 9 + pick) * d.imax;
  for (int s = 0; s < spb; s++) {
    const float* p0 = reinterpret_cast<const float*>(s_tile[s * KS][0]);
    float gs = p0[tid], us = p0[256 + tid];
    for (int q = 1; q < KS; q++) {  // parts in order
      const float* pq = reinterpret_cast<const float*>(s_tile[s * KS + q][0]);
      gs += pq[tid];
      us += pq[256 + tid];
    }
    const float gt = gs * rs, ut = us * rs;
    mrow[(b * spb + s) * 16 + n] = gt / (1.0f + expf(-gt)) * ut;
  }
}

}  // namespace moe
