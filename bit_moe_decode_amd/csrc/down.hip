// down.hip -- down GEMV of the shared expert and of every distinct routed
// expert from mid, per (row, pick); then the gate-weighted combine.
//
// #85 Mod. row 16: down units take one expert's tile against every row that
// uses it, and each row adds its units up in the order a lone row would,
// so dedup changes no output bit.  Mod. row 1: down reads mid as FP8
// bytes with one fp32 scale per 1x128 block, quantised once per (row, pick)
// and expert.  Mod. rows 18 and 21: 16-byte, nontemporal weight loads.
//
// moe_down_kernel: block = WPB waves of T 16-row tiles each = 16 * WPB * T
// output rows of one expert (the shared expert's blocks first, then those of
// each of the step's possible routed groups; blocks of groups past the step's
// D exit at once).  Many small blocks let the hardware dispatcher even out the
// load per CU: WPB = 2, T = 1 for FP8 steps of one or two rows, where larger
// blocks would leave some CUs with a block more than others (a CU streams at
// most about 1/256 of the chip's bandwidth); else WPB = 4.
//
// FP8 experts.  The block first puts the first K blocks of its weight stream
// in flight, then quantises the fp32 mid of each of its columns (one per row
// that uses the expert) into LDS: per 1x128 block s = amax / 448 (fp32) and
// codes = E4M3(mid / s) by the hardware's round-to-nearest-even conversion, an
// all-zero block giving s = 0 and zero codes.  Every block of an expert does
// this the same way, so all use the same bytes; the first block also stores
// them as the step's midq / midqs.  A wave then owns 16 output rows over the
// whole K (from 3 rows, two tiles of 16: each read of the mid codes from LDS
// then serves 32 rows): for each 128-wide K block it loads its weight rows
// row-contiguously, re-lays each tile through LDS into MFMA operand order and
// runs one 16x16x128 FP8 MFMA per tile against the mid codes, scaled by weight
// scale x mid scale and accumulated in fp32.  It stores y[row, pick][h]; every
// (row, pick) belongs to exactly one expert of the step, so no two writes
// collide.
//
// MXFP4 routed experts (mid kept in fp32, as the oracle does): the block
// splits its columns' mid into bf16 hi + lo (mid = hi + lo to about 2^-17) in
// LDS; a wave streams its rows in whole 128-byte lines (256 inputs; half
// lines when I % 256 != 0), converts each lane's 8 E2M1 weights of an MFMA
// step to bf16 with the hardware's scaled conversion (the lane's E8M0 as the
// scale) and runs two 16x16x32 bf16 MFMAs, one against hi and one against
// lo, accumulating in fp32.  From 3 rows a wave
// takes two 16-row tiles, so that each LDS read of the mid operand serves
// both (the block's LDS, 4 bytes per mid element and column, then allows only
// two or three blocks a CU).
//
// moe_combine_kernel:
//   out[r][h] = bf16( sum_{j<8} g_rj * y_rj[h] + y_r8[h] )
// in pick order, the same arithmetic whether or not experts were deduplicated.
#include "device_common.h"

namespace moe {

template <int TF>
struct DnStage {
  u32x4 w0[TF], w1[TF];  // rows l/8 and 8 + l/8 of each 16-row tile
  float sd;              // weight block scale (the tiles share a 128-row block)
};

// Dynamic LDS of the down kernel: mid codes of each column (row stride
// I + 16 bytes, so that the columns of one MFMA read start on different
// banks), then their scales.
__host__ __device__ inline int dn_code_stride(int inter) { return inter + 16; }
__host__ __device__ inline size_t dn_lds_bytes(int rows, int inter) {
  return (size_t)rows * dn_code_stride(inter) + (size_t)rows * (inter / 128) * 4;
}

// The (row, pick) index u = row * 9 + pick of column c of a block: the shared
// expert's columns are the rows in order (pick 8); a routed group's are its
// using rows (`rows8`, one byte each) with their picks (`picks8`, byte per row).
struct DnCols {
  int g;  // -1: shared expert
  uint64_t rows8, picks8;
  __device__ __forceinline__ int u(int c) const {
    if (g < 0) return c * 9 + 8;
    const int r = (int)((rows8 >> (8 * c)) & 0xFF);
    return r * 9 + (int)((picks8 >> (8 * r)) & 0xFF);
  }
};

// Four fp32 -> four E4M3FN bytes (hardware conversion, round to nearest even).
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float e) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, e, lo, true);
}

// Quantises the fp32 mid of the block's columns into LDS, per 1x128 block:
// half-wave h of the block's n halves takes blocks h, h + n, ..., 4 values a
// lane.  The
// first block of an expert (`publish`) also stores codes and scales as the
// step's midq / midqs.
__device__ __forceinline__ void dn_quant_mid(const Ws& ws, const Dims& d, int nrows,
                                             const DnCols& cols, bool publish, uint8_t* s_q,
                                             float* s_qs, bool q1_order = false) {
  const int tid = threadIdx.x, hw = tid >> 5, l = tid & 31, nhw = blockDim.x >> 5;
  const int nkb = d.I / 128, cs = dn_code_stride(d.I), T = nrows * nkb;
  for (int t = hw; t < T; t += nhw) {
    const int c = t / nkb, kb = t - c * nkb;
    const int uc = cols.u(c);
    const size_t src = (size_t)uc * d.imax + kb * 128 + 4 * l;
    const v4f v = *reinterpret_cast<const v4f*>(ws.mid + src);
    uint32_t m = max(max(__float_as_uint(fabsf(v[0])), __float_as_uint(fabsf(v[1]))),
                     max(__float_as_uint(fabsf(v[2])), __float_as_uint(fabsf(v[3]))));
    m = row16_umax(m);
    m = max(m, (uint32_t)__shfl_xor((int)m, 16, kWave));
    const float s = __uint_as_float(m) / 448.0f;
    const uint32_t q = s > 0.f ? f32x4_to_e4m3(v[0] / s, v[1] / s, v[2] / s, v[3] / s) : 0u;
    if (!q1_order) {
      *reinterpret_cast<uint32_t*>(s_q + c * cs + kb * 128 + 4 * l) = q;
    } else {
      // the 1-bit operand order of the block (as the router's act_qp): code
      // 4l + j sits at the B byte of K h = 32(l/8) + 8j + l%8
      uint8_t* qb = s_q + c * cs + kb * 128;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int h = 32 * (l >> 3) + 8 * j + (l & 7);
        const int pos = h < 64 ? 32 * (h >> 4) + (h & 15) : 32 * ((h - 64) >> 4) + 16 + (h & 15);
        qb[pos] = (uint8_t)(q >> (8 * j));
      }
    }
    if (l == 0) s_qs[c * nkb + kb] = s;
    if (publish) {
      *reinterpret_cast<uint32_t*>(ws.midq + src) = q;
      if (l == 0) ws.midqs[(size_t)uc * (d.imax / 128) + kb] = s;
    }
  }
}

typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// 2^(e-127) as fp32 for an E8M0 code (0xFF, NaN, is not produced by the
// generator; it decodes to a NaN here as well).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  uint32_t b = e << 23;
  b = e == 0 ? 0x00400000u : b;
  b = e == 255 ? 0x7FC00000u : b;
  return __uint_as_float(b);
}

// LDS of an MXFP4 block's mid columns: per column, K bf16 "hi" values then K
// bf16 "lo" values (mid = hi + lo to about 2^-17), the column stride padded by
// 32 bytes so that the columns of one MFMA read start on different banks.
__host__ __device__ inline int dn4_col_stride(int inter) { return 4 * inter + 32; }
__host__ __device__ inline size_t dn4_lds_bytes(int rows, int inter) {
  return (size_t)rows * dn4_col_stride(inter);
}


// The MXFP4 down GEMV of one wave: output rows h0 .. h0 + 16*T of routed
// expert e over the whole K, against the block's nrows mid columns (fp32 mid,
// unquantised, split into bf16 hi + lo in LDS by the block).  This form, for
// I % 256 != 0, takes half-line items: item k = the 128 inputs 128k .. +128
// of every row (64 bytes a row): per tile, lane L
// loads row L/4, 16-byte chunk L%4 (row-contiguous), re-laid through the
// wave's LDS tile into MFMA operand order; then per 32 inputs (one E8M0
// block) lane l converts 8 E2M1 of row l%16 to bf16 scaled by 2^(E8M0-127)
// (v_cvt_scalef32_pk_bf16_fp4) and runs two 16x16x32 bf16 MFMAs per tile,
// against the hi and the lo parts of mid.  The mid operand is read from LDS
// once per 32 inputs for all T tiles.
template <int P, int T>
__device__ __forceinline__ void down_fp4_wave(const Weights& w, const Dims& d, int e, int nrows,
                                              int h0, uint8_t* tile, const uint8_t* smid,
                                              const float* e8tab, float (*acc)[4]) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const int H = d.H, I = d.I, nki = I / 128;
  const size_t rbytes = I / 2, ebytes = I / 32;
  const uint8_t* wrow = w.down_c + ((size_t)e * H + h0 + (lane >> 2)) * rbytes + (lane & 3) * 16;
  const uint8_t* erow =
      reinterpret_cast<const uint8_t*>(w.down_s) + ((size_t)e * H + h0 + col) * ebytes;
  const int cc = col < nrows ? col : 0;  // columns past the rows reuse column 0
  const uint8_t* mh = smid + cc * dn4_col_stride(I) + 16 * g;  // hi of K 8g.. of a 32-step
  const uint8_t* ml = mh + 2 * I;                               // lo
  struct It {
    u32x4 w[T];
    uint32_t e[T];
  };
  auto issue = [&](It& s, int k) {
#pragma unroll
    for (int t = 0; t < T; t++) {
      s.w[t] = ld_nt16(wrow + (size_t)t * 16 * rbytes + (size_t)k * 64);
      s.e[t] = *reinterpret_cast<const uint32_t*>(erow + (size_t)t * 16 * ebytes + 4 * k);
    }
  };
  v4f c[T];
#pragma unroll
  for (int t = 0; t < T; t++) c[t] = v4f{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](It& s, int k) {
    uint32_t a4[T][4];
#pragma unroll
    for (int t = 0; t < T; t++) {  // re-lay each tile through the wave's LDS tile
      *reinterpret_cast<u32x4*>(tile + (lane >> 2) * kTileStride + (lane & 3) * 16) = s.w[t];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int st = 0; st < 4; st++)
        a4[t][st] = *reinterpret_cast<const uint32_t*>(tile + col * kTileStride + 16 * st + 4 * g);
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int st = 0; st < 4; st++) {
      const int ko = 2 * (128 * k + 32 * st);
      const v8bf bh = *reinterpret_cast<const v8bf*>(mh + ko);
      const v8bf bl = *reinterpret_cast<const v8bf*>(ml + ko);
#pragma unroll
      for (int t = 0; t < T; t++) {
        const float sc = e8tab[__builtin_amdgcn_ubfe(s.e[t], 8 * st, 8)];
        const v2bf_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a4[t][st], sc, 0);
        const v2bf_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a4[t][st], sc, 1);
        const v2bf_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a4[t][st], sc, 2);
        const v2bf_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a4[t][st], sc, 3);
        const v8bf a = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        c[t] = mfma_bf16(a, bh, c[t]);
        c[t] = mfma_bf16(a, bl, c[t]);
      }
    }
  };
  // ring of P items (P divides I/128): every issued load is used
  It st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  for (int k0 = 0; k0 < nki - P; k0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p], k0 + p);
      issue(st[p], k0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p], nki - P + p);
#pragma unroll
  for (int t = 0; t < T; t++) {
    acc[t][0] = c[t][0];
    acc[t][1] = c[t][1];
    acc[t][2] = c[t][2];
    acc[t][3] = c[t][3];
  }
}

// The same GEMV with whole-line items (I % 256 == 0), which stream faster
// than half lines: item k = the 256 inputs 256k .. +256 of every row (a
// 128-byte line a row).  Per tile, lane L loads rows L/8 and 8 + L/8, 16-byte
// chunk L%8 (row-contiguous, as the FP8 path), re-laid through the wave's LDS
// tile; lane l then reads the 16 bytes of row l%16 at 64h + 16(l/16), h = 0, 1:
// the 32 inputs of E8M0 block 4h + l/16 of the item.  The item's 8 MFMA steps
// give each lane 8 of those 32 inputs in turn (step 4h + j: inputs 8j .. +8),
// so the 32 K terms of one step come from four E8M0 blocks, each lane
// converting its own 8 with its own block's exponent; the mid operand is read
// at the same K indices, so the sum is the same set of products.
template <int P, int T, typename Pro>
__device__ __forceinline__ void down_fp4_wave_line(const Weights& w, const Dims& d, int e,
                                                   int nrows, int h0, uint8_t* tile,
                                                   const uint8_t* smid, const float* e8tab,
                                                   float (*acc)[4], Pro pro) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const int H = d.H, I = d.I, nki = I / 256;
  const size_t rbytes = I / 2, ebytes = I / 32, r8 = 8 * rbytes;
  const uint8_t* wrow = w.down_c + ((size_t)e * H + h0 + (lane >> 3)) * rbytes + (lane & 7) * 16;
  const uint8_t* erow =
      reinterpret_cast<const uint8_t*>(w.down_s) + ((size_t)e * H + h0 + col) * ebytes;
  const int cc = col < nrows ? col : 0;  // columns past the rows reuse column 0
  const uint8_t* mh = smid + cc * dn4_col_stride(I) + 64 * g;  // hi at inputs 32g of each 128
  const uint8_t* ml = mh + 2 * I;                               // lo
  struct It {
    u32x4 w0[T], w1[T];
    uint2 e[T];  // the 8 E8M0 of the lane's MFMA row in the item
  };
  auto issue = [&](It& s, int k) {
#pragma unroll
    for (int t = 0; t < T; t++) {
      const uint8_t* p = wrow + (size_t)t * 16 * rbytes + (size_t)k * 128;
      s.w0[t] = ld_nt16(p);
      s.w1[t] = ld_nt16(p + r8);
      s.e[t] = *reinterpret_cast<const uint2*>(erow + (size_t)t * 16 * ebytes + 8 * k);
    }
  };
  v4f c[T];
#pragma unroll
  for (int t = 0; t < T; t++) c[t] = v4f{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](It& s, int k) {
    u32x4 a4[T][2];
#pragma unroll
    for (int t = 0; t < T; t++) {  // re-lay each tile through the wave's LDS tile
      tile_put(tile, lane, s.w0[t], s.w1[t]);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int h = 0; h < 2; h++)
        a4[t][h] = *reinterpret_cast<const u32x4*>(tile + col * kTileStride + 64 * h + 16 * g);
      asm volatile("" ::: "memory");
    }
    // the item's exponents are used here, not earlier: without this the
    // compiler hoisted every ring item's extraction to the top of the loop,
    // which waited for all loads in flight (the ring drained each round)
    uint2 ev[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
      ev[t] = s.e[t];
      asm volatile("" : "+v"(ev[t].x), "+v"(ev[t].y));
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      float sc[T];
#pragma unroll
      for (int t = 0; t < T; t++) sc[t] = e8tab[__builtin_amdgcn_ubfe(h ? ev[t].y : ev[t].x, 8 * g, 8)];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int ko = 512 * k + 256 * h + 16 * j;
        const v8bf bh = *reinterpret_cast<const v8bf*>(mh + ko);
        const v8bf bl = *reinterpret_cast<const v8bf*>(ml + ko);
#pragma unroll
        for (int t = 0; t < T; t++) {
          const uint32_t q = a4[t][h][j];
          const v2bf_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc[t], 0);
          const v2bf_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc[t], 1);
          const v2bf_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc[t], 2);
          const v2bf_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sc[t], 3);
          const v8bf a = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          c[t] = mfma_bf16(a, bh, c[t]);
          c[t] = mfma_bf16(a, bl, c[t]);
        }
      }
    }
  };
  // ring of P items (P divides I/256): every issued load is used
  It st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  pro();  // the block's mid split and barrier, with the first items in flight
  for (int k0 = 0; k0 < nki - P; k0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p], k0 + p);
      issue(st[p], k0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p], nki - P + p);
#pragma unroll
  for (int t = 0; t < T; t++) {
    acc[t][0] = c[t][0];
    acc[t][1] = c[t][1];
    acc[t][2] = c[t][2];
    acc[t][3] = c[t][3];
  }
}

// The block's mid columns as bf16 hi + lo: hi = bf16(m), lo = bf16(m - hi)
// (m - hi is exact in fp32), 4 values a thread per pass.
__device__ __forceinline__ void dn4_store_split(uint8_t* smid, int I, int c, int k, const v4f& m) {
  uint16_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    hi[i] = f32_to_bf16(m[i]);
    lo[i] = f32_to_bf16(m[i] - bf16_to_f32(hi[i]));
  }
  uint8_t* p = smid + c * dn4_col_stride(I) + 2 * k;
  *reinterpret_cast<uint2*>(p) = uint2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
  *reinterpret_cast<uint2*>(p + 2 * I) =
      uint2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
}
__device__ __forceinline__ void dn4_split_mid(const Ws& ws, const Dims& d, int nrows,
                                              const DnCols& cols, uint8_t* smid) {
  const int I = d.I, n4 = I / 4;
  for (int t = threadIdx.x; t < nrows * n4; t += blockDim.x) {
    const int c = t / n4, k = 4 * (t - c * n4);
    dn4_store_split(smid, I, c, k,
                    *reinterpret_cast<const v4f*>(ws.mid + (size_t)cols.u(c) * d.imax + k));
  }
}

// The 1-bit down GEMV of one wave: output rows h0 .. h0 + 16 of routed expert
// e over the whole K (I <= 4096: up to 4 items of 4 chunks), against the
// block's FP8 mid codes in LDS (pm: the lane's column at inputs 32(l/16) ..,
// psm: that column's block scales).  Item i = chunks 4i .. 4i+3 of every row:
// lane l loads chunk 4i + l%4 of row h0 + l/4 (9 dwords, nontemporal; lanes
// past the row's chunks load chunk 0 and do not use it), all items at once,
// before the block quantises mid.  Per item the chunks are re-aligned into the
// wave's LDS tile; per group the lane reads sign dword l/16 of its MFMA row
// l%16, builds E4M3 +-1 operands and runs one FP8 MFMA against the mid codes;
// each row's sum is scaled by its group d and the mid block scale.
struct DnQ1Items {
  uint32_t w[4][9];
};
__device__ __forceinline__ void down_q1_issue(const Weights& w, const Dims& d, int e, int h0,
                                              DnQ1Items& it) {
  const int lane = threadIdx.x & 63, I = d.I;
  const size_t rb = (size_t)18 * (I / 128);
  const int nchunk = I / 256;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(
      w.down_c + ((size_t)e * d.H + h0 + (lane >> 2)) * rb);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (4 * i < nchunk) {  // wave-uniform
      const int c = 4 * i + (lane & 3);
      ld_nt_chunk36(row + 9 * (c < nchunk ? c : 0), it.w[i]);
    }
  }
}
__device__ __forceinline__ void down_q1_consume(const Dims& d, const DnQ1Items& it,
                                                uint32_t* lds, const uint8_t* pm,
                                                const float* psm, float* acc) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const int lrow = lane >> 2, lq = lane & 3;
  const int nchunk = d.I / 256;
  const uint32_t m8 = q1_in_vgpr(0x88888888u), o2 = q1_in_vgpr(0x22222222u);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (4 * i >= nchunk) break;  // wave-uniform
    uint32_t u[8], dd;
    q1_chunk_split(it.w[i], u, &dd);
#pragma unroll
    for (int q = 0; q < 8; q++) lds[(lq * 8 + q) * 16 + lrow] = u[q];
    lds[512 + lq * 16 + lrow] = dd;
    asm volatile("" ::: "memory");
    const int nc = nchunk - 4 * i < 4 ? nchunk - 4 * i : 4;
    for (int q = 0; q < nc; q++) {
      const u32x4 dv = *reinterpret_cast<const u32x4*>(lds + 512 + q * 16 + 4 * g);
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int kb = 2 * (4 * i + q) + h;  // group = mid block
        const uint32_t ws = lds[(q * 8 + 4 * h + g) * 16 + col];
        const v4f c = mfma_fp4_fp8(q1_fp4_operand(ws, m8, o2),
                                   cat8(ld16(pm + kb * 128), ld16(pm + kb * 128 + 16)));
        const float sm = psm[kb];
#pragma unroll
        for (int v = 0; v < 4; v++) acc[v] = fmaf(c[v], q1_d(dv[v], h) * sm, acc[v]);
      }
    }
    asm volatile("" ::: "memory");
  }
}

// 1-bit routed down when I % 1024 == 0: a wave's 16 output rows are
// contiguous, so it loads them in octets of 8 groups (144 bytes a row, 2304
// bytes a wave: 144 consecutive 16-byte units, lane l taking units l, l + 64
// and l + 128) instead of 36-byte chunks of 16 rows a load, parks each octet
// in its tile (rows 144 bytes = 36 dwords apart: distinct banks) and reads its
// MFMA operands from there; two octets are in flight (octets past K load the
// last one again and are not used).
struct DnQ1Oct {
  u32x4 v[3];
};
__device__ __forceinline__ void dn_q1_oct_load(const uint8_t* wb, size_t rb, int o, int lane,
                                               DnQ1Oct& t) {
#pragma unroll
  for (int i = 0; i < 3; i++) {
    int u = lane + 64 * i;
    u = u < 144 ? u : 143;
    const int row = u / 9, k = u - row * 9;
    t.v[i] = ld_nt16(wb + (size_t)row * rb + 144 * o + 16 * k);
  }
}
__device__ __forceinline__ void dn_q1_oct_consume(const DnQ1Oct& t, uint8_t* tile, int o,
                                                  const uint8_t* pm, const float* psm,
                                                  uint32_t m8, uint32_t o2, float* acc) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 3; i++)
    if (lane + 64 * i < 144) *reinterpret_cast<u32x4*>(tile + 16 * (lane + 64 * i)) = t.v[i];
  asm volatile("" ::: "memory");
#pragma unroll
  for (int gi = 0; gi < 8; gi++) {
    const int go = 18 * gi;  // the group's d, then its 16 sign bytes
    const int so = go + 2 + 4 * g;
    const uint8_t* pr = tile + col * 144;
    const uint32_t ws = gi % 2 == 0
                            ? __builtin_amdgcn_alignbyte(*reinterpret_cast<const uint32_t*>(pr + so + 2),
                                                         *reinterpret_cast<const uint32_t*>(pr + so - 2), 2)
                            : *reinterpret_cast<const uint32_t*>(pr + so);
    const int kb = 8 * o + gi;  // group = mid block
    const v4f c = mfma_fp4_fp8(q1_fp4_operand(ws, m8, o2),
                               cat8(ld16(pm + kb * 128), ld16(pm + kb * 128 + 16)));
    const float sm = psm[kb];
    const int dq = go & ~3, dh = (go & 2) * 8;
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const uint32_t dw = *reinterpret_cast<const uint32_t*>(tile + (4 * g + v) * 144 + dq);
      acc[v] = fmaf(c[v], q1_d(dw >> dh, 0) * sm, acc[v]);
    }
  }
  asm volatile("" ::: "memory");  // this octet's reads before the next octet's writes
}

// (1-bit layers' down blocks held to 4 waves a SIMD: their octet loads need
// more registers than the one-row step pays for in occupancy)
template <int RF, int P, int WPB, int T4>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(RF == kFmtQ1 ? 4 : 1))) void moe_down_kernel(Weights w, Ws ws, Dims d) {
  __shared__ __align__(16) uint8_t s_tile[WPB][kTileBytes];
  __shared__ float s_e8tab[RF == kFmtMxfp4 ? 256 : 1];  // 2^(e-127) for each E8M0 code
  static_assert(RF != kFmtMxfp4 || WPB == 4, "the E8M0 table takes one code a thread");
  extern __shared__ __align__(16) uint8_t dyn[];  // dn_lds_bytes(rows, I)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = d.H, I = d.I, nkb = I / 128;
  const int col = lane & 15;

  // ---- the block's expert and rows (MXFP4 routed blocks: T4 times the rows
  // of an FP8 block)
  // FP8 waves take TF 16-row tiles (T4 in FP8 layers; the shared expert of
  // an MXFP4 layer keeps one)
  constexpr int TF = RF == kFmtFp8 ? T4 : 1;
  const int per = H / (16 * WPB);
  const int nb_sh = d.Is > 0 ? per / TF : 0;
  int b = blockIdx.x, g = -1, nrows, e;
  uint64_t rows8 = 0, picks8 = 0;
  if (b < nb_sh) {
    nrows = d.rows;
    e = -1;
  } else {
    b -= nb_sh;
    const int perg = per / T4;
    g = b / perg;
    b -= g * perg;
    // one round of independent loads; the table of a group past D is stale
    // but in bounds, and unused
    const int D = *ws.n_groups;
    e = ws.grp_expert[g];
    nrows = ws.grp_nrows[g];
    rows8 = *reinterpret_cast<const uint64_t*>(ws.grp_rows + g * 8);
    picks8 = *reinterpret_cast<const uint64_t*>(ws.grp_slot + g * 8);
    if (g >= D) return;
  }
  const DnCols cols{g, rows8, picks8};
  if (RF == kFmtMxfp4 && g >= 0) {
    // MXFP4 routed expert: mid columns split into bf16 hi + lo in LDS while
    // the first weight items are in flight (issued inside down_fp4_wave after
    // the barrier below; the split is short next to the stream)
    float acc[T4][4];
    const int h0 = (b * WPB + wv) * 16 * T4;
    // whole-line items when I % 256 == 0 (then P, which divides I/128, is
    // even): P/2 of them hold the bytes of P half-line items (a ring of P
    // whole-line items measured slower: 8 rows 225.2 -> 229.1 us a step)
    if (I % 256 == 0) {
      // a block whose mid is at most 4 x 4 values a thread loads it before
      // its weight ring and splits it once the ring is out; else it splits
      // first (loads with a runtime count would make the split wait for the
      // whole ring)
      const int n4 = I / 4, tot = nrows * n4;
      const bool early = tot <= 4 * 256;  // blockDim.x == 256 here
      v4f mv[4];
      if (early) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          int t = tid + 256 * i;
          t = t < tot ? t : tot - 1;
          const int c = t / n4;
          mv[i] = *reinterpret_cast<const v4f*>(ws.mid + (size_t)cols.u(c) * d.imax + 4 * (t - c * n4));
        }
        asm volatile("" ::: "memory");  // keep them ahead of the weight ring
      }
      if (!early) {
        dn4_split_mid(ws, d, nrows, cols, dyn);
        s_e8tab[tid] = e8m0_scale(tid);  // blockDim.x >= 256 for the MXFP4 path
        __syncthreads();
      }
      auto pro = [&]() {
        if (early) {
#pragma unroll
          for (int i = 0; i < 4; i++) {  // unconditional: clamped slots rewrite their own value
            int t = tid + 256 * i;
            t = t < tot ? t : tot - 1;
            const int c = t / n4;
            dn4_store_split(dyn, I, c, 4 * (t - c * n4), mv[i]);
          }
          s_e8tab[tid] = e8m0_scale(tid);
          __syncthreads();
        }
      };
      down_fp4_wave_line<(P > 1 ? P / 2 : 1), T4>(w, d, e, nrows, h0, s_tile[wv], dyn, s_e8tab,
                                                  acc, pro);
    } else {
      dn4_split_mid(ws, d, nrows, cols, dyn);
      s_e8tab[tid] = e8m0_scale(tid);
      __syncthreads();
      down_fp4_wave<P, T4>(w, d, e, nrows, h0, s_tile[wv], dyn, s_e8tab, acc);
    }
#pragma unroll
    for (int t = 0; t < T4; t++) pin4(acc[t]);
    if (col < nrows) {
#pragma unroll
      for (int t = 0; t < T4; t++)
        *reinterpret_cast<v4f*>(ws.ypart + (size_t)cols.u(col) * H + h0 + 16 * t +
                                4 * (lane >> 4)) = v4f{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
    }
    return;
  }
  if (RF == kFmtQ1 && g >= 0 && I % 1024 == 0) {
    // 1-bit routed expert, octets of the wave's contiguous rows (above): the
    // first two in flight while the block quantises mid into LDS
    const int h0 = (b * WPB + wv) * 16;
    const size_t rb = (size_t)18 * nkb;
    const uint8_t* wb = w.down_c + ((size_t)e * H + h0) * rb;
    const int no = I / 1024;
    DnQ1Oct t0, t1;
    dn_q1_oct_load(wb, rb, 0, lane, t0);
    dn_q1_oct_load(wb, rb, no > 1 ? 1 : 0, lane, t1);
    uint8_t* s_q = dyn;
    float* s_qs = reinterpret_cast<float*>(dyn + (size_t)d.rows * dn_code_stride(I));
    dn_quant_mid(ws, d, nrows, cols, b == 0, s_q, s_qs, true);
    __syncthreads();
    const int cq = col < nrows ? col : 0;
    const uint8_t* pm = s_q + cq * dn_code_stride(I) + (lane >> 4) * 32;
    const float* psm = s_qs + cq * nkb;
    const uint32_t m8 = q1_in_vgpr(0x88888888u), o2 = q1_in_vgpr(0x22222222u);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int o = 0; o < no; o += 2) {
      dn_q1_oct_consume(t0, s_tile[wv], o, pm, psm, m8, o2, acc);
      dn_q1_oct_load(wb, rb, o + 2 < no ? o + 2 : no - 1, lane, t0);
      if (o + 1 < no) dn_q1_oct_consume(t1, s_tile[wv], o + 1, pm, psm, m8, o2, acc);
      dn_q1_oct_load(wb, rb, o + 3 < no ? o + 3 : no - 1, lane, t1);
    }
    pin4(acc);  // the MFMAs run with every lane, before the divergent store
    if (col < nrows)
      *reinterpret_cast<v4f*>(ws.ypart + (size_t)cols.u(col) * H + h0 + 4 * (lane >> 4)) =
          v4f{acc[0], acc[1], acc[2], acc[3]};
    return;
  }
  if (RF == kFmtQ1 && g >= 0) {
    // 1-bit routed expert: all its weight items in flight while the block
    // quantises mid into LDS, then one 16-row tile a wave
    const int h0 = (b * WPB + wv) * 16;
    DnQ1Items it;
    down_q1_issue(w, d, e, h0, it);
    uint8_t* s_q = dyn;
    float* s_qs = reinterpret_cast<float*>(dyn + (size_t)d.rows * dn_code_stride(I));
    dn_quant_mid(ws, d, nrows, cols, b == 0, s_q, s_qs, true);
    __syncthreads();
    const int cq = col < nrows ? col : 0;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    down_q1_consume(d, it, reinterpret_cast<uint32_t*>(s_tile[wv]),
                    s_q + cq * dn_code_stride(I) + (lane >> 4) * 32, s_qs + cq * nkb, acc);
    pin4(acc);  // the MFMAs run with every lane, before the divergent store
    if (col < nrows)
      *reinterpret_cast<v4f*>(ws.ypart + (size_t)cols.u(col) * H + h0 + 4 * (lane >> 4)) =
          v4f{acc[0], acc[1], acc[2], acc[3]};
    return;
  }
  const int cc = col < nrows ? col : 0;  // columns past the rows reuse column 0
  const int h0 = (b * WPB + wv) * 16 * TF;

  const uint8_t* wb = e < 0 ? w.sd_c : w.down_c + (size_t)e * H * I;
  const float* sb =
      e < 0 ? w.sd_s : reinterpret_cast<const float*>(w.down_s) + (size_t)e * (H / 128) * nkb;
  // lane l loads rows h0 + 16t + l/8 and h0 + 16t + 8 + l/8 of tile t, 16-byte chunk l%8
  const uint8_t* pw = wb + (size_t)(h0 + (lane >> 3)) * I + (lane & 7) * 16;
  const size_t r8 = (size_t)8 * I;
  const float* psd = sb + (size_t)(h0 / 128) * nkb;
  uint8_t* tile = s_tile[wv];
  uint8_t* s_q = dyn;
  float* s_qs = reinterpret_cast<float*>(dyn + (size_t)d.rows * dn_code_stride(I));
  const uint8_t* pm = s_q + cc * dn_code_stride(I) + (lane >> 4) * 32;
  const float* psm = s_qs + cc * nkb;

  auto issue = [&](DnStage<TF>& s, int k) {
    const size_t o = (size_t)k * 128;
#pragma unroll
    for (int t = 0; t < TF; t++) {
      s.w0[t] = ld_nt16(pw + (size_t)t * 2 * r8 + o);
      s.w1[t] = ld_nt16(pw + (size_t)t * 2 * r8 + r8 + o);
    }
    s.sd = psd[k];
  };
  float acc[TF][4];
#pragma unroll
  for (int t = 0; t < TF; t++)
#pragma unroll
    for (int v = 0; v < 4; v++) acc[t][v] = 0.f;
  auto consume = [&](DnStage<TF>& s, int k) {
    v8i a[TF];  // each tile re-laid through the wave's LDS tile in turn
#pragma unroll
    for (int t = 0; t < TF; t++) {
      tile_put(tile, lane, s.w0[t], s.w1[t]);
      asm volatile("" ::: "memory");
      a[t] = tile_get(tile, lane);
      asm volatile("" ::: "memory");
    }
    const u32x4 m0 = ld16(pm + k * 128), m1 = ld16(pm + k * 128 + 16);
    const float f = s.sd * psm[k];
#pragma unroll
    for (int t = 0; t < TF; t++) {
      const v4f c = mfma_fp8(a[t], cat8(m0, m1));
#pragma unroll
      for (int v = 0; v < 4; v++) acc[t][v] = fmaf(c[v], f, acc[t][v]);
    }
  };
  // ring of P K blocks (P divides nkb): every issued load is used.  The first
  // P are in flight while the block quantises mid.
  DnStage<TF> st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  dn_quant_mid(ws, d, nrows, cols, b == 0, s_q, s_qs);
  __syncthreads();
  for (int k0 = 0; k0 < nkb - P; k0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p], k0 + p);
      issue(st[p], k0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p], nkb - P + p);
#pragma unroll
  for (int t = 0; t < TF; t++) pin4(acc[t]);  // the MFMAs run with every lane, before the divergent store
  if (col < nrows) {
#pragma unroll
    for (int t = 0; t < TF; t++)
      *reinterpret_cast<v4f*>(ws.ypart + (size_t)cols.u(col) * H + h0 + 16 * t + 4 * (lane >> 4)) =
          v4f{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
  }
}

// out[r][h] for 4 consecutive h per thread.
__global__ __launch_bounds__(256) void moe_combine_kernel(Ws ws, Dims d,
                                                          uint16_t* __restrict__ out) {
  const int r = blockIdx.y, h = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (h >= d.H) return;
  const size_t H = d.H;
  v4f y[9];
#pragma unroll
  for (int j = 0; j < 9; j++)
    y[j] = (j < 8 || d.Is > 0) ? *reinterpret_cast<const v4f*>(ws.ypart + (r * 9 + j) * H + h)
                               : v4f{0.f, 0.f, 0.f, 0.f};
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const float gj = ws.gates[r * 8 + j];
#pragma unroll
    for (int v = 0; v < 4; v++) a[v] = fmaf(gj, y[j][v], a[v]);
  }
  if (d.Is > 0) {
#pragma unroll
    for (int v = 0; v < 4; v++) a[v] += y[8][v];
  }
  uint2 pk;
  pk.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
  pk.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)r * H + h) = pk;
}

// K blocks in flight per wave: the largest of 8, 4, 2, 1 dividing I/128.
static int down_ring(int inter) {
  const int nkb = inter / 128;
  return nkb % 8 == 0 ? 8 : (nkb % 4 == 0 ? 4 : (nkb % 2 == 0 ? 2 : 1));
}

// Launches one instantiation with `lds` bytes of dynamic LDS, raising the
// kernel's dynamic-LDS limit first when it is above the default 64 KB.
template <int RF, int P, int WPB, int T4>
static hipError_t launch_one(int max_groups, size_t lds, const Weights& w, const Ws& ws,
                             const Dims& d, hipStream_t stream) {
  static size_t raised[kLdsDevices] = {};  // the limit set per device, this instantiation
  const hipError_t e =
      ensure_dyn_lds(reinterpret_cast<const void*>(&moe_down_kernel<RF, P, WPB, T4>), lds, raised);
  if (e != hipSuccess) return e;
  constexpr int TF = RF == kFmtFp8 ? T4 : 1;  // tiles of the FP8 (shared and routed) waves
  const int per = d.H / (16 * WPB);
  const dim3 grid((d.Is > 0 ? per / TF : 0) + (per / T4) * max_groups);
  hipLaunchKernelGGL((moe_down_kernel<RF, P, WPB, T4>), grid, dim3(64 * WPB), lds, stream, w, ws,
                     d);
  return hipGetLastError();
}

// FP8: blocks of 2 waves of one tile (32 output rows) for steps of one or two
// rows, whose few experts otherwise leave some CUs a block more than others;
// else 4 waves of two tiles (128 rows; measured against one tile, same ring:
// 150.5 -> 149.9, 190.3 -> 188.9, 269.1 -> 266.8 and 339.9 -> 337.2 us per
// GLM step at 3, 4, 6 and 8 rows; half the ring with two tiles was between).
// MXFP4 routed waves take 2 tiles of 16 rows from kDn4TwoTileRows rows up
// (the mid operand's LDS reads then serve 32 rows), else 1 (more blocks for
// the few experts of small steps); measured with whole-line items: 2 tiles
// are faster from 3 rows (4 rows 136.1 -> 132.8, 5 rows 163.3 -> 158.8, 8
// rows 245.4 -> 225.1 us a step).
constexpr int kDn4TwoTileRows = 3;

template <int RF, int P>
static hipError_t launch_wpb(int max_groups, size_t lds, const Weights& w, const Ws& ws,
                             const Dims& d, hipStream_t stream) {
  if constexpr (RF == kFmtQ1)  // 1-bit routed experts: one 16-row tile a wave
    return launch_one<RF, P, 4, 1>(max_groups, lds, w, ws, d, stream);
  else if constexpr (RF == kFmtFp8)
    return d.rows <= 2 ? launch_one<RF, P, 2, 1>(max_groups, lds, w, ws, d, stream)
                       : launch_one<RF, P, 4, 2>(max_groups, lds, w, ws, d, stream);
  else
    return d.rows >= kDn4TwoTileRows
               ? launch_one<RF, P, 4, 2>(max_groups, lds, w, ws, d, stream)
               : launch_one<RF, P, 4, 1>(max_groups, lds, w, ws, d, stream);
}

template <int RF>
static hipError_t launch_rf(int max_groups, size_t lds, const Weights& w, const Ws& ws,
                            const Dims& d, hipStream_t stream) {
  switch (down_ring(d.I)) {
    case 8: return launch_wpb<RF, 8>(max_groups, lds, w, ws, d, stream);
    case 4: return launch_wpb<RF, 4>(max_groups, lds, w, ws, d, stream);
    case 2: return launch_wpb<RF, 2>(max_groups, lds, w, ws, d, stream);
    default: return launch_wpb<RF, 1>(max_groups, lds, w, ws, d, stream);
  }
}

hipError_t launch_down(int rfmt, int max_groups, const Weights& w, const Ws& ws, const Dims& d,
                       hipStream_t stream) {
  size_t lds = dn_lds_bytes(d.rows, d.I);
  if (rfmt == kFmtMxfp4 && dn4_lds_bytes(d.rows, d.I) > lds) lds = dn4_lds_bytes(d.rows, d.I);
  if (rfmt == kFmtFp8) return launch_rf<kFmtFp8>(max_groups, lds, w, ws, d, stream);
  if (rfmt == kFmtMxfp4) return launch_rf<kFmtMxfp4>(max_groups, lds, w, ws, d, stream);
  if (rfmt == kFmtQ1) return launch_rf<kFmtQ1>(max_groups, lds, w, ws, d, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const Ws& ws, const Dims& d, uint16_t* out, hipStream_t stream) {
  const dim3 grid((d.H / 4 + 255) / 256, d.rows);
  hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(256), 0, stream, ws, d, out);
  return hipGetLastError();
}

}  // namespace moe
