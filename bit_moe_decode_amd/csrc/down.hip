// down.hip -- down GEMV of the shared expert and of every distinct routed
// expert from the FP8 mid, per (row, pick); then the gate-weighted combine.
//
// #85 Mod. row 16: down units take one expert's tile against every row that
// uses it; a row's output is summed over its units in the one-row form's
// order, so dedup changes no output bit.  Mod. row 1: down reads mid as the
// FP8 bytes and scales quantised once.  Mod. rows 18 and 21: 16-byte,
// nontemporal weight loads.
//
// moe_down_kernel: block = 4 waves = 64 output rows of one expert (the shared
// expert's H/64 blocks first, then H/64 for each of the step's possible routed
// groups; blocks of groups past the step's D exit at once).  Many small
// blocks let the hardware dispatcher even out the load per CU.  A wave owns 16
// output rows over the whole K: for each 128-wide K block it loads its 16
// weight rows row-contiguously, re-lays them through LDS into MFMA operand
// order and runs one 16x16x128 FP8 MFMA against the expert's midq columns (one
// column per using row), scaled by weight scale x mid scale and accumulated in
// fp32.  It stores y[row, pick][h]; every (row, pick) belongs to exactly one
// expert of the step, so no two writes collide.
//
// MXFP4 routed experts (mid kept in fp32, as the oracle does): a VALU path in
// the same blocks, one mid column at a time.  Per K chunk of 512 the block
// stages the column's fp32 mid in LDS (4 pad floats per 32, so the 4 lanes of
// a row read disjoint banks); each 16-byte run of weights -- 32 inputs, one
// E8M0 block -- is decoded with the hardware FP4 -> fp32 conversion scaled by
// 2^(E8M0-127) and multiplied into an fp32 sum.
//
// moe_combine_kernel:
//   out[r][h] = bf16( sum_{j<8} g_rj * y_rj[h] + y_r8[h] )
// in pick order, the same arithmetic whether or not experts were deduplicated.
#include "device_common.h"

namespace moe {

struct DnStage {
  u32x4 w0, w1, m0, m1;
  float sd, sm;
};

constexpr int kDnChunk = 512;                  // K inputs per staged mid chunk (MXFP4)
constexpr int kDnMidStride = kDnChunk + kDnChunk / 8;  // 4 pad floats per 32

typedef float v2f_t __attribute__((ext_vector_type(2)));

// 2^(e-127) as fp32 for an E8M0 code (0xFF, NaN, is not produced by the
// generator; it decodes to a NaN here as well).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  uint32_t b = e << 23;
  b = e == 0 ? 0x00400000u : b;
  b = e == 255 ? 0x7FC00000u : b;
  return __uint_as_float(b);
}

// The MXFP4 down GEMV of one block: 64 output rows of routed expert e against
// its nrows mid columns u_c (fp32, unquantised), one column at a time.  Lane l
// takes row hb + 16*wave + l/4 and, of each staged K chunk, the 16-byte runs
// 16(l%4) + 64i (32 inputs, one E8M0 block each); the 4 lanes of a row are
// summed at the end.
__device__ __forceinline__ void down_fp4_block(const Weights& w, const Ws& ws, const Dims& d,
                                               int e, int nrows, const int* ucol, int hb,
                                               float* s_mid) {
  constexpr int R = kDnChunk / 128;  // runs of a lane per chunk
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = d.H, I = d.I;
  const size_t rbytes = I / 2;
  const int h = hb + wv * 16 + (lane >> 2), q = lane & 3;
  const uint8_t* wrow = w.down_c + ((size_t)e * H + h) * rbytes;
  const uint8_t* erow = reinterpret_cast<const uint8_t*>(w.down_s) + ((size_t)e * H + h) * (I / 32);
#pragma unroll 1
  for (int c = 0; c < nrows; c++) {
    const float* mcol = ws.mid + (size_t)ucol[c] * d.imax;
    float a = 0.f;
#pragma unroll 1
    for (int k0 = 0; k0 < I; k0 += kDnChunk) {
      const int kc = I - k0 < kDnChunk ? I - k0 : kDnChunk;  // a multiple of 128
      const int nrun = kc / 128;
      u32x4 wq[R];
      uint32_t ev[R];
#pragma unroll
      for (int i = 0; i < R; i++)
        if (i < nrun) {
          const int byte = k0 / 2 + 64 * i + 16 * q;
          wq[i] = ld_nt16(wrow + byte);
          ev[i] = erow[byte / 16];
        }
      __syncthreads();  // the previous chunk's readers are done
      for (int f4 = tid; f4 < kc / 4; f4 += 256)
        *reinterpret_cast<v4f*>(s_mid + 4 * f4 + (f4 / 8) * 4) =
            *reinterpret_cast<const v4f*>(mcol + k0 + 4 * f4);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < R; i++) {
        if (i >= nrun) break;
        const float sc = e8m0_scale(ev[i]);
        const int kl = 128 * i + 32 * q;  // first input of the run within the chunk
        const float* mp = s_mid + kl + (kl / 32) * 4;
#pragma unroll
        for (int j = 0; j < 4; j++) {  // 8 inputs per dword of codes
          const v2f_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq[i][j], sc, 0);
          const v2f_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq[i][j], sc, 1);
          const v2f_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq[i][j], sc, 2);
          const v2f_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq[i][j], sc, 3);
          const v4f m0 = *reinterpret_cast<const v4f*>(mp + 8 * j);
          const v4f m1 = *reinterpret_cast<const v4f*>(mp + 8 * j + 4);
          a = fmaf(p0[0], m0[0], a);
          a = fmaf(p0[1], m0[1], a);
          a = fmaf(p1[0], m0[2], a);
          a = fmaf(p1[1], m0[3], a);
          a = fmaf(p2[0], m1[0], a);
          a = fmaf(p2[1], m1[1], a);
          a = fmaf(p3[0], m1[2], a);
          a = fmaf(p3[1], m1[3], a);
        }
        __builtin_amdgcn_sched_barrier(0);  // one run decoded at a time
      }
    }
    // sum over the 4 lanes of the row (xor 1, xor 2 within quads)
    a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false));
    a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false));
    if (q == 0) ws.ypart[(size_t)ucol[c] * H + h] = a;
  }
}

template <int RF, int P>
__global__ __launch_bounds__(256) void moe_down_kernel(Weights w, Ws ws, Dims d) {
  __shared__ uint8_t s_tile[4][kTileBytes];
  __shared__ float s_mid[RF == kFmtMxfp4 ? kDnMidStride : 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = d.H, I = d.I, nkb = I / 128;
  const int col = lane & 15;

  // ---- the block's expert and rows
  const int per = H / 64;
  const int nb_sh = d.Is > 0 ? per : 0;
  int b = blockIdx.x, g = -1, nrows, e;
  uint64_t rows8 = 0, picks8 = 0;
  if (b < nb_sh) {
    nrows = d.rows;
    e = -1;
  } else {
    b -= nb_sh;
    g = b / per;
    b -= g * per;
    // one round of independent loads; the table of a group past D is stale
    // but in bounds, and unused
    const int D = *ws.n_groups;
    e = ws.grp_expert[g];
    nrows = ws.grp_nrows[g];
    rows8 = *reinterpret_cast<const uint64_t*>(ws.grp_rows + g * 8);
    picks8 = *reinterpret_cast<const uint64_t*>(ws.grp_slot + g * 8);
    if (g >= D) return;
  }
  if (RF == kFmtMxfp4 && g >= 0) {
    int ucol[kMaxRows];
#pragma unroll
    for (int c = 0; c < kMaxRows; c++) {
      const int r = (int)((rows8 >> (8 * c)) & 0xFF);
      ucol[c] = c < nrows ? r * 9 + (int)((picks8 >> (8 * r)) & 0xFF) : 0;
    }
    down_fp4_block(w, ws, d, e, nrows, ucol, b * 64, s_mid);
    return;
  }
  const int row = col < nrows ? (g < 0 ? col : (int)((rows8 >> (8 * (col & 7))) & 0xFF)) : 0;
  const int pick = g < 0 ? 8 : (int)((picks8 >> (8 * row)) & 0xFF);
  const int u = col < nrows ? row * 9 + pick : 0;  // (row, pick) of this column
  const int h0 = b * 64 + wv * 16;

  const uint8_t* wb = e < 0 ? w.sd_c : w.down_c + (size_t)e * H * I;
  const float* sb =
      e < 0 ? w.sd_s : reinterpret_cast<const float*>(w.down_s) + (size_t)e * (H / 128) * nkb;
  // lane l loads rows h0 + l/8 and h0 + 8 + l/8, 16-byte chunk l%8
  const uint8_t* pw = wb + (size_t)(h0 + (lane >> 3)) * I + (lane & 7) * 16;
  const size_t r8 = (size_t)8 * I;
  const uint8_t* pm = ws.midq + (size_t)u * d.imax + (lane >> 4) * 32;
  const float* psd = sb + (size_t)(h0 / 128) * nkb;
  const float* psm = ws.midqs + (size_t)u * (d.imax / 128);
  uint8_t* tile = s_tile[wv];

  auto issue = [&](DnStage& s, int k) {
    const size_t o = (size_t)k * 128;
    s.w0 = ld_nt16(pw + o);
    s.w1 = ld_nt16(pw + r8 + o);
    s.m0 = ld16(pm + o);
    s.m1 = ld16(pm + o + 16);
    s.sd = psd[k];
    s.sm = psm[k];
  };
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](DnStage& s) {
    tile_put(tile, lane, s.w0, s.w1);
    asm volatile("" ::: "memory");
    const v4f c = mfma_fp8(tile_get(tile, lane), cat8(s.m0, s.m1));
    asm volatile("" ::: "memory");
    const float f = s.sd * s.sm;
#pragma unroll
    for (int v = 0; v < 4; v++) acc[v] = fmaf(c[v], f, acc[v]);
  };
  // ring of P K blocks (P divides nkb): every issued load is used
  DnStage st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  for (int k0 = 0; k0 < nkb - P; k0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p]);
      issue(st[p], k0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p]);
  pin4(acc);  // the MFMAs run with every lane, before the divergent store
  if (col < nrows)
    *reinterpret_cast<v4f*>(ws.ypart + (size_t)u * H + h0 + 4 * (lane >> 4)) =
        v4f{acc[0], acc[1], acc[2], acc[3]};
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

template <int RF>
static void launch_rf(dim3 grid, const Weights& w, const Ws& ws, const Dims& d,
                      hipStream_t stream) {
  switch (down_ring(d.I)) {
    case 8: hipLaunchKernelGGL((moe_down_kernel<RF, 8>), grid, dim3(256), 0, stream, w, ws, d); break;
    case 4: hipLaunchKernelGGL((moe_down_kernel<RF, 4>), grid, dim3(256), 0, stream, w, ws, d); break;
    case 2: hipLaunchKernelGGL((moe_down_kernel<RF, 2>), grid, dim3(256), 0, stream, w, ws, d); break;
    default: hipLaunchKernelGGL((moe_down_kernel<RF, 1>), grid, dim3(256), 0, stream, w, ws, d); break;
  }
}

hipError_t launch_down(int rfmt, int max_groups, const Weights& w, const Ws& ws, const Dims& d,
                       hipStream_t stream) {
  const dim3 grid((d.H / 64) * ((d.Is > 0 ? 1 : 0) + max_groups));
  if (rfmt == kFmtFp8)
    launch_rf<kFmtFp8>(grid, w, ws, d, stream);
  else if (rfmt == kFmtMxfp4)
    launch_rf<kFmtMxfp4>(grid, w, ws, d, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_combine(const Ws& ws, const Dims& d, uint16_t* out, hipStream_t stream) {
  const dim3 grid((d.H / 4 + 255) / 256, d.rows);
  hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(256), 0, stream, ws, d, out);
  return hipGetLastError();
}

}  // namespace moe
