// dense_gemv.hip -- decode GEMV against 1 to 8 bf16 input rows over FP8 E4M3
// weights with one fp32 scale per 128x128 block, or over bf16 weights: the
// tail's LM-head GEMV after the last layer (#85 Mod. row 24: a tail wave keeps
// its next weights in flight while the current tile is reduced and stored).
//   FP8:  y[r][n] = bf16( sum_k dec(W[n][k]) * s[n/128][k/128] * x[r][k] )
//   bf16: y[r][n] = bf16( sum_k W[n][k] * x[r][k] )
//
// The description below is the FP8 form's; the bf16 form differs only in
// that a K block (128 bytes of a row) holds 64 weights, read from the tile as
// they are (two MFMA steps a K block instead of four, no scale).
//
// Block = 4 waves = 4/KS groups of T = 2 slabs of 16 weight rows x KS parts
// of K (KS the largest of 4, 2, 1 dividing K/128): each wave keeps two tiles'
// weights in flight and each load of the input operands serves 32 weight
// rows.  A wave streams its two slabs' K part: per 128-wide K block its lanes
// load each slab's 16 rows row-contiguously (8 lanes per 128-byte line,
// nontemporal: every weight byte is read once), P K blocks in
// flight (P the largest of 4, 2, 1 dividing the part's K blocks, so every
// issued load is used).  Each K block is re-laid through the wave's LDS tiles
// into MFMA operand order; per 32 inputs a lane converts the 8 codes of row
// l%16 at inputs 8(l/16) .. +8 to bf16 (exact) and runs one 16x16x32 bf16 MFMA
// against the input rows at the same inputs (the MFMA's columns are the input
// rows; columns past them repeat row 0 and are not stored).  The K block's
// fp32 result is scaled by its weight scale and accumulated.  The block then
// adds its K parts in part order through LDS and stores y as bf16.
#include "device_common.h"

namespace moe {

// A K block is 128 bytes of each weight row: 128 FP8 codes (S = 4 MFMA steps
// of 32 inputs) or 64 bf16 weights (S = 2).
template <bool BF, int T>
struct DgStage {
  static constexpr int S = BF ? 2 : 4;
  u32x4 w0[T], w1[T];  // rows l/8 and 8 + l/8 of each 16-row tile, 16-byte chunk l%8
  u32x4 a[S];          // the lane's input row at inputs 32s + 8(l/16) .. +8, s < S
  float sw;            // FP8: weight block scale (the T tiles share a 128-row block)
};

// BF: bf16 weights (no scales), else FP8 codes with block scales.  T = 16-row
// tiles a wave.
template <bool BF, int P, int T>
__global__ __launch_bounds__(256) void dense_gemv_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scales,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int rows, int n, int k, int ks) {
  constexpr int S = DgStage<BF, T>::S, EPB = 32 * S;  // MFMA steps, inputs per K block
  __shared__ __align__(16) uint8_t s_tile[4][T][kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int spb = 4 / ks;  // wave groups (of T slabs) per block
  const int grp = blockIdx.x * spb + wv / ks, kp = wv % ks;
  const int n0 = grp * 16 * T;
  const int nkb = k / EPB, nk = nkb / ks, kb0 = kp * nk;

  const size_t rb = BF ? (size_t)2 * k : (size_t)k;  // bytes of a weight row
  const uint8_t* pw = codes + (size_t)(n0 + (lane >> 3)) * rb + (lane & 7) * 16 + (size_t)kb0 * 128;
  const size_t r8 = 8 * rb, r16 = 16 * rb;
  // FP8: T * 16 rows share a 128-row scale block
  const float* psw = BF ? nullptr : scales + (size_t)(n0 / 128) * (k / 128) + kb0;
  const uint16_t* pa = x + (size_t)(col < rows ? col : 0) * k + 8 * g + (size_t)kb0 * EPB;

  auto issue = [&](DgStage<BF, T>& st, int kk) {
    const size_t o = (size_t)kk * 128, oe = (size_t)kk * EPB;  // weight bytes, inputs
#pragma unroll
    for (int t = 0; t < T; t++) {
      st.w0[t] = ld_nt16(pw + t * r16 + o);
      st.w1[t] = ld_nt16(pw + t * r16 + r8 + o);
    }
#pragma unroll
    for (int s = 0; s < S; s++) st.a[s] = ld16(pa + oe + 32 * s);
    if constexpr (!BF) st.sw = psw[kk];
  };
  float acc[T][4];
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int v = 0; v < 4; v++) acc[t][v] = 0.f;
  auto consume = [&](DgStage<BF, T>& st) {
#pragma unroll
    for (int t = 0; t < T; t++) tile_put(s_tile[wv][t], lane, st.w0[t], st.w1[t]);
    asm volatile("" ::: "memory");
    v4f c[T];
#pragma unroll
    for (int t = 0; t < T; t++) c[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; s++) {
      const v8bf b = __builtin_bit_cast(v8bf, st.a[s]);
#pragma unroll
      for (int t = 0; t < T; t++) {
        const uint8_t* row = s_tile[wv][t] + col * kTileStride;
        const v8bf a = BF ? *reinterpret_cast<const v8bf*>(row + 64 * s + 16 * g)
                          : fp8x8_to_bf16(*reinterpret_cast<const uint2*>(row + 32 * s + 8 * g));
        c[t] = mfma_bf16(a, b, c[t]);
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < T; t++)
#pragma unroll
      for (int v = 0; v < 4; v++)
        acc[t][v] = BF ? acc[t][v] + c[t][v] : fmaf(c[t][v], st.sw, acc[t][v]);
  };
  DgStage<BF, T> st[P];
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
#pragma unroll
  for (int t = 0; t < T; t++) pin4(acc[t]);  // the MFMAs run with every lane, before any divergent use

  // ---- K parts -> y.  Each wave parks its (16 T) x 16 sums in its own tiles,
  // column-major per tile (weight row i, input row c at c*16 + i); lane l
  // holds rows 4(l/16) .. +4 of column l%16 of each tile.
  __syncthreads();  // every wave is done with its tiles' weights
#pragma unroll
  for (int t = 0; t < T; t++)
    *reinterpret_cast<v4f*>(reinterpret_cast<float*>(s_tile[wv][t]) + col * 16 + 4 * g) =
        v4f{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
  __syncthreads();
  const int c = tid >> 4, i = tid & 15;  // input row c, weight row i of each tile
  if (c >= rows) return;
  for (int s = 0; s < spb; s++) {
#pragma unroll
    for (int t = 0; t < T; t++) {
      float v = reinterpret_cast<const float*>(s_tile[s * ks][t])[c * 16 + i];
      for (int q = 1; q < ks; q++) v += reinterpret_cast<const float*>(s_tile[s * ks + q][t])[c * 16 + i];
      y[(size_t)c * n + ((blockIdx.x * spb + s) * T + t) * 16 + i] = f32_to_bf16(v);
    }
  }
}

template <bool BF, int T>
static void launch_gemv_t(const uint8_t* codes, const float* scales, const uint16_t* x,
                          uint16_t* y, int rows, int n, int k, int ks, int nk,
                          hipStream_t stream) {
  const dim3 grid(n / (16 * T * (4 / ks)));  // n is a multiple of 128 >= 16 * T * (4 / ks)
  if (nk % 4 == 0)
    hipLaunchKernelGGL((dense_gemv_kernel<BF, 4, T>), grid, dim3(256), 0, stream, codes, scales,
                       x, y, rows, n, k, ks);
  else if (nk % 2 == 0)
    hipLaunchKernelGGL((dense_gemv_kernel<BF, 2, T>), grid, dim3(256), 0, stream, codes, scales,
                       x, y, rows, n, k, ks);
  else
    hipLaunchKernelGGL((dense_gemv_kernel<BF, 1, T>), grid, dim3(256), 0, stream, codes, scales,
                       x, y, rows, n, k, ks);
}

// K parts of a wave group: the largest of 4, 2, 1 dividing K/128; ring depth:
// the largest of 4, 2, 1 dividing a part's K blocks; two 16-row tiles a wave
// at every row count (measured on the [151936, 6144] LM head against one
// tile: 149.8 -> 132.8 us at one row, 187.3 -> 147.4 us at 8; four tiles
// with a 2-deep ring: 141.6 us at one row, and 148.1 against 147.2 us at 8).
hipError_t launch_gemv_fp8(const uint8_t* codes, const float* scales, const uint16_t* x,
                           uint16_t* y, int rows, int n, int k, hipStream_t stream) {
  const int nkb = k / 128;
  const int ks = nkb % 4 == 0 ? 4 : (nkb % 2 == 0 ? 2 : 1);
  const int nk = nkb / ks;
  launch_gemv_t<false, 2>(codes, scales, x, y, rows, n, k, ks, nk, stream);
  return hipGetLastError();
}

// bf16 weights [n, k]: K blocks of 64 inputs (128 bytes a row), the same K
// parts, ring and tiles as the FP8 form.  n a multiple of 128, k of 64.
hipError_t launch_gemv_bf16(const uint16_t* w, const uint16_t* x, uint16_t* y, int rows, int n,
                            int k, hipStream_t stream) {
  const int nkb = k / 64;
  const int ks = nkb % 4 == 0 ? 4 : (nkb % 2 == 0 ? 2 : 1);
  const int nk = nkb / ks;
  launch_gemv_t<true, 2>(reinterpret_cast<const uint8_t*>(w), nullptr, x, y, rows, n, k, ks, nk,
                         stream);
  return hipGetLastError();
}

}  // namespace moe
