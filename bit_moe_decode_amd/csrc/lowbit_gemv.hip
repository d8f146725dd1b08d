// lowbit_gemv.hip -- dense decode GEMV over 1-bit group-128 weights.
//
// 1-Bit Turbo, Q1_0_G128: 1-bit weights with one fp16 scale per group of 128
// (about 18 bytes a group: 572 MB for 4B parameters).  Layout: [N, K/128]
// blocks of 18 bytes = fp16 d (little-endian) + 16 bytes of bits; bit i of
// byte b is element 8b+i; bit 1 means -d.
//   y[n] = bf16( sum_g d[n,g] * sum_{k in g} sign[n,k] * x[k] )
//
// Any K (a multiple of 128): block = 4 waves; x (bf16) is staged once per
// block into LDS as fp32, with
// the sum of every 8 consecutive x beside it.  A wave takes one row at a time
// (grid-stride over rows); lane l covers byte l%16 of group 4i + l/16, i.e. 8
// elements: their signed sum is S8 - 2 * (sum of the x whose bit is 1), the
// mask of each bit coming from a signed 1-bit field extract.  Partial sums
// are scaled by d, summed over the row's groups per lane, then across the
// wave.
#include "device_common.h"

namespace moe {

constexpr int kQ1KMax = 16384;

__global__ __launch_bounds__(256) void lowbit_gemv_q1_kernel(const uint8_t* __restrict__ blocks,
                                                             const uint16_t* __restrict__ x,
                                                             uint16_t* __restrict__ y, int n, int k) {
  __shared__ float xs[kQ1KMax];
  __shared__ float s8[kQ1KMax / 8];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < k / 8; i += 256) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float v = bf16_to_f32(x[8 * i + j]);
      xs[8 * i + j] = v;
      s += v;
    }
    s8[i] = s;
  }
  __syncthreads();
  const int groups = k / 128;
  const size_t row_bytes = (size_t)groups * 18;
  const int byte = lane & 15, gsub = lane >> 4;
  for (int row = blockIdx.x * 4 + wv; row < n; row += gridDim.x * 4) {
    const uint8_t* rb = blocks + (size_t)row * row_bytes;
    float acc = 0.f;
    for (int g = gsub; g < groups; g += 4) {
      const uint8_t* blk = rb + (size_t)g * 18;
      const uint32_t bits = blk[2 + byte];
      const uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
      const float d = (float)__builtin_bit_cast(_Float16, dh);
      const int e0 = g * 128 + byte * 8;
      float set = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)bits, i, 1);  // 0 or ~0
        set += __uint_as_float(__float_as_uint(xs[e0 + i]) & m);
      }
      acc = fmaf(d, fmaf(-2.f, set, s8[e0 / 8]), acc);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (lane == 0) y[row] = f32_to_bf16(acc);
  }
}

// Nibble-table form, for K a multiple of 256 (an even number of groups: a row
// is a whole number of 36-byte, dword-aligned pairs of groups).  Block = 256
// threads = RB rows x KP = 256/RB parts of K.  K is taken in chunks of 256
// inputs (two groups, 64 positions of 4 inputs), CH = KP * M chunks a round
// (M = 1..5: all of K in one round when the round's tables fit).  Each thread
// reads the 36 bytes of each of its row's chunks of the round straight from
// memory at the start of the round (the lanes of a load touch one line per
// row; staging the rows through LDS first measured slower, 23.5 against
// 21.4 us on the LM head).  The block fills, for the CH chunks at once, a
// table of the signed sums of every position's 4 inputs for all 16 nibble
// values,
//   T[p][v] = sum_{i<4} (bit i of v ? -x : +x)[256c + 4p + i],
// and thread (row r, part q) adds T[p][nibble] over the 64 nibbles of chunks
// c0 + q, c0 + q + KP, ... of its row, scales each group's sum by its d and
// accumulates in fp32: one table read per 4 weights.  The parts of a row are
// added in part order at the end.  The lanes of a wave read one position's
// 16 entries at a time (a broadcast or a distinct bank each), and the tables
// of different parts are offset by 16 floats so that they use different banks.
constexpr int kLbTab = 64 * 16 + 16;  // floats per chunk table, padded
// chunks whose tables one round may hold (19 x 4160 bytes: two blocks a CU)
constexpr int kLbRoundChunks = 19;

// Bits o .. o+3 of v as one v_bfe_u32 (the compiler would otherwise split a
// constant-offset field extract into a shift and a mask).
template <int O>
__device__ __forceinline__ uint32_t nib4_at(uint32_t v) {
  uint32_t r;
  asm("v_bfe_u32 %0, %1, %2, 4" : "=v"(r) : "v"(v), "n"(O));
  return r;
}
__device__ __forceinline__ uint32_t nib4(uint32_t v, int o) {
  switch (o) {
    case 0: return nib4_at<0>(v);
    case 4: return nib4_at<4>(v);
    case 8: return nib4_at<8>(v);
    case 12: return nib4_at<12>(v);
    case 16: return nib4_at<16>(v);
    case 20: return nib4_at<20>(v);
    case 24: return nib4_at<24>(v);
    default: return v >> 28;
  }
}

__device__ __forceinline__ float lb_f16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// One chunk (two groups) of a row: w = its 9 dwords (d of group 0, 16 bit
// bytes, d of group 1, 16 bit bytes), tab = the chunk's 64 positions x 16
// entries.  Returns acc + d0 * s0 + d1 * s1, s = the sum of the entries of
// the group's 32 nibbles.
__device__ __forceinline__ float lb_chunk(const uint32_t* w, const float* tab, float acc) {
  // the 16 bit-bytes of each group as 4 aligned dwords (group 0 starts 2
  // bytes in)
  uint32_t u[8];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    u[q] = __builtin_amdgcn_alignbyte(w[q + 1], w[q], 2);
    u[4 + q] = w[5 + q];
  }
  // nibble t of dword q is the 4 inputs of position 8(q%4) + t of its group;
  // its entry is float `nibble` of that position's 16
  const float* tg[2] = {tab, tab + 32 * 16};
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 8; q++) {
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
      const int pos = 8 * (q & 3) + t;
      const uint32_t n0 = nib4(u[q], 4 * t), n1 = nib4(u[q], 4 * t + 4);
      s[q >> 2] += tg[q >> 2][pos * 16 + n0] + tg[q >> 2][pos * 16 + 16 + n1];
    }
  }
  acc = fmaf(lb_f16(w[0] & 0xFFFFu), s[0], acc);
  return fmaf(lb_f16(w[4] >> 16), s[1], acc);
}

// The 16 entries of one position, t[v] = sum_{i<4} (bit i of v ? -x : +x)[i],
// from its 4 bf16 inputs (packed in xv, input 0 in the low half of xv.x).
__device__ __forceinline__ void lb_fill_pos(float* t, uint2 xv) {
  const float x0 = bf16_to_f32((uint16_t)(xv.x & 0xFFFFu)), x1 = bf16_to_f32((uint16_t)(xv.x >> 16));
  const float x2 = bf16_to_f32((uint16_t)(xv.y & 0xFFFFu)), x3 = bf16_to_f32((uint16_t)(xv.y >> 16));
  // bits 0-1 and bits 2-3 of the nibble
  const float a0 = x0 + x1, a1 = -x0 + x1, a2 = x0 - x1, a3 = -x0 - x1;
  const float b[4] = {x2 + x3, -x2 + x3, x2 - x3, -x2 - x3};
#pragma unroll
  for (int hb = 0; hb < 4; hb++)
    *reinterpret_cast<float4*>(t + 4 * hb) = float4{a0 + b[hb], a1 + b[hb], a2 + b[hb], a3 + b[hb]};
}

template <int RB, int M>
__global__ __launch_bounds__(256) void lowbit_gemv_q1_nib_kernel(
    const uint8_t* __restrict__ blocks, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, int n, int k) {
  constexpr int KP = 256 / RB;
  constexpr int CH = KP * M;  // chunks a round: part q takes q, q + KP, ..
  extern __shared__ __align__(16) uint8_t smem[];
  float* tab = reinterpret_cast<float*>(smem);                    // [CH][kLbTab]
  float* red = tab + CH * kLbTab;                                  // [KP][RB]
  const int tid = threadIdx.x;
  const int G = k / 128, nch = G / 2, rb = 18 * G;
  const int r0 = blockIdx.x * RB;
  const int nr = n - r0 < RB ? n - r0 : RB;

  const int rl = tid % RB, part = tid / RB;
  const int rowl = rl < nr ? rl : nr - 1;  // threads past n decode the last row
  const uint32_t* myrow = reinterpret_cast<const uint32_t*>(blocks + (size_t)(r0 + rowl) * rb);

  // table positions of this thread in a round: e = tid + 256 j (j < NE), the
  // inputs of each loaded one round ahead
  constexpr int NE = (CH * 64 + 255) / 256;
  uint2 xn[NE];
  auto xload = [&](int c0) {
#pragma unroll
    for (int j = 0; j < NE; j++) {
      const int e = tid + 256 * j;
      if (e < CH * 64 && c0 + (e >> 6) < nch)
        xn[j] = *reinterpret_cast<const uint2*>(x + 256 * c0 + 4 * e);
    }
  };
  xload(0);
  float acc = 0.f;
  for (int c0 = 0; c0 < nch; c0 += CH) {
    // this thread's chunks of its row, loaded before the table fill
    uint32_t w9[M][9];
#pragma unroll
    for (int m = 0; m < M; m++) {
      const int c = c0 + part + KP * m;
      if (c < nch) {
#pragma unroll
        for (int i = 0; i < 9; i++) w9[m][i] = myrow[9 * c + i];
      }
    }
    // ---- tables of chunks c0 .. c0 + CH - 1: one position (4 inputs) at a time
#pragma unroll
    for (int j = 0; j < NE; j++) {
      const int e = tid + 256 * j;
      if (e < CH * 64 && c0 + (e >> 6) < nch)
        lb_fill_pos(tab + (e >> 6) * kLbTab + (e & 63) * 16, xn[j]);
    }
    if (c0 + CH < nch) xload(c0 + CH);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; m++)
      if (c0 + part + KP * m < nch) acc = lb_chunk(w9[m], tab + (part + KP * m) * kLbTab, acc);
    if (c0 + CH < nch) __syncthreads();
  }
  red[part * RB + rl] = acc;
  __syncthreads();
  if (tid < nr) {
    float v = red[tid];
#pragma unroll
    for (int q = 1; q < KP; q++) v += red[q * RB + tid];
    y[r0 + tid] = f32_to_bf16(v);
  }
}

static size_t lb_nib_lds(int rbk, int m) { return (size_t)(256 / rbk) * m * kLbTab * 4 + 256 * 4; }

template <int RB, int M>
static hipError_t lb_nib_launch(const uint8_t* blocks, const uint16_t* x, uint16_t* y, int n,
                                int k, hipStream_t stream) {
  const size_t sh = lb_nib_lds(RB, M);
  static size_t raised[kLdsDevices] = {};  // the limit set per device
  if (ensure_dyn_lds(reinterpret_cast<const void*>(lowbit_gemv_q1_nib_kernel<RB, M>), sh,
                     raised) != hipSuccess)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((lowbit_gemv_q1_nib_kernel<RB, M>), dim3((n + RB - 1) / RB), dim3(256), sh,
                     stream, blocks, x, y, n, k);
  return hipGetLastError();
}

hipError_t launch_lowbit_q1(const uint8_t* blocks, const uint16_t* x, uint16_t* y, int n, int k,
                            hipStream_t stream) {
  // the nibble-table form: rows per block RB the largest of 128, 64, 32 that
  // gives 2048 blocks, else the largest that gives 256, else 16; chunks per
  // thread and round M the fewest (up to 5) that take all of K in one round,
  // as long as the round's tables stay within kLbRoundChunks chunks
  if (k % 256 == 0) {
    int rbk = 16;
    for (int want : {2048, 256}) {
      for (int c = 128; c >= 32 && rbk == 16; c >>= 1)
        if ((n + c - 1) / c >= want) rbk = c;
      if (rbk != 16) break;
    }
    const int nch = k / 256, kp = 256 / rbk;
    int m = (nch + kp - 1) / kp;
    if (m > 5) m = 5;
    while (m > 1 && kp * m > kLbRoundChunks) m--;
#define LB_CASE(R)                                                           \
  case R:                                                                    \
    switch (m) {                                                             \
      case 5: return lb_nib_launch<R, 5>(blocks, x, y, n, k, stream);        \
      case 4: return lb_nib_launch<R, 4>(blocks, x, y, n, k, stream);        \
      case 3: return lb_nib_launch<R, 3>(blocks, x, y, n, k, stream);        \
      case 2: return lb_nib_launch<R, 2>(blocks, x, y, n, k, stream);        \
      default: return lb_nib_launch<R, 1>(blocks, x, y, n, k, stream);       \
    }
    switch (rbk) {
      LB_CASE(128)
      LB_CASE(64)
      LB_CASE(32)
      LB_CASE(16)
    }
#undef LB_CASE
  }
  int rows_blocks = (n + 3) / 4;
  int grid = rows_blocks < 1024 ? rows_blocks : 1024;
  hipLaunchKernelGGL(lowbit_gemv_q1_kernel, dim3(grid), dim3(256), 0, stream, blocks, x, y, n, k);
  return hipGetLastError();
}

}  // namespace moe
