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
// added in part order at the end.
//
// LDS layout: the tables of the KP parts' m-th chunks are interleaved per
// position, slot P = 64 m + p holding part q's 16 entries at floats
// S P + 16 q .. +16 (S = 16 KP + 4: the fill writes one chunk's positions
// from consecutive lanes, S floats apart, and S mod 64 = 4 or 36 puts the 16
// lanes of a b128 pass on distinct banks).  A lookup's
// address is then 4 (16 q + nibble) + 4 S P: the sign dword, masked to its
// even or odd nibbles with 16 q or'ed into every byte, gives the first term
// for one byte in one SDWA shift, and 4 S P is the read's immediate offset
// (so 2 VALU operations per 4 weights: the shift and the add).  The lanes of
// a wave read one slot's 16 entries at a time (a broadcast or a distinct bank
// each).  The kernel declares no static LDS, so its dynamic LDS starts at
// address 0, and tables and part sums are addressed from there.
template <int KP>
constexpr int lb_slot() { return 16 * KP + 4; }
// chunks whose tables one round may hold (KP * M, at most 16 for the M and KP
// the launcher picks: about 70 KB, two blocks a CU); grids of at most one
// block a CU (gfx950: 256 CUs) may take 32 (at most 136 KB), for fewer rounds
constexpr int kLbRoundChunks = 19;
constexpr int kLbRoundChunksOne = 32;
constexpr int kLbCus = 256;

typedef __attribute__((address_space(3))) float lds_float;
__device__ __forceinline__ float lds_ld(uint32_t a) { return *(lds_float*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st(uint32_t a, float v) { *(lds_float*)(uintptr_t)a = v; }


// Byte B of e, times 4 (one v_lshlrev_b32 with an SDWA byte select; the
// compiler emits a shift and a mask for it otherwise).
template <int B>
__device__ __forceinline__ uint32_t byte_x4(uint32_t e) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(e));
  else if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(e));
  else if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(e));
  else
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(e));
  return r;
}

__device__ __forceinline__ float lb_f16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// One chunk (two groups) of a row: w = its 9 dwords (d of group 0, 16 bit
// bytes, d of group 1, 16 bit bytes), the chunk the thread's m-th of the
// round; pb = 16 q in every byte.  Returns acc + d0 * s0 + d1 * s1, s = the
// sum of the entries of the group's 32 nibbles.
template <int KP, int MI>
__device__ __forceinline__ float lb_chunk(const uint32_t* w, uint32_t pb, float acc) {
  constexpr uint32_t kSlotB = 4 * lb_slot<KP>();  // bytes per slot
  // the 16 bit-bytes of each group as 4 aligned dwords (group 0 starts 2
  // bytes in)
  uint32_t u[8];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    u[q] = __builtin_amdgcn_alignbyte(w[q + 1], w[q], 2);
    u[4 + q] = w[5 + q];
  }
  // nibble t of dword q is the 4 inputs of position 32(q/4) + 8(q%4) + t;
  // even nibbles are the low halves of the bytes of ev, odd ones of od
  // two dwords (16 reads) in flight before their sums
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 8; q += 2) {
    float v[2][8];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t ev = (u[q + h] & 0x0F0F0F0Fu) | pb, od = ((u[q + h] >> 4) & 0x0F0F0F0Fu) | pb;
      const uint32_t p0 = (uint32_t)(64 * MI + 32 * (q >> 2) + 8 * ((q + h) & 3)) * kSlotB;
      v[h][0] = lds_ld(byte_x4<0>(ev) + p0);
      v[h][1] = lds_ld(byte_x4<0>(od) + p0 + kSlotB);
      v[h][2] = lds_ld(byte_x4<1>(ev) + p0 + 2 * kSlotB);
      v[h][3] = lds_ld(byte_x4<1>(od) + p0 + 3 * kSlotB);
      v[h][4] = lds_ld(byte_x4<2>(ev) + p0 + 4 * kSlotB);
      v[h][5] = lds_ld(byte_x4<2>(od) + p0 + 5 * kSlotB);
      v[h][6] = lds_ld(byte_x4<3>(ev) + p0 + 6 * kSlotB);
      v[h][7] = lds_ld(byte_x4<3>(od) + p0 + 7 * kSlotB);
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int t = 0; t < 8; t += 2) s[q >> 2] += v[h][t] + v[h][t + 1];
  }
  acc = fmaf(lb_f16(w[0] & 0xFFFFu), s[0], acc);
  return fmaf(lb_f16(w[4] >> 16), s[1], acc);
}

// The thread's chunks of a round, the m-th being chunk c + KP m, while below
// nch.
template <int KP, int M, int MI = 0>
__device__ __forceinline__ float lb_chunks(const uint32_t (*w9)[9], uint32_t pb, int c, int nch,
                                           float acc) {
  if constexpr (MI < M) {
    if (c + KP * MI < nch) acc = lb_chunk<KP, MI>(w9[MI], pb, acc);
    return lb_chunks<KP, M, MI + 1>(w9, pb, c, nch, acc);
  } else {
    return acc;
  }
}

// The 16 entries of one position, t[v] = sum_{i<4} (bit i of v ? -x : +x)[i],
// from its 4 bf16 inputs (packed in xv, input 0 in the low half of xv.x), to
// LDS bytes a .. a + 64 (a % 16 == 0) of smem, the kernel's dynamic LDS.
__device__ __forceinline__ void lb_fill_pos(uint8_t* smem, uint32_t a, uint2 xv) {
  const float x0 = bf16_to_f32((uint16_t)(xv.x & 0xFFFFu)), x1 = bf16_to_f32((uint16_t)(xv.x >> 16));
  const float x2 = bf16_to_f32((uint16_t)(xv.y & 0xFFFFu)), x3 = bf16_to_f32((uint16_t)(xv.y >> 16));
  // bits 0-1 and bits 2-3 of the nibble
  const float a0 = x0 + x1, a1 = -x0 + x1, a2 = x0 - x1, a3 = -x0 - x1;
  const float b[4] = {x2 + x3, -x2 + x3, x2 - x3, -x2 - x3};
#pragma unroll
  for (int hb = 0; hb < 4; hb++)
    *reinterpret_cast<float4*>(smem + a + 16 * hb) = float4{a0 + b[hb], a1 + b[hb], a2 + b[hb], a3 + b[hb]};
}

// (its LDS allows 3 blocks a CU, so the compiler may schedule for 3 waves a SIMD)
template <int RB, int M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 3))) void lowbit_gemv_q1_nib_kernel(
    const uint8_t* __restrict__ blocks, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, int n, int k) {
  constexpr int KP = 256 / RB;
  constexpr int CH = KP * M;  // chunks a round: part q takes q, q + KP, ..
  constexpr uint32_t kSlotB = 4 * lb_slot<KP>();
  constexpr uint32_t kRed = 64 * M * kSlotB;  // LDS bytes of the tables; then [KP][RB] sums
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int G = k / 128, nch = G / 2, rb = 18 * G;
  const int r0 = blockIdx.x * RB;
  const int nr = n - r0 < RB ? n - r0 : RB;
  // the lookups address LDS from 0 (immediate offsets), the table fill from
  // smem: with no static LDS in this kernel they coincide; were they ever to
  // differ, every output is NaN rather than silently wrong
  if ((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem != 0u) {
    if (tid < nr) y[r0 + tid] = 0x7FC0;
    return;
  }

  const int rl = tid % RB, part = tid / RB;
  const int rowl = rl < nr ? rl : nr - 1;  // threads past n decode the last row
  const uint32_t* myrow = reinterpret_cast<const uint32_t*>(blocks + (size_t)(r0 + rowl) * rb);
  const uint32_t pb = (uint32_t)(16 * part) * 0x01010101u;

  // table positions of this thread in a round: e = tid + 256 j (j < NE) is
  // position e % 64 of chunk c0 + e / 64 (part (e / 64) % KP's chunk
  // (e / 64) / KP), the inputs of each loaded one round ahead
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
      if (e < CH * 64 && c0 + (e >> 6) < nch) {
        const int c = e >> 6;
        lb_fill_pos(smem, (uint32_t)(64 * (c / KP) + (e & 63)) * kSlotB + 64u * (uint32_t)(c % KP),
                    xn[j]);
      }
    }
    if (c0 + CH < nch) xload(c0 + CH);
    __syncthreads();
    acc = lb_chunks<KP, M>(w9, pb, c0 + part, nch, acc);
    if (c0 + CH < nch) __syncthreads();
  }
  lds_st(kRed + 4u * (uint32_t)(part * RB + rl), acc);
  __syncthreads();
  if (tid < nr) {
    float v = lds_ld(kRed + 4u * (uint32_t)tid);
#pragma unroll
    for (int q = 1; q < KP; q++) v += lds_ld(kRed + 4u * (uint32_t)(q * RB + tid));
    y[r0 + tid] = f32_to_bf16(v);
  }
}

static size_t lb_nib_lds(int rbk, int m) {
  return (size_t)64 * m * 4 * (16 * (256 / rbk) + 4) + 256 * 4;  // tables + part sums
}

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

// MFMA form, for 1 to 8 input rows (K a multiple of 256): y[r][n] for every
// input row r at once.  Block = 4 waves = 4/KS slabs of 16 weight rows x KS
// parts of K (KS = 4, 2 or 1 dividing the chunks of 256 inputs).  Per chunk
// (two groups, 36 bytes a row) lane l holds its row l%16's 9 dwords and, per
// 32 inputs, turns the byte of its row at inputs 8(l/16) .. +8 into 8 bf16
// values +-1 in registers (bf16 1.0 is 0x3F80; bit i of the byte becomes the
// sign bit of value i) and runs one 16x16x32 bf16 MFMA against the input rows
// at the same inputs (the MFMA's columns; those past the rows repeat row 0
// and are not stored): the products are +-x exactly.  A group's fp32 sum (4
// MFMAs) is scaled by its d (fp16) and accumulated; the block adds its K
// parts in part order through LDS and stores bf16.

// Sign bits to bf16 +-1 operands.  bf16 1.0 is 0x3F80; bit i of a sign word
// becomes the sign bit of value i, values paired per dword (value 2p in the
// low half, 2p+1 in the high half).  For a pair of bits (i, i+1), i even:
// R = rotl(w, 15) holds bit i+1 at (i+16) mod 32, so Z = the half of w that
// holds bit i merged with the other half of R holds bit i at i and bit i+1 at
// i+16 (mod 32), and rotr(Z, i - 15) puts them at bits 15 and 31; a mask and
// an or with 1.0 in both halves finish the pair.  The three constants come in
// registers (kernel arguments): gfx950's three-operand instructions take no
// literal, and with constants in sight the compiler folds the rotations into
// quarter-rate multiplies.
struct SignK {
  uint32_t half;  // 0x0000FFFF
  uint32_t sign;  // 0x80008000
  uint32_t one;   // 0x3F803F80
};
// Z for the pairs whose low bit lies in the low half of w (lo = true) or in
// the high half.
__device__ __forceinline__ uint32_t q1_spread(uint32_t w, bool lo, const SignK& k) {
  const uint32_t r = __builtin_amdgcn_alignbit(w, w, 17);  // rotl(w, 15)
  return lo ? ((w & k.half) | (r & ~k.half)) : ((w & ~k.half) | (r & k.half));
}
// The 8 values of sign bits i0 .. i0+7 (i0 = 8 * byte) from their Z; `one`
// is k.one held in a vector register (so that the mask and the or are one
// v_and_or_b32 with the mask as its scalar operand).
__device__ __forceinline__ v8bf q1_pairs(uint32_t z, uint32_t i0, const SignK& k, uint32_t one) {
  uint32_t r[4];
#pragma unroll
  for (int p = 0; p < 4; p++)
    r[p] = (__builtin_amdgcn_alignbit(z, z, (i0 + 2 * p - 15) & 31) & k.sign) | one;
  return __builtin_bit_cast(v8bf, r);
}
// A kernel argument copied into a vector register (a DPP move the compiler
// does not fold back into a scalar).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xE4, 0xF, 0xF, false);
}

constexpr SignK kSignK = {0x0000FFFFu, 0x80008000u, 0x3F803F80u};

struct QmStage {
  uint32_t w[9];  // the chunk of the lane's row: d0, 16 bit-bytes, d1, 16 bit-bytes
  u32x4 xb[8];    // the lane's input row at inputs 128h + 32s + 8(l/16) .. +8
};

template <int P, int WPB>
__global__ __launch_bounds__(64 * WPB) void lowbit_gemv_q1_mfma_kernel(
    const uint8_t* __restrict__ blocks, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, int rows, int n, int k, int ks, SignK sk) {
  __shared__ __align__(16) float s_part[WPB][256];  // per wave 16 x 16 sums, column-major
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int spb = WPB / ks;
  const int slab = blockIdx.x * spb + wv / ks, kp = wv % ks;
  // part kp: chunks kp nch / ks .. (kp + 1) nch / ks - 1 (at least one: ks <= nch)
  const int nch = k / 256, c0 = kp * nch / ks, nc = (kp + 1) * nch / ks - c0;
  const int row = slab * 16 + col;
  const int rowc = row < n ? row : n - 1;  // rows past n decode the last row (not stored)
  const uint32_t* wrow = reinterpret_cast<const uint32_t*>(blocks + (size_t)rowc * 36 * nch);
  const uint16_t* pa = x + (size_t)(col < rows ? col : 0) * k + 8 * g;
  const uint32_t one = in_vgpr(sk.one);

  auto issue = [&](QmStage& st, int c) {
#pragma unroll
    for (int i = 0; i < 9; i++) st.w[i] = wrow[9 * c + i];
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int s2 = 0; s2 < 4; s2++)
        st.xb[4 * h + s2] = ld16(pa + (size_t)c * 256 + h * 128 + 32 * s2);
  };
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](QmStage& st) {
    // the 16 bit-bytes of each group as 4 aligned dwords (group 0 starts 2
    // bytes in); byte 4s + l/16 of a group is byte l/16 of its dword s
    uint32_t u[8];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      u[q] = __builtin_amdgcn_alignbyte(st.w[q + 1], st.w[q], 2);
      u[4 + q] = st.w[5 + q];
    }
    const float dg[2] = {lb_f16(st.w[0] & 0xFFFFu), lb_f16(st.w[4] >> 16)};
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 4; s2++) {
        // byte g of sign word s2: bits 8g .. 8g+7 (low half of the word for g < 2)
        const v8bf a = q1_pairs(q1_spread(u[4 * h + s2], g < 2, sk), 8 * g, sk, one);
        c = mfma_bf16(a, __builtin_bit_cast(v8bf, st.xb[4 * h + s2]), c);
      }
      // lane l holds weight rows 4(l/16) + v; their d is held by lanes 4(l/16) + v
#pragma unroll
      for (int v = 0; v < 4; v++) acc[v] = fmaf(c[v], __shfl(dg[h], 4 * g + v, kWave), acc[v]);
    }
  };
  QmStage st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], c0 + p);
  for (int i0 = 0; i0 < nc - P; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p]);
      issue(st[p], c0 + i0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p]);
  pin4(acc);  // the MFMAs run with every lane, before any divergent use

  *reinterpret_cast<v4f*>(&s_part[wv][col * 16 + 4 * g]) = v4f{acc[0], acc[1], acc[2], acc[3]};
  __syncthreads();
  const int cc = tid >> 4, i = tid & 15;  // input row cc, weight row i of each slab
  if (cc >= rows) return;
  for (int s2 = 0; s2 < spb; s2++) {
    float v = s_part[s2 * ks][cc * 16 + i];
    for (int q = 1; q < ks; q++) v += s_part[s2 * ks + q][cc * 16 + i];
    const int r = (blockIdx.x * spb + s2) * 16 + i;
    if (r < n) y[(size_t)cc * n + r] = f32_to_bf16(v);
  }
}

// Wide MFMA form, for 1 to 8 input rows (K a multiple of 256, the input
// rows within kQ4XBytes) and many weight rows: a wave owns 64 weight rows
// (four 16-row tiles) over its part of K, so each read of the input rows
// serves four MFMAs, and lane l loads the 36 contiguous bytes of row l's
// chunk (two dwordx4 and a dword) instead of every lane loading its tile
// row's 9 dwords one at a time.  The block first copies the input rows into
// LDS (row stride padded by 16 bytes, so the 16 columns of a read fall on
// different banks).  Per chunk the lane re-aligns its chunk (two groups of 16
// bit-bytes as 8 dwords; d0 | d1 << 16) into the wave's LDS area, and the
// tiles read back their rows' sign dwords.  The K order inside a 128-group is
// permuted so that one sign dword serves a lane for four MFMA steps: lane
// quarter g (l/16) takes sign dword g of the group (bytes 4g .. 4g+3, inputs
// 32g .. 32g+31), step s its byte s (inputs 32g + 8s .. +8), and reads the
// input rows at the same inputs.  A group's fp32 sum is scaled by its d (the
// d of the lane's 4 result rows: one 16-byte LDS read) and accumulated; K
// parts are added in part order.
constexpr int kQ4Stride = 10;           // LDS dwords per row of sign words (8 used)
constexpr int kQ4XBytes = 48 * 1024;    // the largest rows x K x 2 staged in LDS

struct Q4Stage {
  uint32_t w[9];  // this lane's row, one chunk: d0, 16 bit-bytes, d1, 16 bit-bytes
};

template <int P>
__global__ __launch_bounds__(256) void lowbit_gemv_q1_mfma4_kernel(
    const uint8_t* __restrict__ blocks, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, int rows, int n, int k, int ks, SignK sk) {
  constexpr int T = 4;
  extern __shared__ __align__(16) uint8_t q4_dyn[];           // input rows, [rows][k + 8] bf16
  __shared__ __align__(16) uint32_t s_u[4][64 * kQ4Stride];  // per wave: sign dwords by row
  __shared__ __align__(16) uint32_t s_d[4][64];               // per wave: d0 | d1 << 16 by row
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int xs = k + 8;  // LDS row stride of the input rows (elements)
  uint16_t* sx = reinterpret_cast<uint16_t*>(q4_dyn);
  for (int i = tid; i < rows * (k / 8); i += 256) {
    const int r = i / (k / 8), e = 8 * (i - r * (k / 8));
    *reinterpret_cast<u32x4*>(sx + r * xs + e) = ld16(x + (size_t)r * k + e);
  }
  const int spb = 4 / ks;
  const int slab = blockIdx.x * spb + wv / ks, kp = wv % ks;
  const int nch = k / 256, nc = nch / ks, c0 = kp * nc;
  const int lrow = slab * 64 + lane;
  const int rowc = lrow < n ? lrow : n - 1;  // rows past n decode the last row (not stored)
  const uint32_t* wrow = reinterpret_cast<const uint32_t*>(blocks + (size_t)rowc * 36 * nch);
  const uint16_t* pa = sx + (col < rows ? col : 0) * xs + 32 * g;
  const uint32_t one = in_vgpr(sk.one);
  uint32_t* su = s_u[wv];
  uint32_t* sd = s_d[wv];
  __syncthreads();

  auto issue = [&](Q4Stage& st, int c) {
    const uint32_t* src = wrow + 9 * c;
    const u32x4 a = *reinterpret_cast<const u32x4*>(src);
    const u32x4 b = *reinterpret_cast<const u32x4*>(src + 4);
    st.w[0] = a[0]; st.w[1] = a[1]; st.w[2] = a[2]; st.w[3] = a[3];
    st.w[4] = b[0]; st.w[5] = b[1]; st.w[6] = b[2]; st.w[7] = b[3];
    st.w[8] = src[8];
  };
  float acc[T][4];
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int v = 0; v < 4; v++) acc[t][v] = 0.f;
  auto consume = [&](Q4Stage& st, int c) {
    // this lane's chunk re-aligned into the wave's LDS area
    uint32_t* dst = su + lane * kQ4Stride;
#pragma unroll
    for (int q = 0; q < 4; q += 2) {
      uint2 p0, p1;
      p0.x = __builtin_amdgcn_alignbyte(st.w[q + 1], st.w[q], 2);
      p0.y = __builtin_amdgcn_alignbyte(st.w[q + 2], st.w[q + 1], 2);
      p1.x = st.w[5 + q];
      p1.y = st.w[6 + q];
      *reinterpret_cast<uint2*>(dst + q) = p0;
      *reinterpret_cast<uint2*>(dst + 4 + q) = p1;
    }
    sd[lane] = (st.w[0] & 0xFFFFu) | (st.w[4] & 0xFFFF0000u);
    asm volatile("" ::: "memory");
    u32x4 dd[T];
#pragma unroll
    for (int t = 0; t < T; t++) dd[t] = *reinterpret_cast<const u32x4*>(sd + 16 * t + 4 * g);
    // per group: the four tiles' MFMA chains interleaved, their results
    // read after all of them
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v4f cv[T];
      uint32_t z[T][2];  // spread of the sign word's low and high halves
#pragma unroll
      for (int t = 0; t < T; t++) {
        const uint32_t uw = su[(16 * t + col) * kQ4Stride + g + 4 * h];
        z[t][0] = q1_spread(uw, true, sk);
        z[t][1] = q1_spread(uw, false, sk);
        cv[t] = v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s2 = 0; s2 < 4; s2++) {
        const v8bf b = *reinterpret_cast<const v8bf*>(pa + c * 256 + 128 * h + 8 * s2);
#pragma unroll
        for (int t = 0; t < T; t++) {
          // byte s2 of the sign word: bits 8 s2 .. 8 s2 + 7
          cv[t] = mfma_bf16(q1_pairs(z[t][s2 >> 1], 8 * s2, sk, one), b, cv[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < T; t++)
#pragma unroll
        for (int v = 0; v < 4; v++)
          acc[t][v] = fmaf(cv[t][v], lb_f16(h ? (dd[t][v] >> 16) : (dd[t][v] & 0xFFFFu)), acc[t][v]);
    }
    asm volatile("" ::: "memory");
  };
  // ring of P chunks (P divides the part's chunks: every load is used)
  Q4Stage st[P];
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], c0 + p);
  for (int i0 = 0; i0 < nc - P; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p], c0 + i0 + p);
      issue(st[p], c0 + i0 + P + p);
    }
  }
#pragma unroll
  for (int p = 0; p < P; p++) consume(st[p], c0 + nc - P + p);
#pragma unroll
  for (int t = 0; t < T; t++) pin4(acc[t]);  // the MFMAs run with every lane, before any divergent use

  // K-part sums per wave and tile, column-major, over the input rows' LDS
  // once every wave is done with them (rows * (k + 8) * 2 >= 16 KB: k >= 1024)
  __syncthreads();
  float(*s_part)[T][256] = reinterpret_cast<float(*)[T][256]>(q4_dyn);
#pragma unroll
  for (int t = 0; t < T; t++)
    *reinterpret_cast<v4f*>(&s_part[wv][t][col * 16 + 4 * g]) =
        v4f{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
  __syncthreads();
  const int cc = tid >> 4, i = tid & 15;  // input row cc, weight row i of each tile
  if (cc >= rows) return;
  for (int s2 = 0; s2 < spb; s2++) {
#pragma unroll
    for (int t = 0; t < T; t++) {
      float v = s_part[s2 * ks][t][cc * 16 + i];
      for (int q = 1; q < ks; q++) v += s_part[s2 * ks + q][t][cc * 16 + i];
      const int rr = (blockIdx.x * spb + s2) * 64 + 16 * t + i;
      if (rr < n) y[(size_t)cc * n + rr] = f32_to_bf16(v);
    }
  }
}

// The wide form's launch: K parts the fewest of 1, 2, 4 dividing the chunks
// that gives at least 4096 waves, else the most that divide; ring depth the
// largest divisor of a part's chunks up to 8 (a whole part of 8 chunks or
// fewer is loaded at once).
template <int P>
static void lb_mfma4_one(dim3 grid, size_t lds, const uint8_t* blocks, const uint16_t* x,
                         uint16_t* y, int rows, int n, int k, int ks, hipStream_t stream) {
  hipLaunchKernelGGL(lowbit_gemv_q1_mfma4_kernel<P>, grid, dim3(256), lds, stream, blocks, x, y,
                     rows, n, k, ks, kSignK);
}
template <int P>
static hipError_t lb_mfma4_lds(size_t lds) {
  static size_t raised[kLdsDevices] = {};
  return ensure_dyn_lds(reinterpret_cast<const void*>(lowbit_gemv_q1_mfma4_kernel<P>), lds, raised);
}
static hipError_t lb_mfma4_launch(const uint8_t* blocks, const uint16_t* x, uint16_t* y,
                                  int rows, int n, int k, hipStream_t stream) {
  const int nch = k / 256, slabs = (n + 63) / 64;
  int ks = 1;
  for (int c : {1, 2, 4}) {
    if (nch % c) continue;
    ks = c;
    if (slabs * c >= 4096) break;
  }
  const int nc = nch / ks;
  int p = 1;
  for (int d = 8; d >= 1; d--)
    if (nc % d == 0) {
      p = d;
      break;
    }
  const int spb = 4 / ks;
  size_t lds = (size_t)rows * (k + 8) * 2;
  if (lds < 4 * 4 * 256 * 4) lds = 4 * 4 * 256 * 4;  // the K-part sums reuse it
  const dim3 grid((slabs + spb - 1) / spb);
  hipError_t e = hipSuccess;
  switch (p) {
#define Q4_CASE(P)                                                          \
  case P:                                                                   \
    e = lb_mfma4_lds<P>(lds);                                               \
    if (e == hipSuccess) lb_mfma4_one<P>(grid, lds, blocks, x, y, rows, n, k, ks, stream); \
    break;
    Q4_CASE(8)
    Q4_CASE(7)
    Q4_CASE(6)
    Q4_CASE(5)
    Q4_CASE(4)
    Q4_CASE(3)
    Q4_CASE(2)
    Q4_CASE(1)
#undef Q4_CASE
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

// The MFMA form's launch: K parts the fewest of 1, 2, 4 dividing the chunks
// that gives at least 512 blocks, else the most that divide (more parts, more
// blocks); ring depth 2 where it divides a part's chunks, else 1.
static hipError_t lb_mfma_launch(const uint8_t* blocks, const uint16_t* x, uint16_t* y, int rows,
                                 int n, int k, hipStream_t stream) {
  const int nch = k / 256, slabs = (n + 15) / 16;
  // K parts a block (4 waves: 4 / ks slabs of ks parts): the fewest of 1 and
  // 2 that give 512 blocks, else 4 (more waves for few weight rows), at most
  // nch; parts of nch / ks chunks rounded down or up.  Fewer than 256 slabs
  // (a block a slab would leave CUs idle): blocks of 8 waves, one slab of 8
  // parts.  A ring of 2 chunks when every part's count is even, else 1.
  int ks = 4;
  for (int c : {1, 2})
    if ((slabs + 4 / c - 1) / (4 / c) >= 512) {
      ks = c;
      break;
    }
  const bool w8 = ks == 4 && slabs < 256 && nch >= 8;
  if (w8) ks = 8;
  while (ks > nch) ks >>= 1;
  const int spb = (w8 ? 8 : 4) / ks;
  const dim3 grid((slabs + spb - 1) / spb);
  const bool p2 = nch % ks == 0 && (nch / ks) % 2 == 0;
  if (w8) {
    if (p2)
      hipLaunchKernelGGL((lowbit_gemv_q1_mfma_kernel<2, 8>), grid, dim3(512), 0, stream, blocks,
                         x, y, rows, n, k, ks, kSignK);
    else
      hipLaunchKernelGGL((lowbit_gemv_q1_mfma_kernel<1, 8>), grid, dim3(512), 0, stream, blocks,
                         x, y, rows, n, k, ks, kSignK);
  } else if (p2) {
    hipLaunchKernelGGL((lowbit_gemv_q1_mfma_kernel<2, 4>), grid, dim3(256), 0, stream, blocks, x,
                       y, rows, n, k, ks, kSignK);
  } else {
    hipLaunchKernelGGL((lowbit_gemv_q1_mfma_kernel<1, 4>), grid, dim3(256), 0, stream, blocks, x,
                       y, rows, n, k, ks, kSignK);
  }
  return hipGetLastError();
}

// Weight rows from which several-row calls take the wide form (64 rows a
// wave): below it there are too few waves to spread over the CUs.
constexpr int kQ4MinRows = 32768;

hipError_t launch_lowbit_q1(const uint8_t* blocks, const uint16_t* x, uint16_t* y, int rows,
                            int n, int k, hipStream_t stream) {
  if (rows > 1) {  // K % 256 == 0
    if (n >= kQ4MinRows && (size_t)rows * (k + 8) * 2 <= kQ4XBytes)
      return lb_mfma4_launch(blocks, x, y, rows, n, k, stream);
    return lb_mfma_launch(blocks, x, y, rows, n, k, stream);
  }
  // the nibble-table form: rows per block RB the largest of 128, 64, 32 that
  // gives 2048 blocks, else the largest that gives 256, else 16; chunks per
  // thread and round M the fewest (up to 5) that take all of K in one round,
  // as long as the round's tables stay within kLbRoundChunks chunks
  // (kLbRoundChunksOne when the grid has at most one block a CU)
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
    const int lim = (n + rbk - 1) / rbk <= kLbCus ? kLbRoundChunksOne : kLbRoundChunks;
    while (m > 1 && kp * m > lim) m--;
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
