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

// Table-lookup form, for many rows (the LM head) and K a multiple of 256 (an
// even number of groups: a row is a whole number of 36-byte, dword-aligned
// pairs of groups).  Block = RW waves = 64*RW rows, one per lane.  The block's
// rows are one contiguous run of bytes; they are staged into LDS with
// coalesced 16-byte loads (a lane reading its own row straight from memory
// would touch a different cache line per lane).  Then for each chunk of 256
// inputs (two groups, 32 byte positions) the block fills an LDS table with,
// for every byte position p and byte value v, the signed sum of its 8 inputs:
//   T[p][v] = sum_{i<8} (bit i of v ? -x : +x)[256c + 8p + i]
// (a thread fills one position's values for some of the top bits, from pair
// sums), and each lane adds T[p][byte] over the 16 bytes of each group of its
// row -- one table read per 8 weights instead of 8 masked adds -- scales by
// the group's d and accumulates in fp32.
constexpr int kLbLutBytes = 32 * 256 * 4;
constexpr int kLbStageMax = 96 * 1024;

__device__ __forceinline__ float lb_bf16(uint32_t w, int hi) {
  return bf16_to_f32((uint16_t)(hi ? (w >> 16) : (w & 0xFFFFu)));
}
__device__ __forceinline__ float lb_f16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int RW>
__global__ __launch_bounds__(64 * RW) void lowbit_gemv_q1_lut_kernel(
    const uint8_t* __restrict__ blocks, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, int n, int k) {
  constexpr int NT = 64 * RW;        // threads = rows per block
  constexpr int VPT = 256 * 32 / NT;  // table values per thread per chunk
  extern __shared__ __align__(16) uint8_t smem[];
  float(*lut)[256] = reinterpret_cast<float(*)[256]>(smem);
  uint8_t* stage = smem + kLbLutBytes;
  const int tid = threadIdx.x;
  const int G = k / 128, nch = G / 2, rb = 18 * G;
  const int r0 = blockIdx.x * NT;
  const int nr = n - r0 < NT ? n - r0 : NT;

  // ---- stage the block's rows: [r0 * rb, (r0 + nr) * rb), 16-byte aligned
  // start (64 rows are 1152 * G bytes); a tail shorter than 16 bytes goes by
  // 2-byte loads, so nothing past the matrix is read
  {
    const uint8_t* src = blocks + (size_t)r0 * rb;
    const int bytes = nr * rb, n16 = bytes >> 4;
    for (int i0 = tid; i0 < n16; i0 += 8 * NT) {  // 8 loads in flight per thread
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; u++)
        if (i0 + u * NT < n16) v[u] = ld_nt16(src + 16 * (i0 + u * NT));
#pragma unroll
      for (int u = 0; u < 8; u++)
        if (i0 + u * NT < n16) *reinterpret_cast<u32x4*>(stage + 16 * (i0 + u * NT)) = v[u];
    }
    const int tail = bytes - 16 * n16;  // even
    if (tid < (tail >> 1))
      *reinterpret_cast<uint16_t*>(stage + 16 * n16 + 2 * tid) =
          *reinterpret_cast<const uint16_t*>(src + 16 * n16 + 2 * tid);
  }
  const int rowl = tid < nr ? tid : nr - 1;  // lanes past n decode the last row
  const uint32_t* myrow = reinterpret_cast<const uint32_t*>(stage + rowl * rb);
  // table role: byte position bp, values v = vb * VPT .. + VPT
  const int bp = tid / (256 / VPT), vb = tid % (256 / VPT);

  float acc = 0.f;
  for (int c = 0; c < nch; c++) {
    {
      const u32x4 xv = ld16(x + 256 * c + 8 * bp);
      float xs[8];
#pragma unroll
      for (int i = 0; i < 8; i++) xs[i] = lb_bf16(xv[i >> 1], i & 1);
      // values v = vb * VPT + 16 q + m: pair sums over bits 0..3, bits 4..7 added
      float ab[16];
#pragma unroll
      for (int m = 0; m < 16; m++)
        ab[m] = ((m & 1) ? -xs[0] : xs[0]) + ((m & 2) ? -xs[1] : xs[1]) +
                ((m & 4) ? -xs[2] : xs[2]) + ((m & 8) ? -xs[3] : xs[3]);
      float* dst = &lut[bp][vb * VPT];
#pragma unroll
      for (int q = 0; q < VPT / 16; q++) {
        const int hi = vb * VPT + 16 * q;  // bits 4..7 of v
        float hs = 0.f;
#pragma unroll
        for (int i = 4; i < 8; i++) hs += ((hi >> i) & 1) ? -xs[i] : xs[i];
#pragma unroll
        for (int m = 0; m < 16; m += 4)
          *reinterpret_cast<float4*>(dst + 16 * q + m) =
              float4{ab[m] + hs, ab[m + 1] + hs, ab[m + 2] + hs, ab[m + 3] + hs};
      }
    }
    __syncthreads();  // (the first pass also waits for the staged rows)
    uint32_t w[9];
#pragma unroll
    for (int i = 0; i < 9; i++) w[i] = myrow[9 * c + i];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const int b0 = 2 + j, b1 = 20 + j;  // bits of group 2c and of group 2c+1
      s0 += lut[j][(w[b0 >> 2] >> (8 * (b0 & 3))) & 0xFFu];
      s1 += lut[16 + j][(w[b1 >> 2] >> (8 * (b1 & 3))) & 0xFFu];
    }
    acc = fmaf(lb_f16(w[0] & 0xFFFFu), s0, acc);
    acc = fmaf(lb_f16(w[4] >> 16), s1, acc);
    __syncthreads();
  }
  if (tid < nr) y[r0 + tid] = f32_to_bf16(acc);
}

hipError_t launch_lowbit_q1(const uint8_t* blocks, const uint16_t* x, uint16_t* y, int n, int k,
                            hipStream_t stream) {
  // many rows: the table form, 128 rows a block where they fit the staging
  // area, else 64
  const int rb = 18 * (k / 128);
  if (n >= 16384 && k % 256 == 0 && 64 * rb <= kLbStageMax) {
    static const bool attrs = [] {
      const int mx = kLbLutBytes + kLbStageMax;
      return hipFuncSetAttribute(reinterpret_cast<const void*>(lowbit_gemv_q1_lut_kernel<2>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, mx) == hipSuccess &&
             hipFuncSetAttribute(reinterpret_cast<const void*>(lowbit_gemv_q1_lut_kernel<1>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, mx) == hipSuccess;
    }();
    if (!attrs) return hipErrorInvalidValue;
    if (128 * rb <= kLbStageMax) {
      const size_t sh = kLbLutBytes + 128 * rb;
      hipLaunchKernelGGL(lowbit_gemv_q1_lut_kernel<2>, dim3((n + 127) / 128), dim3(128), sh,
                         stream, blocks, x, y, n, k);
    } else {
      const size_t sh = kLbLutBytes + 64 * rb;
      hipLaunchKernelGGL(lowbit_gemv_q1_lut_kernel<1>, dim3((n + 63) / 64), dim3(64), sh, stream,
                         blocks, x, y, n, k);
    }
    return hipGetLastError();
  }
  int rows_blocks = (n + 3) / 4;
  int grid = rows_blocks < 1024 ? rows_blocks : 1024;
  hipLaunchKernelGGL(lowbit_gemv_q1_kernel, dim3(grid), dim3(256), 0, stream, blocks, x, y, n, k);
  return hipGetLastError();
}

}  // namespace moe
