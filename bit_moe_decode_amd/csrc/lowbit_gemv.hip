// lowbit_gemv.hip -- dense decode GEMV over 1-bit group-128 weights.
//
// 1-Bit Turbo, Q1_0_G128: 1-bit weights with one fp16 scale per group of 128
// (about 18 bytes a group: 572 MB for 4B parameters).  Layout: [N, K/128]
// blocks of 18 bytes = fp16 d (little-endian) + 16 bytes of bits; bit i of
// byte b is element 8b+i; bit 1 means -d.
//   y[n] = bf16( sum_g d[n,g] * sum_{k in g} sign[n,k] * x[k] )
//
// Block = 4 waves; x (bf16) is staged once per block into LDS as fp32, with
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

hipError_t launch_lowbit_q1(const uint8_t* blocks, const uint16_t* x, uint16_t* y, int n, int k,
                            hipStream_t stream) {
  int rows_blocks = (n + 3) / 4;
  int grid = rows_blocks < 1024 ? rows_blocks : 1024;
  hipLaunchKernelGGL(lowbit_gemv_q1_kernel, dim3(grid), dim3(256), 0, stream, blocks, x, y, n, k);
  return hipGetLastError();
}

}  // namespace moe
