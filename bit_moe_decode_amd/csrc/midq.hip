// midq.hip -- mid from the up/gate K-part sums, and its FP8 re-quantisation
// once per 1x128 block.
//
// #85 Mod. row 1: mid is quantised to FP8 once, with one scale per block of
// 128, and published as code bytes plus scale, which is what the down GEMV
// reads; MXFP4 experts keep mid in fp32.
//
// Block (b, pick, row), 128 threads: thread t owns intermediate element
// i = 128 b + t of (row, pick), pick 8 being the shared expert.  It adds the
// ks K-part sums of gate and of up in part order, then
//   mid = silu(gate * rstd) * (up * rstd)          (fp32)
// and the block quantises its 128 values: s = amax / 448 (fp32),
// codes = E4M3(mid / s) with the hardware's round-to-nearest-even conversion;
// an all-zero block gets s = 0 and zero codes.
#include "device_common.h"

namespace moe {

constexpr int kKsMax = 16;

__global__ __launch_bounds__(128) void moe_midq_kernel(Ws ws, Dims d, int routed_fp8) {
  __shared__ float s_max[2];
  const int b = blockIdx.x, j = blockIdx.y, r = blockIdx.z, t = threadIdx.x;
  const bool shared = j == 8;
  if (shared && d.Is == 0) return;
  const int width = shared ? d.Is : d.I;
  if (b * 128 >= width) return;
  const int u = r * 9 + j, i = b * 128 + t, KS = d.ks;
  const size_t base = (size_t)u * KS * d.imax + i;
  float gp[kKsMax], up[kKsMax];
#pragma unroll
  for (int q = 0; q < kKsMax; q++) {
    gp[q] = q < KS ? ws.gpart[base + (size_t)q * d.imax] : 0.f;
    up[q] = q < KS ? ws.upart[base + (size_t)q * d.imax] : 0.f;
  }
  float g = gp[0], v = up[0];
#pragma unroll
  for (int q = 1; q < kKsMax; q++)
    if (q < KS) {
      g += gp[q];
      v += up[q];
    }
  const float rs = ws.rstd[r];
  const float gt = g * rs, ut = v * rs;
  const float m = gt / (1.0f + expf(-gt)) * ut;
  ws.mid[(size_t)u * d.imax + i] = m;
  if (!shared && !routed_fp8) return;
  const float wm = wave_max_nonneg(fabsf(m));
  if ((t & 63) == 0) s_max[t >> 6] = wm;
  __syncthreads();
  const float amax = fmaxf(s_max[0], s_max[1]);
  const float s = amax / 448.0f;
  const uint32_t q = (s > 0.f) ? f32x2_to_e4m3(m / s, 0.f) : 0u;
  ws.midq[(size_t)u * d.imax + i] = (uint8_t)(q & 0xFFu);
  if (t == 0) ws.midqs[(size_t)u * (d.imax / 128) + b] = s;
}

hipError_t launch_midq(int rfmt, const Ws& ws, const Dims& d, hipStream_t stream) {
  const dim3 grid(d.imax / 128, 9, d.rows);
  hipLaunchKernelGGL(moe_midq_kernel, grid, dim3(128), 0, stream, ws, d, rfmt == kFmtFp8 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
