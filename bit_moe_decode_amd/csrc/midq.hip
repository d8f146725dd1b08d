// midq.hip -- mid re-quantised to FP8 once per 1x128 block.
//
// #85 Mod. row 1 ("mid as FP8 once"): mid is quantised to FP8 with one scale
// per block and published as code bytes plus scale (Layout bullet: 128 code
// bytes and a 4-byte scale per block), which is what the down GEMV reads.
// Per block: s = amax / 448 (fp32), codes = E4M3(mid / s) with the hardware's
// round-to-nearest-even conversion; an all-zero block gets s = 0 and zero
// codes.  MXFP4 experts keep mid in fp32 (Mod. row 1) and are skipped.
//
// Grid (expert slots, max_rows): block (slot, c) quantises the c-th using row
// of that slot, one wave per 128-block, all loads issued before any reduction.
#include "device_common.h"

namespace moe {

__global__ __launch_bounds__(256) void moe_midq_kernel(Ws ws, Dims d, int routed_fp8) {
  const int slot = blockIdx.x, c = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int nrows, row, width;
  if (slot == 0) {
    if (d.Is == 0) return;
    nrows = d.rows;
    row = c;
    width = d.Is;
  } else {
    const int g = slot - 1;
    if (!routed_fp8 || g >= *ws.n_groups) return;
    nrows = ws.grp_nrows[g];
    row = c < nrows ? ws.grp_rows[g * 8 + c] : 0;
    width = d.I;
  }
  if (c >= nrows) return;
  const size_t base = ((size_t)slot * d.max_rows + row) * d.imax;
  const int nb = width / 128;
  constexpr int kPer = 8;  // 128-blocks per wave per pass, loads in flight together
  for (int b0 = wv * kPer; b0 < nb; b0 += 4 * kPer) {
    v2f v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int b = b0 + i < nb ? b0 + i : nb - 1;
      v[i] = *reinterpret_cast<const v2f*>(ws.mid + base + b * 128 + 2 * lane);
    }
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      if (b0 + i >= nb) break;
      const int b = b0 + i;
      const float amax = wave_max_nonneg(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])));
      const float s = amax / 448.0f;
      const uint32_t q = (s > 0.f) ? f32x2_to_e4m3(v[i][0] / s, v[i][1] / s) : 0u;
      *reinterpret_cast<uint16_t*>(ws.midq + base + b * 128 + 2 * lane) = (uint16_t)q;
      if (lane == 0) ws.midqs[((size_t)slot * d.max_rows + row) * (d.imax / 128) + b] = s;
    }
  }
}

hipError_t launch_midq(int rfmt, int max_groups, const Ws& ws, const Dims& d,
                       hipStream_t stream) {
  dim3 grid(1 + max_groups, d.rows);
  hipLaunchKernelGGL(moe_midq_kernel, grid, dim3(256), 0, stream, ws, d, rfmt == kFmtFp8 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
