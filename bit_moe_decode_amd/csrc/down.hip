// down.hip -- down GEMV of the shared expert and of every distinct routed
// expert from the FP8 mid, and the gate-weighted combine.
//
// #85 Mod. row 16: down units take one expert's tile against every row that
// uses it; a row's output is summed over its units in the one-row form's
// order, so dedup changes no output bit.  Mod. row 1: down reads mid as the
// FP8 bytes and scales quantised once.  Mod. rows 18 and 21: 16-byte,
// nontemporal weight loads.
//
// Block = 4 waves, one expert slot, 64 output rows (16 a wave), full K.  Each
// wave runs one 16x16x128 FP8 MFMA per K block against the using rows' midq
// columns, scaled by weight scale x mid scale.  Results go to the per-row,
// per-pick buffer ybuf[row][pick][h] (pick 8 = shared expert).  The blocks of
// one 64-row output tile count their arrivals (D routed groups + the shared
// expert); the last one combines every row in pick order:
//   out = bf16(sum_{j<8} g_j * y_j + y_shared).
#include "device_common.h"

namespace moe {

template <int RFMT>
__global__ __launch_bounds__(256) void moe_down_kernel(Weights w, Ws ws, Dims d,
                                                       uint16_t* __restrict__ out) {
  constexpr int P = 8;  // K blocks in flight per wave
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = d.H, HT = H / 64;
  const int slot = blockIdx.x / HT, ht = blockIdx.x - slot * HT;
  const int has_sh = d.Is > 0;
  const int D = *ws.n_groups;
  int g = -1, nrows, K;
  const uint8_t* cd;
  const float* sd;
  if (slot == 0) {
    if (!has_sh) return;
    K = d.Is;
    nrows = d.rows;
    cd = w.sd_c;
    sd = w.sd_s;
  } else {
    g = slot - 1;
    if (g >= D) return;
    K = d.I;
    nrows = ws.grp_nrows[g];
    const size_t e = (size_t)ws.grp_expert[g];
    cd = w.down_c + e * (size_t)H * K;
    sd = reinterpret_cast<const float*>(w.down_s) + e * (size_t)(H / 128) * (K / 128);
  }
  const int nkb = K / 128;
  const int h0 = ht * 64 + wv * 16;
  const int col = lane & 15;
  const bool live = col < nrows;
  const int row = live ? (g < 0 ? col : (int)ws.grp_rows[g * 8 + col]) : 0;

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (RFMT == kFmtFp8 || g < 0) {
    const uint8_t* pw = cd + (size_t)(h0 + col) * K + (lane >> 4) * 32;
    const size_t mrow = ((size_t)slot * d.max_rows + row);
    const uint8_t* pm = ws.midq + mrow * d.imax + (lane >> 4) * 32;
    const float* psm = ws.midqs + mrow * (d.imax / 128);
    const float* psd = sd + (size_t)(h0 / 128) * nkb;
    struct Stage {
      u32x4 w0, w1, m0, m1;
      float sd, sm;
    } st[P];
    auto issue = [&](Stage& s, int kb) {
      s.w0 = ld_nt16(pw + kb * 128);
      s.w1 = ld_nt16(pw + kb * 128 + 16);
      if (live) {
        s.m0 = ld16(pm + kb * 128);
        s.m1 = ld16(pm + kb * 128 + 16);
        s.sm = psm[kb];
      } else {
        s.m0 = u32x4{0u, 0u, 0u, 0u};
        s.m1 = s.m0;
        s.sm = 0.f;
      }
      s.sd = psd[kb];
    };
#pragma unroll
    for (int p = 0; p < P; p++)
      if (p < nkb) issue(st[p], p);
    for (int kb = 0; kb < nkb; kb += P) {
#pragma unroll
      for (int p = 0; p < P; p++) {
        const int k = kb + p;
        if (k < nkb) {
          const v4f c = mfma_fp8(cat8(st[p].w0, st[p].w1), cat8(st[p].m0, st[p].m1));
          const float f = st[p].sd * st[p].sm;
#pragma unroll
          for (int v = 0; v < 4; v++) acc[v] = fmaf(c[v], f, acc[v]);
          if (k + P < nkb) issue(st[p], k + P);
        }
      }
    }
  }
  if (live) {
    const int pick = (g < 0) ? 8 : (int)ws.grp_slot[g * 8 + row];
    v4f y = {acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<v4f*>(ws.ybuf + ((size_t)row * 9 + pick) * H + h0 + 4 * (lane >> 4)) = y;
  }

  // ---- arrival per 64-row output tile; the last block combines
  __threadfence();
  __syncthreads();
  uint32_t* cnt = ws.ctrl_down + ht;
  if (tid == 0) s_last = (atomicAdd(cnt, 1u) == (uint32_t)(D + has_sh - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int hh = ht * 64 + lane;
  for (int r = wv; r < d.rows; r += 4) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) a = fmaf(ws.gates[r * 8 + j], ws.ybuf[((size_t)r * 9 + j) * H + hh], a);
    if (has_sh) a += ws.ybuf[((size_t)r * 9 + 8) * H + hh];
    out[(size_t)r * H + hh] = f32_to_bf16(a);
  }
  if (tid == 0) *cnt = 0u;
}

template __global__ void moe_down_kernel<kFmtFp8>(Weights, Ws, Dims, uint16_t*);

}  // namespace moe

namespace moe {
hipError_t launch_down(int rfmt, int max_groups, const Weights& w, const Ws& ws, const Dims& d,
                       uint16_t* out, hipStream_t stream) {
  dim3 grid((1 + max_groups) * (d.H / 64));
  if (rfmt != kFmtFp8) return hipErrorInvalidValue;
  hipLaunchKernelGGL((moe_down_kernel<kFmtFp8>), grid, dim3(256), 0, stream, w, ws, d, out);
  return hipGetLastError();
}
}  // namespace moe
