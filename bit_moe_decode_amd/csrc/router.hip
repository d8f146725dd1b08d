// router.hip -- router logits with the RMSNorm folded in, and the FP8
// activation blocks, in one launch with no cross-block synchronisation.
//
// #85 Mod. row 10: the router multiplies u = bf16(x * gamma) (the product is
// exact in fp32, rounded once) and scales each row's dots by its rstd; the
// same u, quantised per 1x128 block, is the activation of the up/gate GEMV,
// whose results take the rstd afterwards.  The routing launch (route.hip) then
// derives the top-8, gates and dedup table from these logits in one block
// (route.h).
//
// Grid E/EB blocks of 16 waves.  A block owns EB experts (1) over the whole
// hidden dimension, so its logits need no partial sums from
// other blocks: lane (wave w, q = lane/16, s = lane%16) takes columns
// 8s..8s+7 of the 128-blocks w + 16*(q + 4*it), keeps fp32 dots for its EB
// experts and every row and the row's sum of x^2; the 16 lanes of a DPP row
// are summed, then the 64 rows of the block in a fixed order, so every block
// derives the same rstd.  Row r's
// 128-block kb of activations is quantised by block (kb*R + r) modulo the
// grid, from the 16 lanes that hold it: s = amax/448, q = e4m3(u/s).  With at
// least R blocks, the R rows of a 128-block go to R different blocks, so a
// lane quantises at most one row of each 128-block it holds.  With bf16
// activations the owner stores u itself instead.
#include "device_common.h"

namespace moe {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two packed bf16 as the operand of v_dot2.  The value goes through a scalar
// parameter: a bit cast applied directly to an element of a vector variable
// (v[p]) compiles to a cast of element 0 with this compiler.
__device__ __forceinline__ v2bf as_bf16x2(uint32_t v) { return __builtin_bit_cast(v2bf, v); }

constexpr int kRtWaves = 16;   // waves per block
// experts per block: 1 at every width (E blocks spread the router's bytes
// over more CUs; against 2 a block from 2 rows up: 4 rows 188.0 -> 187.2,
// 8 rows 336.5 -> 335.9 us a step, outputs bitwise equal)
__host__ __device__ constexpr int router_experts(int rows) { return 1 + 0 * rows; }

// Element j (0..7) of eight packed bf16 values.
__device__ __forceinline__ float bf16_elem(const u32x4& v, int j) {
  const uint32_t w = v[j >> 1];
  return bf16_to_f32((uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// Lane (wave w, q = lane/16, s = lane%16) owns columns 8s .. 8s+7 of the
// 128-blocks kb = w + 16*(q + 4*it).
template <int R>
__global__ __launch_bounds__(1024) void moe_router_kernel(const uint16_t* __restrict__ x,
                                                          Weights w, Ws ws, Dims d) {
  constexpr int EB = router_experts(R);
  __shared__ float s_dot[kRtWaves * 4][EB][R];
  __shared__ float s_ss[kRtWaves * 4][R];
  __shared__ float s_rstd[R];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane >> 4, s = lane & 15;
  const int H = d.H, E = d.E, nkb = H / 128;
  const int e0 = blockIdx.x * EB;

  // the routing launch's records (route.hip) start unpublished
  const int nrec = (d.Is + d.groups * d.I) / (16 * (4 / d.ks));
  for (int t = blockIdx.x * blockDim.x + tid; t < nrec; t += gridDim.x * blockDim.x)
    ws.blk_rec[t] = 0u;

  float dot[EB][R], ss[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    ss[r] = 0.f;
#pragma unroll
    for (int e = 0; e < EB; e++) dot[e][r] = 0.f;
  }
  // 128-blocks per wave: at most 2 rounds for H <= 16384.  Every lane loads
  // (rows of 16 lanes past the last 128-block read block 0 and zero it), so
  // the loads carry no condition.
  for (int it = 0; it * 64 < nkb; it++) {
    const int kb = wv + 16 * (q + 4 * it);
    const bool on = kb < nkb;  // uniform over a row of 16 lanes
    const uint32_t col = (uint32_t)(on ? kb : 0) * 128u + 8u * s;  // 32-bit offsets
    u32x4 wr[EB], xv[R];
#pragma unroll
    for (int e = 0; e < EB; e++) wr[e] = ld16(w.router + ((uint32_t)(e0 + e) * H + col));
    const u32x4 gm = ld16(w.gamma + col);
#pragma unroll
    for (int r = 0; r < R; r++) xv[r] = ld16(x + ((uint32_t)r * H + col));
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < R; r++) xv[r] = on ? xv[r] : zero;
    // u = bf16(x * gamma) two columns at a time; the dots take bf16 pairs
    // (v_dot2 with fp32 accumulation)
#pragma unroll
    for (int r = 0; r < R; r++) {
#pragma unroll
      for (int p = 0; p < 4; p++) {
        const float x0 = bf16_elem(xv[r], 2 * p), x1 = bf16_elem(xv[r], 2 * p + 1);
        const uint32_t up = (uint32_t)f32_to_bf16(x0 * bf16_elem(gm, 2 * p)) |
                            ((uint32_t)f32_to_bf16(x1 * bf16_elem(gm, 2 * p + 1)) << 16);
        ss[r] = fmaf(x1, x1, fmaf(x0, x0, ss[r]));
#pragma unroll
        for (int e = 0; e < EB; e++)
          dot[e][r] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wr[e][p]), as_bf16x2(up),
                                                      dot[e][r], false);
      }
    }
    // The owner of (row, 128-block) quantises it from the 16 lanes that hold
    // it: s = amax/448, q = e4m3(u/s).
    // With at least R blocks, the R pairs (row, kb) of a 128-block go to R
    // different blocks, so this block owns at most one of them: row r with
    // kb * R + r = blockIdx.x (mod grid).  Its 8 inputs are still in
    // registers (picked by a select chain: an indexed register array would
    // go to scratch).
    const int r = (int)(((uint32_t)blockIdx.x + gridDim.x - ((uint32_t)(kb * R) % gridDim.x)) %
                        gridDim.x);
    if (on && r < R) {  // uniform over 16 lanes
      u32x4 xr = xv[0];
#pragma unroll
      for (int i = 1; i < R; i++) xr = i == r ? xv[i] : xr;
      do {
        if (d.act_bf16) {  // the experts take u itself: store its 8 bf16
          u32x4 ub;
#pragma unroll
          for (int p = 0; p < 4; p++)
            ub[p] = (uint32_t)f32_to_bf16(bf16_elem(xr, 2 * p) * bf16_elem(gm, 2 * p)) |
                    ((uint32_t)f32_to_bf16(bf16_elem(xr, 2 * p + 1) * bf16_elem(gm, 2 * p + 1))
                     << 16);
          *reinterpret_cast<u32x4*>(ws.act_u + ((uint32_t)r * H + col)) = ub;
          break;
        }
        float u[8], m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
          u[j] = bf16_to_f32(f32_to_bf16(bf16_elem(xr, j) * bf16_elem(gm, j)));
          m = fmaxf(m, fabsf(u[j]));
        }
        const float amax = __uint_as_float(row16_umax(__float_as_uint(m)));
        const float sc = amax / 448.0f;
        uint32_t c[4] = {0u, 0u, 0u, 0u};
        if (sc > 0.f) {
#pragma unroll
          for (int p = 0; p < 4; p++) c[p] = f32x2_to_e4m3(u[2 * p] / sc, u[2 * p + 1] / sc);
        }
        uint2 pk;
        pk.x = c[0] | (c[1] << 16);
        pk.y = c[2] | (c[3] << 16);
        *reinterpret_cast<uint2*>(ws.act_q + ((uint32_t)r * H + col)) = pk;
        if (d.act_q1) {  // the same codes in 1-bit operand order: 4 adjacent pairs
          uint8_t* qb = ws.act_qp + ((uint32_t)r * H + (col & ~127));
          const int t = (col & 127) >> 3;
#pragma unroll
          for (int j = 0; j < 4; j++)
            *reinterpret_cast<uint16_t*>(qb + q1_act_pos(t, j)) =
                (uint16_t)__builtin_amdgcn_perm(pk.y, pk.x, (uint32_t)((4 + j) << 8 | j));
        }
        if (s == 0) ws.act_s[r * nkb + kb] = sc;
      } while (false);
    }
  }

  // sums over the 16 lanes of a row, then over the rows of every wave in order
#pragma unroll
  for (int r = 0; r < R; r++) {
    ss[r] = row16_sum(ss[r]);
#pragma unroll
    for (int e = 0; e < EB; e++) dot[e][r] = row16_sum(dot[e][r]);
  }
  if (s == 0) {
#pragma unroll
    for (int r = 0; r < R; r++) {
      s_ss[wv * 4 + q][r] = ss[r];
#pragma unroll
      for (int e = 0; e < EB; e++) s_dot[wv * 4 + q][e][r] = dot[e][r];
    }
  }
  __syncthreads();
  if (tid < R) {
    float a = 0.f;
    for (int i = 0; i < kRtWaves * 4; i++) a += s_ss[i][tid];
    const float rs = 1.0f / sqrtf(a / (float)H + d.eps);
    s_rstd[tid] = rs;
    if (blockIdx.x == 0) ws.rstd[tid] = rs;
  }
  __syncthreads();
  if (tid < EB * R) {
    const int e = tid / R, r = tid - e * R;
    float a = 0.f;
    for (int i = 0; i < kRtWaves * 4; i++) a += s_dot[i][e][r];
    ws.logits[(size_t)r * E + e0 + e] = s_rstd[r] * a;
  }
}

hipError_t launch_router(const uint16_t* x, const Weights& w, const Ws& ws, const Dims& d,
                         hipStream_t stream) {
  const dim3 grid(d.E / router_experts(d.rows)), block(kRtWaves * kWave);
  switch (d.rows) {
    case 1: hipLaunchKernelGGL(moe_router_kernel<1>, grid, block, 0, stream, x, w, ws, d); break;
    case 2: hipLaunchKernelGGL(moe_router_kernel<2>, grid, block, 0, stream, x, w, ws, d); break;
    case 3: hipLaunchKernelGGL(moe_router_kernel<3>, grid, block, 0, stream, x, w, ws, d); break;
    case 4: hipLaunchKernelGGL(moe_router_kernel<4>, grid, block, 0, stream, x, w, ws, d); break;
    case 5: hipLaunchKernelGGL(moe_router_kernel<5>, grid, block, 0, stream, x, w, ws, d); break;
    case 6: hipLaunchKernelGGL(moe_router_kernel<6>, grid, block, 0, stream, x, w, ws, d); break;
    case 7: hipLaunchKernelGGL(moe_router_kernel<7>, grid, block, 0, stream, x, w, ws, d); break;
    case 8: hipLaunchKernelGGL(moe_router_kernel<8>, grid, block, 0, stream, x, w, ws, d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
