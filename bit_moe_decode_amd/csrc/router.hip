// router.hip -- RMSNorm folded into the router logits, top-8, gates, the
// expert dedup table and the FP8 activation blocks, in one launch.
//
// #85 Mod. row 10 ("router norm in its logits"): the router multiplies
// bf16(x * gamma) and scales the logits by the row's rstd, which also scales
// the FP8 activation blocks.  Mod. row 9: top-8 rounds take the maximum and
// break exact ties by the lower expert ID; picks keep their order.
// Mod. rows 16 and 20: the step's distinct experts, first use slot-major,
// owner = the earliest job (lowest row on a tie).
//
// Grid (nc, ceil(E/64)), 256 threads.  Block (c, eg) handles the K chunk
// [c*chunk, (c+1)*chunk) for experts eg*64 .. eg*64+63 (16 per wave) with a
// bf16 16x16x32 MFMA whose columns are the token rows; the partial dots go to
// the workspace.  Blocks with eg == 0 also write the chunk's x^2 partial sums
// and quantise the chunk's activation blocks.  The last block to arrive sums
// the partials in chunk order and finishes the routing for every row.
#include "device_common.h"

namespace moe {

constexpr int kChunkMax = 1024;
constexpr int kEMax = 1024;

typedef short v8s __attribute__((ext_vector_type(8)));

// Order key of a logit: unsigned compare = float order, -0 == +0, NaN (1)
// below every number (-inf maps to 0x007FFFFF), 0 = already picked.
__device__ __forceinline__ uint32_t topk_vkey(float z) {
  if (z != z) return 1u;
  const uint32_t b = (z == 0.0f) ? 0u : __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct RouterSmem {
  union {
    uint16_t u[kMaxRows][kChunkMax + 8];  // bf16(x * gamma) of this chunk
    float z[kMaxRows * kEMax];            // finish: logits of every row
  };
  float red[4][kMaxRows];
  float rstd[kMaxRows];
  int ids[kMaxRows][8];
  float zsel[kMaxRows][8];
  int g_expert[64];
  uint32_t g_mask[64];
  uint8_t g_slot[64][8];
  uint8_t g_owner[64][2];
  int n_groups;
  int last;
};

template <int CB>  // K blocks of 128 per chunk
__global__ __launch_bounds__(256) void moe_router_kernel(const uint16_t* __restrict__ x,
                                                         Weights w, Ws ws, Dims d) {
  __shared__ RouterSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = blockIdx.x, eg = blockIdx.y;
  const int H = d.H, R = d.rows, E = d.E;
  constexpr int chunk = CB * 128;
  const int k0 = c * chunk;

  // the router weights of this wave's 16 experts over the chunk: issued first,
  // they do not depend on the staged activations
  constexpr int NKS = CB * 4;  // 32-wide K steps of the chunk
  const int e0 = __builtin_amdgcn_readfirstlane(eg * 64 + wv * 16);  // wave-uniform
  const int col = lane & 15, kq = (lane >> 4) * 8;
  u32x4 a[NKS];
  if (e0 < E) {
    const uint16_t* wr = w.router + (size_t)(e0 + col) * H + k0 + kq;
#pragma unroll
    for (int i = 0; i < NKS; i++) a[i] = ld16(wr + i * 32);
  }

  // -- 1. stage u = bf16(x * gamma) for the chunk and the x^2 partial sums
  float ss[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; r++) ss[r] = 0.f;
  for (int k = tid; k < chunk; k += 256) {
    const float gk = bf16_to_f32(w.gamma[k0 + k]);
#pragma unroll
    for (int r = 0; r < kMaxRows; r++) {
      if (r < R) {
        const float xv = bf16_to_f32(x[(size_t)r * H + k0 + k]);
        sm.u[r][k] = f32_to_bf16(xv * gk);  // exact product, one rounding
        ss[r] = fmaf(xv, xv, ss[r]);
      }
    }
  }
  if (eg == 0) {
#pragma unroll
    for (int r = 0; r < kMaxRows; r++) {
      float v = ss[r];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
      if (lane == 0) sm.red[wv][r] = v;
    }
  }
  __syncthreads();
  if (eg == 0) {
    if (tid < R)
      ws.ss_part[c * d.max_rows + tid] =
          ((sm.red[0][tid] + sm.red[1][tid]) + sm.red[2][tid]) + sm.red[3][tid];
    // -- 2. FP8 activation blocks of this chunk: s = amax/448, q = e4m3(u/s)
    const int nkc = chunk / 128;
    for (int p = wv; p < R * nkc; p += 4) {
      const int r = p / nkc, kb = p % nkc;
      const float u0 = bf16_to_f32(sm.u[r][kb * 128 + 2 * lane]);
      const float u1 = bf16_to_f32(sm.u[r][kb * 128 + 2 * lane + 1]);
      const float amax = wave_max_nonneg(fmaxf(fabsf(u0), fabsf(u1)));
      const float s = amax / 448.0f;
      const uint32_t q = (s > 0.f) ? f32x2_to_e4m3(u0 / s, u1 / s) : 0u;
      *reinterpret_cast<uint16_t*>(ws.act_q + (size_t)r * H + k0 + kb * 128 + 2 * lane) =
          (uint16_t)q;
      if (lane == 0) ws.act_s[r * (H / 128) + k0 / 128 + kb] = s;
    }
  }

  // -- 3. router partial dots: 16 experts per wave x token-row columns
  if (e0 < E) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    // columns past the step's rows read row 0 of the staged u and are never stored
    const int brow = col < R ? col : 0;
#pragma unroll
    for (int i = 0; i < NKS; i++) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(&sm.u[brow][i * 32 + kq]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[i]),
                                                    __builtin_bit_cast(v8bf, b), acc, 0, 0, 0);
    }
    pin4(acc);  // the MFMA chain runs with every lane, before the row-dependent store
    if (col < R) {
      float* dst = ws.part + ((size_t)c * d.max_rows + col) * E + e0 + 4 * (lane >> 4);
#pragma unroll
      for (int v = 0; v < 4; v++) dst[v] = acc[v];
    }
  }

  // -- 4. arrival; the last block finishes the routing.  Producers release
  // (L2 write-back), only the last block acquires (L2 invalidate).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) sm.last = (atomicAdd(ws.ctrl_router, 1u) == gridDim.x * gridDim.y - 1);
  __syncthreads();
  if (!sm.last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // sums over the K chunks, in chunk order; every thread issues all of its
  // loads (float4 over 4 experts, all chunks, two groups) before adding
  constexpr int kNcMax = 16;
  if (tid < R) {
    float v[kNcMax];
#pragma unroll
    for (int q = 0; q < kNcMax; q++) v[q] = q < d.nc ? ws.ss_part[q * d.max_rows + tid] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kNcMax; q++)
      if (q < d.nc) s += v[q];
    const float rs = 1.0f / sqrtf(s / (float)H + d.eps);
    sm.rstd[tid] = rs;
    ws.rstd[tid] = rs;
  }
  __syncthreads();
  {
    const int n4 = R * E / 4;  // groups of 4 (row, expert) logits
    for (int i0 = tid; i0 < n4; i0 += 512) {
      v4f v[2][kNcMax];
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int i = i0 + 256 * h < n4 ? i0 + 256 * h : i0;
        const int r = (4 * i) / E, e = 4 * i - r * E;
#pragma unroll
        for (int q = 0; q < kNcMax; q++)
          if (q < d.nc)
            v[h][q] = *reinterpret_cast<const v4f*>(&ws.part[((size_t)q * d.max_rows + r) * E + e]);
      }
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int i = i0 + 256 * h;
        if (i >= n4) break;
        const int r = (4 * i) / E, e = 4 * i - r * E;
        v4f acc = v[h][0];
#pragma unroll
        for (int q = 1; q < kNcMax; q++)
          if (q < d.nc) acc += v[h][q];
        const float rs = sm.rstd[r];
        v4f z = {rs * acc[0], rs * acc[1], rs * acc[2], rs * acc[3]};
        *reinterpret_cast<v4f*>(&sm.z[r * E + e]) = z;
        *reinterpret_cast<v4f*>(&ws.logits[(size_t)r * E + e]) = z;
      }
    }
  }
  if (tid < 64) {
    sm.g_mask[tid] = 0u;
#pragma unroll
    for (int r = 0; r < 8; r++) sm.g_slot[tid][r] = 0xFF;
  }
  __syncthreads();

  // top-8 per row, one wave a row; lane l holds experts l, l+64, ...  A round
  // takes the largest value key across the wave (DPP max); when one lane holds
  // it (ballot) that lane's expert is the pick, and only an exact tie runs the
  // expert-ID reduction (#85 Mod. row 9).  Within a lane, scanning experts in
  // increasing order with a strict compare keeps the lowest ID among equals.
  for (int r = wv; r < R; r += 4) {
    uint32_t key[kEMax / kWave];
#pragma unroll
    for (int i = 0; i < kEMax / kWave; i++) {
      const int e = lane + kWave * i;
      key[i] = (e < E) ? topk_vkey(sm.z[r * E + e]) : 0u;
    }
    for (int j = 0; j < 8; j++) {
      uint32_t best = 0, bid = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < kEMax / kWave; i++)
        if (key[i] > best) {
          best = key[i];
          bid = lane + kWave * i;
        }
      const uint32_t m = dpp_umax(best);
      const uint64_t holders = __ballot(best == m);
      uint32_t e;
      if (__popcll(holders) == 1)
        e = __builtin_amdgcn_readlane(bid, __ffsll((unsigned long long)holders) - 1);
      else
        e = dpp_umin(best == m ? bid : 0xFFFFFFFFu);
#pragma unroll
      for (int i = 0; i < kEMax / kWave; i++)
        if (lane + kWave * i == (int)e) key[i] = 0u;
      if (lane == 0) {
        sm.ids[r][j] = (int)e;
        sm.zsel[r][j] = sm.z[r * E + e];
      }
    }
    if (lane == 0) {
      float mz = sm.zsel[r][0];
      for (int j = 1; j < 8; j++) mz = fmaxf(mz, sm.zsel[r][j]);
      float g[8], sum = 0.f;
      for (int j = 0; j < 8; j++) {
        g[j] = expf(sm.zsel[r][j] - mz);
        sum += g[j];
      }
      for (int j = 0; j < 8; j++) {
        ws.gates[r * 8 + j] = g[j] / sum;
        ws.ids[r * 8 + j] = sm.ids[r][j];
      }
    }
  }
  __syncthreads();

  // dedup table: lane p holds pick p in slot-major order (p = j*R + r).  The
  // lanes holding the same expert are found with one ballot per ID bit; the
  // lowest of them owns the group (first use), and a group's index is the
  // number of first uses before its owner.
  if (wv == 0) {
    const int P = 8 * R;
    const bool valid = lane < P;
    int ep = 0, jp = 0, rp = 0;
    if (valid) {
      jp = lane / R;
      rp = lane - jp * R;
      ep = sm.ids[rp][jp];
    }
    uint64_t same = __ballot(valid);
    if (d.no_dedup) {
      same = 1ull << lane;
    } else {
#pragma unroll
      for (int b = 0; b < 10; b++) {  // expert IDs < 1024
        const uint64_t bb = __ballot(valid && ((ep >> b) & 1));
        same &= ((ep >> b) & 1) ? bb : ~bb;
      }
    }
    const int owner = valid ? __ffsll((unsigned long long)same) - 1 : lane;
    const uint64_t first = __ballot(valid && owner == lane);
    const int gidx = __popcll(first & ((1ull << owner) - 1ull));
    if (valid) {
      atomicOr(&sm.g_mask[gidx], 1u << rp);
      sm.g_slot[gidx][rp] = (uint8_t)jp;
      if (owner == lane) {
        sm.g_expert[gidx] = ep;
        sm.g_owner[gidx][0] = (uint8_t)jp;
        sm.g_owner[gidx][1] = (uint8_t)rp;
      }
    }
    if (lane == 0) sm.n_groups = __popcll(first);
  }
  __syncthreads();
  const int D = sm.n_groups;
  if (tid < D) {
    const uint32_t m = sm.g_mask[tid];
    ws.grp_expert[tid] = sm.g_expert[tid];
    ws.grp_owner[2 * tid] = sm.g_owner[tid][0];
    ws.grp_owner[2 * tid + 1] = sm.g_owner[tid][1];
    ws.grp_mask[tid] = (uint8_t)m;
    int n = 0;
    for (int r = 0; r < 8; r++) {
      ws.grp_slot[tid * 8 + r] = sm.g_slot[tid][r];
      if ((m >> r) & 1u) ws.grp_rows[tid * 8 + n++] = (uint8_t)r;
    }
    ws.grp_nrows[tid] = (uint8_t)n;
  }
  if (tid == 0) {
    *ws.n_groups = D;
    *ws.ctrl_router = 0u;
  }
}

}  // namespace moe

namespace moe {
hipError_t launch_router(const uint16_t* x, const Weights& w, const Ws& ws, const Dims& d,
                         hipStream_t stream) {
  dim3 grid(d.nc, (d.E + 63) / 64);
  switch (d.chunk / 128) {
    case 1: hipLaunchKernelGGL(moe_router_kernel<1>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    case 2: hipLaunchKernelGGL(moe_router_kernel<2>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    case 3: hipLaunchKernelGGL(moe_router_kernel<3>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    case 4: hipLaunchKernelGGL(moe_router_kernel<4>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    case 5: hipLaunchKernelGGL(moe_router_kernel<5>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    case 6: hipLaunchKernelGGL(moe_router_kernel<6>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    case 7: hipLaunchKernelGGL(moe_router_kernel<7>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    case 8: hipLaunchKernelGGL(moe_router_kernel<8>, grid, dim3(256), 0, stream, x, w, ws, d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace moe
