// down.hip -- down GEMV of the shared expert and of every distinct routed
// expert from the FP8 mid, and the gate-weighted combine, in one launch with
// no cross-block synchronisation.
//
// #85 Mod. row 16: down units take one expert's tile against every row that
// uses it; a row's output is summed over its units in the one-row form's
// order, so dedup changes no output bit.  Mod. row 1: down reads mid as the
// FP8 bytes and scales quantised once.  Mod. rows 18 and 21: 16-byte,
// nontemporal weight loads.
//
// Block = 4 waves = HW sub-tiles of 16 output rows x KSD parts of K; the
// block owns 16*HW output rows and walks every expert of the step (shared
// first, then the routed groups in table order).  For each 128-wide K block of
// its part a wave loads its 16 weight rows row-contiguously, re-lays them
// through LDS into MFMA operand order and runs one 16x16x128 FP8 MFMA against
// the group's midq columns (one column per using row), scaled by weight scale
// x mid scale.  At the end of each group the wave files its partial into
// part[K part][row][pick][h] (pick 8 = shared expert): every (row, pick) has
// exactly one group, so no two writes collide.  Finally the block combines
//   out[r][h] = bf16( sum_{j<8} g_rj * y_rj[h] + y_r8[h] ),
//   y_rj = ((part_0 + part_1) + ...) in part order,
// the same arithmetic whether or not experts were deduplicated.
#include "device_common.h"

namespace moe {

struct DnStage {
  u32x4 w0, w1, m0, m1;
  float sd, sm;
};

constexpr int kGroupsMax = 65;  // 64 routed groups + the shared expert

template <int KSD, int P>
__global__ __launch_bounds__(256) void moe_down_kernel(Weights w, Ws ws, Dims d,
                                                       uint16_t* __restrict__ out) {
  constexpr int HW = 4 / KSD;   // 16-row output sub-tiles per block
  constexpr int BH = 16 * HW;   // output rows per block
  __shared__ uint8_t s_tile[4][kTileBytes];
  __shared__ float s_part[KSD][kMaxRows][9][BH];
  __shared__ int s_expert[kGroupsMax];
  __shared__ uint8_t s_nrows[kGroupsMax];
  __shared__ uint8_t s_row[kGroupsMax][16];
  __shared__ uint8_t s_pick[kGroupsMax][16];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hs = wv % HW, kp = wv / HW;
  const int H = d.H, I = d.I, nkb = I / 128, nkw = nkb / KSD;
  const int hb = blockIdx.x * BH, h0 = hb + hs * 16;
  const int has_sh = d.Is > 0;
  const int ng = *ws.n_groups + has_sh;

  // ---- the step's groups: index 0 is the shared expert when there is one.
  // One round of independent loads copies the routed table into LDS ...
  __shared__ uint64_t s_grows[kGroupsMax], s_gslot[kGroupsMax];
  const int D = ng - has_sh;
  if (tid < D) {
    s_expert[tid + has_sh] = ws.grp_expert[tid];
    s_nrows[tid + has_sh] = ws.grp_nrows[tid];
    s_grows[tid] = reinterpret_cast<const uint64_t*>(ws.grp_rows)[tid];
    s_gslot[tid] = reinterpret_cast<const uint64_t*>(ws.grp_slot)[tid];
  }
  if (has_sh && tid == 0) {
    s_expert[0] = -1;
    s_nrows[0] = (uint8_t)d.rows;
  }
  __syncthreads();
  // ... and the per-column rows and picks are derived there
  for (int idx = tid; idx < ng * 16; idx += 256) {
    const int gi = idx >> 4, c = idx & 15, g = gi - has_sh;
    const int nr = s_nrows[gi];
    int r = 0, pk = 0;
    if (c < nr) {
      r = g < 0 ? c : (int)((s_grows[g] >> (8 * c)) & 0xFF);
      pk = g < 0 ? 8 : (int)((s_gslot[g] >> (8 * r)) & 0xFF);
    }
    s_row[gi][c] = (uint8_t)r;
    s_pick[gi][c] = (uint8_t)pk;
  }
  __syncthreads();

  const int col = lane & 15;
  const int nitems = ng * nkw;  // (group, K block) pairs of this wave
  uint8_t* tile = s_tile[wv];
  // lane l loads rows h0 + l/8 and h0 + 8 + l/8, 16-byte chunk l%8
  const size_t wrow = (size_t)(h0 + (lane >> 3)) * I + (lane & 7) * 16;
  const size_t r8 = (size_t)8 * I;
  const int hblk = h0 / 128;

  DnStage st[P];
  // Item i = K block (kp*nkw + i%nkw) of group i/nkw.  Items past the end
  // read the workspace's zero pad (cache-resident) for weights and the last
  // item's mid (weight 0), so the ring has no branches and no extra HBM reads.
  auto issue = [&](DnStage& s, int i) {
    const bool pad = i >= nitems;
    i = pad ? nitems - 1 : i;
    const int gi = i / nkw, kb = kp * nkw + (i - gi * nkw);
    const int e = s_expert[gi];
    const uint8_t* wb = e < 0 ? w.sd_c : w.down_c + (size_t)e * H * I;
    const float* sb = e < 0 ? w.sd_s
                            : reinterpret_cast<const float*>(w.down_s) + (size_t)e * (H / 128) * nkb;
    const size_t mrow = (size_t)s_row[gi][col] * 9 + s_pick[gi][col];  // (row, pick)
    const uint8_t* p0 = pad ? ws.pad + lane * 16 : wb + wrow + (size_t)kb * 128;
    const uint8_t* p1 = pad ? p0 + 1024 : p0 + r8;
    s.w0 = ld_nt16(p0);
    s.w1 = ld_nt16(p1);
    s.m0 = ld16(ws.midq + mrow * d.imax + kb * 128 + (lane >> 4) * 32);
    s.m1 = ld16(ws.midq + mrow * d.imax + kb * 128 + (lane >> 4) * 32 + 16);
    s.sm = ws.midqs[mrow * (d.imax / 128) + kb];
    s.sd = sb[(size_t)hblk * nkb + kb];
  };
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](DnStage& s, int i) {
    tile_put(tile, lane, s.w0, s.w1);
    asm volatile("" ::: "memory");
    const v4f c = mfma_fp8(tile_get(tile, lane), cat8(s.m0, s.m1));
    asm volatile("" ::: "memory");
    const float f = i < nitems ? s.sd * s.sm : 0.f;
#pragma unroll
    for (int v = 0; v < 4; v++) acc[v] = fmaf(c[v], f, acc[v]);
    if (i < nitems && (i + 1) % nkw == 0) {  // last K block of a group: file it
      pin4(acc);
      const int gi = i / nkw;
      if (col < s_nrows[gi]) {
        float* dst = &s_part[kp][s_row[gi][col]][s_pick[gi][col]][hs * 16 + 4 * (lane >> 4)];
#pragma unroll
        for (int v = 0; v < 4; v++) dst[v] = acc[v];
      }
#pragma unroll
      for (int v = 0; v < 4; v++) acc[v] = 0.f;
    }
  };
#pragma unroll
  for (int p = 0; p < P; p++) issue(st[p], p);
  for (int i0 = 0; i0 < nitems; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      consume(st[p], i0 + p);
      issue(st[p], i0 + P + p);
    }
  }
  __syncthreads();

  // ---- combine in pick order, K parts in part order
  for (int idx = tid; idx < d.rows * BH; idx += 256) {
    const int r = idx / BH, hh = idx - r * BH;
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      float y = s_part[0][r][j][hh];
#pragma unroll
      for (int q = 1; q < KSD; q++) y += s_part[q][r][j][hh];
      a = fmaf(ws.gates[r * 8 + j], y, a);
    }
    if (has_sh) {
      float y = s_part[0][r][8][hh];
#pragma unroll
      for (int q = 1; q < KSD; q++) y += s_part[q][r][8][hh];
      a += y;
    }
    out[(size_t)r * H + hb + hh] = f32_to_bf16(a);
  }
}

// K parts per block for the down GEMV: the largest of 4, 2, 1 dividing the
// expert's K blocks.
int down_k_split(int inter) {
  const int nkb = inter / 128;
  return nkb % 4 == 0 ? 4 : (nkb % 2 == 0 ? 2 : 1);
}

template <int KSD>
static void launch_ksd(dim3 grid, const Weights& w, const Ws& ws, const Dims& d, uint16_t* out,
                       hipStream_t stream) {
  hipLaunchKernelGGL((moe_down_kernel<KSD, 8>), grid, dim3(256), 0, stream, w, ws, d, out);
}

hipError_t launch_down(int rfmt, const Weights& w, const Ws& ws, const Dims& d, uint16_t* out,
                       hipStream_t stream) {
  if (rfmt != kFmtFp8) return hipErrorInvalidValue;
  const int ksd = down_k_split(d.I);
  dim3 grid(d.H / (16 * (4 / ksd)));
  switch (ksd) {
    case 4: launch_ksd<4>(grid, w, ws, d, out, stream); break;
    case 2: launch_ksd<2>(grid, w, ws, d, out, stream); break;
    default: launch_ksd<1>(grid, w, ws, d, out, stream); break;
  }
  return hipGetLastError();
}

}  // namespace moe
