// route.h -- the routing decisions of a step, computed inside one block from
// the final router logits: top-8 per row, the softmax gates and the expert
// dedup table, published to the workspace for the kernels that follow.
//
// #85 Mod. row 9: a row's picks are its 8 largest logits in decreasing order,
// exact ties going to the lower expert ID.  Mod. rows 16 and 20: the distinct
// experts of the step are numbered by first use in slot-major order (slot j of
// every row before slot j + 1), the owner of a group being that first use.
//
// Top-8 in 8 rounds on one wave: lane l holds experts l, l + 64, ... as order
// keys; a round takes the wave's largest remaining key (DPP max) and, among
// the slots holding it, the lowest expert ID, then clears that slot, so the
// picks come out in top-8 order.  (A radix select of the 8th largest key, 32
// ballot rounds, then ranking the 8 picks, took about three times as long.)
#pragma once
#include "device_common.h"

namespace moe {

// Order key of a logit: unsigned compare = float order, -0 == +0, NaN (1)
// below every number (-inf maps to 0x007FFFFF), 0 = no expert.
__device__ __forceinline__ uint32_t topk_vkey(float z) {
  if (z != z) return 1u;
  const uint32_t b = (z == 0.0f) ? 0u : __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// The logit back from its key (-0 comes back as +0, NaN as a NaN).
__device__ __forceinline__ float topk_vkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct RouteSmem {
  int ids[kMaxRows][8];        // picks in top-8 order
  float zsel[kMaxRows][8];
  int g_expert[64];
  uint32_t g_mask[64];
  uint8_t g_slot[64][8];
  uint8_t g_owner[64][2];
  uint8_t g_rows[64][8];
  uint8_t g_nrows[64];
  uint64_t g_rec[64];  // published record of each group (group_record)
  int n_groups;
};

// Record of a routed up/gate block in moe_route_kernel, 64 bits: bit 0 set
// when published; bits 1-10 the group's expert, 11-14 its number of using
// rows (0: the step has no such group), 15 + 3c its c-th using row, 39 + 3r
// the pick that row r of the group made (rows of the group only).  Expert IDs
// are below 1024 and rows below 8, so the fields hold them whole.
__device__ __forceinline__ uint64_t group_record(int expert, int nrows, const uint8_t* rows,
                                                 const uint8_t* slot) {
  uint64_t rec = 1u | ((uint64_t)expert << 1) | ((uint64_t)nrows << 11);
  for (int c = 0; c < nrows; c++) {
    const int r = rows[c];
    rec |= (uint64_t)r << (15 + 3 * c);
    rec |= (uint64_t)(slot[r] & 7) << (39 + 3 * r);
  }
  return rec;
}

// Order keys of the logits z[0 .. E) of one row: lane l holds experts l,
// l + 64, ... in KPL = ceil(E / 64) key slots (key 0, below every logit, past E).
template <int KPL>
__device__ __forceinline__ void load_keys(const float* z, int E, int lane, uint32_t* key) {
#pragma unroll
  for (int i = 0; i < KPL; i++) {
    const int e = lane + kWave * i;
    const float v = z[e < E ? e : E - 1];  // lanes past E load in bounds
    key[i] = e < E ? topk_vkey(v) : 0u;
  }
}

// The 8 largest of a row's order keys (load_keys) in top-8 order, equal keys
// by increasing expert ID, as wave-uniform values okey[j], oid[j].  Runs with
// one full wave; clears the picked slots of `key` (key 0 is below every
// logit's key, and E >= 16 leaves 8 real keys).
template <int KPL>
__device__ __forceinline__ void top8_sorted(uint32_t* key, int lane, uint32_t* okey, int* oid) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < KPL; i++) m = max(m, key[i]);
    const uint32_t M = dpp_umax(m);
    // the lowest expert ID holding M: the lowest slot, then the lowest lane
    int id = 0;
#pragma unroll
    for (int i = 0; i < KPL; i++) {
      const uint64_t b = __ballot(key[i] == M);
      if (b) {
        id = kWave * i + (int)__builtin_ctzll(b);
        break;
      }
    }
#pragma unroll
    for (int i = 0; i < KPL; i++)
      if (kWave * i + lane == id) key[i] = 0u;
    okey[j] = M;
    oid[j] = id;
  }
}

// Gates of row r: softmax of its 8 picked logits in pick order (zsel), one
// thread, published with the row's IDs.
__device__ __forceinline__ void publish_gates(const Ws& ws, int r, const float* zsel,
                                              const int* ids) {
  float mz = zsel[0];
  for (int j = 1; j < 8; j++) mz = fmaxf(mz, zsel[j]);
  float g[8], sum = 0.f;
  for (int j = 0; j < 8; j++) {
    g[j] = expf(zsel[j] - mz);
    sum += g[j];
  }
  for (int j = 0; j < 8; j++) {
    ws.gates[r * 8 + j] = g[j] / sum;
    ws.ids[r * 8 + j] = ids[j];
  }
}

// Wave 0 of the routing launch's block 0, once row 0's logits are loaded:
// publishes the go records 0 .. go - 1 of the launch's shared-expert blocks.
__device__ __forceinline__ void publish_go(const Ws& ws, int go, int lane) {
  // the logits loads have returned (the wait), so the stores come after them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int i = lane; i < go; i += kWave)
    __hip_atomic_store(ws.blk_rec + i, (uint64_t)1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Runs with every thread of the block (it contains block barriers).  Fills
// `rs` for rows 0..d.rows-1; when `publish`, also writes ids, gates and the
// group table to the workspace.  KPL = key slots per lane, ceil(E / 64).
// go > 0 (the routing launch): once row 0's logits are in registers, wave 0
// publishes the records 0 .. go - 1 of the launch's first up/gate blocks
// (the shared expert's), which hold back their weight loads until then, so
// that the logits' loads do not queue behind those streams.
template <int KPL>
__device__ __forceinline__ void route_block(const Ws& ws, const Dims& d, RouteSmem& rs,
                                            bool publish, int go = 0) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  const int R = d.rows, E = d.E;

  for (int r = wv; r < R; r += nw) {
    uint32_t key[KPL];
    load_keys<KPL>(ws.logits + (size_t)r * E, E, lane, key);
    if (go > 0 && r == 0) publish_go(ws, go, lane);
    uint32_t okey[8];
    int oid[8];
    top8_sorted<KPL>(key, lane, okey, oid);
#pragma unroll
    for (int j = 0; j < 8; j++)
      if (lane == j) {
        rs.ids[r][j] = oid[j];
        rs.zsel[r][j] = topk_vkey_value(okey[j]);
      }
  }
  if (tid < 64) {
    rs.g_mask[tid] = 0u;
#pragma unroll
    for (int r = 0; r < 8; r++) rs.g_slot[tid][r] = 0xFF;
  }
  __syncthreads();

  // gates: softmax of a row's 8 picked logits, in pick order (on wave 1, so
  // that they overlap the dedup on wave 0; one wave does both when the block
  // has one)
  const int gt0 = nw > 1 ? 64 : 0;
  if (publish && tid >= gt0 && tid < gt0 + R) publish_gates(ws, tid - gt0, rs.zsel[tid - gt0], rs.ids[tid - gt0]);

  // dedup: lane p holds pick p in slot-major order (p = j*R + r).  Lanes with
  // the same expert are found with one ballot per ID bit; the lowest of them
  // owns the group, and a group's index counts the first uses before it.
  if (wv == 0) {
    const int P = 8 * R;
    const bool valid = lane < P;
    int ep = 0, jp = 0, rp = 0;
    if (valid) {
      jp = lane / R;
      rp = lane - jp * R;
      ep = rs.ids[rp][jp];
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
      atomicOr(&rs.g_mask[gidx], 1u << rp);
      rs.g_slot[gidx][rp] = (uint8_t)jp;
      if (owner == lane) {
        rs.g_expert[gidx] = ep;
        rs.g_owner[gidx][0] = (uint8_t)jp;
        rs.g_owner[gidx][1] = (uint8_t)rp;
      }
    }
    if (lane == 0) rs.n_groups = __popcll(first);
  }
  __syncthreads();
  const int D = rs.n_groups;
  if (tid < D) {
    const uint32_t m = rs.g_mask[tid];
    int n = 0;
    for (int r = 0; r < 8; r++)
      if ((m >> r) & 1u) rs.g_rows[tid][n++] = (uint8_t)r;
    rs.g_nrows[tid] = (uint8_t)n;
    rs.g_rec[tid] = group_record(rs.g_expert[tid], n, rs.g_rows[tid], rs.g_slot[tid]);
    if (publish) {
      ws.grp_expert[tid] = rs.g_expert[tid];
      ws.grp_owner[2 * tid] = rs.g_owner[tid][0];
      ws.grp_owner[2 * tid + 1] = rs.g_owner[tid][1];
      ws.grp_mask[tid] = (uint8_t)m;
      uint64_t slots = 0, rows = 0;  // the 8 bytes of each, stored at once
      for (int r = 0; r < 8; r++) {
        slots |= (uint64_t)rs.g_slot[tid][r] << (8 * r);
        if (r < n) rows |= (uint64_t)rs.g_rows[tid][r] << (8 * r);
      }
      *reinterpret_cast<uint64_t*>(ws.grp_slot + tid * 8) = slots;
      *reinterpret_cast<uint64_t*>(ws.grp_rows + tid * 8) = rows;
      ws.grp_nrows[tid] = (uint8_t)n;
    }
  }
  if (publish && tid == 0) *ws.n_groups = D;
  __syncthreads();
}

}  // namespace moe
