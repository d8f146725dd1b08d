// route.hip -- the routing launch of a step.
//
// #85 Mod. row 3 and its `poll` section: the routed experts' weights should
// start streaming as soon as the routing has chosen them, not after a launch
// boundary, and the shared expert's (which need no routing) from the start.
// So one launch holds three kinds of block of 256 threads:
//
//   block 0          the routing (route.h): top-8, gates and dedup table from
//                    the router logits, published to the workspace for the
//                    down and combine launches; then one record per routed
//                    up/gate block of this launch (group_record), stored with
//                    relaxed agent-scope atomics;
//   blocks 1 ..      the shared expert's up/gate slabs, which start streaming
//                    as soon as block 0 has its logits in registers (a go
//                    record: their loads would otherwise delay those few);
//   then             the routed groups' up/gate slabs (upgate.h), each of
//                    which waits for its own record (await_record) and then
//                    streams its expert's weights.
//
// Only block 0 is waited for, and it waits for nothing: it is the first block
// of the grid, so it is dispatched no later than any block that waits for it,
// and every wait is capped besides (a routed block that reaches the cap
// counts itself in the workspace and does no work, so every block exits).
// Each routed block clears its record after reading it, and the router
// clears them all, so a record is never read twice.
//
// Steps of more rows than fused_route() takes run the routing alone on 8
// waves (moe_route_only_kernel) and the up/gate in its own launch
// (upgate.hip).
#include "upgate.h"

#ifndef MOE_FUSE_MAX_ROWS
#define MOE_FUSE_MAX_ROWS 4
#endif

namespace moe {

// Whether the step's up/gate runs in the routing launch.
bool fused_route(const Dims& d) { return d.rows <= MOE_FUSE_MAX_ROWS; }

// Routed up/gate blocks per group (slabs of 16 intermediate rows, 4/ks a block).
__host__ __device__ inline int routed_blocks_per_group(const Dims& d) {
  return d.I / (16 * (4 / d.ks));
}

// Shared-expert up/gate blocks of the launch (their records come first).
__host__ __device__ inline int shared_blocks(const Dims& d) { return d.Is / (16 * (4 / d.ks)); }

// Block 0, after route_block: routed block rb gets the record of its group
// rb / per (at index shared_blocks + rb), or an empty published record (no
// using rows) for groups past the step's D.  Low blocks first: they are the
// first to be dispatched.
__device__ __forceinline__ void publish_records(const Ws& ws, const Dims& d,
                                                const RouteSmem& rs) {
  const int per = routed_blocks_per_group(d), n = d.groups * per, D = rs.n_groups;
  uint64_t* rec0 = ws.blk_rec + shared_blocks(d);
  for (int rb = threadIdx.x; rb < n; rb += blockDim.x) {
    const int g = rb / per;
    const uint64_t rec = g < D ? rs.g_rec[g] : (uint64_t)1u;
    __hip_atomic_store(rec0 + rb, rec, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int KPL, int RF, int P, int P4, bool AB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RF == kFmtQ1 ? 4 : 1))) void moe_route_kernel(Weights w, Ws ws, Dims d) {
  __shared__ RouteSmem rs;
  __shared__ __align__(16) UgTiles s_tile;
  __shared__ __align__(16) uint8_t s_e8[ug_e8_lds<RF>()];
  __shared__ uint64_t s_rec;
  if (blockIdx.x == 0) {
    route_block<KPL>(ws, d, rs, true, shared_blocks(d));
    if (!d.withhold) publish_records(ws, d, rs);
  } else {
    upgate_block<RF, P, P4, AB, true>(w, ws, d, blockIdx.x - 1, s_tile, s_e8, &s_rec);
  }
}

// The routing alone, 8 waves (steps whose up/gate runs in its own launch).
template <int KPL>
__global__ __launch_bounds__(512) void moe_route_only_kernel(Ws ws, Dims d) {
  __shared__ RouteSmem rs;
  route_block<KPL>(ws, d, rs, true);
}

template <int KPL, int RF, int P, int P4>
static void launch_fused(dim3 grid, const Weights& w, const Ws& ws, const Dims& d,
                         hipStream_t stream) {
  if constexpr (RF == kFmtFp8) {  // bf16 activations: FP8 routed experts only
    if (d.act_bf16) {
      hipLaunchKernelGGL((moe_route_kernel<KPL, RF, P, P4, true>), grid, dim3(256), 0, stream, w,
                         ws, d);
      return;
    }
  }
  hipLaunchKernelGGL((moe_route_kernel<KPL, RF, P, P4, false>), grid, dim3(256), 0, stream, w,
                     ws, d);
}

template <int KPL, int RF, int P>
static void launch_fused_p4(int p4, dim3 grid, const Weights& w, const Ws& ws, const Dims& d,
                            hipStream_t stream) {
  if constexpr (RF != kFmtQ1) {  // 1-bit items are never two deep
    if (p4 == 2) {
      launch_fused<KPL, RF, P, 2>(grid, w, ws, d, stream);
      return;
    }
  }
  launch_fused<KPL, RF, P, 1>(grid, w, ws, d, stream);
}

template <int KPL, int RF>
static void launch_fused_p(int p, int p4, dim3 grid, const Weights& w, const Ws& ws,
                           const Dims& d, hipStream_t stream) {
  if constexpr (RF == kFmtFp8) {
    switch (p) {
      case 4: launch_fused<KPL, RF, 4, 1>(grid, w, ws, d, stream); break;
      case 2: launch_fused<KPL, RF, 2, 1>(grid, w, ws, d, stream); break;
      default: launch_fused<KPL, RF, 1, 1>(grid, w, ws, d, stream); break;
    }
  } else if constexpr (RF == kFmtMxfp4) {  // shared rings of at most 2
    if (p >= 2)
      launch_fused_p4<KPL, RF, 2>(p4, grid, w, ws, d, stream);
    else
      launch_fused_p4<KPL, RF, 1>(p4, grid, w, ws, d, stream);
  } else {  // 1-bit layers: a shared ring of 1 (see launch_upgate)
    launch_fused_p4<KPL, RF, 1>(p4, grid, w, ws, d, stream);
  }
}

template <int KPL>
static hipError_t launch_route_k(int rfmt, const Weights& w, const Ws& ws, const Dims& d,
                                 hipStream_t stream) {
  if (!fused_route(d)) {
    hipLaunchKernelGGL((moe_route_only_kernel<KPL>), dim3(1), dim3(512), 0, stream, ws, d);
    return hipSuccess;
  }
  const dim3 grid(1 + shared_blocks(d) + d.groups * routed_blocks_per_group(d));
  // FP8 items in flight (the shared expert's, and FP8 routed experts'); MXFP4
  // and 1-bit items in flight
  const int p = ring_depth(d.H / 128 / d.ks);
  switch (rfmt) {
    case kFmtFp8: launch_fused_p<KPL, kFmtFp8>(p, 1, grid, w, ws, d, stream); break;
    case kFmtMxfp4:  // rings of at most 2 (MXFP4 items and FP8 shared): see launch_upgate
      launch_fused_p<KPL, kFmtMxfp4>(p > 2 ? 2 : p, ring_depth2(d.H / 256 / d.ks), grid, w, ws,
                                     d, stream);
      break;
    case kFmtQ1:  // rings of 1 (1-bit and FP8 shared): see launch_upgate
      launch_fused_p<KPL, kFmtQ1>(1, 1, grid, w, ws, d, stream);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_route(int rfmt, const Weights& w, const Ws& ws, const Dims& d,
                        hipStream_t stream) {
  // key slots per lane of the top-8: 4, 8 or 16 (E <= 256, 512, 1024)
  hipError_t e;
  if (d.E <= 256)
    e = launch_route_k<4>(rfmt, w, ws, d, stream);
  else if (d.E <= 512)
    e = launch_route_k<8>(rfmt, w, ws, d, stream);
  else
    e = launch_route_k<16>(rfmt, w, ws, d, stream);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace moe
