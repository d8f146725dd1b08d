// upgate.hip -- the up/gate launch of steps whose routing runs alone
// (moe_route_only_kernel): the shared expert's slabs and every routed
// group's, which read the published table (the block's code is in upgate.h).
#include "upgate.h"

namespace moe {

// Up/gate blocks: the shared expert's slabs, then the routed groups'.
template <int RF, int P, int P4, bool AB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RF == kFmtQ1 ? 4 : 1))) void moe_upgate_kernel(Weights w, Ws ws, Dims d) {
  __shared__ __align__(16) UgTiles s_tile;
  __shared__ __align__(16) uint8_t s_e8[ug_e8_lds<RF>()];
  __shared__ uint64_t s_rec;
  upgate_block<RF, P, P4, AB, false>(w, ws, d, blockIdx.x, s_tile, s_e8, &s_rec);
}

// K parts of the up/gate slabs: the largest of 4, 2, 1 dividing H/128, or
// H/256 when routed experts are MXFP4 (their items are two K blocks).
int upgate_k_parts(int hidden, int routed_fmt) {
  // parts hold whole items: K blocks (FP8), pairs of them (MXFP4), or 4-group
  // items (1-bit experts: hidden a multiple of 512)
  const int n = routed_fmt == kFmtMxfp4 ? hidden / 256
                                          : (routed_fmt == kFmtQ1 ? hidden / 512 : hidden / 128);
  return n % 4 == 0 ? 4 : (n % 2 == 0 ? 2 : 1);
}

template <int RF, int P, int P4>
static void launch_one(dim3 grid, const Weights& w, const Ws& ws, const Dims& d,
                       hipStream_t stream) {
  if constexpr (RF == kFmtFp8) {  // bf16 activations: FP8 routed experts only
    if (d.act_bf16) {
      hipLaunchKernelGGL((moe_upgate_kernel<RF, P, P4, true>), grid, dim3(256), 0, stream, w, ws,
                         d);
      return;
    }
  }
  hipLaunchKernelGGL((moe_upgate_kernel<RF, P, P4, false>), grid, dim3(256), 0, stream, w, ws, d);
}

template <int RF, int P>
static void launch_p4(int p4, dim3 grid, const Weights& w, const Ws& ws,
                      const Dims& d, hipStream_t stream) {
  if constexpr (RF != kFmtQ1) {  // 1-bit items are never two deep
    if (p4 == 2) {
      launch_one<RF, P, 2>(grid, w, ws, d, stream);
      return;
    }
  }
  launch_one<RF, P, 1>(grid, w, ws, d, stream);
}

hipError_t launch_upgate(int rfmt, int max_groups, const Weights& w, const Ws& ws,
                         const Dims& d, hipStream_t stream) {
  const int br = 16 * (4 / d.ks);
  const dim3 grid(d.Is / br + max_groups * (d.I / br));
  const int p = ring_depth(d.H / 128 / d.ks);
  if (rfmt == kFmtFp8) {
    switch (p) {
      case 4: launch_one<kFmtFp8, 4, 1>(grid, w, ws, d, stream); break;
      case 2: launch_one<kFmtFp8, 2, 1>(grid, w, ws, d, stream); break;
      default: launch_one<kFmtFp8, 1, 1>(grid, w, ws, d, stream); break;
    }
  } else if (rfmt == kFmtMxfp4) {
    // at most 2 MXFP4 items and 2 FP8 shared K blocks in flight: 164
    // registers, 3 waves a SIMD against 216 and 2 with rings of 3 and 4 (GLM
    // step 209.5 -> 202.8 us at 8 rows, 123.5 -> 118.4 at 4, 49.6 -> 48.4 at
    // 1, outputs bitwise equal; rings of 1 were between)
    const int p4 = ring_depth2(d.H / 256 / d.ks);
    if (p >= 2)
      launch_p4<kFmtMxfp4, 2>(p4, grid, w, ws, d, stream);
    else
      launch_p4<kFmtMxfp4, 1>(p4, grid, w, ws, d, stream);
  } else if (rfmt == kFmtQ1) {
    // one 1-bit item in flight (a round of the block's rows, or a wave's
    // item) and one K block of the FP8 shared expert: the 1-bit path gains
    // from more waves, not from deeper rings; at 4 waves a SIMD (the kernels'
    // register cap) a shared ring of 2 spilled registers and ran no faster
    // (GLM step 130.2 against 130.6 us at 8 rows, 39.8 against 40.1 at 1)
    launch_p4<kFmtQ1, 1>(1, grid, w, ws, d, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
