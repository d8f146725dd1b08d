// device_common.h -- shared device helpers and the workspace view for the
// gfx950 MoE decode kernels (router.hip, upgate.hip, down.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace moe {

// Host side: sets kernel `fn`'s dynamic-LDS limit on the current device to at
// least `bytes` when that is above the 64 KB default.  `raised` (kLdsDevices
// slots, one per device, kept by the caller for this kernel) records what
// each device already has, so the attribute call is made once per device and
// size; the check and the call run under one lock, so concurrent callers
// never leave a device below what a recorded size promises.
constexpr int kLdsDevices = 64;
inline hipError_t ensure_dyn_lds(const void* fn, size_t bytes, size_t* raised) {
  if (bytes <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < kLdsDevices && raised[dev] >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && dev >= 0 && dev < kLdsDevices) raised[dev] = bytes;
  return e;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxRows = 8;

enum : int { kFmtFp8 = 1, kFmtMxfp4 = 2, kFmtQ1 = 3 };

// Everything a step keeps in the caller's workspace (device pointers).
struct Ws {
  float* logits;          // [max_rows][E]
  float* rstd;            // [max_rows]
  int32_t* ids;           // [max_rows][8]
  float* gates;           // [max_rows][8]
  int32_t* n_groups;      // [1]
  int32_t* grp_expert;    // [G]
  uint8_t* grp_owner;     // [G][2]
  uint8_t* grp_mask;      // [G]
  uint8_t* grp_slot;      // [G][8]
  uint8_t* grp_rows;      // [G][8] using rows, ascending
  uint8_t* grp_nrows;     // [G]
  uint8_t* act_q;         // [max_rows][H]
  uint8_t* act_qp;        // [max_rows][H] act_q with each 128-block in 1-bit operand order (1-bit experts)
  float* act_s;           // [max_rows][H/128]
  uint16_t* act_u;        // [max_rows][H] u = bf16(x * gamma) (bf16 activations only)
  // per (row, pick) with pick 8 = the shared expert: u = row * 9 + pick
  float* mid;             // [max_rows * 9][imax]
  uint8_t* midq;          // [max_rows * 9][imax]
  float* midqs;           // [max_rows * 9][imax/128]
  float* ypart;           // [max_rows * 9][H] down output per (row, pick)
  // routing launch: one record per up/gate block (the shared expert's go,
  // then each routed block's group_record, route.h), cleared by the router
  // and by the block that reads it
  uint64_t* blk_rec;      // [Is/16 + G * I/16]
  uint32_t* wait_timeouts;  // [1] routed blocks that gave up waiting for their record
};

// Shapes of the step (all multiples as validated on the host).
struct Dims {
  int H, I, E, Is;     // hidden, routed inter, experts, shared inter (0: none)
  int rows, max_rows;  // this step's rows, the context's maximum
  int imax;            // max(I, Is)
  int ks;              // up/gate K parts (divides H/128)
  int no_dedup;        // 1: one group per (row, pick)
  int act_bf16;        // 1: the experts take u (bf16), not FP8 activation blocks
  int act_q1;          // 1: the router also writes act_qp (1-bit routed experts)
  int groups;          // routed groups the up/gate grid covers (8 * rows, or E if fewer)
  uint32_t wait_ticks; // cap of a routed block's wait for its record (100 MHz ticks)
  int withhold;        // 1: the routing block publishes no records (failure tests)
  float eps;
};

struct Weights {
  const uint16_t* gamma;
  const uint16_t* router;
  const uint8_t *gate_c, *up_c, *down_c;  // routed codes
  const void *gate_s, *up_s, *down_s;     // routed scales (fp32 or E8M0 bytes)
  const uint8_t *sg_c, *su_c, *sd_c;      // shared codes (FP8)
  const float *sg_s, *su_s, *sd_s;        // shared scales
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32): round to
// nearest even, NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> two E4M3FN bytes (hardware conversion: round to nearest even,
// OCP E4M3FN as on gfx950), returned in the low 16 bits.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// 16x16x128 FP8 x FP8 -> fp32 MFMA, unit scales.  A: lane l holds row l%16,
// K bytes 32*(l/16)..+32; B: lane l holds column l%16, same K bytes;
// D: lane l holds rows 4*(l/16)+v (v=0..3) of column l%16.
__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// Pins a value in registers at this point of the program.  Results of MFMA
// chains must be pinned before any lane-divergent branch that consumes them:
// otherwise the compiler may sink the last MFMA into that branch, where it
// would run under a partial EXEC mask and read the masked lanes' operands as
// missing (the 16 rows and columns of an MFMA come from all 64 lanes).
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin4(float* a) {
  pin(a[0]);
  pin(a[1]);
  pin(a[2]);
  pin(a[3]);
}
__device__ __forceinline__ void pin4(v4f& a) {
  float t[4] = {a[0], a[1], a[2], a[3]};
  pin4(t);
  a = v4f{t[0], t[1], t[2], t[3]};
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Wave-wide unsigned max / min with DPP row operations: xor 1 and xor 2
// within quads, half-row and row mirrors, then row broadcasts 15 and 31; lane
// 63 ends with the result, which is read back as a uniform value.
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t dpp_umin(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum and unsigned max over each row of 16 lanes: xor 1 and xor 2 within
// quads, then the half-row and row mirrors.  Every lane of a row ends with the
// row's result; for the sum the association differs from lane to lane, so a
// caller takes one fixed lane's value.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}
__device__ __forceinline__ uint32_t row16_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// Number of set bits of `m` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave max of non-negative floats (their bit patterns order as unsigned).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  return __uint_as_float(dpp_umax(__float_as_uint(v)));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

// Nontemporal 16-byte load for weights read once per step.
__device__ __forceinline__ u32x4 ld_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Row-contiguous weight tile -> MFMA operand order, through a per-wave LDS
// tile of 16 rows x 128 bytes (row stride 144 B so that the 16 rows of a
// column read fall on different banks).  `lo`/`hi` were loaded by lane l from
// rows (l/8) and 8 + (l/8), 16-byte chunk (l%8) of one 128-wide K block; the
// result is lane l's A operand: row l%16, bytes 32*(l/16) .. +32.  Only this
// wave touches `tile`, and LDS operations of one wave complete in order.
constexpr int kTileStride = 144;
constexpr int kTileBytes = 16 * kTileStride;
__device__ __forceinline__ void tile_put(uint8_t* tile, int lane, const u32x4& lo, const u32x4& hi) {
  *reinterpret_cast<u32x4*>(tile + (lane >> 3) * kTileStride + (lane & 7) * 16) = lo;
  *reinterpret_cast<u32x4*>(tile + (8 + (lane >> 3)) * kTileStride + (lane & 7) * 16) = hi;
}
__device__ __forceinline__ v8i tile_get(const uint8_t* tile, int lane) {
  const uint8_t* p = tile + (lane & 15) * kTileStride + (lane >> 4) * 32;
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
  v8i r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__device__ __forceinline__ v8i cat8(const u32x4& lo, const u32x4& hi) {
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  A: lane l holds row l%16, K
// 8*(l/16) .. +8; B: lane l holds column l%16, same K; D: lane l holds rows
// 4*(l/16)+v of column l%16 (layout checked on the device).
// Eight E4M3 codes (c.x bytes 0..3, then c.y) as eight bf16 values: every
// E4M3 value is a bf16 value, so the hardware conversion with scale 1 is exact.
typedef __bf16 v2bf_u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint2 c) {
  const v2bf_u p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false);
  const v2bf_u p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true);
  const v2bf_u p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false);
  const v2bf_u p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- 1-bit (Q1_0_G128) weights.  A group of 128 weights is an fp16 d and
// 16 sign bytes; weight k of the group is -d when bit k%8 of byte k/8 is set,
// else +d.  Two groups (36 bytes) make a dword-aligned chunk.  The MFMA takes
// the weights as +-1 and the group's sum is scaled by d afterwards.
//
// A constant copied into a vector register (a DPP move the compiler does not
// fold back): gfx950's three-operand instructions take no literal, and with
// both operand constants in registers a mask and an or are one v_and_or_b32.
__device__ __forceinline__ uint32_t q1_in_vgpr(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xE4, 0xF, 0xF, false);
}

// ---- 1-bit weights as FP4 (E2M1) MFMA operands, against FP8 codes.
// +-1 in E2M1 is 0x2 / 0xA, so a weight is a nibble with its sign bit at bit
// 3.  In the 16x16x128 f8f6f4 MFMA, lane group g = l/16 of an FP4 A operand
// holds K 32g .. 32g+31 (nibble s%8 of dword s/8 is K 32g + s), while an FP8 B
// operand's 32 bytes hold K 16g .. 16g+15 (bytes 0-15) and 64+16g .. +15
// (bytes 16-31); the pairing of A and B is by that K.  Lane group g's A is
// built from the sign dword g of the group (weights 32g .. 32g+31) with the
// weights permuted: dword d, nibble i (K 32g + 8d + i) takes weight
// 32g + d + 4i, so dword d is the sign word shifted left by 3 - d, masked to
// the nibble sign bits and or'ed with 1.0 in every nibble (two operations a
// dword).  The activation codes then go to the B operand permuted the same
// way, which the router writes once per step (q1_act_pos, act_qp): lane group
// g reads bytes 32g .. 32g+31 of each 128-block of that copy as its B.
// `m8` and `o2` are 0x88888888 and 0x22222222 held in vector registers (see
// q1_in_vgpr), so that the mask and the or are one v_and_or_b32.
__device__ __forceinline__ v8i q1_fp4_operand(uint32_t w, uint32_t m8, uint32_t o2) {
  v8i a;
  a[0] = (int)(((w << 3) & m8) | o2);
  a[1] = (int)(((w << 2) & m8) | o2);
  a[2] = (int)(((w << 1) & m8) | o2);
  a[3] = (int)((w & m8) | o2);
  a[4] = a[5] = a[6] = a[7] = 0;  // not read for an FP4 operand
  return a;
}
// Byte offset, inside a 128-block of act_qp, of the pair of activations
// 8t + j and 8t + j + 4 (t < 16, j < 4; the two are adjacent there): the K of
// the A slot holding activation n = 32g + r is h = 32g + 8(r%4) + r/4, and h
// sits at byte 32(h/16) + h%16 of the copy for h < 64, else at
// 32((h-64)/16) + 16 + h%16.
__device__ __forceinline__ uint32_t q1_act_pos(int t, int j) {
  const int g = t >> 2, tt = t & 3;
  return g < 2 ? (uint32_t)(32 * (2 * g + (j >> 1)) + 8 * (j & 1) + 2 * tt)
               : (uint32_t)(32 * (2 * (g - 2) + (j >> 1)) + 16 + 8 * (j & 1) + 2 * tt);
}
// 16x16x128 FP4 (A) x FP8 (B) -> fp32 MFMA, unit scales.
__device__ __forceinline__ v4f mfma_fp4_fp8(const v8i& a, const v8i& b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 0, 0, 127, 0, 127);
}

// One 36-byte chunk (9 dwords, as loaded) re-aligned: the 16 sign bytes of
// each group as 4 dwords (u[0..3] group 0, which starts 2 bytes in, u[4..7]
// group 1), and both groups' fp16 d as one dword (d0 | d1 << 16).
__device__ __forceinline__ void q1_chunk_split(const uint32_t* w, uint32_t* u, uint32_t* dd) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    u[q] = __builtin_amdgcn_alignbyte(w[q + 1], w[q], 2);
    u[4 + q] = w[5 + q];
  }
  *dd = (w[0] & 0xFFFFu) | (w[4] & 0xFFFF0000u);
}

__device__ __forceinline__ float q1_d(uint32_t dd, int h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h ? (dd >> 16) : (dd & 0xFFFFu)));
}

// A 36-byte chunk (dword-aligned) as two 16-byte and one 4-byte nontemporal
// loads (the hardware takes 16-byte loads at any dword alignment).
__device__ __forceinline__ void ld_nt_chunk36(const uint32_t* p, uint32_t* w) {
  const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
  w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  w[8] = __builtin_nontemporal_load(p + 8);
}

}  // namespace moe
