// Device-side helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element storage types: bf16 is carried as its 16-bit pattern.
struct Bf16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};
struct Fp32 {
  using storage = float;
  static constexpr int kBytes = 4;
};

// bf16 pattern (low or high half of a 32-bit word) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 p;
  p.x = (__bf16)lo;
  p.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// 16-byte load with the nontemporal (streaming) hint: K/V rows are read
// once per kernel, and streaming loads sustain ~10% more HBM read bandwidth
// on gfx950 than ordinary ones.
__device__ __forceinline__ u32x4 stream_load(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Raw buffer resource over `bytes` bytes at `base` (word 3: 32-bit data
// format, the value used for untyped buffer access on gfx9-family parts).
// A load at or past `bytes` returns zero and reads no memory.  Both
// arguments must be the same in every lane; readfirstlane states that for
// the compiler (otherwise a load through the resource may be wrapped in a
// loop over the lanes' distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bounded_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 16-byte nontemporal load at byte offset `off` through a buffer resource
// (cache policy: nt, as stream_load).
__device__ __forceinline__ u32x4 stream_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the 64 lanes of a wavefront; every lane gets the result.
// Within each row of 16 lanes: DPP quad_perm (xor 1, xor 2), half-row mirror
// and row mirror, so all 16 lanes of a row hold the row result; the four row
// results are then read out as scalars and combined.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

}  // namespace pkv
