// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core contraction: v_mfma_f32_32x32x16_bf16, one 64-lane wavefront
// computes C[32x32] += A[32x16] * B[16x32] in fp32.  Lane layout (checked on
// the device):
//   A operand: lane l holds row (l % 32), k = 8*(l / 32) + s, s = 0..7
//   B operand: lane l holds column (l % 32), the same k slots
//   C/D      : lane l holds column (l % 32), register i holds row
//              8*(i / 4) + 4*(l / 32) + (i % 4), i = 0..15
// A contraction only needs the A and B operands to agree on which logical k
// sits in which (lane group, slot); the kernels below rely on that to feed a
// C-layout result (P, dS) straight back in as an operand, with the other
// operand read in the matching key order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type of a bfloat16 in global memory

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row of the C/D layout held by register i of lane group g = lane / 32.
__device__ __forceinline__ constexpr int crow(int i, int g) { return 8 * (i / 4) + 4 * g + (i % 4); }

// Eight consecutive fp32 registers (C-layout rows of one 16-wide k step) to a
// bf16 operand fragment, round-to-nearest-even.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int half) {
  bf16x8 r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = (__bf16)c[8 * half + s];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 positions away (the other half of a C column).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// 16-byte global load / store helpers.
__device__ __forceinline__ uint4 ldg16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 lds_read16(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// receives element e (e = 0..3) from the 8-byte row chunk addressed by lane
// 4*e + i/4 of the same group, at position i % 4 of that chunk.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Per-lane offset (in elements, row pitch `pitch`) used to gather an A
// operand whose rows run along the tile's columns ("transposed" operand) from
// a row-major LDS tile with two transposed reads.  The operand covers tile
// rows r0 + 8*(s/4) + 4*(l/32) + (s%4) (the key order of a C-layout result,
// see crow) and tile columns c0 + (l % 32).  Lane l addresses row
// 4*(l/32) + (l/4)%4 and column 16*((l/16)%2) + 4*(l%4); the second read adds
// 8 rows.
__device__ __forceinline__ int tr_lane_offset(int lane, int pitch) {
  return (4 * (lane >> 5) + ((lane >> 2) & 3)) * pitch + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}

__device__ __forceinline__ bf16x8 lds_read_trA(const bf16_t* tile, int lane_off, int r0, int c0, int pitch) {
  const bf16_t* p = tile + lane_off + r0 * pitch + c0;
  return cat8(lds_read_tr4(p), lds_read_tr4(p + 8 * pitch));
}

// Map a launch-order block id to a logical work id so that the blocks the
// hardware places on one XCD (block id mod 8, round robin) get a contiguous
// range of logical ids, which share key/value heads and so hit one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd, rem = nblocks % kXcd;
  const int x = bid % kXcd, idx = bid / kXcd;
  return x * per + min(x, rem) + idx;
}

}  // namespace cgqa
