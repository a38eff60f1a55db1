// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core contraction: v_mfma_f32_32x32x16_bf16 (or _f16), one 64-lane
// wavefront computes C[32x32] += A[32x16] * B[16x32] in fp32.  Lane layout (checked on
// the device):
//   A operand: lane l holds row (l % 32), k = 8*(l / 32) + s, s = 0..7
//   B operand: lane l holds column (l % 32), the same k slots
//   C/D      : lane l holds column (l % 32), register i holds row
//              8*(i / 4) + 4*(l / 32) + (i % 4), i = 0..15
// A contraction only needs the A and B operands to agree on which logical k
// sits in which (lane group, slot); the kernels rely on that to feed a
// C-layout result (P, dS) straight back in as an operand, with the other
// operand read in the matching key order.
//
// LDS tiles are row-major with 16-byte chunks, unpadded, with the chunk index
// XOR-swizzled per row (see Tile below), so a wave's 64 x 16-byte direct
// global->LDS load fills 1 KiB of consecutive chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type of a 16-bit element in global memory and LDS

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ element formats
// Q, K, V, O, dO and the gradients are bfloat16 (BF16) or IEEE half (FP16).
// Operand fragments travel as 16-bit payloads in bf16x8 registers in either
// case; only the matrix instruction (v_mfma_f32_32x32x16_bf16 / _f16, same
// lane layout) and the conversions from and to fp32 read them as numbers.
// Conversions from fp32 round to nearest even.
struct BF16 {
  __device__ __forceinline__ static f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // registers 8*half .. 8*half+7 of a C-layout result as an operand fragment
  __device__ __forceinline__ static bf16x8 pack8(const f32x16& c, int half) {
    bf16x8 r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = (__bf16)c[8 * half + s];
    return r;
  }
  // v_mfma_f32_16x16x32_bf16: C[16x16] += A[16x32] * B[32x16]; lane l holds
  // A row / B column l % 16 with k = 8*(l / 16) + s, and C column l % 16,
  // rows 4*(l / 16) + i
  __device__ __forceinline__ static f32x4 mma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint2 pack4(float x0, float x1, float x2, float x3) {
    const bf16x4 r = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
    return __builtin_bit_cast(uint2, r);
  }
  __device__ __forceinline__ static float get(const uint4& u, int e) {
    return (float)__builtin_bit_cast(bf16x8, u)[e];
  }
};

struct FP16 {
  __device__ __forceinline__ static f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  }
  __device__ __forceinline__ static bf16x8 pack8(const f32x16& c, int half) {
    f16x8 r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = (_Float16)c[8 * half + s];
    return __builtin_bit_cast(bf16x8, r);
  }
  __device__ __forceinline__ static f32x4 mma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  }
  __device__ __forceinline__ static uint2 pack4(float x0, float x1, float x2, float x3) {
    const f16x4 r = {(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
    return __builtin_bit_cast(uint2, r);
  }
  __device__ __forceinline__ static float get(const uint4& u, int e) {
    return (float)__builtin_bit_cast(f16x8, u)[e];
  }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// c *= alpha for an accumulator the compiler keeps in AGPRs (kernels at one
// wavefront per SIMD with a 128-register accumulator).  Written as inline
// assembly on the AGPRs themselves: as plain code the compiler copies every
// accumulator register to a VGPR at the top of the loop, on every tile, for
// a rescale that runs on few of them.
__device__ __forceinline__ void scale_agpr(f32x16& c, float alpha) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(c[i]), "=&v"(t)
                 : "v"(alpha));
  }
}

// Row of the C/D layout held by register i of lane group g = lane / 32.
__device__ __forceinline__ constexpr int crow(int i, int g) { return 8 * (i / 4) + 4 * g + (i % 4); }

// Wave priority around matrix-core phases: a wave about to issue a run of
// MFMAs asks the sequencer to prefer it, so a co-resident wave's vector work
// fills the matrix-core time instead of competing with it.
#ifndef CGQA_SETPRIO
#define CGQA_SETPRIO 0
#endif
__device__ __forceinline__ void prio_hi() {
  if (CGQA_SETPRIO) __builtin_amdgcn_s_setprio(1);
}
__device__ __forceinline__ void prio_lo() {
  if (CGQA_SETPRIO) __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 positions away (the other half of a C column).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x, x[lane ^ 32]) on the VALU: v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second; starting from
// two copies of x, lane l then holds x[l] in one and x[l ^ 32] in the other.
// (Inline assembly: the compiler folds an fmax over the pair of results of
// the intrinsic to its first result.  The s_nop covers the VALU-write to
// permlane-read hazard.)
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// v_permlane16_swap: within each pair of 16-lane rows, the odd row of `a`
// and the even row of `b` trade places.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

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

// ------------------------------------------------------------ tile layout
//
// LDS has 64 banks of 4 bytes.  A 16-byte read is served 16 lanes at a time,
// an 8-byte transposed read 32 lanes at a time; a read runs at full rate when
// the lanes served together touch 16 distinct 16-byte bank groups.  The row
// swizzle below gives that for both patterns the kernels use: 16 consecutive
// rows at one logical chunk (row reads), and 4 rows x 4 consecutive chunks
// (transposed reads).  Measured on gfx950 both then run near the LDS peak.

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;                  // logical 16-byte chunks per row
  static constexpr int PC = (D == 96) ? 16 : CPR;    // physical chunks per row (power of two)
  static constexpr int P = PC * 8;                   // row pitch in elements
  // physical chunk of logical chunk c in row r is c ^ swz(r)
  __device__ __forceinline__ static constexpr int swz(int r) {
    return PC >= 16 ? 4 * (r & 3) + ((r >> 2) & 3)          // rows of >= 256 bytes
                    : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);  // 128-byte rows: two per bank row
  }
};

// Per-lane element offsets for reading a tile from LDS.
//  row16(tile, r0, kd): A/B operand fragment of rows r0 + (lane % 32) (r0 a
//    multiple of 16), head-dim slots 16*kd + 8*(lane/32) + s (one 16-byte read).
//  trA(tile, r0, db): A operand whose rows are tile columns 32*db + lane % 32
//    and whose k slots are tile rows r0 + 8*(s/4) + 4*(lane/32) + s%4 (the row
//    order of a C-layout result), r0 a multiple of 16; two transposed reads.
// The swizzle mixes the low four chunk bits, so the offsets for the first
// 8 k steps / 4 column blocks are precomputed per lane and higher steps add a
// constant.
template <int D>
struct TileReader {
  using T = Tile<D>;
  static constexpr int P = T::P;
  static constexpr int NRA = (D / 16) < 8 ? (D / 16) : 8;
  static constexpr int NTR = (D / 32) < 4 ? (D / 32) : 4;
  int ra[NRA];      // byte offsets
  int tr[2][NTR];   // byte offsets
  __device__ __forceinline__ explicit TileReader(int lane) {
    const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int j = 0; j < NRA; ++j) ra[j] = 2 * (lr * P + (((2 * j + lg) ^ T::swz(lr)) << 3));
    // transposed read: lane addresses row rl (+8), chunk 4*db + y, 8-byte half `within`
    const int rl = 4 * (lane >> 5) + ((lane >> 2) & 3);
    const int y = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int within = 4 * (lane & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dm = 0; dm < NTR; ++dm)
        tr[h][dm] = 2 * ((rl + 8 * h) * P + (((4 * dm + y) ^ T::swz(rl + 8 * h)) << 3) + within);
  }
  // Move every offset to the other half of a double buffer whose halves sit
  // `half` elements apart (`half` a power of two above every offset used):
  // one XOR per register per tile instead of an address add per read.
  __device__ __forceinline__ void flip(int half) {
    flip_ra(half);
    flip_tr(half);
  }
  __device__ __forceinline__ void flip_ra(int half) {
#pragma unroll
    for (int j = 0; j < NRA; ++j) ra[j] ^= 2 * half;
  }
  __device__ __forceinline__ void flip_tr(int half) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dm = 0; dm < NTR; ++dm) tr[h][dm] ^= 2 * half;
  }
  // Carry a fixed row offset (bytes, a multiple of 32 P, below the flip's
  // half) in every offset, so that reads take a constant row offset: an
  // instruction immediate instead of a vector add per address.
  __device__ __forceinline__ void shift(int bytes) {
#pragma unroll
    for (int j = 0; j < NRA; ++j) ra[j] += bytes;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dm = 0; dm < NTR; ++dm) tr[h][dm] += bytes;
  }
  __device__ __forceinline__ bf16x8 row16(const bf16_t* tile, int r0, int kd) const {
    const char* p = reinterpret_cast<const char*>(tile + r0 * P + 128 * (kd / NRA)) + ra[kd % NRA];
    return lds_read16(reinterpret_cast<const bf16_t*>(p));
  }
  __device__ __forceinline__ bf16x8 trA(const bf16_t* tile, int r0, int db) const {
    const char* p = reinterpret_cast<const char*>(tile + r0 * P + 128 * (db / NTR));
    return cat8(lds_read_tr4(reinterpret_cast<const bf16_t*>(p + tr[0][db % NTR])),
                lds_read_tr4(reinterpret_cast<const bf16_t*>(p + tr[1][db % NTR])));
  }
};

// The same reads from two registers.  Within a row the chunk of k step j is
// (2j | lane/32) ^ swz = 2j ^ (lane/32 ^ swz), so ra[j] = ra[0] ^ 32 j; the
// transposed chunk of column block dm is 4 dm ^ (y ^ swz), and row r + 8 has
// swz(r) ^ 2 with the row term's bit 16 P clear in every offset, so
// tr[h][dm] = tr[0][0] ^ 64 dm ^ h (32 | 16 P).  One XOR per read instead of
// 2 + 2 * NTR + NRA - 2 more offset registers.
template <int D>
struct TileReaderX {
  using T = Tile<D>;
  static constexpr int P = T::P;
  static constexpr int NRA = (D / 16) < 8 ? (D / 16) : 8;
  static constexpr int NTR = (D / 32) < 4 ? (D / 32) : 4;
  static_assert(2 * 7 * P + 16 * (T::PC - 1) + 8 < 16 * P, "offsets of rows 0-7 must clear bit 16 P");
  int ra0, tr0;  // byte offsets
  __device__ __forceinline__ explicit TileReaderX(int lane) {
    const int lr = lane & 31, lg = lane >> 5;
    ra0 = 2 * (lr * P + ((lg ^ T::swz(lr)) << 3));
    const int rl = 4 * (lane >> 5) + ((lane >> 2) & 3);
    const int y = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr0 = 2 * (rl * P + ((y ^ T::swz(rl)) << 3) + 4 * (lane & 1));
  }
  __device__ __forceinline__ void flip_ra(int half) { ra0 ^= 2 * half; }
  __device__ __forceinline__ void flip_tr(int half) { tr0 ^= 2 * half; }
  __device__ __forceinline__ void flip(int half) {
    flip_ra(half);
    flip_tr(half);
  }
  // Carry a tile's distance from the base pointer the reads are given in the
  // transposed-read offset (bytes; a multiple of 32 P, clear of the bits the
  // XORs touch).  A ds_read's immediate offset holds 16 bits: with a tile
  // 64 KB or more into LDS the compiler otherwise adds the base to every
  // read's address.
  __device__ __forceinline__ void shift_tr(int bytes) { tr0 += bytes; }
  __device__ __forceinline__ void shift(int bytes) {
    ra0 += bytes;
    tr0 += bytes;
  }
  __device__ __forceinline__ bf16x8 row16(const bf16_t* tile, int r0, int kd) const {
    const char* p = reinterpret_cast<const char*>(tile + r0 * P + 128 * (kd / NRA)) + (ra0 ^ (32 * (kd % NRA)));
    return lds_read16(reinterpret_cast<const bf16_t*>(p));
  }
  __device__ __forceinline__ bf16x8 trA(const bf16_t* tile, int r0, int db) const {
    const char* p = reinterpret_cast<const char*>(tile + r0 * P + 128 * (db / NTR));
    const int o = tr0 ^ (64 * (db % NTR));
    return cat8(lds_read_tr4(reinterpret_cast<const bf16_t*>(p + o)),
                lds_read_tr4(reinterpret_cast<const bf16_t*>(p + (o ^ (32 | 16 * P)))));
  }
};

// Reads for a wavefront that owns 16 rows of a tile (rows of >= 256 bytes).
//  a16(tile, r0, s): 16x16x32 A/B fragment of rows r0 + lane % 16, head-dim
//    slots 32*s + 8*(lane/16) + e (one 16-byte read).
//  trA(tile, r0, db): 32x32x16 A operand whose rows are tile columns
//    32*db + lane % 32 and whose k slots are tile rows r0 + 8*(lane/32) + e,
//    e = 0..7 in order; two transposed reads of four rows each.
// The chunk of step s is (4s + lane/16) ^ swz = 4s ^ (lane/16 ^ swz), and of
// column block db (4db + y) ^ swz = 4db ^ (y ^ swz), so one base offset per
// read kind and an XOR per read cover them; row r + 4 (r % 8 < 4) has
// swz(r) ^ 1 and sits 4 P elements further, a bit the row term leaves clear.
template <int D>
struct TileReader16 {
  using T = Tile<D>;
  static constexpr int P = T::P;
  static_assert(T::PC >= 16 && T::PC == T::CPR, "16-row reads need unpadded rows of >= 256 bytes");
  int ra0, tr0;  // byte offsets
  __device__ __forceinline__ explicit TileReader16(int lane) {
    const int r = lane & 15;
    ra0 = 2 * (r * P + (((lane >> 4) ^ T::swz(r)) << 3));
    const int rl = 8 * (lane >> 5) + ((lane >> 2) & 3);
    const int y = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    tr0 = 2 * (rl * P + ((y ^ T::swz(rl)) << 3) + 4 * (lane & 1));
  }
  __device__ __forceinline__ void flip(int half) {
    ra0 ^= 2 * half;
    tr0 ^= 2 * half;
  }
  __device__ __forceinline__ bf16x8 a16(const bf16_t* tile, int r0, int s) const {
    const char* p = reinterpret_cast<const char*>(tile + r0 * P) + (ra0 ^ (64 * s));
    return lds_read16(reinterpret_cast<const bf16_t*>(p));
  }
  __device__ __forceinline__ bf16x8 trA(const bf16_t* tile, int r0, int db) const {
    const char* p = reinterpret_cast<const char*>(tile + r0 * P);
    const int o = tr0 ^ (64 * db);
    return cat8(lds_read_tr4(reinterpret_cast<const bf16_t*>(p + o)),
                lds_read_tr4(reinterpret_cast<const bf16_t*>(p + (o ^ (8 * P | 16)))));
  }
};

// Direct global->LDS copy of a ROWS x D tile of 16-bit elements into the
// swizzled layout.
// Load round i of wave w fills the 1 KiB block 4*i + w of the tile, i.e. tile
// rows 4*RW*i + RW*w + lane / PC (RW = 64 / PC rows per block), physical
// chunk lane % PC; the lane's source chunk follows from the row's swizzle.
template <int D>
struct TileLoader {
  using T = Tile<D>;
  static constexpr int PC = T::PC, CPR = T::CPR;
  static constexpr int RW = 64 / PC;  // tile rows per wave block
  int rl;    // this lane's row within a round's rows
  int x;     // physical chunk this lane fills
  int rs;     // row stride of the source in elements (wave-uniform; rs * 128 < 2^31)
  int rstep;  // 4 * RW * rs: source elements between two load rounds
  int lro;    // rl * rs
  __device__ __forceinline__ TileLoader(int w, int lane, int row_stride)
      : rl(RW * w + lane / PC), x(lane % PC), rs(row_stride), rstep(4 * RW * row_stride),
        lro(rl * row_stride) {}
  __device__ __forceinline__ int src_off(int r) const {  // element offset within the source row
    int c = x ^ T::swz(r);
    return (c < CPR ? c : 0) * 8;  // padding slots (D = 96): any in-bounds data
  }
  // Rows row0 .. row0+ROWS-1 of `g`, whose rows sit rs elements apart (the
  // D elements of a row contiguous).  Rows at or past `nrows` repeat row
  // nrows-1, which keeps every value finite; kernels mask them.
  // Each wave issues ROWS*PC/256 loads of 64 x 16 bytes; the caller waits on
  // vmcnt and synchronises before reading.  ASM issues them as inline
  // assembly (see lds_dma16); without it they go through the compiler's
  // builtin, which makes every later LDS read wait for them.
  template <int ROWS, bool ASM = true>
  __device__ __forceinline__ void load(bf16_t* tile, const bf16_t* g, int row0, int nrows, int w) const {
    constexpr int ROUNDS = ROWS * PC / 256;
    static_assert(ROWS * PC % 256 == 0, "tile must split evenly over four waves");
    const bf16_t* const g0 = g + (int64_t)row0 * rs;  // wave-uniform
    if (row0 + ROWS <= nrows) {
      // whole tile: the per-lane offsets do not depend on the tile, so they
      // stay in registers across the loop; the row step goes in the scalar base
#pragma unroll
      for (int i = 0; i < ROUNDS; ++i) {
        const int r = 4 * RW * i + rl;
        const bf16_t* base = g0 + i * rstep;  // wave-uniform
        if constexpr (ASM)
          lds_dma16(tile + (4 * i + w) * 512, base, (uint32_t)(lro + src_off(r)) * 2u);
        else
          __builtin_amdgcn_global_load_lds((const void*)(base + lro + src_off(r)),
                                           (LDS_AS void*)(tile + (4 * i + w) * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < ROUNDS; ++i) {
        const int r = 4 * RW * i + rl;
        if constexpr (ASM) {
          const int last = nrows - 1 - row0;  // last tile row that exists
          lds_dma16(tile + (4 * i + w) * 512, g0, (uint32_t)(min(r, last) * rs + src_off(r)) * 2u);
        } else {
          const int gr = min(row0 + r, nrows - 1);
          __builtin_amdgcn_global_load_lds((const void*)(g + (int64_t)gr * rs + src_off(r)),
                                           (LDS_AS void*)(tile + (4 * i + w) * 512), 16, 0, 0);
        }
      }
    }
  }

  // The same layout from rows at arbitrary offsets: tile row r comes from
  // g + rowoff(r) (elements, per lane, < 2^30), e.g. rows gathered from
  // several heads.  Issued like load(): ROWS * PC / 256 loads per wave.
  template <int ROWS, class RowOff>
  __device__ __forceinline__ void gather(bf16_t* tile, const bf16_t* g, RowOff rowoff, int w) const {
    constexpr int ROUNDS = ROWS * PC / 256;
    static_assert(ROWS * PC % 256 == 0, "tile must split evenly over four waves");
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int r = 4 * RW * i + rl;
      lds_dma16(tile + (4 * i + w) * 512, g, (uint32_t)(rowoff(r) + src_off(r)) * 2u);
    }
  }

  // The same as load() with the tile given by its LDS byte address (from
  // lds_addr): no generic-pointer conversion per load, which the compiler
  // otherwise rebuilds from the shared aperture with a null check each time.
  template <int ROWS>
  __device__ __forceinline__ void load_at(uint32_t tile, const bf16_t* g, int row0, int nrows, int w) const {
    constexpr int ROUNDS = ROWS * PC / 256;
    static_assert(ROWS * PC % 256 == 0, "tile must split evenly over four waves");
    const bf16_t* const g0 = g + (int64_t)row0 * rs;  // wave-uniform
    const uint32_t t0 = tile + (uint32_t)w * 1024u;
    if (row0 + ROWS <= nrows) {
#pragma unroll
      for (int i = 0; i < ROUNDS; ++i)
        lds_dma16_at(t0 + 4096u * i, g0 + i * rstep, (uint32_t)(lro + src_off(4 * RW * i + rl)) * 2u);
    } else {
      const int last = nrows - 1 - row0;  // last tile row that exists
#pragma unroll
      for (int i = 0; i < ROUNDS; ++i) {
        const int r = 4 * RW * i + rl;
        lds_dma16_at(t0 + 4096u * i, g0, (uint32_t)(min(r, last) * rs + src_off(r)) * 2u);
      }
    }
  }

  // One global_load_lds_dwordx4: lane l's 16 bytes at sbase + voff go to LDS
  // address dst + 16*l (dst and sbase wave-uniform).  Issued as inline
  // assembly so that the compiler does not treat the load as a write to LDS
  // that every later LDS read must wait for: the kernels read the other
  // buffer meanwhile and wait (vmcnt) and synchronise before reading this one.
  __device__ __forceinline__ static void lds_dma16(bf16_t* dst, const bf16_t* sbase, uint32_t voff) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(LDS_AS void*)(dst));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0v), "v"(voff), "s"(sbase) : "memory");
  }
  // the same with the LDS byte address itself (wave-uniform)
  __device__ __forceinline__ static void lds_dma16_at(uint32_t dst, const bf16_t* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(dst), "v"(voff), "s"(sbase) : "memory");
  }
};

// LDS byte address of a pointer into a __shared__ array (the value an LDS
// instruction or the DMA's m0 takes).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const LDS_AS void*)(p));
}

// Direct global->LDS copy of a ROWS x D tile by ONE wavefront, into the
// layout TileLoader<D> produces with four: 1 KiB block b holds tile rows
// RW * b .. RW * b + RW - 1, lane l filling physical chunk l % PC of row
// RW * b + l / PC.  The per-lane source offsets repeat every 16 / RW blocks
// (the swizzle depends on the row modulo 16), so they are kept for one period;
// each block adds its rows' offset to the wave-uniform base.
template <int D, int ROWS>
struct WaveTileLoader {
  using T = Tile<D>;
  static constexpr int PC = T::PC, CPR = T::CPR;
  static constexpr int RW = 64 / PC;               // tile rows per 1 KiB block
  static constexpr int NBLK = ROWS / RW;           // blocks (loads) per tile
  static constexpr int PER = 16 / RW < NBLK ? 16 / RW : NBLK;  // blocks per swizzle period
  static_assert(ROWS % RW == 0 && NBLK % PER == 0, "tile rows");
  int rs;         // row stride of the source in elements (wave-uniform)
  int lrow;       // this lane's row within a block
  int so[PER];    // per-lane source element offset of block b % PER, row offset included
  __device__ __forceinline__ WaveTileLoader(int lane, int row_stride) : rs(row_stride), lrow(lane / PC) {
    const int x = lane % PC;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = x ^ T::swz(RW * j + lrow);
      so[j] = lrow * row_stride + (c < CPR ? c : 0) * 8;  // padding slots (D = 96): any in-bounds data
    }
  }
  // Rows row0 .. row0 + ROWS - 1 of g; rows at or past nrows repeat row
  // nrows - 1 (row0 < nrows).  NBLK loads; the caller waits on vmcnt.
  __device__ __forceinline__ void load(bf16_t* tile, const bf16_t* g, int row0, int nrows) const {
    const bf16_t* const g0 = g + (int64_t)row0 * rs;  // wave-uniform
    if (row0 + ROWS <= nrows) {
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
        TileLoader<D>::lds_dma16(tile + b * 512, g0 + (int64_t)(RW * b) * rs, (uint32_t)so[b % PER] * 2u);
    } else {
      const int last = nrows - 1 - row0;
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int r = RW * b + lrow;
        const int c = (so[b % PER] - lrow * rs);  // the chunk's element offset
        TileLoader<D>::lds_dma16(tile + b * 512, g0, (uint32_t)(min(r, last) * rs + c) * 2u);
      }
    }
  }
};

// One global_load_lds_dword: lane l's 4 bytes at sbase + voff go to LDS
// address dst + 4*l (dst and sbase wave-uniform); inline assembly for the
// reason given at TileLoader::lds_dma16.
__device__ __forceinline__ void lds_dma4(void* dst, const void* sbase, uint32_t voff) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS void*)(dst));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(m0v), "v"(voff), "s"(sbase) : "memory");
}

// Per-row fp32 statistics of one query tile into LDS: dst[l] = src[row0 + l]
// for the 64 lanes l of the calling wave, rows past nrows-1 repeating the
// last row (row0 < nrows).  Waited for like the tile loads.
__device__ __forceinline__ void load_row_stat(float* dst, const float* src, int row0, int nrows, int lane) {
  lds_dma4(dst, src + row0, (uint32_t)min(lane, nrows - 1 - row0) * 4u);
}
// the same with dst given by its LDS byte address
__device__ __forceinline__ void load_row_stat_at(uint32_t dst, const float* src, int row0, int nrows, int lane) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(dst), "v"((uint32_t)min(lane, nrows - 1 - row0) * 4u), "s"(src + row0) : "memory");
}

// Scheduling pattern for a block of NM MFMAs that each consume RPM LDS reads:
// the first LA reads go out ahead, then every MFMA is followed by the reads
// of the one LA reads later.  Placed after the block's code; the compiler
// drops a pattern it cannot meet (for instance for want of registers).
template <int NM, int RPM, int LA = 6>
__device__ __forceinline__ void read_ahead() {
  constexpr int NR = NM * RPM;
  constexpr int L = LA < NR ? LA : NR;
  constexpr int MID = (NR - L) / RPM;
  static_assert((NR - L) % RPM == 0, "read pattern");
  __builtin_amdgcn_sched_group_barrier(0x100, L, 0);
#pragma unroll
  for (int t = 0; t < MID; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - MID, 0);
}

// ------------------------------------------------------------ block-sparse lists
// Under a block mask (one byte per 64 query rows x 64 keys, nonzero = kept) a
// workgroup visits only the tiles that some of its rows need.  One wavefront
// builds that list in LDS: for i = 0 .. n-1 it takes candidate c = order(i)
// and keeps it when covers(c) (some mask entry the tile touches is nonzero),
// preserving the order.  Returns the number kept (the same in every lane).
template <class Order, class Covers>
__device__ __forceinline__ int build_list(int* list, int n, int lane, Order order, Covers covers) {
  int count = 0;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const int c = i < n ? order(i) : 0;
    const bool keep = i < n && covers(c);
    const uint64_t bal = __ballot(keep);
    const int pos = count + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (keep) list[pos] = c;
    count += __popcll(bal);
  }
  return count;
}

// s_waitcnt lgkmcnt(0), leaving vmcnt/expcnt unconstrained: this wavefront's
// LDS reads have returned (before a direct load overwrites what they read).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(0), leaving expcnt/lgkmcnt unconstrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but the N most recent vector-memory loads done
// (vmcnt's low four bits in 3:0, its high two in 15:14).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Tile t and head h of workgroup `bid` in a grid of (tiles) x nh heads
// numbered tile-major, so that tile 0 (the caller's heaviest) goes first.
// Workgroups are dealt round-robin over the 8 XCDs: with nh a multiple of 8,
// XCD bid % 8 = j % 8 (j = bid mod nh) for every tile, and it is given heads
// (j % 8) nh / 8 .. + nh / 8 - 1, consecutive ones (those of one key/value
// head share K and V in that XCD's L2); every XCD gets every tile, so a
// causal triangle's heavy tiles spread over all of them.  Otherwise heads go
// round-robin.
struct TileHead {
  int t, h;
};
__device__ __forceinline__ TileHead tile_major(int bid, int nh) {
  const int t = bid / nh, j = bid - t * nh;
  const int h = (nh & 7) == 0 ? (j & 7) * (nh >> 3) + (j >> 3) : j;
  return {t, h};
}

}  // namespace cgqa
