// Internal helpers shared by the DASH HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed pair of bf16, round to nearest even (v_cvt_pk_bf16_f32 on
// gfx950); low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Logical tile order for a grid spread over the 8 XCDs (each with its own L2).
// Chunks of `chunk` consecutive logical ids are dealt to the XCDs in turn
// (chunk c runs on XCD c % 8, its ids in order), so a chunk shares one L2 and
// any prefix of the logical order (the tiles that hold rows when the row
// count is only known on the device) is spread over all XCDs.  Grids smaller
// than 8 chunks use chunks of nblocks / 8; ids past the last whole round of 8
// chunks map to themselves.  (Workgroup ids are dispatched to XCD bid % 8.)
__device__ __forceinline__ int xcd_remap_chunked(int bid, int nblocks, int chunk) {
  constexpr int kXcd = 8;
  if (chunk > nblocks / kXcd) chunk = nblocks / kXcd;
  if (chunk == 0) return bid;
  const int round = kXcd * chunk;
  const int full = (nblocks / round) * round;
  if (bid >= full) return bid;
  const int xcd = bid % kXcd;
  const int j = bid / kXcd;  // j-th workgroup dispatched to this XCD
  return ((j / chunk) * kXcd + xcd) * chunk + j % chunk;
}

}  // namespace dash
