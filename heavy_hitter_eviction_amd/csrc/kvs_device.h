// Device-side helpers shared by the libkvs kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvs_internal.h"

namespace kvs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kTile = 16;          // slots per tile == tokens per block

__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 (stored as the upper 16 bits of a float) to float: exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return bits_to_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bits_to_f32(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// using the gfx950 row-swap permutes. The combine order is the same in every
// lane, so all four rows end up with bit-identical results.
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f32_bits(x), f32_bits(x), false, false);
  x = fmaxf(bits_to_f32(a[0]), bits_to_f32(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return fmaxf(bits_to_f32(b[0]), bits_to_f32(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f32_bits(x), f32_bits(x), false, false);
  x = bits_to_f32(a[0]) + bits_to_f32(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return bits_to_f32(b[0]) + bits_to_f32(b[1]);
}

// Reductions over each group of eight consecutive lanes (l ^ 1 and l ^ 2
// within a quad by DPP quad permutes, then lane 7 - l of the group by the
// half-row mirror). The pairs combine in the same order in every lane up to
// commutation, so all eight lanes of a group hold bit-identical results.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return bits_to_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_bits(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppRowMirror = 0x140;   // row_mirror

__device__ __forceinline__ float oct_max(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  return fmaxf(x, dpp_f32<kDppHalfMirror>(x));
}

__device__ __forceinline__ float oct_sum(float x) {
  x = x + dpp_f32<kDppXor1>(x);
  x = x + dpp_f32<kDppXor2>(x);
  return x + dpp_f32<kDppHalfMirror>(x);
}

// Maximum over the whole wave, in every lane: groups of eight, then each
// 16-lane row (lane 15 - l), then the four rows. fmaxf is exact and drops
// NaNs in any order, so the result does not depend on the order.
__device__ __forceinline__ float wave_max(float x) {
  x = oct_max(x);
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return rows_max(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform "any lane" / "all lanes" votes.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
__device__ __forceinline__ bool wave_all(bool p) {
  return __builtin_amdgcn_ballot_w64(p) == __builtin_amdgcn_read_exec();
}

// ---------------------------------------------------------------------------
// FP8 E4M3 (OCP: bias 7, no infinity, NaN = 0x7F/0xFF, largest finite 448).
// Encoding follows the format definition directly: clip to 448, pick the
// binade (the subnormal range shares the 2^-9 quantum of the lowest binade),
// scale to an integer grid by a power of two (exact), round half to even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = f32_bits(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = bits_to_f32(u & 0x7FFFFFFFu);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                 // below 2^-6: quantum 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);          // 0..8, ties to even
  } else {
    const int e = (int)((f32_bits(a) >> 23) & 0xFF) - 127;  // -6 .. 8
    const float n = __builtin_rintf(a * bits_to_f32((uint32_t)(127 + 3 - e) << 23));  // 8..16
    code = (uint32_t)((e + 7) * 8) + (uint32_t)n - 8u;
  }
  return code | sign;
}

// absmax / 240, correctly rounded (the pages' per-position scale).
__device__ __forceinline__ float fp8_scale_of(float absmax) { return __fdiv_rn(absmax, 240.0f); }

// Element i of a row of float32 or (src_bf16) bf16 values, widened exactly.
__device__ __forceinline__ float load_src(const void* p, size_t i, int src_bf16) {
  if (src_bf16) return bf16_lo((uint32_t)((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

// E4M3 code of x / s (the quotient rounded once); a zero scale (all-zero row)
// gives code 0.
__device__ __forceinline__ uint32_t encode_with_scale(float x, float s) {
  return s > 0.0f ? e4m3_encode(__fdiv_rn(x, s)) : 0u;
}

// Four FP8 codes (one dword) to four bf16 values, exact (E4M3 is a subset of bf16).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// ---------------------------------------------------------------------------
// Cache tile layout. A tile is 16 consecutive slots of one (sequence, KV head),
// 16*D elements of K and as many of V. Both are stored fragment-major: the
// 16-byte chunk i that MFMA lane l (l = 16*kg + j) of the decode kernel reads
// sits at byte 1024*i + 16*l of the tile, so one load instruction covers one
// contiguous KiB.
//   K: lane (j, kg) chunk i holds slot j, row bytes [64 i + 16 kg, +16).
//   V: lane (j, kg) chunk i holds bytes [16 i, +16) of the run
//      {slot 4 kg + e, dim (D/16) j + n : n < D/16, e < 4}, element 4 n + e.
// Byte offsets inside the tile of element (slot t, dim x), element size eb:
__host__ __device__ __forceinline__ uint32_t k_tile_offset(int t, int x, int eb) {
  const int xb = x * eb;
  return (uint32_t)(((xb / 64 * 4 + (xb % 64) / 16) * 16 + t) * 16 + xb % 16);
}
__host__ __device__ __forceinline__ uint32_t v_tile_offset(int t, int x, int D, int eb) {
  const int kg = t / 4, e = t % 4, j = x / (D / 16), n = x % (D / 16);
  const int ub = (4 * n + e) * eb;
  return (uint32_t)(((ub / 16 * 4 + kg) * 16 + j) * 16 + ub % 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
}

}  // namespace kvs
