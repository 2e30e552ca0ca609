// ssd_device.h -- device-side helpers shared by the gfx950 SSD kernels.
//
// Storage conventions: bf16 tensors are held as raw 16-bit words; conversion
// to fp32 is exact (shift), conversion from fp32 rounds to nearest even with
// the gfx950 hardware instruction (v_cvt_pk_bf16_f32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Two floats -> two bf16 (round to nearest even) packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One 16x16x32 bf16 MFMA with fp32 accumulation (gfx950).
// A: lane l holds row (l % 16), 8 consecutive k of slot group (l / 16).
// B: lane l holds column (l % 16), the same 8 k. D: lane l holds column
// (l % 16), rows 4 * (l / 16) + r for r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Chunk-slot record written by the cumsum stage: sequence (row when unpacked),
// first token in the row, number of tokens (0: empty slot), chunk index in sequence.
struct SlotRec {
  int seq;
  int tok0;  // first token, flattened over rows (row * T + t)
  int len;
  int kidx;
};

__device__ __forceinline__ SlotRec load_slot(const int4* table, long slot) {
  int4 v = table[slot];
  return SlotRec{v.x, v.y, v.z, v.w};
}

// Transposing 8x8 block of 16-bit values: in[r] holds row r (8 values, 4
// words); out[q] receives column q (the 8 row values at column q).
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = in[2 * k][c];
      const uint32_t b = in[2 * k + 1][c];
      // column 2c: low halves of rows 2k, 2k+1; column 2c+1: high halves.
      out[2 * c][k] = __builtin_amdgcn_perm(b, a, 0x05040100u);
      out[2 * c + 1][k] = __builtin_amdgcn_perm(b, a, 0x07060302u);
    }
  }
}

}  // namespace ssd
