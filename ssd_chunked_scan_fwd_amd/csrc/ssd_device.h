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

// silu(v) = v / (1 + e^-v), with the hardware exp2 and reciprocal (a few ulp
// of fp32); v far below zero gives -0 through 1 / inf.
__device__ __forceinline__ float silu_f32(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + fast_exp2(-v * kLog2e));
}

// Inclusive sum over lanes 0..l of a wave (DPP): shifts of 1, 2, 4 and 8
// within each row of 16 lanes, then each row's total broadcast into the rows
// above it.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_pick(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_pick<0x111, 0xF>(v);   // row_shr:1
  v += dpp_pick<0x112, 0xF>(v);   // row_shr:2
  v += dpp_pick<0x114, 0xF>(v);   // row_shr:4
  v += dpp_pick<0x118, 0xF>(v);   // row_shr:8
  v += dpp_pick<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_pick<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// One 16x16x32 bf16 MFMA with fp32 accumulation (gfx950).
// A: lane l holds row (l % 16), 8 consecutive k of slot group (l / 16).
// B: lane l holds column (l % 16), the same 8 k. D: lane l holds column
// (l % 16), rows 4 * (l / 16) + r for r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Buffer resources (raw, unswizzled): loads at byte offsets at or beyond
// `bytes` return zero and touch no memory, and stores there are dropped. The
// kernels use them so that ragged rows and surplus lanes need no branch around
// a load: branches around loads make the compiler wait for every outstanding
// load where the paths join, which would serialise prefetches. The base must
// be the same in every lane; `bytes` must be below 2^31 (checked on the host).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;   // dword 3 of a raw buffer descriptor on gfx950
constexpr uint32_t kOffNone = 0x80000000u;    // an offset no descriptor here covers

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferFlags);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint16_t buf_load_u16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(u32x4 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2 v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// MI355X deals consecutive workgroups of a launch round-robin over its 8 XCDs,
// each with its own L2. Renumber them so that XCD x runs one contiguous range
// of units: the heads of one state block, which read the same B and C rows,
// then share one L2 instead of each XCD fetching every block's B and C. The map
// is a bijection of [0, n).
constexpr int kXcds = 8;
__device__ __forceinline__ long xcd_unit(long bid, long n) {
  const long q = n / kXcds, r = n % kXcds;
  const long x = bid % kXcds, local = bid / kXcds;
  return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

// The unit (state block slot m, head group k of `per` per block) that
// workgroup `bid` of the chunk-scan stage takes, n = slots * per workgroups.
// When the state-passing stage has ranked the block slots (btable[r].w =
// (slot + 1) | (nfull << 16) for rank r, slots with the most chunks first and
// nfull of them full), each XCD gets an equal share of the full blocks' units,
// in contiguous runs (one block's heads stay on one XCD's L2), ahead of an
// equal share of the others, which are dealt round robin by decreasing length:
// with one workgroup per CU the short sequence-end blocks then fill the last
// round instead of full blocks landing there. With every block full this is
// xcd_unit's order; without a ranking (ranked = 0, or w = 0) it is
// xcd_unit's order.
__device__ __forceinline__ void scan_unit(const int4* __restrict__ btable, long bid, long n, int per, int ranked,
                                          long& m, int& k) {
  const int w0 = ranked ? btable[0].w : 0;
  if (w0 == 0) {
    const long u = xcd_unit(bid, n);
    m = u / per;
    k = (int)(u % per);
    return;
  }
  const long F = (long)(w0 >> 16) * per;  // units of full blocks, ranked first
  const int x = (int)(bid % kXcds);
  const long l = bid / kXcds;
  const long fq = F / kXcds;
  const int fr = (int)(F % kXcds);
  const long fx = fq + (x < fr ? 1 : 0);
  long g;
  if (l < fx) {
    g = x * fq + (x < fr ? x : fr) + l;
  } else {
    // XCD xx holds ceil((n - xx) / 8) workgroups, fq + (xx < fr) of them full;
    // the rest counts differ by at most one between XCDs.
    auto rest = [&](int xx) { return (n - xx + kXcds - 1) / kXcds - (fq + (xx < fr ? 1 : 0)); };
    long mn = rest(0);
    for (int xx = 1; xx < kXcds; ++xx) mn = rest(xx) < mn ? rest(xx) : mn;
    const long j = l - fx;
    long sig = j * kXcds + x;
    if (j >= mn) {
      sig = kXcds * mn;
      for (int xx = 0; xx < x; ++xx) sig += rest(xx) > mn ? 1 : 0;
    }
    g = F + sig;
  }
  m = (long)(btable[g / per].w & 0xFFFF) - 1;
  k = (int)(g % per);
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

namespace ssd {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// gfx950 LDS transpose read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte pieces addressed by
// lanes 4k + i / 4, k = 0..3. When the 16 lanes of a group address a 4-row by
// 16-column block of 16-bit values (lane 4k + c: row k, columns 4c..4c+3), lane
// i receives column i of the 4 rows.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// MFMA operand with k along the rows of a row-major LDS tile W (pitch in
// elements): lane (c = l % 16, g = l / 16) receives W[row(s)][col0 + c] for
// its 8 slots s. Natural order: row(s) = row0 + 8g + s (the MFMA's own k order).
__device__ __forceinline__ u32x4 frag_k_rows_natural(const uint16_t* W, int pitch, int row0, int col0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const uint16_t* p0 = W + (row0 + 8 * g + (i >> 2)) * pitch + col0 + 4 * (i & 3);
  const u32x2 lo = lds_read_tr16(p0);
  const u32x2 hi = lds_read_tr16(p0 + 4 * pitch);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Same, with the slot order of a 16x16 accumulator pair: slots 0..3 hold rows
// row0 + 4g + 0..3 and slots 4..7 hold rows row0 + 16 + 4g + 0..3.
__device__ __forceinline__ u32x4 frag_k_rows_accpair(const uint16_t* W, int pitch, int row0, int col0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const uint16_t* p0 = W + (row0 + 4 * g + (i >> 2)) * pitch + col0 + 4 * (i & 3);
  const u32x2 lo = lds_read_tr16(p0);
  const u32x2 hi = lds_read_tr16(p0 + 16 * pitch);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// MFMA operand with k along the columns: lane (r = l % 16, g = l / 16) reads
// W[row0 + r][col0 + 8g .. col0 + 8g + 7] (one 16-byte read).
__device__ __forceinline__ u32x4 frag_k_cols(const uint16_t* W, int pitch, int row0, int col0, int lane) {
  return *reinterpret_cast<const u32x4*>(W + (row0 + (lane & 15)) * pitch + col0 + 8 * (lane >> 4));
}

// LDS row pitch (elements of 16 bits) for a row of `cols` values: an odd
// multiple of 32 bytes, which makes 16-byte row reads of 16 consecutive rows and
// the pair-order transpose read (frag_k_rows_accpair) free of bank conflicts
// on gfx950.
__host__ __device__ constexpr int lds_pitch(int cols) { return ((cols / 16) % 2 == 0) ? cols + 16 : cols + 32; }

// Row permutation within blocks of 32 rows under which a pair-order transpose
// read returns rows in natural order: data row 8g + 4t + k is stored at row
// 16t + 4g + k. frag_k_rows_accpair on rows stored at perm32(r) yields, in slot
// s of lane group g, data row 8g + s.
__device__ __forceinline__ int perm32(int r) {
  return (r & ~31) | (((r >> 2) & 1) << 4) | (((r >> 3) & 3) << 2) | (r & 3);
}

// Transposed-state tiles ([n][p] rows stored at perm32(n)) shift the upper 16
// rows of every 32-row block by 8 elements (inside the row padding): the
// state's 8-byte row stores by 32 lanes (16 rows, two pieces each) then cover
// all 64 banks once, where rows r and r + 16 would otherwise share banks. A
// transposed read stays within one 16-row half, so its pattern only moves.
constexpr int kHalfShift = 8;
__host__ __device__ constexpr int hs_row(int r, int pitch) { return r * pitch + ((r >> 4) & 1) * kHalfShift; }

// frag_k_rows_accpair on a tile stored with that shift: slots 4..7 come from
// the shifted half.
__device__ __forceinline__ u32x4 frag_k_rows_accpair_hs(const uint16_t* W, int pitch, int row0, int col0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const uint16_t* p0 = W + (row0 + 4 * g + (i >> 2)) * pitch + col0 + 4 * (i & 3);
  const u32x2 lo = lds_read_tr16(p0);
  const u32x2 hi = lds_read_tr16(p0 + 16 * pitch + kHalfShift);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Scale the 8 bf16 values of an operand by 8 fp32 weights and round back to bf16.
__device__ __forceinline__ u32x4 scale_frag(u32x4 v, const float* w) {
  u32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = pack_bf16x2(bf16_lo(v[c]) * w[2 * c], bf16_hi(v[c]) * w[2 * c + 1]);
  return r;
}

// Block-slot record written by the cumsum stage: sequence, first chunk slot,
// number of chunks (0: empty block slot).
struct BlockRec {
  int seq;
  int slot0;
  int nchunks;
};

__device__ __forceinline__ BlockRec load_block(const int4* table, long b) {
  int4 v = table[b];
  return BlockRec{v.x, v.y, v.z};
}

}  // namespace ssd
