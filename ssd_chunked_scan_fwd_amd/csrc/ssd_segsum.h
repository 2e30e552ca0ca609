// ssd_segsum.h -- chunk and state-block records and the per-chunk segment sums
// of the log decay, shared by the stand-alone cumsum stage and the chunk-state
// stage that computes them itself.
//
// Segment sums: within each chunk the cumulative log decay restarts at zero
// ("Transformers are SSMs" paper card, Method 5 / paper section 6: the
// 1-semiseparable mask of a chunk is exp of differences of these sums, and the
// last one is the chunk's total decay). Values are scaled by log2(e) so that
// later stages use exp2. The Mamba-2 block's call discretises first (paper card
// Method 6 block sketch; Paper vs code items 7-8): dt' = softplus(dt + dt_bias),
// log a = dt' A with A = -exp(A_log), and the key-side exponent
// ck_j = cs_j - log2(dt'_j) carries the input scale dt'_j into every weight.
#pragma once

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// log(1 + e^v); beyond v = 20 the correction log1p(e^-v) < 3e-9 is below fp32 resolution.
__device__ __forceinline__ float softplus_f32(float v) { return v > 20.f ? v : log1pf(expf(v)); }

// Packed rows: base_s = floor(cu[s]/span) + s is strictly increasing in s; the
// last s with base_s <= x owns slot x (span = Q for chunk slots, Gs*Q for
// state-block slots).
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int S, long x, int span) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const long base = cu[mid] / span + mid;
    if (base <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Record of chunk slot x of row `row` (x < slots_per_row): sequence, first
// token flattened over rows, length (0: a slot that holds no chunk), chunk index.
__device__ __forceinline__ int4 chunk_record(const int32_t* __restrict__ cu, int S, int row, long x, int T, int Q,
                                             long slots_per_row) {
  if (cu == nullptr) {
    const int t0 = (int)x * Q;
    return make_int4(row, row * T + t0, min(Q, T - t0), (int)x);
  }
  const int seq = find_seq(cu, S, x, Q);
  const int b = cu[seq], e = cu[seq + 1];
  const long j = x - (long)(b / Q + seq);
  const int nch = (e - b + Q - 1) / Q;
  if (j < 0 || j >= nch) return make_int4(seq, 0, 0, -1);
  const int t0 = b + (int)j * Q;
  return make_int4(seq, t0, min(Q, e - t0), (int)j);
}

// Record of state-block slot x of row `row` (x < blocks_per_row): sequence,
// first chunk slot (absolute), number of chunks (0: an empty block slot), 0.
__device__ __forceinline__ int4 block_record(const int32_t* __restrict__ cu, int S, int row, long x, int Q, int Gs,
                                             long slots_per_row) {
  if (cu == nullptr) {
    const int nch = (int)min((long)Gs, slots_per_row - x * Gs);
    return make_int4(row, (int)(row * slots_per_row + x * Gs), nch, 0);
  }
  const int span = Gs * Q;
  const int seq = find_seq(cu, S, x, span);
  const int b = cu[seq], e = cu[seq + 1];
  const long j = x - (long)(b / span + seq);
  const int nblk = (e - b + span - 1) / span;
  if (j < 0 || j >= nblk) return make_int4(seq, 0, 0, 0);
  const int nchs = (e - b + Q - 1) / Q;
  return make_int4(seq, b / Q + seq + (int)j * Gs, min(Gs, nchs - (int)j * Gs), 0);
}

// One wave writes the segment sums of one chunk and head: `tval(j)` gives the
// value of token j < len (log a, or dt' for Mamba-2 calls, where it is scanned
// as dt' A). out[j] = log2(e) (v_0 + .. + v_j) for j < Q, positions from len on
// repeating the total; outk[j] = out[j] - log2(dt'_j) for Mamba-2 calls (the
// total past len). lk, when given, receives outk (or out) as well. Returns the
// chunk total (log2-scaled) in every lane.
template <class F>
__device__ __forceinline__ float wave_segsum(F tval, int len, int Q, bool m2, float A, float* __restrict__ out,
                                             float* __restrict__ outk, float* __restrict__ lk, int lane) {
  // Every value is fetched before the scan, so their latencies overlap.
  constexpr int kMaxPieces = 256 / 64;
  float tv[kMaxPieces];
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    const int j = 64 * i + lane;
    tv[i] = (j < len && j < Q) ? tval(j) : 0.f;
  }
  float carry = 0.f;  // inclusive sum up to the last valid token seen so far
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    const int jb = 64 * i;
    if (jb >= Q) break;
    const int j = jb + lane;
    if (jb < len) {
      const float t = tv[i];
      float v = wave_incl_scan(m2 ? t * A : t);
      v += carry;
      carry = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), min(len - jb, 64) - 1));
      if (j < Q) {
        const float c = (j < len ? v : carry) * kLog2e;
        const float k = m2 && j < len ? c - log2f(t) : c;
        out[j] = c;
        if (m2) outk[j] = k;
        if (lk) lk[j] = k;
      }
    } else if (j < Q) {
      out[j] = carry * kLog2e;
      if (m2) outk[j] = carry * kLog2e;
      if (lk) lk[j] = carry * kLog2e;
    }
  }
  return carry * kLog2e;
}

}  // namespace ssd
