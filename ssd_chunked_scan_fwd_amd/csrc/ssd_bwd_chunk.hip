// ssd_bwd_chunk.hip -- the backward pass of one chunk in one kernel (bf16, MFMA).
//
// The output of the chunked algorithm is y = M x with M = L o (C B^T) inside a
// chunk plus the contributions that pass through the chunk-entering state
// ("Transformers are SSMs" paper card, Method 5, the four terms of the chunked
// algorithm). Its reverse mode for one chunk and head, with h the state
// entering the chunk, lam the adjoint leaving it (the gradient reaching the
// chunk's last state from later outputs, decayed onto it), cs the cumulative
// log decay inside the chunk, e_s = 2^{cs_last - cs_s} and W = L o (dY X^T):
//   dX = (L o C B^T)^T dY + diag(e) B lam^T
//   dC = W B               + diag(2^cs) dY h      (summed over the group's heads)
//   dB = W^T C             + diag(e) X lam        (summed over the group's heads)
//   d log a_t = sum over pairs (s, u) with s < t <= u of M_us (dY_u . x_s),
// the pairs being both inside the chunk, s before it (through h), u after it
// (through lam) or both outside. The last form is a_t <lam_t, h_{t-1}> written
// out: every token pair whose decay product contains a_t contributes once.
//
// One workgroup (Q/16 waves) takes one chunk, one group and a slice of its
// heads: B, C and C B^T are loaded once, dB and dC accumulate over the slice's
// heads in registers, and each head's X, dY, h and lam pass through LDS once
// (the next head's are fetched while the current one's state terms are
// computed). The
// products run as 16x16x32 bf16 MFMAs with fp32 accumulation, transposed so
// that each lane holds four consecutive output channels of one token. Wave w
// owns one 16-token strip, as keys (dX, dB: queries from the strip on) and as
// queries (dC: keys up to the strip); the pair tiles of both roles are computed
// by the owner in the orientation whose accumulator layout is directly the
// B operand of the next product, so L o C B^T and L o dY X^T never go through
// LDS. Both enter their products as bf16 hi and lo pairs (two MFMAs on the same
// other operand), so the pair tiles are not rounded to bf16 once: the masked
// decayed products carry the full fp32 value into dX, dB and dC. Waves w and
// w + Q/32 share a SIMD and own strips w and Q/16 - 1 - w, which evens out the
// causal work.
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_segsum.h"

namespace ssd {

template <int P, int N, int Q>
struct BwdCfg {
  static constexpr int QT = Q / 16;         // 16-token strips, one per wave
  static constexpr int NW = QT, NTHR = 64 * NW;
  static constexpr int NT = N / 16, PT = P / 16;
  static constexpr int pN = lds_pitch(N), pP = lds_pitch(P);
  // 16-bit LDS tiles: B, C [Q][pN]; X, dY [Q][pP]; the states h, lam [P][pN].
  static constexpr int offB = 0, offC = Q * pN, offX = 2 * Q * pN, offY = offX + Q * pP, offH = offY + Q * pP,
                       offL = offH + P * pN, halfElems = offL + P * pN;
  // fp32 after the tiles, two heads in flight: cs [2][Q], the per-token pair
  // terms v and b [2][Q] each, the state dot products [2][NW]; and the row
  // sums of the pair tiles, one partial per wave, [NW][Q].
  static constexpr int floats = 6 * Q + 2 * NW + NW * Q;
  static constexpr size_t lds_bytes = (size_t)halfElems * 2 + (size_t)floats * 4;
  static_assert(Q == 64 || Q == 128, "chunk of 64 or 128 tokens");
  static_assert(P % 32 == 0 && N % 32 == 0, "head and state sizes in multiples of 32");
  static_assert(halfElems % 8 == 0, "fp32 area 16-byte aligned");
  static_assert(lds_bytes <= kMaxLdsBytes, "LDS of one workgroup");
};

// The 8 bf16 values of an operand scaled by one factor, rounded back to bf16.
__device__ __forceinline__ u32x4 scale_frag1(u32x4 v, float f) {
  u32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = pack_bf16x2(bf16_lo(v[c]) * f, bf16_hi(v[c]) * f);
  return r;
}

// Sums across lanes without the LDS crossbar: over the 16 lanes of each DPP
// row (quad swaps, then the half-row and row mirrors, which pair lanes of
// different quads and halves), and over the four rows (gfx950 row swaps).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_row16(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float sum_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// MFMA operand with k along the columns of a row-major LDS tile, in the slot
// order of frag_k_rows_accpair: lane (r = l % 16, g = l / 16) reads
// W[row0 + r][col0 + 4g .. 4g + 3] and W[row0 + r][col0 + 16 + 4g .. 16 + 4g + 3].
// Paired with a pair-order transposed read of the other operand (whose reads
// are free of bank conflicts at the lds_pitch pitches), the contraction runs
// over the same 32 k in a permuted order.
__device__ __forceinline__ u32x4 frag_k_cols_pair(const uint16_t* W, int pitch, int row0, int col0, int lane) {
  const uint16_t* p = W + (row0 + (lane & 15)) * pitch + col0 + 4 * (lane >> 4);
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Dot product of 4 fp32 values with 4 bf16 values (two words).
__device__ __forceinline__ float dot4_bf16(f32x4 a, u32x2 b) {
  return a[0] * bf16_lo(b.x) + a[1] * bf16_hi(b.x) + a[2] * bf16_lo(b.y) + a[3] * bf16_hi(b.y);
}

// Tile staging by NTHR threads: ROWS x COLS 16-bit values from global memory
// (row stride `gstride` bytes; offsets past the descriptor's range read as
// zero) into registers, then into LDS with row pitch PITCH.
template <int ROWS, int COLS, int NTHR>
struct StageT {
  static constexpr int kTotal = ROWS * COLS / 8;                 // 16-byte pieces
  static constexpr int kPieces = (kTotal + NTHR - 1) / NTHR;     // per thread
  static_assert(kTotal % NTHR == 0 || kTotal < NTHR, "whole pieces per thread");
  u32x4 v[kPieces];
  __device__ __forceinline__ void load(rsrc_t r, uint32_t gstride, int tid) {
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int i = tid + k * NTHR;
      v[k] = buf_load16(r, i < kTotal ? (uint32_t)(i / (COLS / 8)) * gstride + (uint32_t)(i % (COLS / 8)) * 16
                                      : kOffNone);
    }
  }
  template <int PITCH>
  __device__ __forceinline__ void store(uint16_t* dst, int tid) const {
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int i = tid + k * NTHR;
      if (i < kTotal) *reinterpret_cast<u32x4*>(dst + (i / (COLS / 8)) * PITCH + (i % (COLS / 8)) * 8) = v[k];
    }
  }
};

template <int P, int N, int Q>
__global__ __launch_bounds__(Q / 16 * 64, 1) void bwd_chunk_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ dY, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ Cm, const float* __restrict__ la, const float* __restrict__ fcs,
    const uint16_t* __restrict__ fstart, const uint16_t* __restrict__ rstart, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cur, int S, int T, long spr, long spr_r, uint16_t* __restrict__ dX,
    float* __restrict__ dla, void* __restrict__ dBo, void* __restrict__ dCo, long tokens, int H, int G, int nsl) {
  using K = BwdCfg<P, N, Q>;
  constexpr int QT = K::QT, NW = K::NW, NTHR = K::NTHR, NT = K::NT, PT = K::PT, HALF = QT / 2;
  constexpr int pN = K::pN, pP = K::pP;
  const long unit = xcd_unit(blockIdx.x, gridDim.x);
  const int sl = (int)(unit % nsl);
  const long rest = unit / nsl;
  const int g = (int)(rest % G);
  const long slot = rest / G;
  // The chunk of this slot (none for the slots between packed sequences).
  const int4 rec = cu == nullptr ? chunk_record(nullptr, 0, (int)(slot / spr), slot % spr, T, Q, spr)
                                 : chunk_record(cu, S, 0, slot, T, Q, spr);
  const int len = rec.z;
  if (len <= 0) return;
  const int seq = rec.x, tok0 = rec.y, jc = rec.w;
  const int hpg = H / G;
  const int hbeg = g * hpg + (int)((long)sl * hpg / nsl);
  const int hend = g * hpg + (int)((long)(sl + 1) * hpg / nsl);
  // The reversed run's slot of this chunk: reversed chunk nch - 1 - jc.
  int nch;
  long rslot;
  if (cu == nullptr) {
    nch = (int)spr;
    rslot = (long)seq * spr_r + (nch - 1 - jc);
  } else {
    nch = (cu[seq + 1] - cu[seq] + Q - 1) / Q;
    rslot = cur[seq] / Q + seq + (nch - 1 - jc);
  }
  const bool last_chunk = jc == nch - 1;

  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* Bs = lds + K::offB;
  uint16_t* Cs = lds + K::offC;
  uint16_t* Xs = lds + K::offX;
  uint16_t* Ys = lds + K::offY;
  uint16_t* Hs = lds + K::offH;
  uint16_t* Ls = lds + K::offL;
  float* csl = reinterpret_cast<float*>(lds + K::halfElems);  // [2][Q]
  float* vb = csl + 2 * Q;                                    // [2][Q] col_k - row_k + c_k
  float* bb = vb + 2 * Q;                                     // [2][Q] b_u
  float* red = bb + 2 * Q;                                    // [2][NW]
  float* rowp = red + 2 * NW;                                 // [NW][Q] row sums over this wave's keys

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g4 = lane >> 4;
  const int i = uniform(w < HALF ? w : QT - 1 - (w - HALF));  // the wave's strip
  const int u = 16 * i + c;  // the lane's token (a query in the query tiles, a key in the key tiles)

  const uint32_t xstride = (uint32_t)(H * P * 2), bstride = (uint32_t)(G * N * 2);
  auto x_rsrc = [&](const uint16_t* base, int h) {
    return make_rsrc(base + ((long)tok0 * H + h) * P, (uint32_t)len * xstride);
  };
  auto state_rsrc = [&](const uint16_t* base, long s, int h) {
    return make_rsrc(base + (s * H + h) * (long)(P * N), (uint32_t)(P * N * 2));
  };
  // <lam, h> of a head from its staged states: this wave's part to red.
  auto state_dot = [&](const StageT<P, N, NTHR>& sh, const StageT<P, N, NTHR>& sl2, float* dst) {
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < StageT<P, N, NTHR>::kPieces; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        d += bf16_lo(sh.v[k][q]) * bf16_lo(sl2.v[k][q]) + bf16_hi(sh.v[k][q]) * bf16_hi(sl2.v[k][q]);
    d = sum_rows4(sum_row16(d));
    if (lane == 0) dst[w] = d;
  };

  // ---- prologue: B, C and the first head's X, dY, states and segment sums
  {
    StageT<Q, N, NTHR> sb, sc;
    sb.load(make_rsrc(Bm + ((long)tok0 * G + g) * N, (uint32_t)len * bstride), bstride, tid);
    sc.load(make_rsrc(Cm + ((long)tok0 * G + g) * N, (uint32_t)len * bstride), bstride, tid);
    StageT<Q, P, NTHR> sx, sy;
    sx.load(x_rsrc(X, hbeg), xstride, tid);
    sy.load(x_rsrc(dY, hbeg), xstride, tid);
    StageT<P, N, NTHR> sh, sl2;
    sh.load(state_rsrc(fstart, slot, hbeg), (uint32_t)(N * 2), tid);
    sl2.load(state_rsrc(rstart, rslot, hbeg), (uint32_t)(N * 2), tid);
    if (tid < Q) csl[tid] = fcs[(slot * H + hbeg) * (long)Q + tid];
    sb.template store<pN>(Bs, tid);
    sc.template store<pN>(Cs, tid);
    sx.template store<pP>(Xs, tid);
    sy.template store<pP>(Ys, tid);
    sh.template store<pN>(Hs, tid);
    sl2.template store<pN>(Ls, tid);
    state_dot(sh, sl2, red);
  }
  __syncthreads();

  // C B^T of one tile, recomputed for every head (registers are the limit):
  // key orientation (query tile t as rows u, the strip as column s) or query
  // orientation (key tile t as rows s, the strip as column u).
  auto cbt = [&](int t, bool key) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < N / 32; ++kk)
      a = key ? mfma16x16x32(frag_k_cols(Cs, pN, 16 * t, 32 * kk, lane), frag_k_cols(Bs, pN, 16 * i, 32 * kk, lane), a)
              : mfma16x16x32(frag_k_cols(Bs, pN, 16 * t, 32 * kk, lane), frag_k_cols(Cs, pN, 16 * i, 32 * kk, lane), a);
    return a;
  };

  f32x4 dc[NT], db[NT];  // dC^T, dB^T of the strip: row n, column token
#pragma unroll
  for (int m = 0; m < NT; ++m) dc[m] = db[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int h = hbeg; h < hend; ++h) {
    const int hb = (h - hbeg) & 1;
    const float* cs = csl + hb * Q;
    const float anext = last_chunk ? 1.f : fast_exp2(la[(long)(tok0 + len) * H + h] * kLog2e);
    const float csu = cs[u];
    for (int q = lane; q < Q; q += 64) rowp[w * Q + q] = 0.f;  // this wave's row only

    // ---- the strip as keys: query tiles ut >= i in pairs (one 32-token k block
    // of the pair-order operands). W1 = L o C B^T (bf16 hi and lo parts) and
    // W2 = L o dY X^T feed dX^T += dY^T W1 and dB^T += C^T W2; the column
    // sums of S = W1 o dY X^T (queries u > s) and its row sums (keys s < u of
    // this strip, partial per wave) feed d log a.
    f32x4 dx[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) dx[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float colsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < HALF; ++kk) {
      if (2 * kk + 1 < i) continue;
      uint32_t w1h[4], w1l[4], w2[4], w2l[4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int ut = 2 * kk + hf;
        w1h[2 * hf] = w1h[2 * hf + 1] = w1l[2 * hf] = w1l[2 * hf + 1] = w2[2 * hf] = w2[2 * hf + 1] = 0u;
        w2l[2 * hf] = w2l[2 * hf + 1] = 0u;
        if (ut < i) continue;  // queries before the strip: zero
        f32x4 m2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < P / 32; ++kp)
          m2 = mfma16x16x32(frag_k_cols(Ys, pP, 16 * ut, 32 * kp, lane), frag_k_cols(Xs, pP, 16 * i, 32 * kp, lane),
                            m2);
        const f32x4 csq = *reinterpret_cast<const f32x4*>(cs + 16 * ut + 4 * g4);
        const f32x4 mk = cbt(ut, true);
        float a1[4], a2[4], sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int uq = 16 * ut + 4 * g4 + r;  // query row; the key is the lane's token
          const float l = uq >= u ? fast_exp2(csq[r] - csu) : 0.f;
          a1[r] = l * mk[r];
          a2[r] = l * m2[r];
          sv[r] = uq > u ? a1[r] * m2[r] : 0.f;
          colsum += sv[r];
        }
        // row sums of the query rows over this strip's keys
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = sum_row16(sv[r]);
        if (c == 0) {
          f32x4* rp = reinterpret_cast<f32x4*>(rowp + w * Q + 16 * ut + 4 * g4);
          *rp += f32x4{sv[0], sv[1], sv[2], sv[3]};
        }
        w1h[2 * hf] = pack_bf16x2(a1[0], a1[1]);
        w1h[2 * hf + 1] = pack_bf16x2(a1[2], a1[3]);
        w1l[2 * hf] = pack_bf16x2(a1[0] - bf16_lo(w1h[2 * hf]), a1[1] - bf16_hi(w1h[2 * hf]));
        w1l[2 * hf + 1] = pack_bf16x2(a1[2] - bf16_lo(w1h[2 * hf + 1]), a1[3] - bf16_hi(w1h[2 * hf + 1]));
        w2[2 * hf] = pack_bf16x2(a2[0], a2[1]);
        w2[2 * hf + 1] = pack_bf16x2(a2[2], a2[3]);
        w2l[2 * hf] = pack_bf16x2(a2[0] - bf16_lo(w2[2 * hf]), a2[1] - bf16_hi(w2[2 * hf]));
        w2l[2 * hf + 1] = pack_bf16x2(a2[2] - bf16_lo(w2[2 * hf + 1]), a2[3] - bf16_hi(w2[2 * hf + 1]));
      }
      const u32x4 bh = {w1h[0], w1h[1], w1h[2], w1h[3]}, bl = {w1l[0], w1l[1], w1l[2], w1l[3]};
      const u32x4 b2 = {w2[0], w2[1], w2[2], w2[3]}, b2l = {w2l[0], w2l[1], w2l[2], w2l[3]};
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const u32x4 ya = frag_k_rows_accpair(Ys, pP, 32 * kk, 16 * pt, lane);
        dx[pt] = mfma16x16x32(ya, bh, dx[pt]);
        dx[pt] = mfma16x16x32(ya, bl, dx[pt]);
      }
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const u32x4 ca = frag_k_rows_accpair(Cs, pN, 32 * kk, 16 * m, lane);
        db[m] = mfma16x16x32(ca, b2, db[m]);
        db[m] = mfma16x16x32(ca, b2l, db[m]);
      }
    }

    // ---- the strip as queries: key tiles st <= i in pairs. W2 = L o dY X^T in
    // this orientation feeds dC^T += B^T W2^T.
#pragma unroll
    for (int kk = 0; kk < HALF; ++kk) {
      if (2 * kk > i) continue;
      uint32_t w2q[4], w2ql[4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int st = 2 * kk + hf;
        w2q[2 * hf] = w2q[2 * hf + 1] = w2ql[2 * hf] = w2ql[2 * hf + 1] = 0u;
        if (st > i) continue;  // keys after the strip: zero
        f32x4 m2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < P / 32; ++kp)
          m2 = mfma16x16x32(frag_k_cols(Xs, pP, 16 * st, 32 * kp, lane), frag_k_cols(Ys, pP, 16 * i, 32 * kp, lane),
                            m2);
        const f32x4 csk = *reinterpret_cast<const f32x4*>(cs + 16 * st + 4 * g4);
        float a2[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sk = 16 * st + 4 * g4 + r;  // key row; the query is the lane's token
          const float l = sk <= u ? fast_exp2(csu - csk[r]) : 0.f;
          a2[r] = l * m2[r];
        }
        w2q[2 * hf] = pack_bf16x2(a2[0], a2[1]);
        w2q[2 * hf + 1] = pack_bf16x2(a2[2], a2[3]);
        w2ql[2 * hf] = pack_bf16x2(a2[0] - bf16_lo(w2q[2 * hf]), a2[1] - bf16_hi(w2q[2 * hf]));
        w2ql[2 * hf + 1] = pack_bf16x2(a2[2] - bf16_lo(w2q[2 * hf + 1]), a2[3] - bf16_hi(w2q[2 * hf + 1]));
      }
      const u32x4 bq = {w2q[0], w2q[1], w2q[2], w2q[3]}, bql = {w2ql[0], w2ql[1], w2ql[2], w2ql[3]};
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const u32x4 ba = frag_k_rows_accpair(Bs, pN, 32 * kk, 16 * m, lane);
        dc[m] = mfma16x16x32(ba, bq, dc[m]);
        dc[m] = mfma16x16x32(ba, bql, dc[m]);
      }
    }
    colsum = sum_rows4(colsum);

    // The next head's inputs, fetched into registers while this head's state
    // terms are computed.
    const bool more = h + 1 < hend;
    StageT<Q, P, NTHR> nx, ny;
    StageT<P, N, NTHR> nh, nl;
    float ncs = 0.f;
    if (more) {
      nx.load(x_rsrc(X, h + 1), xstride, tid);
      ny.load(x_rsrc(dY, h + 1), xstride, tid);
      nh.load(state_rsrc(fstart, slot, h + 1), (uint32_t)(N * 2), tid);
      nl.load(state_rsrc(rstart, rslot, h + 1), (uint32_t)(N * 2), tid);
      if (tid < Q) ncs = fcs[(slot * H + h + 1) * (long)Q + tid];
    }

    // ---- terms through the states
    const float cs_last = cs[Q - 1];
    {
      const float fu = fast_exp2(csu);
      const float es = anext * fast_exp2(cs_last - csu);
      // b_u = 2^{cs_u} dY_u . (h C_u)
      f32x4 t[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) t[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk) {
        const u32x4 bop = frag_k_cols(Cs, pN, 16 * i, 32 * kk, lane);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) t[pt] = mfma16x16x32(frag_k_cols(Hs, pN, 16 * pt, 32 * kk, lane), bop, t[pt]);
      }
      float b = 0.f;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
        b += dot4_bf16(t[pt], *reinterpret_cast<const u32x2*>(Ys + u * pP + 16 * pt + 4 * g4));
      b = sum_rows4(b);
      // dX_off = e_s lam B_s; c_s = x_s . dX_off
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) t[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk) {
        const u32x4 bop = frag_k_cols(Bs, pN, 16 * i, 32 * kk, lane);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) t[pt] = mfma16x16x32(frag_k_cols(Ls, pN, 16 * pt, 32 * kk, lane), bop, t[pt]);
      }
      float cc = 0.f;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        t[pt] *= es;
        cc += dot4_bf16(t[pt], *reinterpret_cast<const u32x2*>(Xs + u * pP + 16 * pt + 4 * g4));
        dx[pt] += t[pt];
      }
      cc = sum_rows4(cc);
      if (g4 == 0) {
        vb[hb * Q + u] = colsum + cc;
        bb[hb * Q + u] = b * fu;
      }
      // dC^T += h^T (2^cs dY)^T ; dB^T += lam^T (e X)^T
#pragma unroll
      for (int kk = 0; kk < P / 32; ++kk) {
        const u32x4 yop = scale_frag1(frag_k_cols_pair(Ys, pP, 16 * i, 32 * kk, lane), fu);
        const u32x4 xop = scale_frag1(frag_k_cols_pair(Xs, pP, 16 * i, 32 * kk, lane), es);
#pragma unroll
        for (int m = 0; m < NT; ++m) {
          dc[m] = mfma16x16x32(frag_k_rows_accpair(Hs, pN, 32 * kk, 16 * m, lane), yop, dc[m]);
          db[m] = mfma16x16x32(frag_k_rows_accpair(Ls, pN, 32 * kk, 16 * m, lane), xop, db[m]);
        }
      }
      // dX of the lane's token, four consecutive channels per P tile
      const rsrc_t rdx = x_rsrc(dX, h);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
        buf_store8(u32x2{pack_bf16x2(dx[pt][0], dx[pt][1]), pack_bf16x2(dx[pt][2], dx[pt][3])}, rdx,
                   (uint32_t)u * xstride + (uint32_t)(16 * pt + 4 * g4) * 2);
    }
    __syncthreads();  // this head's tiles are no longer read; its pair terms are complete

    // ---- d log a of the chunk's tokens: sum_{k<t} (col_k - row_k + c_k) + sum_{u>=t} b_u + D
    if (w == 0) {
      constexpr int EPL = Q / 64;
      const float* vh = vb + hb * Q;
      const float* bh = bb + hb * Q;
      float v[EPL], bv[EPL], pv[EPL], pb[EPL];
      float sv = 0.f, sb = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int t = lane * EPL + e;
        float rsum = 0.f;
#pragma unroll
        for (int k = 0; k < NW; ++k) rsum += rowp[k * Q + t];
        v[e] = vh[t] - rsum;
        bv[e] = bh[t];
        pv[e] = sv;
        pb[e] = sb;
        sv += v[e];
        sb += bv[e];
      }
      const float iv = wave_incl_scan(sv), ib = wave_incl_scan(sb);
      const float totb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ib), 63));
      const float ev = iv - sv, eb = ib - sb;
      float dsum = 0.f;
#pragma unroll
      for (int k = 0; k < NW; ++k) dsum += red[hb * NW + k];
      const float dspan = anext * fast_exp2(cs_last) * dsum;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int t = lane * EPL + e;
        if (t < len) dla[(long)(tok0 + t) * H + h] = ev + pv[e] + (totb - eb - pb[e]) + dspan;
      }
    }
    if (more) {
      nx.template store<pP>(Xs, tid);
      ny.template store<pP>(Ys, tid);
      nh.template store<pN>(Hs, tid);
      nl.template store<pN>(Ls, tid);
      if (tid < Q) csl[(hb ^ 1) * Q + tid] = ncs;
      state_dot(nh, nl, red + (hb ^ 1) * NW);
    }
    __syncthreads();
  }

  // ---- dB, dC of the slice's heads: bf16 when one slice covers the group,
  // else fp32 partials [nsl][tokens][G][N] that a reduction sums.
  if (nsl == 1) {
    const rsrc_t rb = make_rsrc(reinterpret_cast<uint16_t*>(dBo) + ((long)tok0 * G + g) * N, (uint32_t)len * bstride);
    const rsrc_t rc = make_rsrc(reinterpret_cast<uint16_t*>(dCo) + ((long)tok0 * G + g) * N, (uint32_t)len * bstride);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const uint32_t off = (uint32_t)u * bstride + (uint32_t)(16 * m + 4 * g4) * 2;
      buf_store8(u32x2{pack_bf16x2(db[m][0], db[m][1]), pack_bf16x2(db[m][2], db[m][3])}, rb, off);
      buf_store8(u32x2{pack_bf16x2(dc[m][0], dc[m][1]), pack_bf16x2(dc[m][2], dc[m][3])}, rc, off);
    }
  } else {
    const long base = ((long)sl * tokens + tok0) * G * N + (long)g * N;
    const uint32_t fstride = (uint32_t)(G * N * 4);
    const rsrc_t rb = make_rsrc(reinterpret_cast<float*>(dBo) + base, (uint32_t)len * fstride);
    const rsrc_t rc = make_rsrc(reinterpret_cast<float*>(dCo) + base, (uint32_t)len * fstride);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const uint32_t off = (uint32_t)u * fstride + (uint32_t)(16 * m + 4 * g4) * 4;
      buf_store16(__builtin_bit_cast(u32x4, db[m]), rb, off);
      buf_store16(__builtin_bit_cast(u32x4, dc[m]), rc, off);
    }
  }
}

// The state entering every chunk, from the states entering the state blocks:
// h_0 = the block's entering state and h_{j+1} = a_j h_j + S_j, where a_j is
// chunk j's total decay and S_j = sum_t 2^{cs_last - cs_t} x_t B_t^T its state
// term (paper card Method 5: the chunk-state and state-passing terms, here
// taken one chunk at a time inside a block). h stays in fp32 registers; each
// h_j is written in bf16. One workgroup per (state block, head), 4 waves, each
// holding N/64 row tiles of h^T (row n, column p) so that a lane stores four
// consecutive n of one p.
template <int P, int N, int Q>
__global__ __launch_bounds__(256, 2) void chunk_starts_kernel(const uint16_t* __restrict__ X,
                                                             const uint16_t* __restrict__ Bm,
                                                             const int4* __restrict__ table,
                                                             const int4* __restrict__ btable,
                                                             const float* __restrict__ cs,
                                                             const uint16_t* __restrict__ bstart,
                                                             uint16_t* __restrict__ out, int H, int G) {
  constexpr int PT = P / 16, NTW = N / 64, pN = lds_pitch(N), pP = lds_pitch(P);
  static_assert(N % 64 == 0 && P % 16 == 0, "state tiles over four waves");
  // XCD-aware order: each XCD runs whole blocks, so a block's B rows are read
  // into one L2 rather than into every XCD's.
  const long unit = xcd_unit(blockIdx.x, gridDim.x);
  const long blk = unit / H;
  const int h = (int)(unit % H);
  const int4 br = btable[blk];
  const int nch = br.z;
  if (nch <= 0) return;
  const long slot0 = br.y;
  const int g = h / (H / G);
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* Xs = lds;                                        // [Q][pP]
  uint16_t* Bs = Xs + Q * pP;                                // [Q][pN]
  float* wt = reinterpret_cast<float*>(Bs + Q * pN);         // [Q] weights 2^{cs_last - cs_t}
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g4 = lane >> 4;
  const uint32_t xstride = (uint32_t)(H * P * 2), bstride = (uint32_t)(G * N * 2);

  f32x4 hs[NTW][PT];  // h^T: row n = 16 (NTW w + a) + 4 g4 + r, column p = 16 pt + c
  {
    const rsrc_t rs = make_rsrc(bstart + (blk * H + h) * (long)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const u32x2 v = buf_load8(rs, (uint32_t)((16 * pt + c) * N + 16 * (NTW * w + a) + 4 * g4) * 2);
        hs[a][pt] = f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
      }
  }
  // Chunk j + 1's X and B, and its segment sums, are fetched into registers
  // while chunk j is multiplied.
  StageT<Q, P, 256> sx;
  StageT<Q, N, 256> sb;
  float pcs = 0.f, plast = 0.f;
  auto fetch = [&](long slot) {
    const int4 rec = table[slot];
    sx.load(make_rsrc(X + ((long)rec.y * H + h) * P, (uint32_t)rec.z * xstride), xstride, tid);
    sb.load(make_rsrc(Bm + ((long)rec.y * G + g) * N, (uint32_t)rec.z * bstride), bstride, tid);
    const rsrc_t rc = make_rsrc(cs + (slot * H + h) * (long)Q, (uint32_t)(Q * 4));
    pcs = buf_load_f32(rc, tid < Q ? (uint32_t)(tid * 4) : kOffNone);
    plast = buf_load_f32(rc, (uint32_t)((Q - 1) * 4));  // positions past the chunk's end repeat its total
  };
  if (nch > 1) fetch(slot0);
  for (int j = 0; j < nch; ++j) {
    const long slot = slot0 + j;
    {
      const rsrc_t ro = make_rsrc(out + (slot * H + h) * (long)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
      for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          buf_store8(u32x2{pack_bf16x2(hs[a][pt][0], hs[a][pt][1]), pack_bf16x2(hs[a][pt][2], hs[a][pt][3])}, ro,
                     (uint32_t)((16 * pt + c) * N + 16 * (NTW * w + a) + 4 * g4) * 2);
    }
    if (j == nch - 1) break;
    sx.template store<pP>(Xs, tid);
    sb.template store<pN>(Bs, tid);
    const float cs_last = plast;
    if (tid < Q) wt[tid] = fast_exp2(cs_last - pcs);
    __syncthreads();
    if (j + 2 < nch) fetch(slot + 1);
    const float aj = fast_exp2(cs_last);
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) hs[a][pt] *= aj;
#pragma unroll
    for (int kk = 0; kk < Q / 32; ++kk) {
      // token order of the pair-order reads: 4 g4 + (0..3), then 16 + 4 g4 + (0..3)
      float wk[8];
      *reinterpret_cast<f32x4*>(wk) = *reinterpret_cast<const f32x4*>(wt + 32 * kk + 4 * g4);
      *reinterpret_cast<f32x4*>(wk + 4) = *reinterpret_cast<const f32x4*>(wt + 32 * kk + 16 + 4 * g4);
      u32x4 bo[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) bo[pt] = frag_k_rows_accpair(Xs, pP, 32 * kk, 16 * pt, lane);
#pragma unroll
      for (int a = 0; a < NTW; ++a) {
        const u32x4 ao = scale_frag(frag_k_rows_accpair(Bs, pN, 32 * kk, 16 * (NTW * w + a), lane), wk);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) hs[a][pt] = mfma16x16x32(ao, bo[pt], hs[a][pt]);
      }
    }
    __syncthreads();
  }
}

template <int P, int N, int Q>
static hipError_t launch_chunk_starts_t(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                        void* out, hipStream_t stream) {
  constexpr size_t lds = (size_t)Q * (lds_pitch(P) + lds_pitch(N)) * 2 + (size_t)Q * 4;
  auto kern = chunk_starts_kernel<P, N, Q>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(d.nblocks * d.H)), dim3(256), lds, stream,
                     reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B), ws.table, ws.btable,
                     ws.cs, reinterpret_cast<const uint16_t*>(ws.start_states), reinterpret_cast<uint16_t*>(out), d.H,
                     d.G);
  return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_chunk_starts_q(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                        void* out, hipStream_t stream) {
  switch (d.Q) {
    case 64: return launch_chunk_starts_t<P, N, 64>(d, X, B, ws, out, stream);
    case 128: return launch_chunk_starts_t<P, N, 128>(d, X, B, ws, out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_starts(const FwdDims& d, const void* X, const void* B, const Workspace& ws, void* out,
                               hipStream_t stream) {
  if (!d.bf16 || !bwd_chunk_supported(d.P, d.N, d.Q, true)) return hipErrorInvalidValue;
  if (d.P == 32) return d.N == 64 ? launch_chunk_starts_q<32, 64>(d, X, B, ws, out, stream)
                                  : launch_chunk_starts_q<32, 128>(d, X, B, ws, out, stream);
  if (d.P == 64) return d.N == 64 ? launch_chunk_starts_q<64, 64>(d, X, B, ws, out, stream)
                                  : launch_chunk_starts_q<64, 128>(d, X, B, ws, out, stream);
  return launch_chunk_starts_q<128, 64>(d, X, B, ws, out, stream);
}

// The tail of the fused backward, one launch: workgroups [0, sb) sum the dB
// partials over the head slices, [sb, 2 sb) the dC partials (out[t][g][n] =
// sum over slices of part[sl][t][g][n], rounded to bf16, four per thread;
// sb = 0 with one slice), and the rest form the initial-state gradient,
// dinit = exp(log a of the sequence's first token) * lam_first.
__global__ __launch_bounds__(256) void bwd_tail_kernel(const float* __restrict__ part_b,
                                                       const float* __restrict__ part_c, uint16_t* __restrict__ dB,
                                                       uint16_t* __restrict__ dC, long n4, int nsl, long sb,
                                                       const float* __restrict__ la,
                                                       const float* __restrict__ lam_first,
                                                       float* __restrict__ dinit, const int32_t* __restrict__ cu,
                                                       int T, int H, int PN, long dtotal) {
  const long blk = blockIdx.x;
  if (blk < 2 * sb) {
    const bool c = blk >= sb;
    const float* part = c ? part_c : part_b;
    const long i = (blk - (c ? sb : 0)) * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4 a = reinterpret_cast<const f32x4*>(part)[i];
    for (int s = 1; s < nsl; ++s) a += reinterpret_cast<const f32x4*>(part)[(long)s * n4 + i];
    reinterpret_cast<u32x2*>(c ? dC : dB)[i] = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    return;
  }
  const long i = (blk - 2 * sb) * 256 + threadIdx.x;
  if (i >= dtotal) return;
  const long sh = i / PN;
  const int s = (int)(sh / H), h = (int)(sh % H);
  const long first = cu ? (long)cu[s] : (long)s * T;
  dinit[i] = __builtin_amdgcn_exp2f(la[first * H + h] * kLog2e) * lam_first[i];
}

template <int P, int N, int Q>
static hipError_t launch_bwd_chunk_t(const BwdChunkArgs& a, hipStream_t stream) {
  using K = BwdCfg<P, N, Q>;
  auto kern = bwd_chunk_kernel<P, N, Q>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)K::lds_bytes);
  if (e != hipSuccess) return e;
  const long grid = a.nslots * a.G * a.nsl;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(K::NTHR), K::lds_bytes, stream,
                     reinterpret_cast<const uint16_t*>(a.X), reinterpret_cast<const uint16_t*>(a.dY),
                     reinterpret_cast<const uint16_t*>(a.B), reinterpret_cast<const uint16_t*>(a.C), a.la, a.fcs,
                     reinterpret_cast<const uint16_t*>(a.fstart), reinterpret_cast<const uint16_t*>(a.rstart), a.cu,
                     a.cur, a.S, a.T, a.spr, a.spr_r,
                     reinterpret_cast<uint16_t*>(a.dX), a.dla, a.nsl == 1 ? a.dB : a.part_b,
                     a.nsl == 1 ? a.dC : a.part_c, a.tokens, a.H, a.G, a.nsl);
  e = hipGetLastError();
  if (e != hipSuccess || (a.nsl == 1 && !a.dinit)) return e;
  const long n4 = a.tokens * a.G * a.N / 4;
  const long sb = a.nsl > 1 ? (n4 + 255) / 256 : 0;
  const long dtotal = a.dinit ? (long)a.nseq * a.H * a.P * a.N : 0;
  const long blocks = 2 * sb + (dtotal + 255) / 256;
  hipLaunchKernelGGL(bwd_tail_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.part_b, a.part_c,
                     reinterpret_cast<uint16_t*>(a.dB), reinterpret_cast<uint16_t*>(a.dC), n4, a.nsl, sb, a.la,
                     a.lam_first, a.dinit, a.cu, a.T, a.H, a.P * a.N, dtotal);
  return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_bwd_chunk_q(const BwdChunkArgs& a, hipStream_t stream) {
  switch (a.Q) {
    case 64: return launch_bwd_chunk_t<P, N, 64>(a, stream);
    case 128: return launch_bwd_chunk_t<P, N, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// The (P, N) pairs built: P in {32, 64} with N in {64, 128}, and P = 128 with N = 64.
bool bwd_chunk_supported(int P, int N, int Q, bool bf16) {
  if (!bf16 || (Q != 64 && Q != 128)) return false;
  return ((P == 32 || P == 64) && (N == 64 || N == 128)) || (P == 128 && N == 64);
}

// Head slices per (chunk, group). One workgroup runs per CU at a time (256
// CUs), so a launch of wgs * nsl workgroups takes about ceil(wgs * nsl / 256)
// rounds of ceil(hpg / nsl) heads each. Every slice beyond the first also
// writes, and the tail kernel reads, dB and dC partials of its chunks; those of
// 256 chunks cost about one such head-round. The count with the lowest cost
// wins (the smaller on ties), at most 8: for 128 chunks of 32 heads in one
// group, 2 slices (256 workgroups of 16 heads); for 261 chunks of 80 heads, 8,
// where one slice would leave 5 workgroups of all 80 heads to a second round.
int bwd_chunk_slices(long nslots, int G, int H) {
  const int hpg = H / G;
  const long wgs = nslots * G;
  int best = 1;
  long best_cost = -1;
  for (int nsl = 1; nsl <= (hpg < 8 ? hpg : 8); ++nsl) {
    const long rounds = (wgs * nsl + 255) / 256;
    const long cost = rounds * ((hpg + nsl - 1) / nsl) * 256 + (long)(nsl - 1) * wgs;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = nsl;
    }
  }
  return best;
}

hipError_t launch_bwd_chunks(const BwdChunkArgs& a, hipStream_t stream) {
  if (!bwd_chunk_supported(a.P, a.N, a.Q, true)) return hipErrorInvalidValue;
  if (a.P == 32) return a.N == 64 ? launch_bwd_chunk_q<32, 64>(a, stream) : launch_bwd_chunk_q<32, 128>(a, stream);
  if (a.P == 64) return a.N == 64 ? launch_bwd_chunk_q<64, 64>(a, stream) : launch_bwd_chunk_q<64, 128>(a, stream);
  return launch_bwd_chunk_q<128, 64>(a, stream);
}

}  // namespace ssd
