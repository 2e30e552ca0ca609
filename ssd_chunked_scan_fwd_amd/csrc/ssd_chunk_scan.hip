// ssd_chunk_scan.hip -- diagonal blocks and left factors of the chunked SSD
// forward pass on gfx950, with the state carried through each state block.
//
// For every chunk and head, with cs the log2-scaled cumulative decay and h the
// state entering the chunk:
//   Y[i][p] = exp2(cs_i) sum_n C[i][n] h[p][n]                        (left factor)
//           + sum_{j <= i} exp2(cs_i - cs_j) (sum_n C[i][n] B[j][n]) X[j][p]
//                                                                   (diagonal block)
// ("Transformers are SSMs" paper card, Method 5 / paper section 6, "Diagonal
// Blocks" and "Left Factors": the masked within-chunk product and the carry of
// the entering state, decayed from the chunk start). The mask is applied before
// the exponential (paper card, Pitfalls), so no positive exponent is formed.
//
// bf16 path, one workgroup of 8 waves per (state block, head), one workgroup
// per CU. The block's entering state comes from the state-passing stage;
// inside the block the workgroup walks its chunks in order and advances the
// state itself, h <- exp2(A_k) h + sum_j exp2(cs_last - cs_j) X[j] B[j]^T (the
// centre-factor recurrence of paper section 6 with the right factor of each
// chunk), keeping h in fp32 MFMA accumulators. With one chunk per block this
// is exactly the pages' schedule.
//  * Decay factorisation per 16-row query tile with m = cs at its first row:
//    for keys j before the tile, exp2(cs_i - cs_j) = u_i v_j with
//    u_i = exp2(cs_i - m) <= 1 and v_j = exp2(m - cs_j) <= 1 (cs never
//    increases), so neither factor overflows whatever the decay. Y_i =
//    u_i (sum_{j before the tile} (S o V)_ij X_j + exp2(m) (C h^T)_i) + the
//    key block holding the diagonal, which uses the exact masked
//    exp2(cs_i - cs_j) and is added after the accumulator is scaled by u_i.
//    Most of the per-element work is one multiply by a tabulated v_j.
//  * S^T = B C^T is computed tile by tile on 16x16x32 bf16 MFMA. Its
//    accumulator layout (lane = query row i, registers = 4 key rows j) is, after
//    masking and the v_j factor, directly the A operand of the next MFMA, so S
//    never goes through LDS. S o V is carried as a bf16 hi/lo pair (two MFMAs
//    on the same X fragment): one bf16 rounding alone would double the output
//    error of the pass.
//  * X, the decay-weighted X for the state update and B are staged token-major
//    in LDS through registers (the next chunk's rows and C fragments in flight
//    while the current chunk is computed); operands that contract over tokens
//    use the gfx950 LDS transpose read. The state goes to LDS transposed.
//    The waves accumulate Y^T (MFMA operands swapped: lane = query row,
//    registers = consecutive channels), so after one v_permlane16_swap each
//    lane stores 16 contiguous bytes of its token's row straight to HBM.
//  * Mamba-2 block calls: the key-side weights read ck = cs - log2(dt')
//    instead of cs, so x enters unscaled and dt' rides in the weights; the skip
//    D x_i is added on the diagonal of the diagonal key block's L o S; the gate
//    multiplies by silu(z) in fp32 before the one rounding of Y (paper card
//    Method 6 block sketch; Paper vs code items 3 and 7).
//  * Query tiles are dealt so that each SIMD's pair of waves gets one short
//    and one long row of the triangle; the state update is spread over all
//    waves. Two barriers per chunk.
#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_stage.h"

namespace ssd {

namespace {

constexpr int kScanWaves = 8;
constexpr int kScanThreads = kScanWaves * 64;
// Output forms of the bf16 kernels: plain bf16, bf16 through the silu(z) gate,
// or fp32 (per-head partials that the backward pass sums before rounding).
constexpr int kOutPlain = 0, kOutGated = 1, kOutF32 = 2;

template <int P, int N>
struct ScanCfg {
  static constexpr int BP = lds_pitch(N);   // B rows
  static constexpr int XP = lds_pitch(P);   // X rows, weighted X rows
  static constexpr int HP = lds_pitch(P);   // transposed state rows [N][HP] (rows stored at perm32(n))
  static_assert(HP >= P + kHalfShift, "the half shift stays inside the row padding");
  static constexpr int TP = P / 16, TN = N / 16, NB = N / 32;
  static constexpr int WN = TN < 4 ? TN : 4;
  static constexpr int WP = (kScanWaves / WN) < TP ? (kScanWaves / WN) : TP;
  static constexpr int TPW = TP / WP, TNW = TN / WN;
  static constexpr int CBN = N / 8, CBP = P / 8;
  static constexpr int RB = (kPassRows * CBN + kScanThreads - 1) / kScanThreads;
  static constexpr int RX = (kPassRows * CBP + kScanThreads - 1) / kScanThreads;
};

// Query tile of wave w in round k: SIMD s = w % 4 pairs tile s with tile 7 - s.
__device__ __forceinline__ int scan_tile(int k, int w) { return 8 * k + (w < 4 ? w : 11 - w); }

// Output of one wave's transposed tile: acc[pt][r] holds Y[token][pt * 16 +
// 4 * g4 + r] for the lane's token (query row l16 of the tile), and `row` is
// the element offset of that token's row in Y (and in z). For a pair of P
// tiles, v_permlane16_swap exchanges the halves of lane groups so that each
// lane holds 8 consecutive channels of its token: group g4 gets
// p = 32 q + 16 (g4 & 1) + 8 (g4 >> 1) .. + 7, stored as one 16-byte piece (rows
// past the chunk's length fall outside the buffer range and are dropped). A
// single P tile (P = 16) leaves as 8-byte pieces. With GATE the values are
// multiplied by silu(z) in fp32 before the one rounding to bf16 (the Mamba-2
// block's output gate, paper card Method 6), z read in the same pieces.
template <int TP>
struct ZPieces {
  u32x4 q[TP / 2 > 0 ? TP / 2 : 1];
  u32x2 t;
};

__device__ __forceinline__ uint32_t yT_piece(uint32_t row, int q, int g4) {
  return row + 32 * q + 16 * (g4 & 1) + 8 * (g4 >> 1);
}

// fp32 output of a transposed tile (lane: 4 consecutive channels of its token
// per P tile), for partial results that are summed before their one rounding.
template <int TP>
__device__ __forceinline__ void store_yT_f32(const f32x4 (&acc)[TP], rsrc_t ry, uint32_t row, int g4) {
#pragma unroll
  for (int pt = 0; pt < TP; ++pt) buf_store16(__builtin_bit_cast(u32x4, acc[pt]), ry, (row + pt * 16 + 4 * g4) * 4);
}

template <int TP>
__device__ __forceinline__ void load_zT(ZPieces<TP>& z, rsrc_t rz, uint32_t row, int g4) {
#pragma unroll
  for (int q = 0; q < TP / 2; ++q) z.q[q] = buf_load16(rz, yT_piece(row, q, g4) * 2);
  if (TP % 2) z.t = buf_load8(rz, (row + (TP - 1) * 16 + 4 * g4) * 2);
}

template <int TP, bool GATE>
__device__ __forceinline__ void store_yT(const f32x4 (&acc)[TP], rsrc_t ry, uint32_t row, int g4,
                                         const ZPieces<TP>& z) {
#pragma unroll
  for (int q = 0; q < TP / 2; ++q) {
    const f32x4 lo = acc[2 * q], hi = acc[2 * q + 1];
    u32x4 v;
    if (GATE) {
      float y[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo[r]), __float_as_uint(hi[r]), false, false);
        y[r] = __uint_as_float(sw[0]);
        y[4 + r] = __uint_as_float(sw[1]);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w)
        v[w] = pack_bf16x2(y[2 * w] * silu_f32(bf16_lo(z.q[q][w])), y[2 * w + 1] * silu_f32(bf16_hi(z.q[q][w])));
    } else {
      const auto sx = __builtin_amdgcn_permlane16_swap(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(hi[0], hi[1]), false,
                                                       false);
      const auto sy = __builtin_amdgcn_permlane16_swap(pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[2], hi[3]), false,
                                                       false);
      v = u32x4{sx[0], sy[0], sx[1], sy[1]};
    }
    buf_store16(v, ry, yT_piece(row, q, g4) * 2);
  }
  if (TP % 2) {
    const f32x4 lo = acc[TP - 1];
    u32x2 v;
    if (GATE) {
      v = u32x2{pack_bf16x2(lo[0] * silu_f32(bf16_lo(z.t[0])), lo[1] * silu_f32(bf16_hi(z.t[0]))),
                pack_bf16x2(lo[2] * silu_f32(bf16_lo(z.t[1])), lo[3] * silu_f32(bf16_hi(z.t[1])))};
    } else {
      v = u32x2{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
    }
    buf_store8(v, ry, (row + (TP - 1) * 16 + 4 * g4) * 2);
  }
}


}  // namespace

// Chunks of up to 128 tokens with P <= 64 keep a separate decay-weighted copy
// of X (at N = 256 the tiles then fill 153 KB); the others weight X in place
// after the outputs are done (two more barriers).
static bool scan_in_place(int P, int N, int Q) { return Q > 128 || P > 64; }

// The v_j table ([Q/16][Q] fp32) is kept for chunks of up to 128 tokens;
// longer chunks compute v_j where it is used. cs and ck take [Q] each.
size_t chunk_scan_bf16_lds_bytes(int P, int N, int Q) {
  const size_t nIt = Q / 16;
  const size_t xcopies = scan_in_place(P, N, Q) ? 1 : 2;
  const size_t el = (size_t)Q * lds_pitch(N) + xcopies * (size_t)Q * lds_pitch(P) + (size_t)N * lds_pitch(P);
  return el * 2 + ((Q > 128 ? 0 : nIt * Q) + 2 * Q) * 4 + 16 * 16;
}

// ITW: query tiles per wave (1 for chunks of up to 128 tokens, 2 for 256).
template <int P, int N, int ITW, int OUT>
__global__ __launch_bounds__(kScanThreads, 1) void chunk_scan_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ B, const uint16_t* __restrict__ C,
    const int4* __restrict__ ctable, const int4* __restrict__ btable, const float* __restrict__ cs,
    const float* __restrict__ ck, const uint16_t* __restrict__ start, uint16_t* __restrict__ Y,
    const uint16_t* __restrict__ Z, const float* __restrict__ Dskip, int H, int G, int Q) {
  constexpr bool GATE = OUT == kOutGated;  // silu(z) gate on the output
  constexpr bool YF32 = OUT == kOutF32;    // fp32 output (partials summed before one rounding)
  using K = ScanCfg<P, N>;
  const long unit = xcd_unit(blockIdx.x, gridDim.x);
  const int h = (int)(unit % H);
  const long m = unit / H;
  const BlockRec blk = load_block(btable, m);
  if (blk.nchunks <= 0) return;
  const int g = h / (H / G);
  const int nIt = Q / 16;

  // Weight X in place after the outputs when a second copy does not fit.
  constexpr bool kInPlace = ITW > 1 || P > 64;
  extern __shared__ uint16_t lds[];
  uint16_t* bs = lds;                                 // [Q][BP]  B rows
  uint16_t* xs = bs + Q * K::BP;                      // [Q][XP]  X rows
  uint16_t* xw = kInPlace ? xs : xs + Q * K::XP;      // [Q][XP]  X rows times exp2(cs_last - cs_j)
  uint16_t* hsT = xw + Q * K::XP;                     // [N][HP]  state entering the chunk, transposed
  constexpr bool kVTable = ITW == 1;                  // tabulate v_j (chunks of up to 128 tokens)
  int4* recs = reinterpret_cast<int4*>(hsT + N * K::HP);  // [16] chunk records of the block
  float* Vt = reinterpret_cast<float*>(recs + 16);    // [nIt][Q] v_j = exp2(m - ck_j) per query tile
  float* csl = Vt + (kVTable ? nIt * Q : 0);          // [Q] cumulative log2 decay cs
  float* ckl = csl + Q;                               // [Q] key-side exponent ck

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const long ldb = (long)G * N, ldx = (long)H * P;
  const float Dh = Dskip ? Dskip[h] : 0.f;            // skip weight, on the diagonal of L o S

  // Per-thread constant byte offsets of its staged pieces within a chunk (rows
  // past the chunk's length fall outside the chunk's buffer range and load 0).
  uint32_t boff[K::RB], xoff[K::RX];
  int brow[K::RB], xrow[K::RX];
#pragma unroll
  for (int u = 0; u < K::RB; ++u) {
    const int idx = tid + kScanThreads * u;
    brow[u] = idx / K::CBN;
    boff[u] = idx < kPassRows * K::CBN ? (uint32_t)((brow[u] * ldb + (idx % K::CBN) * 8) * 2) : kOffNone;
  }
#pragma unroll
  for (int u = 0; u < K::RX; ++u) {
    const int idx = tid + kScanThreads * u;
    xrow[u] = idx / K::CBP;
    xoff[u] = idx < kPassRows * K::CBP ? (uint32_t)((xrow[u] * ldx + (idx % K::CBP) * 8) * 2) : kOffNone;
  }

  // Byte offset of this lane's C fragment row in each of its query tiles.
  uint32_t cfoff[ITW];
#pragma unroll
  for (int k = 0; k < ITW; ++k) {
    const int it = scan_tile(k, wave);
    cfoff[k] = it < nIt ? (uint32_t)(((it * 16 + l16) * ldb + 8 * g4) * 2) : kOffNone;
  }

  // State tiles of this wave and the state entering the block.
  const int wn = wave % K::WN, wp = wave / K::WN;
  const bool sact = wp < K::WP;
  const int p0t = wp * K::TPW, n0t = wn * K::TNW;
  f32x4 hacc[K::TPW][K::TNW];
  {
    const rsrc_t rs = make_rsrc(start + (m * H + h) * (long)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
    for (int a = 0; a < K::TPW; ++a)
#pragma unroll
      for (int b = 0; b < K::TNW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hacc[a][b][r] = bf16_to_f32(buf_load_u16(
              rs, sact ? (uint32_t)((((p0t + a) * 16 + 4 * g4 + r) * N + (n0t + b) * 16 + l16) * 2) : kOffNone));
  }

  // Registers holding the next chunk.
  u32x4 pb[K::RB], px[K::RX];
  // C fragments of this wave's query tiles: prefetched with the next chunk up
  // to N = 128; beyond, loaded once this chunk's outputs are done (the
  // registers of a second set held through the output phase would spill).
  constexpr bool kPrefetchC = N <= 128;
  u32x4 pcf[ITW][K::NB];
  float pcs_t = 0.f, pck_t = 0.f, pcs_last = 0.f;
  constexpr int VE = kVTable ? 2 : 1;    // v-table entries per thread: nIt*Q <= VE*512
  float pcs_v[VE], pcs_vm[VE];
  float pcs_x[K::RX];

  // Loads of one chunk's B, X, C fragments and decay values into registers.
  // Every load is issued unconditionally (ragged rows and surplus lanes read
  // zeros through the buffer range); with valid == false nothing is read.
  auto prefetch = [&](const SlotRec& r, long slot, bool valid) {
    const int len = valid ? r.len : 0;
    const rsrc_t rb = make_rsrc(B + ((long)r.tok0 * G + g) * N, (uint32_t)(len * ldb * 2));
    const rsrc_t rx = make_rsrc(X + ((long)r.tok0 * H + h) * P, (uint32_t)(len * ldx * 2));
    const rsrc_t rcc = make_rsrc(C + ((long)r.tok0 * G + g) * N, (uint32_t)(len * ldb * 2));
    const rsrc_t rc = make_rsrc(cs + (slot * H + h) * (long)Q, valid ? (uint32_t)(Q * 4) : 0u);
    const rsrc_t rk = make_rsrc(ck + (slot * H + h) * (long)Q, valid ? (uint32_t)(Q * 4) : 0u);
#pragma unroll
    for (int u = 0; u < K::RB; ++u) pb[u] = buf_load16(rb, boff[u]);
#pragma unroll
    for (int u = 0; u < K::RX; ++u) {
      px[u] = buf_load16(rx, xoff[u]);
      pcs_x[u] = buf_load_f32(rk, (uint32_t)(min(xrow[u], Q - 1) * 4));
    }
    if constexpr (kPrefetchC) {
#pragma unroll
      for (int k = 0; k < ITW; ++k)
#pragma unroll
        for (int nb = 0; nb < K::NB; ++nb) pcf[k][nb] = buf_load16(rcc, cfoff[k] + nb * 64);
    }
    pcs_last = buf_load_f32(rc, (uint32_t)((Q - 1) * 4));
    pcs_t = buf_load_f32(rc, (uint32_t)(tid * 4));            // zero for tid >= Q
    pck_t = buf_load_f32(rk, (uint32_t)(tid * 4));
#pragma unroll
    for (int u = 0; u < VE; ++u) {
      const int e = tid + kScanThreads * u;
      if (kVTable) {
        pcs_v[u] = buf_load_f32(rk, (uint32_t)((e % Q) * 4));
        pcs_vm[u] = buf_load_f32(rc, (uint32_t)(16 * (e / Q) * 4));  // zero past the table
      }
    }
  };

  if (tid < blk.nchunks) recs[tid] = ctable[blk.slot0 + tid];
  __syncthreads();
  auto rec_of = [&](int c) {
    const int4 v = recs[c];
    return SlotRec{uniform(v.x), uniform(v.y), uniform(v.z), uniform(v.w)};
  };
  SlotRec rec = rec_of(0);
  prefetch(rec, blk.slot0, true);
  auto load_c = [&](const SlotRec& r, bool valid) {
    const rsrc_t rcc = make_rsrc(C + ((long)r.tok0 * G + g) * N, valid ? (uint32_t)(r.len * ldb * 2) : 0u);
#pragma unroll
    for (int k = 0; k < ITW; ++k)
#pragma unroll
      for (int nb = 0; nb < K::NB; ++nb) pcf[k][nb] = buf_load16(rcc, cfoff[k] + nb * 64);
  };
  if constexpr (!kPrefetchC) load_c(rec, true);

  for (int c = 0; c < blk.nchunks; ++c) {
    const long slot = blk.slot0 + c;
    const int len = rec.len;
    const long tok0 = rec.tok0;
    const float cs_last = pcs_last;

    __syncthreads();  // every wave is done with the previous chunk's tiles
    u32x4 cf[ITW][K::NB];
#pragma unroll
    for (int k = 0; k < ITW; ++k)
#pragma unroll
      for (int nb = 0; nb < K::NB; ++nb) cf[k][nb] = pcf[k][nb];
    // B, X and decay-weighted X rows of the first pass.
#pragma unroll
    for (int u = 0; u < K::RB; ++u)
      if ((tid + kScanThreads * u) < kPassRows * K::CBN && brow[u] < Q)
        *reinterpret_cast<u32x4*>(bs + brow[u] * K::BP + ((tid + kScanThreads * u) % K::CBN) * 8) = pb[u];
#pragma unroll
    for (int u = 0; u < K::RX; ++u) {
      if ((tid + kScanThreads * u) < kPassRows * K::CBP && xrow[u] < Q) {
        const int o = xrow[u] * K::XP + ((tid + kScanThreads * u) % K::CBP) * 8;
        *reinterpret_cast<u32x4*>(xs + o) = px[u];
        if (!kInPlace) {
          const float w = fast_exp2(cs_last - pcs_x[u]);
          u32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(bf16_lo(px[u][q]) * w, bf16_hi(px[u][q]) * w);
          *reinterpret_cast<u32x4*>(xw + o) = v;
        }
      }
    }
    // cs, ck and the v_j table per (query tile, key).
    if (tid < Q) {
      csl[tid] = pcs_t;
      ckl[tid] = pck_t;
    }
#pragma unroll
    for (int u = 0; u < VE; ++u) {
      const int e = tid + kScanThreads * u;
      if (kVTable && e < nIt * Q) Vt[e] = (e % Q) < 16 * (e / Q) ? fast_exp2(pcs_vm[u] - pcs_v[u]) : 0.f;
    }
    // Chunks longer than one pass: the remaining rows, synchronously.
    for (int r0 = kPassRows; r0 < Q; r0 += kPassRows) {
      const float* ckr = ck + (slot * H + h) * (long)Q;
      for (int idx = tid; idx < kPassRows * K::CBN; idx += kScanThreads) {
        const int j = r0 + idx / K::CBN, cc = idx % K::CBN;
        *reinterpret_cast<u32x4*>(bs + j * K::BP + cc * 8) =
            j < len ? *reinterpret_cast<const u32x4*>(B + (tok0 * G + g) * N + j * ldb + cc * 8) : u32x4{0u, 0u, 0u, 0u};
      }
      for (int idx = tid; idx < kPassRows * K::CBP; idx += kScanThreads) {
        const int j = r0 + idx / K::CBP, cc = idx % K::CBP;
        const u32x4 v0 = j < len ? *reinterpret_cast<const u32x4*>(X + (tok0 * H + h) * P + j * ldx + cc * 8)
                                 : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(xs + j * K::XP + cc * 8) = v0;
        if (!kInPlace) {
          const float w = fast_exp2(cs_last - ckr[j]);
          u32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(bf16_lo(v0[q]) * w, bf16_hi(v0[q]) * w);
          *reinterpret_cast<u32x4*>(xw + j * K::XP + cc * 8) = v;
        }
      }
    }
    // State entering the chunk, transposed to [n][p] in bf16.
    if (sact) {
#pragma unroll
      for (int a = 0; a < K::TPW; ++a)
#pragma unroll
        for (int b = 0; b < K::TNW; ++b) {
          const u32x2 v = {pack_bf16x2(hacc[a][b][0], hacc[a][b][1]), pack_bf16x2(hacc[a][b][2], hacc[a][b][3])};
          *reinterpret_cast<u32x2*>(hsT + hs_row(perm32((n0t + b) * 16 + l16), K::HP) + (p0t + a) * 16 + 4 * g4) = v;
        }
    }
    const bool more = c + 1 < blk.nchunks;
    rec = rec_of(more ? c + 1 : c);
    prefetch(rec, slot + (more ? 1 : 0), more);
    __syncthreads();

    // ---------------- outputs of this chunk: Y_i = u_i (sum_j (S o V)_ij X_j + exp2(m) (C h^T)_i)
#pragma unroll
    for (int k = 0; k < ITW; ++k) {
      const int it = scan_tile(k, wave);
      if (it >= nIt || it * 16 >= len) continue;
      const int irow = it * 16 + l16;
      // Y^T accumulators: lane = query row l16, registers = 4 consecutive p.
      f32x4 acc[K::TP];
#pragma unroll
      for (int pt = 0; pt < K::TP; ++pt) {
        acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < K::NB; ++nb)
          acc[pt] = mfma16x16x32(frag_k_rows_accpair_hs(hsT, K::HP, nb * 32, pt * 16, lane), cf[k][nb], acc[pt]);
      }
      const float mref = csl[16 * it];
      const float em = fast_exp2(mref);
#pragma unroll
      for (int pt = 0; pt < K::TP; ++pt) acc[pt] *= em;
      const float* vrow = Vt + it * Q + 4 * g4;
      const float cs_i = csl[irow];
      const int kbd = it >> 1;  // key block holding the diagonal tile
      // One key block of 32 tokens: S^T tiles of both halves (two interleaved
      // MFMA chains), the decay factor, the bf16 hi/lo split, then Y += M X.
      // diag: exact masked decay (a half above the diagonal masks to zero);
      // otherwise the tabulated (or computed) v_j, u_i being applied later.
      auto key_block = [&](int kb, bool diag) {
        u32x4 bfr[2][K::NB];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int nb = 0; nb < K::NB; ++nb) bfr[half][nb] = frag_k_cols(bs, K::BP, (2 * kb + half) * 16, nb * 32, lane);
        f32x4 fac[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int j0 = (2 * kb + half) * 16 + 4 * g4;
          if (diag || !kVTable) {
            const f32x4 cj = *reinterpret_cast<const f32x4*>(ckl + j0);
            const float ref = diag ? cs_i : mref;
#pragma unroll
            for (int r = 0; r < 4; ++r) fac[half][r] = (!diag || j0 + r <= irow) ? fast_exp2(ref - cj[r]) : 0.f;
          } else {
            fac[half] = *reinterpret_cast<const f32x4*>(vrow + (2 * kb + half) * 16);
          }
        }
        f32x4 sv[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int nb = 0; nb < K::NB; ++nb)
#pragma unroll
          for (int half = 0; half < 2; ++half) sv[half] = mfma16x16x32(bfr[half][nb], cf[k][nb], sv[half]);
        uint32_t mw[4], ml[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int j0 = (2 * kb + half) * 16 + 4 * g4;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = sv[half][r] * fac[half][r] + (diag && j0 + r == irow ? Dh : 0.f);
          mw[2 * half] = pack_bf16x2(v[0], v[1]);
          mw[2 * half + 1] = pack_bf16x2(v[2], v[3]);
          ml[2 * half] = pack_bf16x2(v[0] - bf16_lo(mw[2 * half]), v[1] - bf16_hi(mw[2 * half]));
          ml[2 * half + 1] = pack_bf16x2(v[2] - bf16_lo(mw[2 * half + 1]), v[3] - bf16_hi(mw[2 * half + 1]));
        }
        const u32x4 ah = u32x4{mw[0], mw[1], mw[2], mw[3]};
        const u32x4 al = u32x4{ml[0], ml[1], ml[2], ml[3]};
        u32x4 xf[K::TP];
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) xf[pt] = frag_k_rows_accpair(xs, K::XP, 32 * kb, pt * 16, lane);
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) acc[pt] = mfma16x16x32(xf[pt], ah, acc[pt]);
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) acc[pt] = mfma16x16x32(xf[pt], al, acc[pt]);
      };
      for (int kb = 0; kb < kbd; ++kb) key_block(kb, false);
      const uint32_t yrow = (uint32_t)(irow * ldx);
      ZPieces<K::TP> zp;
      if (GATE) load_zT<K::TP>(zp, make_rsrc(Z + (tok0 * H + h) * P, (uint32_t)(len * ldx * 2)), yrow, g4);
      // u_i now (this lane's query row): the diagonal key block uses the exact masked decay.
      const float u = fast_exp2(cs_i - mref);
#pragma unroll
      for (int pt = 0; pt < K::TP; ++pt) acc[pt] *= u;
      key_block(kbd, true);
      if constexpr (YF32)
        store_yT_f32<K::TP>(acc, make_rsrc(reinterpret_cast<float*>(Y) + (tok0 * H + h) * P, (uint32_t)(len * ldx * 4)),
                            yrow, g4);
      else
        store_yT<K::TP, GATE>(acc, make_rsrc(Y + (tok0 * H + h) * P, (uint32_t)(len * ldx * 2)), yrow, g4, zp);
    }

    if constexpr (!kPrefetchC) load_c(rec, more);

    // ---------------- state entering the next chunk of the block
    if (kInPlace && c + 1 < blk.nchunks) {  // weight X in place once every wave is done with it
      __syncthreads();
      for (int idx = tid; idx < Q * K::CBP; idx += kScanThreads) {
        const int j = idx / K::CBP, cc = idx % K::CBP;
        const float w = fast_exp2(cs_last - ckl[j]);
        u32x4 v = *reinterpret_cast<const u32x4*>(xs + j * K::XP + cc * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(bf16_lo(v[q]) * w, bf16_hi(v[q]) * w);
        *reinterpret_cast<u32x4*>(xs + j * K::XP + cc * 8) = v;
      }
      __syncthreads();
    }
    if (c + 1 < blk.nchunks && sact) {
      const float decay = fast_exp2(cs_last);
#pragma unroll
      for (int a = 0; a < K::TPW; ++a)
#pragma unroll
        for (int b = 0; b < K::TNW; ++b) hacc[a][b] *= decay;
      const int nkb = (len + 31) / 32;
      for (int kb = 0; kb < nkb; ++kb) {
        u32x4 xa[K::TPW], bb[K::TNW];
#pragma unroll
        for (int a = 0; a < K::TPW; ++a) xa[a] = frag_k_rows_accpair(xw, K::XP, 32 * kb, (p0t + a) * 16, lane);
#pragma unroll
        for (int b = 0; b < K::TNW; ++b) bb[b] = frag_k_rows_accpair(bs, K::BP, 32 * kb, (n0t + b) * 16, lane);
#pragma unroll
        for (int a = 0; a < K::TPW; ++a)
#pragma unroll
          for (int b = 0; b < K::TNW; ++b) hacc[a][b] = mfma16x16x32(xa[a], bb[b], hacc[a][b]);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 path, two heads per workgroup. When the heads of a B/C group come in
// pairs and the tiles fit, one workgroup takes two heads of the same group
// over one state block: B and C are staged once for both heads and S^T = B C^T
// is formed once, so every key block costs 8 MFMAs of S^T and 8 of (S o V) X
// per head instead of 16 per head. Per chunk the next chunk's loads are issued
// in three groups spread over the output phase. The next key block's S^T is
// issued before the current block's decay and hi/lo work, so its MFMAs run
// under that VALU work. The decay-weighted X of the state update is formed in
// registers from a per-chunk weight table instead of a second LDS copy.
// ----------------------------------------------------------------------------
namespace {

template <int P, int N>
struct PairCfg {
  static constexpr int BP = lds_pitch(N);   // B rows
  static constexpr int XP = lds_pitch(P);   // X rows of each head
  static constexpr int HP = lds_pitch(P);   // transposed state rows of each head [N][HP] (rows at perm32(n))
  static_assert(HP >= P + kHalfShift, "the half shift stays inside the row padding");
  static constexpr int TP = P / 16, TN = N / 16, NB = N / 32;
  // State tiles: whole P tiles per wave first, so that each decay-weighted X
  // fragment of the state update is formed by as few waves as possible.
  static constexpr int WP = TP < kScanWaves ? TP : kScanWaves;
  static constexpr int WN = TN < kScanWaves / WP ? TN : kScanWaves / WP;
  static constexpr int TPW = TP / WP, TNW = TN / WN;
  static constexpr int CBN = N / 8, CBP = P / 8;
  static constexpr int RB = (kPassRows * CBN + kScanThreads - 1) / kScanThreads;
  static constexpr int RX = (kPassRows * CBP + kScanThreads - 1) / kScanThreads;
};

}  // namespace

static size_t pair_lds_elems(int P, int N, int Q) {
  return (size_t)Q * lds_pitch(N) + 2 * (size_t)Q * lds_pitch(P) + 2 * (size_t)N * lds_pitch(P);
}

// LDS: the tiles above, 16 chunk records, cs, ck and the state-update weights
// of both heads ([2][Q] each) and one [2][Q] row of v_j per wave.
static size_t chunk_scan_pair_lds_bytes(int P, int N, int Q) {
  return pair_lds_elems(P, N, Q) * 2 + 16 * 16 + (size_t)(6 + 2 * kScanWaves) * Q * 4;
}

// Head pairs need an even number of heads per group; beyond P = 64 or N = 128
// the doubled state tiles no longer fit the registers of 8 waves per CU.
static constexpr bool pair_shape(int P, int N) { return P <= 64 && N <= 128; }

static bool chunk_scan_pair_fits(int P, int N, int Q, int H, int G) {
  return pair_shape(P, N) && (H / G) % 2 == 0 && Q <= 128 && chunk_scan_pair_lds_bytes(P, N, Q) <= kMaxLdsBytes;
}

template <int P, int N, int OUT>
__global__ __launch_bounds__(kScanThreads, 1) void chunk_scan_pair_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ B, const uint16_t* __restrict__ C,
    const int4* __restrict__ ctable, const int4* __restrict__ btable, const float* __restrict__ cs,
    const float* __restrict__ ck, const uint16_t* __restrict__ start, uint16_t* __restrict__ Y,
    const uint16_t* __restrict__ Z, const float* __restrict__ Dskip, int H, int G, int Q,
    int ranked) {
  constexpr bool GATE = OUT == kOutGated;  // silu(z) gate on the output
  constexpr bool YF32 = OUT == kOutF32;    // fp32 output (partials summed before one rounding)
  using K = PairCfg<P, N>;
  const int HH = H / 2;
  long m;
  int hp;
  scan_unit(btable, blockIdx.x, gridDim.x, HH, ranked, m, hp);
  const int h0 = 2 * hp;
  const BlockRec blk = load_block(btable, m);
  if (blk.nchunks <= 0) return;
  const int g = h0 / (H / G);
  const int nIt = Q / 16;

  extern __shared__ uint16_t lds[];
  uint16_t* bs = lds;                                   // [Q][BP]      B rows
  uint16_t* xs = bs + Q * K::BP;                        // [2][Q][XP]   X rows of both heads
  uint16_t* hsT = xs + 2 * Q * K::XP;                   // [2][N][HP]   entering states, transposed
  int4* recs = reinterpret_cast<int4*>(hsT + 2 * N * K::HP);  // [16] chunk records
  float* csl = reinterpret_cast<float*>(recs + 16);     // [2][Q] cumulative log2 decay cs
  float* wt = csl + 2 * Q;                              // [2][Q] exp2(cs_last - ck_j)
  float* ckl = wt + 2 * Q;                              // [2][Q] key-side exponent ck

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const long ldb = (long)G * N, ldx = (long)H * P;
  float* vt = ckl + 2 * Q + wave * 2 * Q;               // [2][Q] v_j of this wave's query tile
  // Skip weights of both heads (zero without a skip): D x_i rides on the
  // diagonal of the diagonal key block's L o S.
  const float Dh[2] = {Dskip ? Dskip[h0] : 0.f, Dskip ? Dskip[h0 + 1] : 0.f};
  // This wave's query tile: waves 0-3 (the first wave of each SIMD) take the
  // long rows of the triangle, 7 - w, and waves 4-7 the short rows w - 4, so
  // each SIMD pairs a long and a short row.
  const int it = wave < 4 ? 7 - wave : wave - 4;

  // Per-thread constant byte offsets of the staged pieces within a chunk.
  uint32_t boff[K::RB], xoff[K::RX];
  int brow[K::RB], xrow[K::RX];
#pragma unroll
  for (int u = 0; u < K::RB; ++u) {
    const int idx = tid + kScanThreads * u;
    brow[u] = idx < kPassRows * K::CBN ? idx / K::CBN : kPassRows;
    boff[u] = brow[u] < kPassRows ? (uint32_t)((brow[u] * ldb + (idx % K::CBN) * 8) * 2) : kOffNone;
  }
#pragma unroll
  for (int u = 0; u < K::RX; ++u) {
    const int idx = tid + kScanThreads * u;
    xrow[u] = idx < kPassRows * K::CBP ? idx / K::CBP : kPassRows;
    xoff[u] = xrow[u] < kPassRows ? (uint32_t)((xrow[u] * ldx + (idx % K::CBP) * 8) * 2) : kOffNone;
  }
  const uint32_t cfoff = it < nIt ? (uint32_t)(((it * 16 + l16) * ldb + 8 * g4) * 2) : kOffNone;
  const uint32_t csoff = tid < 2 * Q ? (uint32_t)(tid * 4) : kOffNone;

  // State tiles of this wave, both heads, from the state entering the block.
  const int wn = wave % K::WN, wp = wave / K::WN;
  const bool sact = wp < K::WP;
  const int p0t = wp * K::TPW, n0t = wn * K::TNW;
  f32x4 hacc[2][K::TPW][K::TNW];
#pragma unroll
  for (int hd = 0; hd < 2; ++hd) {
    const rsrc_t rs = make_rsrc(start + (m * H + h0 + hd) * (long)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
    for (int a = 0; a < K::TPW; ++a)
#pragma unroll
      for (int b = 0; b < K::TNW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hacc[hd][a][b][r] = bf16_to_f32(buf_load_u16(
              rs, sact ? (uint32_t)((((p0t + a) * 16 + 4 * g4 + r) * N + (n0t + b) * 16 + l16) * 2) : kOffNone));
  }

  // Registers holding the next chunk, filled in three groups.
  u32x4 pb[K::RB], px[2][K::RX], pcf[K::NB];
  float pcs = 0.f, pck = 0.f, plast[2] = {0.f, 0.f};
  struct Next {
    rsrc_t rb, rx0, rx1, rc, rcs, rck;
  };
  auto next_rsrc = [&](const SlotRec& r, long slot, bool valid) {
    const int len = valid ? r.len : 0;
    Next n;
    n.rb = make_rsrc(B + ((long)r.tok0 * G + g) * N, (uint32_t)(len * ldb * 2));
    n.rc = make_rsrc(C + ((long)r.tok0 * G + g) * N, (uint32_t)(len * ldb * 2));
    n.rx0 = make_rsrc(X + ((long)r.tok0 * H + h0) * P, (uint32_t)(len * ldx * 2));
    n.rx1 = make_rsrc(X + ((long)r.tok0 * H + h0 + 1) * P, (uint32_t)(len * ldx * 2));
    n.rcs = make_rsrc(cs + (slot * H + h0) * (long)Q, valid ? (uint32_t)(2 * Q * 4) : 0u);
    n.rck = make_rsrc(ck + (slot * H + h0) * (long)Q, valid ? (uint32_t)(2 * Q * 4) : 0u);
    return n;
  };
  auto load_b = [&](const Next& n) {
#pragma unroll
    for (int u = 0; u < K::RB; ++u) pb[u] = buf_load16(n.rb, boff[u]);
  };
  auto load_x = [&](const Next& n) {
#pragma unroll
    for (int u = 0; u < K::RX; ++u) {
      px[0][u] = buf_load16(n.rx0, xoff[u]);
      px[1][u] = buf_load16(n.rx1, xoff[u]);
    }
    pcs = buf_load_f32(n.rcs, csoff);
    pck = buf_load_f32(n.rck, csoff);
    plast[0] = buf_load_f32(n.rcs, (uint32_t)((Q - 1) * 4));
    plast[1] = buf_load_f32(n.rcs, (uint32_t)((2 * Q - 1) * 4));
  };
  auto load_c = [&](const Next& n) {
#pragma unroll
    for (int nb = 0; nb < K::NB; ++nb) pcf[nb] = buf_load16(n.rc, cfoff + nb * 64);
  };

  if (tid < blk.nchunks) recs[tid] = ctable[blk.slot0 + tid];
  __syncthreads();
  auto rec_of = [&](int c) {
    const int4 v = recs[c];
    return SlotRec{uniform(v.x), uniform(v.y), uniform(v.z), uniform(v.w)};
  };
  SlotRec rec = rec_of(0);
  {
    const Next n0 = next_rsrc(rec, blk.slot0, true);
    load_b(n0);
    load_x(n0);
    load_c(n0);
  }

  for (int c = 0; c < blk.nchunks; ++c) {
    const int len = rec.len;
    const long tok0 = rec.tok0;
    const float cs_last0 = plast[0], cs_last1 = plast[1];

    __syncthreads();  // every wave is done with the previous chunk's tiles
#pragma unroll
    for (int u = 0; u < K::RB; ++u)
      if (brow[u] < Q)
        *reinterpret_cast<u32x4*>(bs + brow[u] * K::BP + ((tid + kScanThreads * u) % K::CBN) * 8) = pb[u];
#pragma unroll
    for (int u = 0; u < K::RX; ++u)
      if (xrow[u] < Q) {
        const int o = xrow[u] * K::XP + ((tid + kScanThreads * u) % K::CBP) * 8;
        *reinterpret_cast<u32x4*>(xs + o) = px[0][u];
        *reinterpret_cast<u32x4*>(xs + Q * K::XP + o) = px[1][u];
      }
    if (tid < 2 * Q) {
      csl[tid] = pcs;
      ckl[tid] = pck;
      wt[tid] = fast_exp2((tid < Q ? cs_last0 : cs_last1) - pck);
    }
    if (sact) {
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
#pragma unroll
        for (int a = 0; a < K::TPW; ++a)
#pragma unroll
          for (int b = 0; b < K::TNW; ++b) {
            const u32x2 v = {pack_bf16x2(hacc[hd][a][b][0], hacc[hd][a][b][1]),
                             pack_bf16x2(hacc[hd][a][b][2], hacc[hd][a][b][3])};
            *reinterpret_cast<u32x2*>(hsT + hd * N * K::HP + hs_row(perm32((n0t + b) * 16 + l16), K::HP) + (p0t + a) * 16 +
                                      4 * g4) = v;
          }
    }
    u32x4 cf[K::NB];
#pragma unroll
    for (int nb = 0; nb < K::NB; ++nb) cf[nb] = pcf[nb];
    const bool more = c + 1 < blk.nchunks;
    const SlotRec nrec = rec_of(more ? c + 1 : c);
    const Next nx = next_rsrc(nrec, blk.slot0 + c + (more ? 1 : 0), more);
    __syncthreads();

    // ---------------- outputs: Y_i = u_i (sum_j (S o V)_ij X_j + exp2(m) (C h^T)_i) per head
    load_b(nx);
    if (it < nIt && it * 16 < len) {
      f32x4 acc[2][K::TP];
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) {
          acc[hd][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int nb = 0; nb < K::NB; ++nb)
            acc[hd][pt] = mfma16x16x32(frag_k_rows_accpair_hs(hsT + hd * N * K::HP, K::HP, nb * 32, pt * 16, lane), cf[nb],
                                       acc[hd][pt]);
        }
      const float mref[2] = {csl[16 * it], csl[Q + 16 * it]};
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        const float em = fast_exp2(mref[hd]);
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) acc[hd][pt] *= em;
      }
      load_x(nx);
      const int irow = it * 16 + l16;
      const float csi[2] = {csl[irow], csl[Q + irow]};
      const int kbd = it >> 1;  // key block holding the diagonal tile
      // v_j = exp2(m - ck_j) of both heads for the keys before this tile
      // (private to the wave: written and read by the same wave, in order).
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
#pragma unroll
        for (int q = 0; q < kPassRows / 64; ++q) {
          const int j = lane + 64 * q;
          if (j < 16 * it) vt[hd * Q + j] = fast_exp2(mref[hd] - ckl[hd * Q + j]);
        }

      // S^T of one key block of 32 tokens (both 16-key halves).
      auto s_block = [&](int kb, f32x4 sv[2]) {
        u32x4 bfr[2][K::NB];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int nb = 0; nb < K::NB; ++nb) bfr[half][nb] = frag_k_cols(bs, K::BP, (2 * kb + half) * 16, nb * 32, lane);
        sv[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sv[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < K::NB; ++nb)
#pragma unroll
          for (int half = 0; half < 2; ++half) sv[half] = mfma16x16x32(bfr[half][nb], cf[nb], sv[half]);
      };
      // Decay, hi/lo split and Y += M X of one key block for both heads.
      auto y_block = [&](int kb, const f32x4 sv[2], bool diag) {
#pragma unroll
        for (int hd = 0; hd < 2; ++hd) {
          const float* kl = ckl + hd * Q;
          uint32_t mw[4], ml[4];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int j0 = (2 * kb + half) * 16 + 4 * g4;
            float v[4];
            if (diag) {
              const f32x4 cj = *reinterpret_cast<const f32x4*>(kl + j0);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                v[r] = (j0 + r <= irow ? sv[half][r] * fast_exp2(csi[hd] - cj[r]) : 0.f) + (j0 + r == irow ? Dh[hd] : 0.f);
            } else {
              const f32x4 fj = *reinterpret_cast<const f32x4*>(vt + hd * Q + j0);
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] = sv[half][r] * fj[r];
            }
            mw[2 * half] = pack_bf16x2(v[0], v[1]);
            mw[2 * half + 1] = pack_bf16x2(v[2], v[3]);
            ml[2 * half] = pack_bf16x2(v[0] - bf16_lo(mw[2 * half]), v[1] - bf16_hi(mw[2 * half]));
            ml[2 * half + 1] = pack_bf16x2(v[2] - bf16_lo(mw[2 * half + 1]), v[3] - bf16_hi(mw[2 * half + 1]));
          }
          const u32x4 ah = u32x4{mw[0], mw[1], mw[2], mw[3]};
          const u32x4 al = u32x4{ml[0], ml[1], ml[2], ml[3]};
          u32x4 xf[K::TP];
#pragma unroll
          for (int pt = 0; pt < K::TP; ++pt)
            xf[pt] = frag_k_rows_accpair(xs + hd * Q * K::XP, K::XP, 32 * kb, pt * 16, lane);
#pragma unroll
          for (int pt = 0; pt < K::TP; ++pt) acc[hd][pt] = mfma16x16x32(xf[pt], ah, acc[hd][pt]);
#pragma unroll
          for (int pt = 0; pt < K::TP; ++pt) acc[hd][pt] = mfma16x16x32(xf[pt], al, acc[hd][pt]);
        }
      };

      // Key blocks before the diagonal (at most three for chunks of up to
      // 128 tokens), unrolled with two S^T register sets: the next block's
      // S^T is issued before this block's decay and hi/lo work.
      f32x4 sa[2], sb[2];
      s_block(0, sa);
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) {
        if (kb < kbd) {
          s_block(kb + 1, (kb & 1) ? sa : sb);
          y_block(kb, (kb & 1) ? sb : sa, false);
        }
      }
      load_c(nx);
      const uint32_t yrow = (uint32_t)((it * 16 + l16) * ldx);
      ZPieces<K::TP> zp[2];
      if (GATE) {
#pragma unroll
        for (int hd = 0; hd < 2; ++hd)
          load_zT<K::TP>(zp[hd], make_rsrc(Z + (tok0 * H + h0 + hd) * P, (uint32_t)(len * ldx * 2)), yrow, g4);
      }
      // u_i now: the diagonal key block uses the exact masked decay.
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        const float u = fast_exp2(csi[hd] - mref[hd]);   // this lane's query row
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) acc[hd][pt] *= u;
      }
      const f32x4 sd[2] = {(kbd & 1) ? sb[0] : sa[0], (kbd & 1) ? sb[1] : sa[1]};
      y_block(kbd, sd, true);

      // Out: the accumulators hold Y^T tiles (lane: query row l16, 4
      // consecutive p of P tile pt in lane group g4).
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
        if constexpr (YF32)
          store_yT_f32<K::TP>(acc[hd],
                              make_rsrc(reinterpret_cast<float*>(Y) + (tok0 * H + h0 + hd) * P, (uint32_t)(len * ldx * 4)),
                              yrow, g4);
        else
          store_yT<K::TP, GATE>(acc[hd], make_rsrc(Y + (tok0 * H + h0 + hd) * P, (uint32_t)(len * ldx * 2)), yrow,
                                g4, zp[hd]);
    } else {
      load_x(nx);
      load_c(nx);
    }

    // ---------------- state entering the next chunk of the block
    if (more && sact) {
      const float d0 = fast_exp2(cs_last0), d1 = fast_exp2(cs_last1);
#pragma unroll
      for (int a = 0; a < K::TPW; ++a)
#pragma unroll
        for (int b = 0; b < K::TNW; ++b) {
          hacc[0][a][b] *= d0;
          hacc[1][a][b] *= d1;
        }
      const int nkb = (len + 31) / 32;
#pragma unroll
      for (int kb = 0; kb < kPassRows / 32; ++kb) {
        if (kb >= nkb) break;
        u32x4 bb[K::TNW];
#pragma unroll
        for (int b = 0; b < K::TNW; ++b) bb[b] = frag_k_rows_accpair(bs, K::BP, 32 * kb, (n0t + b) * 16, lane);
#pragma unroll
        for (int hd = 0; hd < 2; ++hd) {
          const f32x4 wlo = *reinterpret_cast<const f32x4*>(wt + hd * Q + 32 * kb + 4 * g4);
          const f32x4 whi = *reinterpret_cast<const f32x4*>(wt + hd * Q + 32 * kb + 16 + 4 * g4);
          const float w8[8] = {wlo[0], wlo[1], wlo[2], wlo[3], whi[0], whi[1], whi[2], whi[3]};
#pragma unroll
          for (int a = 0; a < K::TPW; ++a) {
            const u32x4 xa =
                scale_frag(frag_k_rows_accpair(xs + hd * Q * K::XP, K::XP, 32 * kb, (p0t + a) * 16, lane), w8);
#pragma unroll
            for (int b = 0; b < K::TNW; ++b) hacc[hd][a][b] = mfma16x16x32(xa, bb[b], hacc[hd][a][b]);
          }
        }
      }
    }
    rec = nrec;
  }
}

// ----------------------------------------------------------------------------
// Two heads per workgroup, chunks walked in halves of 64 tokens. The second
// half of a 128-token chunk sees the first half through the carried state:
// with cs rebased to the half's start (cs' = cs - cs_63), rows i >= 64 take
// exp2(cs'_i) C_i h_mid with h_mid = exp2(cs_63) h + sum_{j < 64}
// exp2(cs_63 - ck_j) X_j B_j^T, the same decomposition one level down (paper
// section 6: the off-diagonal blocks of a chunk factor through the state).
// Up to N = 128 the tiles of one half fill 80 KB of LDS and four waves carry
// them, so two workgroups share a CU and their chains of halves overlap, where
// the eight-wave whole-chunk kernel runs one chain per CU. At N = 256 (139 KB,
// one workgroup per CU) eight waves each take one (query tile, head): each
// half's B rows are staged once for both heads, where the single-head kernel
// stages them per head.
// ----------------------------------------------------------------------------
constexpr int kHalfRows = 64;

// NW waves: 4 (each wave one query tile of the half for both heads) or 8 (each
// wave one query tile for one head; the wider states, N = 256).
template <int P, int N, int NW>
struct HalfCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BP = lds_pitch(N);
  static constexpr int XP = lds_pitch(P);
  static constexpr int HP = lds_pitch(P);
  static_assert(HP >= P + kHalfShift, "the half shift stays inside the row padding");
  static constexpr int TP = P / 16, TN = N / 16, NB = N / 32;
  static constexpr int WP = TP < NW ? TP : NW;
  static constexpr int WN = TN < NW / WP ? TN : NW / WP;
  static constexpr int TPW = TP / WP, TNW = TN / WN;
  static constexpr int CBN = N / 8, CBP = P / 8;
  static constexpr int RB = (kHalfRows * CBN + NT - 1) / NT;
  static constexpr int RX = (kHalfRows * CBP + NT - 1) / NT;
};

// LDS: B rows of a half, X rows of both heads, both entering states, 16 chunk
// records and cs, ck and the state-update weights of both heads ([2][64]).
static size_t chunk_scan_half_lds_bytes(int P, int N) {
  const size_t el = (size_t)kHalfRows * lds_pitch(N) + 2 * (size_t)kHalfRows * lds_pitch(P) +
                    2 * (size_t)N * lds_pitch(P);
  return el * 2 + 16 * 16 + (size_t)3 * 2 * kHalfRows * 4;
}

// Four-wave form: two such workgroups must fit one CU's LDS.
static bool chunk_scan_half_fits(int P, int N, int Q, int H, int G) {
  return pair_shape(P, N) && (H / G) % 2 == 0 && (Q == 64 || Q == 128) &&
         2 * chunk_scan_half_lds_bytes(P, N) <= kMaxLdsBytes;
}

// Eight-wave form for N = 256 (P <= 64): one workgroup per CU.
static constexpr bool half_wide_shape(int P, int N) { return P <= 64 && N == 256; }
static bool chunk_scan_half_wide_fits(int P, int N, int Q, int H, int G) {
  return half_wide_shape(P, N) && (H / G) % 2 == 0 && (Q == 64 || Q == 128) &&
         chunk_scan_half_lds_bytes(P, N) <= kMaxLdsBytes;
}

// The four-wave half-chunk kernel needs two units per CU to fill the chip
// (256 CUs); with fewer, the eight-wave whole-chunk kernel, one per CU, is
// faster (T = 16384, H = 32, N = 128: 56 against 48 us for 256 units). At
// N = 256 the eight-wave half-chunk form replaces the single-head kernel
// (b 8, T 4096, H 32: 173 against 194 us at state blocks of 16 chunks): it
// stages each half's B rows once for both heads.
constexpr long kHalfMinUnits = 2 * 256;

int chunk_scan_kind(const FwdDims& d) {
  if (!d.bf16) return kScanF32;
  const long units = d.nblocks * (d.H / 2);
  if (chunk_scan_half_fits(d.P, d.N, d.Q, d.H, d.G) && units >= kHalfMinUnits) return kScanHalfPair;
  if (chunk_scan_half_wide_fits(d.P, d.N, d.Q, d.H, d.G)) return kScanHalfPairWide;
  if (chunk_scan_pair_fits(d.P, d.N, d.Q, d.H, d.G)) return kScanPair;
  return kScanSingle;
}

// HW: heads per wave in the output phase (2: four waves; 1: eight waves, each
// (query tile, head) on its own wave, S^T formed by both waves of a tile).
template <int P, int N, int OUT, int HW>
__global__ __launch_bounds__((HW == 2 ? 4 : 8) * 64, 2) void chunk_scan_half_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ B, const uint16_t* __restrict__ C,
    const int4* __restrict__ ctable, const int4* __restrict__ btable, const float* __restrict__ cs,
    const float* __restrict__ ck, const uint16_t* __restrict__ start, uint16_t* __restrict__ Y,
    const uint16_t* __restrict__ Z, const float* __restrict__ Dskip, int H, int G, int Q,
    int ranked) {
  constexpr bool GATE = OUT == kOutGated;
  constexpr bool YF32 = OUT == kOutF32;
  constexpr int R = kHalfRows;
  constexpr int NW = HW == 2 ? 4 : 8;
  using K = HalfCfg<P, N, NW>;
  const int HH = H / 2;
  long m;
  int hp;
  scan_unit(btable, blockIdx.x, gridDim.x, HH, ranked, m, hp);
  const int h0 = 2 * hp;
  const BlockRec blk = load_block(btable, m);
  if (blk.nchunks <= 0) return;
  const int g = h0 / (H / G);

  extern __shared__ uint16_t lds[];
  uint16_t* bs = lds;                                   // [R][BP]      B rows of the half
  uint16_t* xs = bs + R * K::BP;                        // [2][R][XP]   X rows of both heads
  uint16_t* hsT = xs + 2 * R * K::XP;                   // [2][N][HP]   entering states, transposed
  int4* recs = reinterpret_cast<int4*>(hsT + 2 * N * K::HP);  // [16] chunk records
  float* csl = reinterpret_cast<float*>(recs + 16);     // [2][R] cs rebased to the half's start
  float* wt = csl + 2 * R;                              // [2][R] exp2(cs_end - ck_j)
  float* ckl = wt + 2 * R;                              // [2][R] ck rebased to the half's start

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const long ldb = (long)G * N, ldx = (long)H * P;
  const float Dh[2] = {Dskip ? Dskip[h0] : 0.f, Dskip ? Dskip[h0 + 1] : 0.f};
  const int it = wave & 3;                  // query tile of the half
  const int h1 = HW == 2 ? 0 : wave >> 2;   // first head of this wave's outputs

  uint32_t boff[K::RB], xoff[K::RX];
  int brow[K::RB], xrow[K::RX];
#pragma unroll
  for (int u = 0; u < K::RB; ++u) {
    const int idx = tid + K::NT * u;
    brow[u] = idx < R * K::CBN ? idx / K::CBN : R;
    boff[u] = brow[u] < R ? (uint32_t)((brow[u] * ldb + (idx % K::CBN) * 8) * 2) : kOffNone;
  }
#pragma unroll
  for (int u = 0; u < K::RX; ++u) {
    const int idx = tid + K::NT * u;
    xrow[u] = idx < R * K::CBP ? idx / K::CBP : R;
    xoff[u] = xrow[u] < R ? (uint32_t)((xrow[u] * ldx + (idx % K::CBP) * 8) * 2) : kOffNone;
  }
  const uint32_t cfoff = (uint32_t)(((it * 16 + l16) * ldb + 8 * g4) * 2);
  // This thread's entry of the chunk's cs / ck tables of both heads ([2][Q]).
  const int th = tid / Q, trow = tid % Q;
  const uint32_t csoff = tid < 2 * Q ? (uint32_t)(tid * 4) : kOffNone;

  const int wn = wave % K::WN, wp = wave / K::WN;
  const bool sact = wp < K::WP;
  const int p0t = wp * K::TPW, n0t = wn * K::TNW;
  f32x4 hacc[2][K::TPW][K::TNW];
#pragma unroll
  for (int hd = 0; hd < 2; ++hd) {
    const rsrc_t rs = make_rsrc(start + (m * H + h0 + hd) * (long)(P * N), (uint32_t)(P * N * 2));
#pragma unroll
    for (int a = 0; a < K::TPW; ++a)
#pragma unroll
      for (int b = 0; b < K::TNW; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hacc[hd][a][b][r] = bf16_to_f32(buf_load_u16(
              rs, sact ? (uint32_t)((((p0t + a) * 16 + 4 * g4 + r) * N + (n0t + b) * 16 + l16) * 2) : kOffNone));
  }

  // The next half's rows and C fragments in flight; its chunk's cs / ck entry
  // and the chunk's cs at the half's base and end rows of both heads.
  u32x4 pb[K::RB], px[2][K::RX], pcf[K::NB];
  float pcs = 0.f, pck = 0.f, pbase[2] = {0.f, 0.f}, pend[2] = {0.f, 0.f};
  struct Next {
    rsrc_t rb, rx0, rx1, rc, rcs, rck;
    uint32_t obase, oend;
  };
  // Half `sh` of chunk record r in slot `slot` (valid = false: nothing left).
  auto next_rsrc = [&](const SlotRec& r, long slot, int sh, bool valid) {
    const int len = valid ? min(R, r.len - R * sh) : 0;
    const long t0 = (long)r.tok0 + R * sh;
    Next n;
    n.rb = make_rsrc(B + (t0 * G + g) * N, (uint32_t)(len * ldb * 2));
    n.rc = make_rsrc(C + (t0 * G + g) * N, (uint32_t)(len * ldb * 2));
    n.rx0 = make_rsrc(X + (t0 * H + h0) * P, (uint32_t)(len * ldx * 2));
    n.rx1 = make_rsrc(X + (t0 * H + h0 + 1) * P, (uint32_t)(len * ldx * 2));
    n.rcs = make_rsrc(cs + (slot * H + h0) * (long)Q, valid ? (uint32_t)(2 * Q * 4) : 0u);
    n.rck = make_rsrc(ck + (slot * H + h0) * (long)Q, valid ? (uint32_t)(2 * Q * 4) : 0u);
    n.obase = sh ? (uint32_t)((R - 1) * 4) : kOffNone;     // cs_63 for the second half, else 0
    n.oend = (uint32_t)((min(R * sh + R, Q) - 1) * 4);     // cs at the half's last row
    return n;
  };
  auto load_b = [&](const Next& n) {
#pragma unroll
    for (int u = 0; u < K::RB; ++u) pb[u] = buf_load16(n.rb, boff[u]);
  };
  auto load_x = [&](const Next& n) {
#pragma unroll
    for (int u = 0; u < K::RX; ++u) {
      px[0][u] = buf_load16(n.rx0, xoff[u]);
      px[1][u] = buf_load16(n.rx1, xoff[u]);
    }
    pcs = buf_load_f32(n.rcs, csoff);
    pck = buf_load_f32(n.rck, csoff);
    pbase[0] = buf_load_f32(n.rcs, n.obase);
    pbase[1] = buf_load_f32(n.rcs, n.obase == kOffNone ? kOffNone : n.obase + (uint32_t)(Q * 4));
    pend[0] = buf_load_f32(n.rcs, n.oend);
    pend[1] = buf_load_f32(n.rcs, n.oend + (uint32_t)(Q * 4));
  };
  auto load_c = [&](const Next& n) {
#pragma unroll
    for (int nb = 0; nb < K::NB; ++nb) pcf[nb] = buf_load16(n.rc, cfoff + nb * 64);
  };

  if (tid < blk.nchunks) recs[tid] = ctable[blk.slot0 + tid];
  __syncthreads();
  auto rec_of = [&](int c) {
    const int4 v = recs[c];
    return SlotRec{uniform(v.x), uniform(v.y), uniform(v.z), uniform(v.w)};
  };
  SlotRec rec = rec_of(0);
  {
    const Next n0 = next_rsrc(rec, blk.slot0, 0, true);
    load_b(n0);
    load_x(n0);
    load_c(n0);
  }

  int c = 0, sh = 0;
  for (;;) {
    const int len = min(R, rec.len - R * sh);
    const long tok0 = (long)rec.tok0 + R * sh;
    const float base0 = pbase[0], base1 = pbase[1], end0 = pend[0], end1 = pend[1];
    // The half after this one: the chunk's second half, or the next chunk.
    const bool second = sh == 0 && rec.len > R;
    const bool more = second || c + 1 < blk.nchunks;
    const int nc = second ? c : c + 1;
    const SlotRec nrec = second ? rec : rec_of(more ? nc : c);
    const Next nx = next_rsrc(nrec, blk.slot0 + (more ? nc : c), second ? 1 : 0, more);

    __syncthreads();  // every wave is done with the previous half's tiles
#pragma unroll
    for (int u = 0; u < K::RB; ++u)
      if (brow[u] < R)
        *reinterpret_cast<u32x4*>(bs + brow[u] * K::BP + ((tid + K::NT * u) % K::CBN) * 8) = pb[u];
#pragma unroll
    for (int u = 0; u < K::RX; ++u)
      if (xrow[u] < R) {
        const int o = xrow[u] * K::XP + ((tid + K::NT * u) % K::CBP) * 8;
        *reinterpret_cast<u32x4*>(xs + o) = px[0][u];
        *reinterpret_cast<u32x4*>(xs + R * K::XP + o) = px[1][u];
      }
    if (tid < 2 * Q && (trow / R) == sh) {
      const int e = th * R + (trow % R);
      const float bse = th ? base1 : base0;
      csl[e] = pcs - bse;
      ckl[e] = pck - bse;
      wt[e] = fast_exp2((th ? end1 : end0) - pck);
    }
    if (sact) {
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
#pragma unroll
        for (int a = 0; a < K::TPW; ++a)
#pragma unroll
          for (int b = 0; b < K::TNW; ++b) {
            const u32x2 v = {pack_bf16x2(hacc[hd][a][b][0], hacc[hd][a][b][1]),
                             pack_bf16x2(hacc[hd][a][b][2], hacc[hd][a][b][3])};
            *reinterpret_cast<u32x2*>(hsT + hd * N * K::HP + hs_row(perm32((n0t + b) * 16 + l16), K::HP) + (p0t + a) * 16 +
                                      4 * g4) = v;
          }
    }
    __syncthreads();
    const u32x4* cf = pcf;  // this half's C fragments, until the outputs are stored

    // ---------------- outputs of this wave's query tile (both heads, or head h1)
    load_b(nx);
    if (it * 16 < len) {
      f32x4 acc[HW][K::TP];
#pragma unroll
      for (int q = 0; q < HW; ++q)
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) {
          acc[q][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int nb = 0; nb < K::NB; ++nb)
            acc[q][pt] = mfma16x16x32(frag_k_rows_accpair_hs(hsT + (h1 + q) * N * K::HP, K::HP, nb * 32, pt * 16, lane),
                                      cf[nb], acc[q][pt]);
        }
      float mref[HW], csi[HW];
      const int irow = it * 16 + l16;
#pragma unroll
      for (int q = 0; q < HW; ++q) {
        mref[q] = csl[(h1 + q) * R + 16 * it];
        csi[q] = csl[(h1 + q) * R + irow];
        const float em = fast_exp2(mref[q]);
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) acc[q][pt] *= em;
      }
      const int kbd = it >> 1;  // key block holding the diagonal tile

      auto s_block = [&](int kb, f32x4 sv[2]) {
        sv[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sv[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        constexpr int NG = K::NB > 4 ? 2 : 1;  // groups of B fragments in registers at once
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
          u32x4 bfr[2][K::NB / NG];
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int nb = 0; nb < K::NB / NG; ++nb)
              bfr[half][nb] = frag_k_cols(bs, K::BP, (2 * kb + half) * 16, (ng * (K::NB / NG) + nb) * 32, lane);
#pragma unroll
          for (int nb = 0; nb < K::NB / NG; ++nb)
#pragma unroll
            for (int half = 0; half < 2; ++half)
              sv[half] = mfma16x16x32(bfr[half][nb], cf[ng * (K::NB / NG) + nb], sv[half]);
        }
      };
      // Decay (v_j = exp2(m - ck_j) before the diagonal block, the exact
      // masked exp2(cs_i - ck_j) on it), hi/lo split and Y += M X.
      auto y_block = [&](int kb, const f32x4 sv[2], bool diag) {
#pragma unroll
        for (int q = 0; q < HW; ++q) {
          const int hd = h1 + q;
          const float* kl = ckl + hd * R;
          uint32_t mw[4], ml[4];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int j0 = (2 * kb + half) * 16 + 4 * g4;
            const f32x4 cj = *reinterpret_cast<const f32x4*>(kl + j0);
            float v[4];
            if (diag) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                v[r] = (j0 + r <= irow ? sv[half][r] * fast_exp2(csi[q] - cj[r]) : 0.f) + (j0 + r == irow ? Dh[hd] : 0.f);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] = sv[half][r] * fast_exp2(mref[q] - cj[r]);
            }
            mw[2 * half] = pack_bf16x2(v[0], v[1]);
            mw[2 * half + 1] = pack_bf16x2(v[2], v[3]);
            ml[2 * half] = pack_bf16x2(v[0] - bf16_lo(mw[2 * half]), v[1] - bf16_hi(mw[2 * half]));
            ml[2 * half + 1] = pack_bf16x2(v[2] - bf16_lo(mw[2 * half + 1]), v[3] - bf16_hi(mw[2 * half + 1]));
          }
          const u32x4 ah = u32x4{mw[0], mw[1], mw[2], mw[3]};
          const u32x4 al = u32x4{ml[0], ml[1], ml[2], ml[3]};
          u32x4 xf[K::TP];
#pragma unroll
          for (int pt = 0; pt < K::TP; ++pt)
            xf[pt] = frag_k_rows_accpair(xs + hd * R * K::XP, K::XP, 32 * kb, pt * 16, lane);
#pragma unroll
          for (int pt = 0; pt < K::TP; ++pt) acc[q][pt] = mfma16x16x32(xf[pt], ah, acc[q][pt]);
#pragma unroll
          for (int pt = 0; pt < K::TP; ++pt) acc[q][pt] = mfma16x16x32(xf[pt], al, acc[q][pt]);
        }
      };

      f32x4 sa[2], sb[2];
      s_block(0, sa);
      if (kbd > 0) {
        s_block(1, sb);
        y_block(0, sa, false);
      }
      const uint32_t yrow = (uint32_t)((it * 16 + l16) * ldx);
      ZPieces<K::TP> zp[HW];
      if (GATE) {
#pragma unroll
        for (int q = 0; q < HW; ++q)
          load_zT<K::TP>(zp[q], make_rsrc(Z + (tok0 * H + h0 + h1 + q) * P, (uint32_t)(len * ldx * 2)), yrow, g4);
      }
#pragma unroll
      for (int q = 0; q < HW; ++q) {
        const float u = fast_exp2(csi[q] - mref[q]);
#pragma unroll
        for (int pt = 0; pt < K::TP; ++pt) acc[q][pt] *= u;
      }
      const f32x4 sd[2] = {kbd ? sb[0] : sa[0], kbd ? sb[1] : sa[1]};
      y_block(kbd, sd, true);

#pragma unroll
      for (int q = 0; q < HW; ++q)
        if constexpr (YF32)
          store_yT_f32<K::TP>(acc[q],
                              make_rsrc(reinterpret_cast<float*>(Y) + (tok0 * H + h0 + h1 + q) * P,
                                        (uint32_t)(len * ldx * 4)),
                              yrow, g4);
        else
          store_yT<K::TP, GATE>(acc[q], make_rsrc(Y + (tok0 * H + h0 + h1 + q) * P, (uint32_t)(len * ldx * 2)),
                                yrow, g4, zp[q]);
      // The next half's X rows and C fragments, issued once this half's
      // outputs are out (one register set of C fragments; the loads' latency
      // runs under the state update and the staging).
      load_x(nx);
      load_c(nx);
    } else {
      load_x(nx);
      load_c(nx);
    }

    // ---------------- state entering the next half
    if (more && sact) {
      const float d0 = fast_exp2(end0 - base0), d1 = fast_exp2(end1 - base1);
#pragma unroll
      for (int a = 0; a < K::TPW; ++a)
#pragma unroll
        for (int b = 0; b < K::TNW; ++b) {
          hacc[0][a][b] *= d0;
          hacc[1][a][b] *= d1;
        }
      const int nkb = (len + 31) / 32;
#pragma unroll
      for (int kb = 0; kb < R / 32; ++kb) {
        if (kb >= nkb) break;
        u32x4 bb[K::TNW];
#pragma unroll
        for (int b = 0; b < K::TNW; ++b) bb[b] = frag_k_rows_accpair(bs, K::BP, 32 * kb, (n0t + b) * 16, lane);
#pragma unroll
        for (int hd = 0; hd < 2; ++hd) {
          const f32x4 wlo = *reinterpret_cast<const f32x4*>(wt + hd * R + 32 * kb + 4 * g4);
          const f32x4 whi = *reinterpret_cast<const f32x4*>(wt + hd * R + 32 * kb + 16 + 4 * g4);
          const float w8[8] = {wlo[0], wlo[1], wlo[2], wlo[3], whi[0], whi[1], whi[2], whi[3]};
#pragma unroll
          for (int a = 0; a < K::TPW; ++a) {
            const u32x4 xa =
                scale_frag(frag_k_rows_accpair(xs + hd * R * K::XP, K::XP, 32 * kb, (p0t + a) * 16, lane), w8);
#pragma unroll
            for (int b = 0; b < K::TNW; ++b) hacc[hd][a][b] = mfma16x16x32(xa, bb[b], hacc[hd][a][b]);
          }
        }
      }
    }
    if (!more) break;
    if (!second) ++c;
    sh = second ? 1 : 0;
    rec = nrec;
  }
}

// ----------------------------------------------------------------------------
// fp32 path (plain FMA, fp32 accumulation; one chunk per state block). Query
// rows in blocks of 32; for
// each key block j0 <= i0 the masked, decayed block of C B^T is formed in LDS
// and multiplied into X.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_scan_f32_kernel(const float* __restrict__ X,
                                                             const float* __restrict__ B,
                                                             const float* __restrict__ C,
                                                             const int4* __restrict__ table,
                                                             const float* __restrict__ cs,
                                                             const float* __restrict__ ck,
                                                             const float* __restrict__ start,
                                                             float* __restrict__ Y,
                                                             const float* __restrict__ Z,
                                                             const float* __restrict__ Dskip, int H, int G,
                                                             int P, int N, int Q) {
  const long unit = xcd_unit(blockIdx.x, gridDim.x);
  const int h = (int)(unit % H);
  const long slot = unit / H;
  const SlotRec rec = load_slot(table, slot);
  const int len = rec.len;
  if (len <= 0) return;
  const int g = h / (H / G);
  constexpr int IB = 32;
  extern __shared__ float sm[];
  float* ci = sm;                  // [IB][N]
  float* bj = ci + IB * N;         // [IB][N]
  float* xj = bj + IB * N;         // [IB][P]
  float* m = xj + IB * P;          // [IB][IB]
  float* csl = m + IB * IB;        // [Q] cs
  float* ckl = csl + Q;            // [Q] key-side exponent ck
  const float* csr = cs + (slot * H + h) * (long)Q;
  const float* ckr = ck + (slot * H + h) * (long)Q;
  for (int i = threadIdx.x; i < Q; i += 256) {
    csl[i] = csr[i];
    ckl[i] = ckr[i];
  }
  const float Dh = Dskip ? Dskip[h] : 0.f;
  const long tok0 = rec.tok0;
  const float* sth = start + (slot * H + h) * (long)(P * N);
  constexpr int kMaxPer = IB * 128 / 256;  // IB*P <= 4096 outputs per block
  const int per = (IB * P + 255) / 256;

  for (int i0 = 0; i0 < len; i0 += IB) {
    const int ni = min(IB, len - i0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < IB * N; idx += 256) {
      const int i = idx / N, n = idx % N;
      ci[idx] = i < ni ? C[((tok0 + i0 + i) * G + g) * N + n] : 0.f;
    }
    __syncthreads();
    float acc[kMaxPer];
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      acc[k] = 0.f;
      const int e = threadIdx.x + 256 * k;
      if (k < per && e < IB * P) {
        const int i = e / P, p = e % P;
        float s = 0.f;
        for (int n = 0; n < N; ++n) s = fmaf(ci[i * N + n], sth[p * N + n], s);
        acc[k] = s * fast_exp2(csl[min(i0 + i, Q - 1)]);
      }
    }
    for (int j0 = 0; j0 <= i0; j0 += IB) {
      const int nj = min(IB, len - j0);
      __syncthreads();
      for (int idx = threadIdx.x; idx < IB * N; idx += 256) {
        const int j = idx / N, n = idx % N;
        bj[idx] = j < nj ? B[((tok0 + j0 + j) * G + g) * N + n] : 0.f;
      }
      for (int idx = threadIdx.x; idx < IB * P; idx += 256) {
        const int j = idx / P, p = idx % P;
        xj[idx] = j < nj ? X[((tok0 + j0 + j) * H + h) * P + p] : 0.f;
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < IB * IB; idx += 256) {
        const int i = idx / IB, j = idx % IB;
        float v = 0.f;
        if (j0 + j <= i0 + i && i < ni && j < nj) {
          float s = 0.f;
          for (int n = 0; n < N; ++n) s = fmaf(ci[i * N + n], bj[j * N + n], s);
          v = s * fast_exp2(csl[i0 + i] - ckl[j0 + j]) + (j0 + j == i0 + i ? Dh : 0.f);
        }
        m[idx] = v;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kMaxPer; ++k) {
        const int e = threadIdx.x + 256 * k;
        if (k < per && e < IB * P) {
          const int i = e / P, p = e % P;
          float s = acc[k];
          for (int j = 0; j < IB; ++j) s = fmaf(m[i * IB + j], xj[j * P + p], s);
          acc[k] = s;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      const int e = threadIdx.x + 256 * k;
      if (k < per && e < IB * P) {
        const int i = e / P, p = e % P;
        const long o = ((tok0 + i0 + i) * H + h) * P + p;
        if (i < ni) Y[o] = Z ? acc[k] * silu_f32(Z[o]) : acc[k];
      }
    }
  }
}

// ----------------------------------------------------------------------------

template <int P, int N, int OUT>
static hipError_t launch_scan_bf16(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                                   const Workspace& ws, hipStream_t stream, const Mamba2Args& m2) {
  if constexpr (pair_shape(P, N)) {
    if (chunk_scan_kind(d) == kScanHalfPair) {
      const size_t lds = chunk_scan_half_lds_bytes(P, N);
      auto kern = chunk_scan_half_kernel<P, N, OUT, 2>;
      if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kern, dim3((unsigned)(d.nblocks * (d.H / 2))), dim3(4 * 64), lds, stream,
                         reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B),
                         reinterpret_cast<const uint16_t*>(C), ws.table, ws.btable, ws.cs, ws.ck,
                         reinterpret_cast<const uint16_t*>(ws.start_states), reinterpret_cast<uint16_t*>(Y),
                         reinterpret_cast<const uint16_t*>(m2.z), m2.D, d.H, d.G, d.Q, (int)ranked_blocks(d));
      return hipGetLastError();
    }
    if (chunk_scan_kind(d) == kScanPair) {
      const size_t lds = chunk_scan_pair_lds_bytes(P, N, d.Q);
      auto kern = chunk_scan_pair_kernel<P, N, OUT>;
      if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kern, dim3((unsigned)(d.nblocks * (d.H / 2))), dim3(kScanThreads), lds, stream,
                         reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B),
                         reinterpret_cast<const uint16_t*>(C), ws.table, ws.btable, ws.cs, ws.ck,
                         reinterpret_cast<const uint16_t*>(ws.start_states), reinterpret_cast<uint16_t*>(Y),
                         reinterpret_cast<const uint16_t*>(m2.z), m2.D, d.H, d.G, d.Q, (int)ranked_blocks(d));
      return hipGetLastError();
    }
  }
  if constexpr (half_wide_shape(P, N)) {
    if (chunk_scan_kind(d) == kScanHalfPairWide) {
      const size_t lds = chunk_scan_half_lds_bytes(P, N);
      auto kern = chunk_scan_half_kernel<P, N, OUT, 1>;
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3((unsigned)(d.nblocks * (d.H / 2))), dim3(8 * 64), lds, stream,
                         reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B),
                         reinterpret_cast<const uint16_t*>(C), ws.table, ws.btable, ws.cs, ws.ck,
                         reinterpret_cast<const uint16_t*>(ws.start_states), reinterpret_cast<uint16_t*>(Y),
                         reinterpret_cast<const uint16_t*>(m2.z), m2.D, d.H, d.G, d.Q, (int)ranked_blocks(d));
      return hipGetLastError();
    }
  }
  const size_t lds = chunk_scan_bf16_lds_bytes(P, N, d.Q);
  auto kern = d.Q > 128 ? chunk_scan_bf16_kernel<P, N, 2, OUT> : chunk_scan_bf16_kernel<P, N, 1, OUT>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(d.nblocks * d.H)), dim3(kScanThreads), lds, stream,
                     reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B),
                     reinterpret_cast<const uint16_t*>(C), ws.table, ws.btable, ws.cs, ws.ck,
                     reinterpret_cast<const uint16_t*>(ws.start_states), reinterpret_cast<uint16_t*>(Y),
                     reinterpret_cast<const uint16_t*>(m2.z), m2.D, d.H, d.G, d.Q);
  return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_scan_gate(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                                   const Workspace& ws, hipStream_t stream, const Mamba2Args& m2) {
  if (d.y_f32) return launch_scan_bf16<P, N, kOutF32>(d, X, B, C, Y, ws, stream, m2);
  return m2.z ? launch_scan_bf16<P, N, kOutGated>(d, X, B, C, Y, ws, stream, m2)
              : launch_scan_bf16<P, N, kOutPlain>(d, X, B, C, Y, ws, stream, m2);
}

template <int P>
static hipError_t dispatch_scan_n(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                                  const Workspace& ws, hipStream_t stream, const Mamba2Args& m2) {
  switch (d.N) {
    case 32: return launch_scan_gate<P, 32>(d, X, B, C, Y, ws, stream, m2);
    case 64: return launch_scan_gate<P, 64>(d, X, B, C, Y, ws, stream, m2);
    case 128: return launch_scan_gate<P, 128>(d, X, B, C, Y, ws, stream, m2);
    case 256: return launch_scan_gate<P, 256>(d, X, B, C, Y, ws, stream, m2);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_scan(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                             const Workspace& ws, hipStream_t stream, const Mamba2Args& m2) {
  if (!d.bf16) {
    const size_t lds = ((size_t)32 * (2 * d.N + d.P) + 32 * 32 + 2 * d.Q) * 4;
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_scan_f32_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(chunk_scan_f32_kernel, dim3((unsigned)(d.nslots * d.H)), dim3(256), lds, stream,
                       reinterpret_cast<const float*>(X), reinterpret_cast<const float*>(B),
                       reinterpret_cast<const float*>(C), ws.table, ws.cs, ws.ck,
                       reinterpret_cast<const float*>(ws.start_states), reinterpret_cast<float*>(Y),
                       reinterpret_cast<const float*>(m2.z), m2.D, d.H, d.G, d.P, d.N, d.Q);
    return hipGetLastError();
  }
  switch (d.P) {
    case 16: return dispatch_scan_n<16>(d, X, B, C, Y, ws, stream, m2);
    case 32: return dispatch_scan_n<32>(d, X, B, C, Y, ws, stream, m2);
    case 64: return dispatch_scan_n<64>(d, X, B, C, Y, ws, stream, m2);
    case 128: return dispatch_scan_n<128>(d, X, B, C, Y, ws, stream, m2);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
