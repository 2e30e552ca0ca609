// ssd_chunk_state.hip -- right factors of the chunked SSD forward pass on gfx950.
//
// For every state block m (Gs consecutive chunks of one sequence) and head h:
//     s_m[p][n] = sum_j exp2(tail_j) X[j][p] B[j][n],
// tail_j = log2-scaled total decay from token j to the end of the block. With
// Gs = 1 this is exactly the chunk state of the pages' algorithm: the state at
// the chunk end from a zero start ("Transformers are SSMs" paper card, Method 5
// / paper section 6, "Right Factors": one batched matrix product per chunk,
// each token weighted by its decay to the chunk end). With Gs > 1 it is the
// same right factor for a longer block, which the chunk-scan stage refines
// chunk by chunk.
//
// Key-side weights: the weight of token j is exp2(tail_j) times the token's
// input scale. The exponent is read from `ck`, which equals the cumulative
// decay cs for plain calls and cs_j - log2(dt_j) for the Mamba-2 block's call,
// whose input is x * dt (paper card, Paper vs code item 7): the step size
// rides in the weight, so x itself is staged unscaled.
//
// bf16 path: one workgroup of 8 waves per (block, head). Token rows of X and B
// are staged into LDS as they lie in HBM (token-major) through registers,
// prefetching the next 128 rows while the current ones are multiplied; the
// decay weight is applied to X in registers before it is rounded to bf16 and
// stored. The contraction over tokens takes both MFMA operands with the gfx950
// LDS transpose read.
// Products run on 16x16x32 bf16 MFMA with fp32 accumulation; the block state
// is written in fp32 together with the block's total log2 decay.
#include <hip/hip_cooperative_groups.h>

#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_passing.h"
#include "ssd_segsum.h"
#include "ssd_stage.h"

namespace ssd {

namespace {

constexpr int kStateThreads = 512;  // 8 waves

__host__ __device__ constexpr int state_pass_rows(int N) { return N > 128 ? 64 : kPassRows; }
// Waves per SIMD the register budget is cut for (the second launch bound):
// two for the largest states (P * N of 16384 with 128-row passes, or 32768),
// else four: with 64-row passes two workgroups then share a CU (their LDS fits).
__host__ __device__ constexpr int state_min_waves(int P, int N) {
  return (P * N >= 32768 || (P * N >= 16384 && N <= 128)) ? 2 : 4;
}

template <int P, int N>
struct StateCfg {
  static constexpr int BP = lds_pitch(N), XP = lds_pitch(P);
  static constexpr int TP = P / 16, TN = N / 16;
  // MFMA waves: with large states, four waves of 2 x 4 tiles read fewer
  // fragments from LDS per product than eight waves of 2 x 2 (the pass loop is
  // bound by LDS reads); all eight waves stage the rows.
  static constexpr int MW = (P * N == 8192) ? 4 : 8;
  static constexpr int WN = TN < 4 ? TN : (MW == 4 ? 2 : 4);
  static constexpr int WP = (MW / WN) < TP ? (MW / WN) : TP;
  static constexpr int TPW = TP / WP, TNW = TN / WN;
  static constexpr int CBN = N / 8, CBP = P / 8;
  // Rows per pass: 128, or 64 for states beyond N = 128, whose B rows would
  // otherwise hold 70 KB of LDS and leave one workgroup per CU.
  static constexpr int PR = state_pass_rows(N);
  static constexpr int RB = (PR * CBN + kStateThreads - 1) / kStateThreads;
  static constexpr int RX = (PR * CBP + kStateThreads - 1) / kStateThreads;
};

}  // namespace

// The fused form (segment sums computed here) also keeps the key-side
// exponents of the block's chunks, [Gs * Q] fp32.
size_t chunk_state_bf16_lds_bytes(int P, int N, int block_tokens) {
  const size_t pr = (size_t)state_pass_rows(N);
  return (pr * lds_pitch(N) + pr * lds_pitch(P)) * 2 + 16 * 16 + 16 * 4 +
         (size_t)block_tokens * 4;
}

// FUSED: the workgroup also writes its block's records and the segment sums of
// its head (the work of chunk_cumsum, for the slots its block covers): head 0
// writes the records, and wave w takes chunks w, w + 8, ... of the block.
template <int P, int N, bool FUSED>
__device__ __forceinline__ void chunk_state_block(const uint16_t* __restrict__ X, const uint16_t* __restrict__ B,
                                                  int4* __restrict__ ctable, int4* __restrict__ btable,
                                                  float* __restrict__ cs, float* __restrict__ ck,
                                                  float* __restrict__ bstates, float* __restrict__ bdecay, int H,
                                                  int G, int Q, int Gs, const SegArgs& sa, long unit) {
  using K = StateCfg<P, N>;
  const int h = (int)(unit % H);
  const long m = unit / H;
  BlockRec blk;
  if constexpr (FUSED) {
    const int row = (int)(m / sa.blocks_per_row);
    const int4 b = block_record(sa.cu, sa.S, row, m - row * sa.blocks_per_row, Q, Gs, sa.slots_per_row);
    if (h == 0 && threadIdx.x == 0) btable[m] = b;
    blk = BlockRec{b.x, b.y, b.z};
  } else {
    blk = load_block(btable, m);
  }
  if (blk.nchunks <= 0) return;
  const int g = h / (H / G);

  extern __shared__ uint16_t lds[];
  uint16_t* bs = lds;                          // [PR][BP] B rows of the pass
  uint16_t* xw = bs + K::PR * K::BP;       // [PR][XP] X rows times their decay to the block end
  int4* recs = reinterpret_cast<int4*>(xw + K::PR * K::XP);   // [16] chunk records of the block
  float* lastcs = reinterpret_cast<float*>(recs + 16);             // [16] chunk totals (log2)
  float* ckl = lastcs + 16;                                        // [Gs][Q] key-side exponents (FUSED)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wn = wave % K::WN, wp = wave / K::WN;
  const bool active = wp < K::WP;
  const int p0t = wp * K::TPW, n0t = wn * K::TNW;
  const long ldb = (long)G * N, ldx = (long)H * P;

  uint32_t boff[K::RB], xoff[K::RX];
  int brow[K::RB], xrow[K::RX];
#pragma unroll
  for (int u = 0; u < K::RB; ++u) {
    const int idx = tid + kStateThreads * u;
    brow[u] = idx < K::PR * K::CBN ? idx / K::CBN : K::PR;
    boff[u] = brow[u] < K::PR ? (uint32_t)((brow[u] * ldb + (idx % K::CBN) * 8) * 2) : kOffNone;
  }
#pragma unroll
  for (int u = 0; u < K::RX; ++u) {
    const int idx = tid + kStateThreads * u;
    xrow[u] = idx < K::PR * K::CBP ? idx / K::CBP : K::PR;
    xoff[u] = xrow[u] < K::PR ? (uint32_t)((xrow[u] * ldx + (idx % K::CBP) * 8) * 2) : kOffNone;
  }

  // The block's chunk records and totals.
  if (tid < blk.nchunks) {
    if constexpr (FUSED) {
      const long slot = blk.slot0 + tid;
      const int row = (int)(slot / sa.slots_per_row);
      const int4 r = chunk_record(sa.cu, sa.S, row, slot - row * sa.slots_per_row, sa.T, Q, sa.slots_per_row);
      recs[tid] = r;
      if (h == 0) ctable[slot] = r;
    } else {
      recs[tid] = ctable[blk.slot0 + tid];
      lastcs[tid] = cs[((blk.slot0 + tid) * H + h) * (long)Q + Q - 1];
    }
  }
  __syncthreads();
  // One pass = rows r0 .. r0+PR-1 of chunk c; the next pass is loaded while the
  // current one is multiplied.
  u32x4 pb[K::RB], px[K::RX];
  float pcs[K::RX];
  // Loads of one pass into registers, issued unconditionally: rows past the
  // chunk's end and surplus lanes read zeros through the buffer range, and
  // with valid == false nothing is read.
  auto load_pass = [&](const SlotRec& r, long slot, int r0, bool valid) {
    const int rows = valid ? r.len - r0 : 0;
    const rsrc_t rb = make_rsrc(B + (((long)r.tok0 + r0) * G + g) * N, (uint32_t)(rows * ldb * 2));
    const rsrc_t rx = make_rsrc(X + (((long)r.tok0 + r0) * H + h) * P, (uint32_t)(rows * ldx * 2));
#pragma unroll
    for (int u = 0; u < K::RB; ++u) pb[u] = buf_load16(rb, boff[u]);
#pragma unroll
    for (int u = 0; u < K::RX; ++u) px[u] = buf_load16(rx, xoff[u]);
    if constexpr (!FUSED) {
      const rsrc_t rc = make_rsrc(ck + (slot * H + h) * (long)Q + r0, valid ? (uint32_t)((Q - r0) * 4) : 0u);
#pragma unroll
      for (int u = 0; u < K::RX; ++u) pcs[u] = buf_load_f32(rc, xrow[u] < K::PR ? (uint32_t)(xrow[u] * 4) : kOffNone);
    }
  };

  auto rec_of = [&](int c) {
    const int4 v = recs[c];
    return SlotRec{uniform(v.x), uniform(v.y), uniform(v.z), uniform(v.w)};
  };
  SlotRec rec = rec_of(0);
  load_pass(rec, blk.slot0, 0, true);
  if constexpr (FUSED) {
    // Segment sums of this head's chunks: to the workspace for the chunk-scan
    // stage, the key-side exponents to LDS for the weights below.
    const bool m2 = sa.dt != nullptr;
    const float A = m2 ? -expf(sa.A_log[h]) : 1.f;
    const float bias = (m2 && sa.dt_bias) ? sa.dt_bias[h] : 0.f;
    for (int c = wave; c < blk.nchunks; c += kStateThreads / 64) {
      const int4 r = recs[c];
      const long slot = blk.slot0 + c;
      const float* src = (m2 ? sa.dt : sa.la) + (long)r.y * H + h;
      const float tot = wave_segsum(
          [&](int j) {
            const float v = src[(long)j * H];
            return m2 ? softplus_f32(v + bias) : v;
          },
          r.z, Q, m2, A, cs + (slot * H + h) * (long)Q, m2 ? ck + (slot * H + h) * (long)Q : nullptr, ckl + c * Q,
          lane);
      if (lane == 0) lastcs[c] = tot;
    }
    __syncthreads();
  }
  // Total log2 decay of the block; the tail of chunk c is total - (A_0 + .. + A_c).
  float total = 0.f;
  for (int c = 0; c < blk.nchunks; ++c) total += lastcs[c];

  f32x4 acc[K::TPW][K::TNW];
#pragma unroll
  for (int a = 0; a < K::TPW; ++a)
#pragma unroll
    for (int b = 0; b < K::TNW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  float prefix = 0.f;
  for (int c = 0; c < blk.nchunks; ++c) {
    const long slot = blk.slot0 + c;
    const float a_last = lastcs[c];
    prefix += a_last;
    const float shift = (total - prefix) + a_last;  // weight of row j: exp2(shift - ck_j)
    const SlotRec cur = rec;
    for (int r0 = 0; r0 < cur.len; r0 += K::PR) {
      const int rows = min(K::PR, cur.len - r0);
      __syncthreads();
      // Row weights first: in the fused form they come from LDS and need not
      // wait for the pass loads.
      float wr[K::RX];
#pragma unroll
      for (int u = 0; u < K::RX; ++u) {
        const float kj = FUSED ? ckl[c * Q + min(r0 + min(xrow[u], K::PR - 1), Q - 1)] : pcs[u];
        const float e = fast_exp2(shift - kj);
        wr[u] = xrow[u] < rows ? e : 0.f;
      }
#pragma unroll
      for (int u = 0; u < K::RB; ++u)
        if (brow[u] < K::PR)
          *reinterpret_cast<u32x4*>(bs + brow[u] * K::BP + ((tid + kStateThreads * u) % K::CBN) * 8) = pb[u];
#pragma unroll
      for (int u = 0; u < K::RX; ++u) {
        if (xrow[u] < K::PR) {
          const float w = wr[u];
          u32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(bf16_lo(px[u][q]) * w, bf16_hi(px[u][q]) * w);
          *reinterpret_cast<u32x4*>(xw + xrow[u] * K::XP + ((tid + kStateThreads * u) % K::CBP) * 8) = v;
        }
      }
      // prefetch the next pass: next rows of this chunk, else the next chunk
      const bool in_chunk = r0 + K::PR < cur.len;
      const bool more = in_chunk || c + 1 < blk.nchunks;
      if (!in_chunk) rec = rec_of(more ? c + 1 : c);
      load_pass(in_chunk ? cur : rec, in_chunk ? slot : slot + (more ? 1 : 0), in_chunk ? r0 + K::PR : 0, more);
      __syncthreads();
      if (active) {
        const int nkb = (rows + 31) / 32;
#pragma unroll
        for (int kb = 0; kb < K::PR / 32; ++kb) {
          if (kb >= nkb) break;
          u32x4 xa[K::TPW], bb[K::TNW];
#pragma unroll
          for (int a = 0; a < K::TPW; ++a) xa[a] = frag_k_rows_accpair(xw, K::XP, 32 * kb, (p0t + a) * 16, lane);
#pragma unroll
          for (int b = 0; b < K::TNW; ++b) bb[b] = frag_k_rows_accpair(bs, K::BP, 32 * kb, (n0t + b) * 16, lane);
#pragma unroll
          for (int a = 0; a < K::TPW; ++a)
#pragma unroll
            for (int b = 0; b < K::TNW; ++b) acc[a][b] = mfma16x16x32(xa[a], bb[b], acc[a][b]);
        }
      }
    }
  }

  if (tid == 0) bdecay[m * H + h] = total;
  if (!active) return;
  float* out = bstates + (m * H + h) * (long)(P * N);
#pragma unroll
  for (int a = 0; a < K::TPW; ++a)
#pragma unroll
    for (int b = 0; b < K::TNW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = (p0t + a) * 16 + 4 * g4 + r;
        const int n = (n0t + b) * 16 + l16;
        out[p * N + n] = acc[a][b][r];
      }
}

template <int P, int N, bool FUSED>
__global__ __launch_bounds__(kStateThreads, state_min_waves(P, N)) void chunk_state_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ B, int4* __restrict__ ctable,
    int4* __restrict__ btable, float* __restrict__ cs, float* __restrict__ ck,
    float* __restrict__ bstates, float* __restrict__ bdecay, int H, int G, int Q, int Gs, SegArgs sa) {
  chunk_state_block<P, N, FUSED>(X, B, ctable, btable, cs, ck, bstates, bdecay, H, G, Q, Gs, sa,
                                 xcd_unit(blockIdx.x, gridDim.x));
}

// Two heads of one group per workgroup, 64-row passes: each pass stages the B
// rows once for both heads. The eight waves hold both heads' states (four
// waves per head). Each state tile accumulates its products in the same
// token order as chunk_state_block, so the results are bitwise the same. With
// more (block, head) units than one round of the one-head form (two
// workgroups per CU), this form runs half the workgroups, each pass half as
// many rows for two heads (b 8, T 4096, H 32, N 128: forward call 155.6 ->
// 141.1 us; packed H = 80 layer 423.7 -> 394.3 us; 47 KB of LDS and 96
// registers at P = 64, N = 128, two workgroups per CU).
template <int P, int N>
struct PairStateCfg {
  static constexpr int BP = lds_pitch(N), XP = lds_pitch(P);
  static constexpr int TP = P / 16, TN = N / 16;
  static constexpr int WN = TN < 2 ? TN : 2;
  static constexpr int WP = (4 / WN) < TP ? (4 / WN) : TP;
  static constexpr int TPW = TP / WP, TNW = TN / WN;
  static constexpr int CBN = N / 8, CBP = P / 8;
  static constexpr int PR = 64;
  static constexpr int RB = (PR * CBN + kStateThreads - 1) / kStateThreads;
  static constexpr int RX = (PR * CBP + kStateThreads - 1) / kStateThreads;
};

size_t chunk_state_pair_lds_bytes(int P, int N, int block_tokens) {
  return ((size_t)64 * lds_pitch(N) + 2 * (size_t)64 * lds_pitch(P)) * 2 + 16 * 16 + 2 * 16 * 4 +
         2 * (size_t)block_tokens * 4;
}

template <int P, int N, bool FUSED>
__device__ __forceinline__ void chunk_state_pair_block(const uint16_t* __restrict__ X, const uint16_t* __restrict__ B,
                                                       int4* __restrict__ ctable, int4* __restrict__ btable,
                                                       float* __restrict__ cs, float* __restrict__ ck,
                                                       float* __restrict__ bstates, float* __restrict__ bdecay,
                                                       int H, int G, int Q, int Gs, const SegArgs& sa, long unit) {
  using K = PairStateCfg<P, N>;
  const int HH = H / 2;
  const int hp = (int)(unit % HH);
  const long m = unit / HH;
  const int h0 = 2 * hp;
  BlockRec blk;
  if constexpr (FUSED) {
    const int row = (int)(m / sa.blocks_per_row);
    const int4 b = block_record(sa.cu, sa.S, row, m - row * sa.blocks_per_row, Q, Gs, sa.slots_per_row);
    if (hp == 0 && threadIdx.x == 0) btable[m] = b;
    blk = BlockRec{b.x, b.y, b.z};
  } else {
    blk = load_block(btable, m);
  }
  if (blk.nchunks <= 0) return;
  const int g = h0 / (H / G);
  const int GQ = Gs * Q;

  extern __shared__ uint16_t lds[];
  uint16_t* bs = lds;                                             // [64][BP] B rows of the pass
  uint16_t* xw = bs + K::PR * K::BP;                              // [2][64][XP] weighted X rows of both heads
  int4* recs = reinterpret_cast<int4*>(xw + 2 * K::PR * K::XP);   // [16] chunk records of the block
  float* lastcs = reinterpret_cast<float*>(recs + 16);            // [2][16] chunk totals (log2)
  float* ckl = lastcs + 32;                                       // [2][Gs * Q] key-side exponents (FUSED)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int hw = wave >> 2;  // head of this wave's state tiles
  const int wq = wave & 3;
  const int wn = wq % K::WN, wp = wq / K::WN;
  const bool active = wp < K::WP;
  const int p0t = wp * K::TPW, n0t = wn * K::TNW;
  const long ldb = (long)G * N, ldx = (long)H * P;

  uint32_t boff[K::RB], xoff[K::RX];
  int brow[K::RB], xrow[K::RX];
#pragma unroll
  for (int u = 0; u < K::RB; ++u) {
    const int idx = tid + kStateThreads * u;
    brow[u] = idx < K::PR * K::CBN ? idx / K::CBN : K::PR;
    boff[u] = brow[u] < K::PR ? (uint32_t)((brow[u] * ldb + (idx % K::CBN) * 8) * 2) : kOffNone;
  }
#pragma unroll
  for (int u = 0; u < K::RX; ++u) {
    const int idx = tid + kStateThreads * u;
    xrow[u] = idx < K::PR * K::CBP ? idx / K::CBP : K::PR;
    xoff[u] = xrow[u] < K::PR ? (uint32_t)((xrow[u] * ldx + (idx % K::CBP) * 8) * 2) : kOffNone;
  }

  if (tid < blk.nchunks) {
    if constexpr (FUSED) {
      const long slot = blk.slot0 + tid;
      const int row = (int)(slot / sa.slots_per_row);
      const int4 r = chunk_record(sa.cu, sa.S, row, slot - row * sa.slots_per_row, sa.T, Q, sa.slots_per_row);
      recs[tid] = r;
      if (hp == 0) ctable[slot] = r;
    } else {
      recs[tid] = ctable[blk.slot0 + tid];
      lastcs[tid] = cs[((blk.slot0 + tid) * H + h0) * (long)Q + Q - 1];
      lastcs[16 + tid] = cs[((blk.slot0 + tid) * H + h0 + 1) * (long)Q + Q - 1];
    }
  }
  __syncthreads();
  u32x4 pb[K::RB], px[2][K::RX];
  float pcs[2][K::RX];
  auto load_pass = [&](const SlotRec& r, long slot, int r0, bool valid) {
    const int rows = valid ? r.len - r0 : 0;
    const rsrc_t rb = make_rsrc(B + (((long)r.tok0 + r0) * G + g) * N, (uint32_t)(rows * ldb * 2));
    const rsrc_t rx0 = make_rsrc(X + (((long)r.tok0 + r0) * H + h0) * P, (uint32_t)(rows * ldx * 2));
    const rsrc_t rx1 = make_rsrc(X + (((long)r.tok0 + r0) * H + h0 + 1) * P, (uint32_t)(rows * ldx * 2));
#pragma unroll
    for (int u = 0; u < K::RB; ++u) pb[u] = buf_load16(rb, boff[u]);
#pragma unroll
    for (int u = 0; u < K::RX; ++u) {
      px[0][u] = buf_load16(rx0, xoff[u]);
      px[1][u] = buf_load16(rx1, xoff[u]);
    }
    if constexpr (!FUSED) {
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        const rsrc_t rc = make_rsrc(ck + (slot * H + h0 + hd) * (long)Q + r0, valid ? (uint32_t)((Q - r0) * 4) : 0u);
#pragma unroll
        for (int u = 0; u < K::RX; ++u)
          pcs[hd][u] = buf_load_f32(rc, xrow[u] < K::PR ? (uint32_t)(xrow[u] * 4) : kOffNone);
      }
    }
  };
  auto rec_of = [&](int c) {
    const int4 v = recs[c];
    return SlotRec{uniform(v.x), uniform(v.y), uniform(v.z), uniform(v.w)};
  };
  SlotRec rec = rec_of(0);
  load_pass(rec, blk.slot0, 0, true);
  if constexpr (FUSED) {
    // Segment sums of both heads' chunks (wave w takes (chunk, head) tasks w, w + 8, ...).
    const bool m2 = sa.dt != nullptr;
    const float A0 = m2 ? -expf(sa.A_log[h0]) : 1.f, A1 = m2 ? -expf(sa.A_log[h0 + 1]) : 1.f;
    const float b0 = (m2 && sa.dt_bias) ? sa.dt_bias[h0] : 0.f, b1 = (m2 && sa.dt_bias) ? sa.dt_bias[h0 + 1] : 0.f;
    for (int t = wave; t < 2 * blk.nchunks; t += kStateThreads / 64) {
      const int hd = t & 1, c = t >> 1;
      const int h = h0 + hd;
      const float A = hd ? A1 : A0;
      const float bias = hd ? b1 : b0;
      const int4 r = recs[c];
      const long slot = blk.slot0 + c;
      const float* src = (m2 ? sa.dt : sa.la) + (long)r.y * H + h;
      const float tot = wave_segsum(
          [&](int j) {
            const float v = src[(long)j * H];
            return m2 ? softplus_f32(v + bias) : v;
          },
          r.z, Q, m2, A, cs + (slot * H + h) * (long)Q, m2 ? ck + (slot * H + h) * (long)Q : nullptr,
          ckl + hd * GQ + c * Q, lane);
      if (lane == 0) lastcs[hd * 16 + c] = tot;
    }
    __syncthreads();
  }
  float total[2] = {0.f, 0.f};
  for (int c = 0; c < blk.nchunks; ++c) {
    total[0] += lastcs[c];
    total[1] += lastcs[16 + c];
  }

  f32x4 acc[K::TPW][K::TNW];
#pragma unroll
  for (int a = 0; a < K::TPW; ++a)
#pragma unroll
    for (int b = 0; b < K::TNW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  float prefix[2] = {0.f, 0.f};
  for (int c = 0; c < blk.nchunks; ++c) {
    const long slot = blk.slot0 + c;
    float shift[2];
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
      const float a_last = lastcs[hd * 16 + c];
      prefix[hd] += a_last;
      shift[hd] = (total[hd] - prefix[hd]) + a_last;  // weight of row j: exp2(shift - ck_j)
    }
    const SlotRec cur = rec;
    for (int r0 = 0; r0 < cur.len; r0 += K::PR) {
      const int rows = min(K::PR, cur.len - r0);
      __syncthreads();
      float wr[2][K::RX];
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
#pragma unroll
        for (int u = 0; u < K::RX; ++u) {
          const float kj = FUSED ? ckl[hd * GQ + c * Q + min(r0 + min(xrow[u], K::PR - 1), Q - 1)] : pcs[hd][u];
          const float e = fast_exp2(shift[hd] - kj);
          wr[hd][u] = xrow[u] < rows ? e : 0.f;
        }
#pragma unroll
      for (int u = 0; u < K::RB; ++u)
        if (brow[u] < K::PR)
          *reinterpret_cast<u32x4*>(bs + brow[u] * K::BP + ((tid + kStateThreads * u) % K::CBN) * 8) = pb[u];
#pragma unroll
      for (int hd = 0; hd < 2; ++hd)
#pragma unroll
        for (int u = 0; u < K::RX; ++u) {
          if (xrow[u] < K::PR) {
            const float w = wr[hd][u];
            u32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(bf16_lo(px[hd][u][q]) * w, bf16_hi(px[hd][u][q]) * w);
            *reinterpret_cast<u32x4*>(xw + hd * K::PR * K::XP + xrow[u] * K::XP +
                                      ((tid + kStateThreads * u) % K::CBP) * 8) = v;
          }
        }
      const bool in_chunk = r0 + K::PR < cur.len;
      const bool more = in_chunk || c + 1 < blk.nchunks;
      if (!in_chunk) rec = rec_of(more ? c + 1 : c);
      load_pass(in_chunk ? cur : rec, in_chunk ? slot : slot + (more ? 1 : 0), in_chunk ? r0 + K::PR : 0, more);
      __syncthreads();
      if (active) {
        const int nkb = (rows + 31) / 32;
        const uint16_t* xh = xw + hw * K::PR * K::XP;
#pragma unroll
        for (int kb = 0; kb < K::PR / 32; ++kb) {
          if (kb >= nkb) break;
          u32x4 xa[K::TPW], bb[K::TNW];
#pragma unroll
          for (int a = 0; a < K::TPW; ++a) xa[a] = frag_k_rows_accpair(xh, K::XP, 32 * kb, (p0t + a) * 16, lane);
#pragma unroll
          for (int b = 0; b < K::TNW; ++b) bb[b] = frag_k_rows_accpair(bs, K::BP, 32 * kb, (n0t + b) * 16, lane);
#pragma unroll
          for (int a = 0; a < K::TPW; ++a)
#pragma unroll
            for (int b = 0; b < K::TNW; ++b) acc[a][b] = mfma16x16x32(xa[a], bb[b], acc[a][b]);
        }
      }
    }
  }

  if (tid == 0) {
    bdecay[m * H + h0] = total[0];
    bdecay[m * H + h0 + 1] = total[1];
  }
  if (!active) return;
  float* out = bstates + (m * H + h0 + hw) * (long)(P * N);
#pragma unroll
  for (int a = 0; a < K::TPW; ++a)
#pragma unroll
    for (int b = 0; b < K::TNW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = (p0t + a) * 16 + 4 * g4 + r;
        const int n = (n0t + b) * 16 + l16;
        out[p * N + n] = acc[a][b][r];
      }
}

template <int P, int N, bool FUSED>
__global__ __launch_bounds__(kStateThreads, 4) void chunk_state_pair_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ B, int4* __restrict__ ctable,
    int4* __restrict__ btable, float* __restrict__ cs, float* __restrict__ ck,
    float* __restrict__ bstates, float* __restrict__ bdecay, int H, int G, int Q, int Gs, SegArgs sa) {
  chunk_state_pair_block<P, N, FUSED>(X, B, ctable, btable, cs, ck, bstates, bdecay, H, G, Q, Gs, sa,
                                      xcd_unit(blockIdx.x, gridDim.x));
}

// The state chain in one launch: every workgroup computes its block's right
// factor as above, a grid-wide barrier (cooperative launch: all workgroups are
// resident) makes them visible, and the same grid then runs the centre-factor
// recurrence of every (sequence, head) and 4 state elements (pass_states),
// writing the block-entering states and the final states.
template <int P, int N>
__global__ __launch_bounds__(kStateThreads, (P * N >= 16384) ? 2 : 4) void chunk_state_chain_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ B, int4* __restrict__ ctable,
    int4* __restrict__ btable, float* __restrict__ cs, float* __restrict__ ck,
    float* __restrict__ bstates, float* __restrict__ bdecay, int H, int G, int Q, int Gs, SegArgs sa,
    void* __restrict__ start, float* __restrict__ final_state, const float* __restrict__ init, int nseq) {
  chunk_state_block<P, N, true>(X, B, ctable, btable, cs, ck, bstates, bdecay, H, G, Q, Gs, sa,
                                xcd_unit(blockIdx.x, gridDim.x));
  cooperative_groups::this_grid().sync();
  constexpr int PN = P * N, E4 = PN / kPassElems;
  const long total = (long)nseq * H * E4;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const long r = i / E4;
    pass_states<true>(bstates, bdecay, start, final_state, init, sa.cu, sa.blocks_per_row, H, PN, Gs * Q,
                      (int)(r / H), (int)(r % H), (int)(i % E4) * kPassElems);
  }
}

// ----------------------------------------------------------------------------
// fp32 path (plain FMA, fp32 accumulation; one chunk per state block): tokens
// staged 32 at a time in LDS.
// ----------------------------------------------------------------------------
template <bool FUSED>
__global__ __launch_bounds__(256) void chunk_state_f32_kernel(const float* __restrict__ X,
                                                              const float* __restrict__ B,
                                                              int4* __restrict__ table,
                                                              int4* __restrict__ btable,
                                                              float* __restrict__ cs,
                                                              float* __restrict__ ck,
                                                              float* __restrict__ states,
                                                              float* __restrict__ bdecay, int H, int G,
                                                              int P, int N, int Q, SegArgs sa) {
  const long unit = xcd_unit(blockIdx.x, gridDim.x);
  const int h = (int)(unit % H);
  const long slot = unit / H;
  SlotRec rec;
  if constexpr (FUSED) {  // records and segment sums of this slot (one chunk per state block)
    const int row = (int)(slot / sa.slots_per_row);
    const long x = slot - row * sa.slots_per_row;
    const int4 r = chunk_record(sa.cu, sa.S, row, x, sa.T, Q, sa.slots_per_row);
    if (h == 0 && threadIdx.x == 0) {
      table[slot] = r;
      btable[slot] = block_record(sa.cu, sa.S, row, x, Q, 1, sa.slots_per_row);
    }
    rec = SlotRec{r.x, r.y, r.z, r.w};
  } else {
    rec = load_slot(table, slot);
  }
  if (rec.len <= 0) return;
  const int g = h / (H / G);
  constexpr int JB = 32;
  extern __shared__ float sm[];
  float* xs = sm;            // [JB][P], scaled by the decay to the chunk end
  float* bs = sm + JB * P;   // [JB][N]
  const float* ckr = ck + (slot * H + h) * (long)Q;
  float cs_last;
  if constexpr (FUSED) {
    float* ckl = bs + JB * N;  // [Q] key-side exponents
    __shared__ float tot;
    if (threadIdx.x < 64) {
      const bool m2 = sa.dt != nullptr;
      const float A = m2 ? -expf(sa.A_log[h]) : 1.f;
      const float bias = (m2 && sa.dt_bias) ? sa.dt_bias[h] : 0.f;
      const float* src = (m2 ? sa.dt : sa.la) + (long)rec.tok0 * H + h;
      const float t = wave_segsum(
          [&](int j) {
            const float v = src[(long)j * H];
            return m2 ? softplus_f32(v + bias) : v;
          },
          rec.len, Q, m2, A, cs + (slot * H + h) * (long)Q, m2 ? ck + (slot * H + h) * (long)Q : nullptr, ckl,
          threadIdx.x);
      if (threadIdx.x == 0) tot = t;
    }
    __syncthreads();
    ckr = ckl;
    cs_last = tot;
  } else {
    cs_last = cs[(slot * H + h) * (long)Q + Q - 1];
  }
  if (threadIdx.x == 0) bdecay[slot * H + h] = cs_last;
  const int PN = P * N;
  constexpr int kPer = 8;  // outputs per thread per pass
  float* out = states + (slot * H + h) * (long)PN;
  for (int e0 = 0; e0 < PN; e0 += 256 * kPer) {
    float acc[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < rec.len; j0 += JB) {
      const int nb = min(JB, rec.len - j0);
      const long tok = (long)rec.tok0 + j0;
      __syncthreads();
      for (int idx = threadIdx.x; idx < JB * P; idx += 256) {
        const int j = idx / P, p = idx % P;
        xs[idx] = j < nb ? X[((tok + j) * H + h) * P + p] * fast_exp2(cs_last - ckr[j0 + j]) : 0.f;
      }
      for (int idx = threadIdx.x; idx < JB * N; idx += 256) {
        const int j = idx / N, n = idx % N;
        bs[idx] = j < nb ? B[((tok + j) * G + g) * N + n] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = e0 + threadIdx.x + 256 * i;
        if (e < PN) {
          const int p = e / N, n = e % N;
          float s = acc[i];
          for (int j = 0; j < nb; ++j) s = fmaf(xs[j * P + p], bs[j * N + n], s);
          acc[i] = s;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = e0 + threadIdx.x + 256 * i;
      if (e < PN) out[e] = acc[i];
    }
  }
}

// ----------------------------------------------------------------------------

// The head-pair form: heads in pairs within a group, states of up to 64 x 128,
// and more (block, head) units than one round of the one-head form (two
// workgroups per CU on 256 CUs).
static bool chunk_state_pair_use(const FwdDims& d) {
  return d.P <= 64 && d.N <= 128 && (d.H / d.G) % 2 == 0 && d.nblocks * d.H > 2 * 256;
}

template <int P, int N, bool FUSED>
static hipError_t launch_state_bf16(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                    hipStream_t stream, const SegArgs& sa) {
  if constexpr (P <= 64 && N <= 128) {
    if (chunk_state_pair_use(d)) {
      const size_t lds = chunk_state_pair_lds_bytes(P, N, FUSED ? d.state_block * d.Q : 0);
      auto kern = chunk_state_pair_kernel<P, N, FUSED>;
      if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kern, dim3((unsigned)(d.nblocks * (d.H / 2))), dim3(kStateThreads), lds, stream,
                         reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B), ws.table,
                         ws.btable, ws.cs, ws.ck, ws.bstates, ws.bdecay, d.H, d.G, d.Q, d.state_block, sa);
      return hipGetLastError();
    }
  }
  const size_t lds = chunk_state_bf16_lds_bytes(P, N, FUSED ? d.state_block * d.Q : 0);
  auto kern = chunk_state_bf16_kernel<P, N, FUSED>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(d.nblocks * d.H)), dim3(kStateThreads), lds, stream,
                     reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B), ws.table,
                     ws.btable, ws.cs, ws.ck, ws.bstates, ws.bdecay, d.H, d.G, d.Q, d.state_block, sa);
  return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_state_fuse(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                    hipStream_t stream, const SegArgs* seg) {
  return seg ? launch_state_bf16<P, N, true>(d, X, B, ws, stream, *seg)
             : launch_state_bf16<P, N, false>(d, X, B, ws, stream, SegArgs{});
}

template <int P>
static hipError_t dispatch_state_n(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                   hipStream_t stream, const SegArgs* seg) {
  switch (d.N) {
    case 32: return launch_state_fuse<P, 32>(d, X, B, ws, stream, seg);
    case 64: return launch_state_fuse<P, 64>(d, X, B, ws, stream, seg);
    case 128: return launch_state_fuse<P, 128>(d, X, B, ws, stream, seg);
    case 256: return launch_state_fuse<P, 256>(d, X, B, ws, stream, seg);
    default: return hipErrorInvalidValue;
  }
}

// Whether the grid of the cooperative chain kernel for these dimensions can be
// resident all at once on the current device (asked on every call: nothing is
// cached, so concurrent host threads share no state here).
template <int P, int N>
static hipError_t chain_fits_device(const FwdDims& d, bool* fits) {
  *fits = false;
  const size_t lds = chunk_state_bf16_lds_bytes(P, N, d.state_block * d.Q);
  auto kern = chunk_state_chain_kernel<P, N>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int per_cu = 0, ncu = 0, dev = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kStateThreads, lds);
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  *fits = d.nblocks * d.H <= (long)per_cu * ncu;
  return hipSuccess;
}

template <int P, int N>
static hipError_t launch_chain_t(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                 hipStream_t stream, const SegArgs& sa, const float* init, float* final_state,
                                 bool* launched) {
  bool fits = false;
  hipError_t e = chain_fits_device<P, N>(d, &fits);
  if (e != hipSuccess || !fits) return e;  // not all resident: the caller runs two launches
  const size_t lds = chunk_state_bf16_lds_bytes(P, N, d.state_block * d.Q);
  auto kern = chunk_state_chain_kernel<P, N>;
  const long grid = d.nblocks * d.H;
  const uint16_t* Xp = reinterpret_cast<const uint16_t*>(X);
  const uint16_t* Bp = reinterpret_cast<const uint16_t*>(B);
  int4* table = ws.table;
  int4* btable = ws.btable;
  float* cs = ws.cs;
  float* ck = ws.ck;
  float* bstates = ws.bstates;
  float* bdecay = ws.bdecay;
  int H = d.H, G = d.G, Q = d.Q, Gs = d.state_block;
  SegArgs sac = sa;
  void* start = ws.start_states;
  float* fin = final_state;
  const float* ini = init;
  int nseq = sa.cu ? d.num_seqs : d.batch;
  void* args[] = {&Xp, &Bp, &table, &btable, &cs, &ck, &bstates, &bdecay, &H, &G, &Q, &Gs, &sac, &start, &fin, &ini,
                  &nseq};
  e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)grid), dim3(kStateThreads), args,
                                 (unsigned)lds, stream);
  if (e == hipSuccess) *launched = true;
  return e;
}

bool chunk_state_chain_fits(const FwdDims& d) {
  return d.bf16 && (d.P * d.N == 8192 || d.P * d.N == 4096 || d.P * d.N == 16384) && d.P >= 32 && d.N >= 64;
}

hipError_t chunk_state_chain_cooperative(const FwdDims& d, bool* cooperative) {
  *cooperative = false;
  if (!chunk_state_chain_fits(d)) return hipSuccess;
  switch (d.P * 1000 + d.N) {
    case 32064: return chain_fits_device<32, 64>(d, cooperative);
    case 32128: return chain_fits_device<32, 128>(d, cooperative);
    case 64064: return chain_fits_device<64, 64>(d, cooperative);
    case 64128: return chain_fits_device<64, 128>(d, cooperative);
    case 128064: return chain_fits_device<128, 64>(d, cooperative);
    case 128128: return chain_fits_device<128, 128>(d, cooperative);
    default: return hipSuccess;
  }
}

hipError_t launch_chunk_state_chain(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                    hipStream_t stream, const SegArgs& sa, const float* init, float* final_state,
                                    bool* launched) {
  *launched = false;
  if (!chunk_state_chain_fits(d)) return hipSuccess;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return e;
  if (cap != hipStreamCaptureStatusNone) return hipSuccess;  // graphs take the two-launch form
  switch (d.P * 1000 + d.N) {
    case 32064: return launch_chain_t<32, 64>(d, X, B, ws, stream, sa, init, final_state, launched);
    case 32128: return launch_chain_t<32, 128>(d, X, B, ws, stream, sa, init, final_state, launched);
    case 64064: return launch_chain_t<64, 64>(d, X, B, ws, stream, sa, init, final_state, launched);
    case 64128: return launch_chain_t<64, 128>(d, X, B, ws, stream, sa, init, final_state, launched);
    case 128064: return launch_chain_t<128, 64>(d, X, B, ws, stream, sa, init, final_state, launched);
    case 128128: return launch_chain_t<128, 128>(d, X, B, ws, stream, sa, init, final_state, launched);
    default: return hipSuccess;
  }
}

hipError_t launch_chunk_state(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                              hipStream_t stream, const SegArgs* seg) {
  if (!d.bf16) {
    const size_t lds = ((size_t)32 * (d.P + d.N) + (seg ? d.Q : 0)) * 4;
    auto kern = seg ? chunk_state_f32_kernel<true> : chunk_state_f32_kernel<false>;
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)(d.nslots * d.H)), dim3(256), lds, stream,
                       reinterpret_cast<const float*>(X), reinterpret_cast<const float*>(B), ws.table, ws.btable,
                       ws.cs, ws.ck, ws.bstates, ws.bdecay, d.H, d.G, d.P, d.N, d.Q, seg ? *seg : SegArgs{});
    return hipGetLastError();
  }
  switch (d.P) {
    case 16: return dispatch_state_n<16>(d, X, B, ws, stream, seg);
    case 32: return dispatch_state_n<32>(d, X, B, ws, stream, seg);
    case 64: return dispatch_state_n<64>(d, X, B, ws, stream, seg);
    case 128: return dispatch_state_n<128>(d, X, B, ws, stream, seg);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
