// ssd_bwd.hip -- the data-movement and reduction kernels of the backward pass.
//
// The backward pass is assembled from forward passes (paper card Method 5:
// the chunked algorithm multiplies by the semiseparable matrix M = L o (C B^T);
// its transpose M^T is the same kind of matrix run backwards in time with the
// roles of B and C exchanged, and the state-space duality of Method 3-4 lets
// every gradient contraction be written as such a product):
//   dX    = M^T dY: a forward pass over each sequence reversed in time, with
//           B and C exchanged and log a shifted by one token, starting from the
//           final-state gradient;
//   dB, dC: forward passes with the roles of x, B, C and dY exchanged, per
//           head, summed over the heads of each group;
//   d log a_t = a_t <lam_t, h_{t-1}>: by chunks (dlog_chunk_kernel).
// The kernels below reverse token order within each sequence (behind padding
// that keeps reversed chunks aligned with forward chunks), broadcast B/C rows
// over heads, sum per-head partials over groups, and form d log a and the
// initial-state gradient.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// Sequence of token t within row `row`: [b, e) with b <= t < e.
__device__ __forceinline__ void seq_bounds(const int32_t* __restrict__ cu, int S, int T, int t, int& b, int& e) {
  if (cu == nullptr) {
    b = 0;
    e = T;
    return;
  }
  int lo = 0, hi = S - 1;  // last s with cu[s] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  b = cu[lo];
  e = cu[lo + 1];
}

// Padded reversed layout. Sequence s of length L becomes, in the reversed
// tensors, pad_s = (Q - L mod Q) mod Q zero tokens followed by its tokens in
// reverse order, so that reversed chunk k covers exactly forward chunk
// nch - 1 - k (chunks start at sequence starts in both directions). Unpacked
// rows have Tr = T + pad tokens each; packed sequences start at cur[s]
// (a prefix sum of the padded lengths, written by padded_offsets_kernel).

// Flattened position in the padded reversed layout of forward token t of row `row`.
__device__ __forceinline__ long reversed_position(const int32_t* __restrict__ cu, const int32_t* __restrict__ cur,
                                                  int S, int T, int Tr, int row, int t) {
  int b, e;
  seq_bounds(cu, S, T, t, b, e);
  if (cu == nullptr) return (long)row * Tr + (Tr - T) + (T - 1 - t);
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int pad = (cur[lo + 1] - cur[lo]) - (e - b);
  return (long)cur[lo] + pad + (e - 1 - t);
}

// Forward token of position p of the padded reversed layout of row `row`, or -1 for padding.
__device__ __forceinline__ long forward_position(const int32_t* __restrict__ cu, const int32_t* __restrict__ cur,
                                                 int S, int T, int Tr, int row, int p) {
  if (cu == nullptr) {
    const int pad = Tr - T;
    return p < pad ? -1 : (long)row * T + (T - 1 - (p - pad));
  }
  if (p >= cur[S]) return -1;
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cur[mid] <= p) lo = mid; else hi = mid - 1;
  }
  const int len = cu[lo + 1] - cu[lo];
  const int pad = (cur[lo + 1] - cur[lo]) - len;
  const int tau = p - cur[lo] - pad;
  return tau < 0 ? -1 : (long)cu[lo + 1] - 1 - tau;
}

__global__ __launch_bounds__(256) void padded_offsets_kernel(const int32_t* __restrict__ cu, int32_t* __restrict__ cur,
                                                             int S, int Q) {
  // One workgroup: cur[s] = sum over s' < s of ceil(len_s' / Q) * Q.
  __shared__ int32_t part[256];
  int carry = 0;
  for (int base = 0; base <= S; base += 256) {
    const int s = base + threadIdx.x;
    int v = 0;
    if (s < S) {
      const int len = cu[s + 1] - cu[s];
      v = (len + Q - 1) / Q * Q;
    }
    part[threadIdx.x] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {  // inclusive scan
      const int u = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
      __syncthreads();
      part[threadIdx.x] += u;
      __syncthreads();
    }
    if (s <= S) cur[s] = carry + part[threadIdx.x] - v;  // exclusive
    const int tot = part[255];
    __syncthreads();
    carry += tot;
  }
}

// Rows [row, t, hout, 0..D) of `out` from `in`, with head hout reading head
// hout / (Hout / Hin) (a B/C row broadcast to heads when Hout > Hin):
//   mode 0: same layout;
//   mode 1: out is the padded reversed layout ([rows * Tr] tokens), in the
//           forward layout; padding positions are zero;
//   mode 2: out is the forward layout ([rows * T]), in the padded reversed layout.
// Rows move in 16-byte pieces (D * esz is a multiple of 16).
__device__ __forceinline__ void gather_rows_block(const uint8_t* __restrict__ in, uint8_t* __restrict__ out,
                                                  const int32_t* __restrict__ cu, const int32_t* __restrict__ cur,
                                                  int S, int T, int Tr, int Hin, int Hout, int row_bytes, int mode,
                                                  int xblocks, int tpw, long ntok, long bid) {
  // A token's row is Hout * pieces 16-byte pieces: xblocks workgroups per
  // token for long rows, tpw tokens per workgroup for short ones.
  const int pieces = row_bytes / 16;  // per head
  const int per_tok = Hout * pieces;
  const long tok = (bid / xblocks) * (long)tpw + (tpw > 1 ? threadIdx.x / per_tok : 0);  // output token
  const int xb = (int)(bid % xblocks);
  const int idx = tpw > 1 ? (int)(threadIdx.x % per_tok) : xb * 256 + (int)threadIdx.x;
  if (idx >= per_tok || tok >= ntok || (tpw > 1 && (int)threadIdx.x >= tpw * per_tok)) return;
  const int ho = idx / pieces, q = idx % pieces;
  const int hi = ho / (Hout / Hin);
  long src = tok;  // mode 0: same layout
  if (mode == 1) {
    const int row = (int)(tok / Tr), p = (int)(tok % Tr);
    src = forward_position(cu, cur, S, T, Tr, row, p);
  } else if (mode == 2) {
    const int row = (int)(tok / T), t = (int)(tok % T);
    src = reversed_position(cu, cur, S, T, Tr, row, t);
  }
  u32x4 v = {0u, 0u, 0u, 0u};
  if (src >= 0) v = *reinterpret_cast<const u32x4*>(in + (src * Hin + hi) * (long)row_bytes + q * 16);
  *reinterpret_cast<u32x4*>(out + (tok * Hout + ho) * (long)row_bytes + q * 16) = v;
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ in, uint8_t* __restrict__ out,
                                                          const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ cur, int S, int T, int Tr,
                                                          int Hin, int Hout, int row_bytes, int mode,
                                                          int xblocks, int tpw, long ntok) {
  gather_rows_block(in, out, cu, cur, S, T, Tr, Hin, Hout, row_bytes, mode, xblocks, tpw, ntok, blockIdx.x);
}

// out[row, t, g, 0..D) = sum over the heads h of group g of in[row, rsrc(t), h, 0..D)
// (fp32 partials of the padded reversed layout when `flip`, else of the forward
// layout), rounded once to the output dtype.
template <bool BF16>
__global__ __launch_bounds__(256) void group_sum_kernel(const float* __restrict__ in, void* __restrict__ out,
                                                        const int32_t* __restrict__ cu,
                                                        const int32_t* __restrict__ cur, int S, int T, int Tr,
                                                        int H, int G, int D, int flip, int xblocks) {
  const long tok = blockIdx.x / xblocks;
  const int xb = (int)(blockIdx.x % xblocks);
  const int row = (int)(tok / T), t = (int)(tok % T);
  const long src = flip ? reversed_position(cu, cur, S, T, Tr, row, t) : tok;
  const int idx = xb * 256 + threadIdx.x;  // one element of [G][D]
  if (idx >= G * D) return;
  const int g = idx / D, d = idx % D;
  const int hpg = H / G;
  float acc = 0.f;
  for (int k = 0; k < hpg; ++k) acc += in[(src * H + g * hpg + k) * D + d];
  const long o = (tok * G + g) * D + d;
  if (BF16) reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(acc);
  else reinterpret_cast<float*>(out)[o] = acc;
}

// Log decays of the reversed run, padded layout: 0 on padding and at the
// first reversed token of each sequence, else la[src + 1] (the reversed
// recurrence applies a_{t+1} to the adjoint of h_t).
__device__ __forceinline__ void reverse_log_decay_block(const float* __restrict__ la, float* __restrict__ out,
                                                        const int32_t* __restrict__ cu, const int32_t* __restrict__ cur,
                                                        int S, int T, int Tr, int H, long ntok, long bid) {
  const long i = bid * 256 + threadIdx.x;
  if (i >= ntok * H) return;
  const long tok = i / H;
  const int h = (int)(i % H);
  const int row = (int)(tok / Tr), p = (int)(tok % Tr);
  const long src = forward_position(cu, cur, S, T, Tr, row, p);
  float v = 0.f;
  if (src >= 0) {
    const int t = (int)(src - (long)row * (cu ? 0 : T));
    int b, e;
    seq_bounds(cu, S, T, t, b, e);
    if (t + 1 < e) v = la[(src + 1) * H + h];
  }
  out[i] = v;
}

__global__ __launch_bounds__(256) void reverse_log_decay_kernel(const float* __restrict__ la, float* __restrict__ out,
                                                                const int32_t* __restrict__ cu,
                                                                const int32_t* __restrict__ cur, int S, int T, int Tr,
                                                                int H, long ntok) {
  reverse_log_decay_block(la, out, cu, cur, S, T, Tr, H, ntok, blockIdx.x);
}

// The fused backward's reversed inputs in one launch: workgroups [0, na) gather
// the rows of dY, [na, na + nc) those of C, the rest reverse the log decay.
struct GatherPlan {
  int xblocks, tpw;
  long ntok, blocks;
};

__host__ __device__ inline GatherPlan gather_plan(int Hout, int row_bytes, long ntok) {
  GatherPlan g;
  const int pieces = Hout * (row_bytes / 16);
  g.xblocks = (pieces + 255) / 256;
  g.tpw = pieces < 256 ? 256 / pieces : 1;  // tokens per workgroup
  g.ntok = ntok;
  g.blocks = (ntok + g.tpw - 1) / g.tpw * g.xblocks;
  return g;
}

__global__ __launch_bounds__(256) void reverse_inputs_kernel(const uint8_t* __restrict__ dy, uint8_t* __restrict__ rev_dy,
                                                             const uint8_t* __restrict__ c, uint8_t* __restrict__ rev_c,
                                                             const float* __restrict__ la, float* __restrict__ la_rev,
                                                             const int32_t* __restrict__ cu,
                                                             const int32_t* __restrict__ cur, int S, int T, int Tr,
                                                             int H, int G, int dy_bytes, int c_bytes, GatherPlan pa,
                                                             GatherPlan pc) {
  const long bid = blockIdx.x;
  if (bid < pa.blocks)
    gather_rows_block(dy, rev_dy, cu, cur, S, T, Tr, H, H, dy_bytes, 1, pa.xblocks, pa.tpw, pa.ntok, bid);
  else if (bid < pa.blocks + pc.blocks)
    gather_rows_block(c, rev_c, cu, cur, S, T, Tr, G, G, c_bytes, 1, pc.xblocks, pc.tpw, pc.ntok, bid - pa.blocks);
  else
    reverse_log_decay_block(la, la_rev, cu, cur, S, T, Tr, H, pa.ntok, bid - pa.blocks - pc.blocks);
}

// [S][H][A][Bdim] -> [S][H][Bdim][A] (fp32), for states handed to runs whose
// roles of headdim and dstate are exchanged.
__global__ __launch_bounds__(256) void transpose_states_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                               int A, int Bd, long total) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long mat = i / ((long)A * Bd);
  const int r = (int)(i % ((long)A * Bd));
  const int a = r / Bd, bb = r % Bd;
  out[mat * A * Bd + (long)bb * A + a] = in[i];
}

// d log a by chunks, without the cancellation of sum_k (dY_k.y_k - x_k.dx_k):
// d log a_t = a_t <lam_t, h_{t-1}> is the sum of R_ij = dY_i . M_ij x_j over the
// pairs i >= t > j. For t in a chunk [s, s + len) it splits into
//   A_t = pairs inside the chunk            (R from C B^T, dY x^T and L, in fp32)
//   B_t = i >= t in the chunk, j before it  = sum_{i >= t} dY_i . 2^{cs_i} C_i^T h_start
//   C_t = i after the chunk, j < t in it    = sum_{j < t} x_j . 2^{cs_last - cs_j} lam_after^T B_j
//   D   = i after, j before                 = 2^{cs_last} <lam_after, h_start>
// with h_start the state entering the chunk (the forward run's chunk start
// state) and lam_after the adjoint reaching the chunk's last state from later
// outputs (the reversed run's chunk start state, times a of the next token).
// A_t - A_{t+1} = sum_{j<t} R_tj - sum_{i>t} R_it, summed within the chunk.
// One workgroup (256 threads, thread = query row) per (chunk slot, head).
template <int P, int N, bool BF16>
__global__ __launch_bounds__(256) void dlog_chunk_kernel(
    const void* __restrict__ X, const void* __restrict__ dY, const void* __restrict__ Bm, const void* __restrict__ Cm,
    const float* __restrict__ la, const int4* __restrict__ ftable, const int4* __restrict__ fbtable,
    const float* __restrict__ fcs, const void* __restrict__ fstart, const void* __restrict__ rstart,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cur, long spr, long spr_r, float* __restrict__ dla,
    int H, int G, int Q) {
  const long slot = blockIdx.x / H;
  const int h = (int)(blockIdx.x % H);
  // With one chunk per state block, block slot = chunk slot. The block table is
  // written for every slot; the chunk table only for slots that hold a chunk
  // (packed rows leave slots between sequences unwritten).
  if (fbtable[slot].z <= 0) return;
  const int4 rec = ftable[slot];
  const int len = rec.z;
  if (len <= 0) return;
  const int seq = rec.x, tok0 = rec.y, jc = rec.w;
  const int g = h / (H / G);
  int nch;
  long rslot;
  if (cu == nullptr) {
    nch = (int)spr;
    rslot = (long)seq * spr_r + (nch - 1 - jc);
  } else {
    nch = (cu[seq + 1] - cu[seq] + Q - 1) / Q;
    rslot = cur[seq] / Q + seq + (nch - 1 - jc);
  }
  const float anext = jc == nch - 1 ? 1.f : __builtin_amdgcn_exp2f(la[(long)(tok0 + len) * H + h] * kLog2e);

  auto ld = [&](const void* p, long i) -> float {
    return BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]) : reinterpret_cast<const float*>(p)[i];
  };
  using E = typename std::conditional<BF16, uint16_t, float>::type;  // LDS tiles keep the input dtype
  auto cv = [](E v) -> float {
    if constexpr (BF16) return bf16_to_f32(v);
    else return v;
  };
  extern __shared__ float sm[];
  E* Bs = reinterpret_cast<E*>(sm);  // [Q][N]
  E* Xs = Bs + Q * N;                // [Q][P]
  float* csl = reinterpret_cast<float*>(Xs + Q * P);  // [Q]
  float* hs = csl + Q;               // [P][N] state entering the chunk (element (p, n) = h[n][p])
  float* ls = hs + P * N;            // [P][N] adjoint from after the chunk (times a_next)
  float* colp = ls + P * N;          // [4][Q] column partials per wave
  float* rs = colp + 4 * Q;          // [Q] row sums
  float* bb = rs + Q;                // [Q] b_i
  float* cc = bb + Q;                // [Q] c_j
  float* red = cc + Q;               // [4]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < len * N; i += 256) Bs[i] = reinterpret_cast<const E*>(Bm)[((long)(tok0 + i / N) * G + g) * N + i % N];
  for (int i = tid; i < len * P; i += 256) Xs[i] = reinterpret_cast<const E*>(X)[((long)(tok0 + i / P) * H + h) * P + i % P];
  for (int i = tid; i < len; i += 256) csl[i] = fcs[(slot * H + h) * (long)Q + i];
  for (int i = tid; i < P * N; i += 256) {
    hs[i] = ld(fstart, (slot * H + h) * (long)(P * N) + i);
    ls[i] = anext * ld(rstart, (rslot * H + h) * (long)(P * N) + i);
  }
  __syncthreads();

  const int i = tid;
  const bool vi = i < len;
  float Ci[N], Yi[P];
#pragma unroll
  for (int n = 0; n < N; ++n) Ci[n] = vi ? ld(Cm, ((long)(tok0 + i) * G + g) * N + n) : 0.f;
#pragma unroll
  for (int q = 0; q < P; ++q) Yi[q] = vi ? ld(dY, ((long)(tok0 + i) * H + h) * P + q) : 0.f;
  const float cs_i = vi ? csl[i] : 0.f;

  // Pairs inside the chunk: row sums per thread, column sums per wave.
  float rowsum = 0.f;
  for (int jj = 0; jj < len; ++jj) {
    float r = 0.f;
    if (vi && jj <= i) {
      float sdot = 0.f, ddot = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) sdot += Ci[n] * cv(Bs[jj * N + n]);
#pragma unroll
      for (int q = 0; q < P; ++q) ddot += Yi[q] * cv(Xs[jj * P + q]);
      r = __builtin_amdgcn_exp2f(cs_i - csl[jj]) * sdot * ddot;
    }
    if (jj < i) rowsum += r;
    float v = i > jj ? r : 0.f;
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) colp[wave * Q + jj] = v;
  }
  // b_i = dY_i . 2^{cs_i} C_i^T h_start;  c_i = x_i . 2^{cs_last - cs_i} lam^T B_i
  const float cs_last = csl[len - 1];
  float bsum = 0.f, csum = 0.f;
  if (vi) {
#pragma unroll 4
    for (int n = 0; n < N; ++n) {
      float u = 0.f;
#pragma unroll
      for (int q = 0; q < P; ++q) u += hs[q * N + n] * Yi[q];
      bsum += Ci[n] * u;
    }
    bsum *= __builtin_amdgcn_exp2f(cs_i);
#pragma unroll 4
    for (int q = 0; q < P; ++q) {
      float u = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) u += ls[q * N + n] * cv(Bs[i * N + n]);
      csum += cv(Xs[i * P + q]) * u;
    }
    csum *= __builtin_amdgcn_exp2f(cs_last - cs_i);
  }
  // D = 2^{cs_last} <lam_after, h_start>
  float dpart = 0.f;
  for (int k = tid; k < P * N; k += 256) dpart += ls[k] * hs[k];
  for (int off = 32; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off);
  if (lane == 0) red[wave] = dpart;
  if (vi) {
    rs[i] = rowsum;
    bb[i] = bsum;
    cc[i] = csum;
  }
  __syncthreads();
  const float D = __builtin_amdgcn_exp2f(cs_last) * (red[0] + red[1] + red[2] + red[3]);
  if (tid == 0) {
    // A_t = sum_{k >= t} (rowsum_k - colsum_k), B_t = sum_{k >= t} b_k, C_t = sum_{k < t} c_k
    float A = 0.f, Bv = 0.f;
    for (int t = len - 1; t >= 0; --t) {
      const float col = colp[t] + colp[Q + t] + colp[2 * Q + t] + colp[3 * Q + t];
      A += rs[t] - col;
      Bv += bb[t];
      rs[t] = A + Bv;
    }
    float Cv = 0.f;
    for (int t = 0; t < len; ++t) {
      const float c = cc[t];
      cc[t] = Cv;
      Cv += c;
    }
  }
  __syncthreads();
  if (vi) dla[(long)(tok0 + i) * H + h] = rs[i] + cc[i] + D;
}

size_t dlog_chunk_lds_bytes(int P, int N, int Q, int esz) {
  return (size_t)Q * (N + P) * esz + (2 * (size_t)P * N + 8 * (size_t)Q + 4) * 4;
}

// d h_init = a_first * lam_first for each (sequence, head): lam_first is the
// adjoint of the first state (the reversed run's final state).
__global__ __launch_bounds__(256) void dinit_kernel(const float* __restrict__ la, const float* __restrict__ lam_first,
                                                    float* __restrict__ dinit, const int32_t* __restrict__ cu,
                                                    int T, int H, int PN, long total) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long sh = i / PN;
  const int s = (int)(sh / H), h = (int)(sh % H);
  const long first = cu ? (long)cu[s] : (long)s * T;
  dinit[i] = __builtin_amdgcn_exp2f(la[first * H + h] * kLog2e) * lam_first[i];
}

// ----------------------------------------------------------------------------

hipError_t launch_padded_offsets(const int32_t* cu, int32_t* cur, int S, int Q, hipStream_t stream) {
  hipLaunchKernelGGL(padded_offsets_kernel, dim3(1), dim3(256), 0, stream, cu, cur, S, Q);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* in, void* out, const int32_t* cu, const int32_t* cur, int S, int rows, int T,
                              int Tr, int Hin, int Hout, int row_bytes, int mode, hipStream_t stream) {
  const int pieces = Hout * (row_bytes / 16);
  const int xblocks = (pieces + 255) / 256;
  const int tpw = pieces < 256 ? 256 / pieces : 1;  // tokens per workgroup
  const long ntok = (long)rows * (mode == 1 ? Tr : T);
  const long groups = (ntok + tpw - 1) / tpw;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)(groups * xblocks)), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(in), reinterpret_cast<uint8_t*>(out), cu, cur, S, T, Tr, Hin,
                     Hout, row_bytes, mode, xblocks, tpw, ntok);
  return hipGetLastError();
}

hipError_t launch_group_sum(const float* in, void* out, const int32_t* cu, const int32_t* cur, int S, int rows, int T,
                            int Tr, int H, int G, int D, bool bf16, bool from_reversed, hipStream_t stream) {
  const int xblocks = (G * D + 255) / 256;
  dim3 grid((unsigned)((long)rows * T * xblocks));
  if (bf16)
    hipLaunchKernelGGL(group_sum_kernel<true>, grid, dim3(256), 0, stream, in, out, cu, cur, S, T, Tr, H, G, D,
                       from_reversed ? 1 : 0, xblocks);
  else
    hipLaunchKernelGGL(group_sum_kernel<false>, grid, dim3(256), 0, stream, in, out, cu, cur, S, T, Tr, H, G, D,
                       from_reversed ? 1 : 0, xblocks);
  return hipGetLastError();
}

hipError_t launch_reverse_log_decay(const float* la, float* out, const int32_t* cu, const int32_t* cur, int S,
                                    int rows, int T, int Tr, int H, hipStream_t stream) {
  const long ntok = (long)rows * Tr;
  hipLaunchKernelGGL(reverse_log_decay_kernel, dim3((unsigned)((ntok * H + 255) / 256)), dim3(256), 0, stream, la,
                     out, cu, cur, S, T, Tr, H, ntok);
  return hipGetLastError();
}

hipError_t launch_reverse_inputs(const void* dY, void* rev_dy, int dy_bytes, const void* C, void* rev_c, int c_bytes,
                                 const float* la, float* la_rev, const int32_t* cu, const int32_t* cur, int S, int rows,
                                 int T, int Tr, int H, int G, hipStream_t stream) {
  const long ntok = (long)rows * Tr;
  const GatherPlan pa = gather_plan(H, dy_bytes, ntok), pc = gather_plan(G, c_bytes, ntok);
  const long blocks = pa.blocks + pc.blocks + (ntok * H + 255) / 256;
  hipLaunchKernelGGL(reverse_inputs_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(dY), reinterpret_cast<uint8_t*>(rev_dy),
                     reinterpret_cast<const uint8_t*>(C), reinterpret_cast<uint8_t*>(rev_c), la, la_rev, cu, cur, S,
                     T, Tr, H, G, dy_bytes, c_bytes, pa, pc);
  return hipGetLastError();
}

hipError_t launch_transpose_states(const float* in, float* out, long nmat, int A, int Bd, hipStream_t stream) {
  const long total = nmat * A * Bd;
  hipLaunchKernelGGL(transpose_states_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, in, out,
                     A, Bd, total);
  return hipGetLastError();
}

hipError_t launch_dinit(const float* la, const float* lam_first, float* dinit, const int32_t* cu, int nseq, int T,
                        int H, int PN, hipStream_t stream) {
  const long total = (long)nseq * H * PN;
  hipLaunchKernelGGL(dinit_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, la, lam_first, dinit,
                     cu, T, H, PN, total);
  return hipGetLastError();
}

template <int P, int N>
static hipError_t launch_dlog_pn(const DlogArgs& a, hipStream_t stream) {
  const size_t lds = dlog_chunk_lds_bytes(P, N, a.Q, a.bf16 ? 2 : 4);
  auto k = a.bf16 ? dlog_chunk_kernel<P, N, true> : dlog_chunk_kernel<P, N, false>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3((unsigned)(a.nslots * a.H)), dim3(256), lds, stream, a.X, a.dY, a.B, a.C, a.la, a.ftable,
                     a.fbtable, a.fcs, a.fstart, a.rstart, a.cu, a.cur, a.spr, a.spr_r, a.dla, a.H, a.G, a.Q);
  return hipGetLastError();
}

template <int P>
static hipError_t launch_dlog_n(const DlogArgs& a, hipStream_t stream) {
  switch (a.N) {
    case 16: return launch_dlog_pn<P, 16>(a, stream);
    case 32: return launch_dlog_pn<P, 32>(a, stream);
    case 64: return launch_dlog_pn<P, 64>(a, stream);
    case 128:
      if constexpr (P <= 64) return launch_dlog_pn<P, 128>(a, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dlog_chunks(const DlogArgs& a, hipStream_t stream) {
  switch (a.P) {
    case 16: return launch_dlog_n<16>(a, stream);
    case 32: return launch_dlog_n<32>(a, stream);
    case 64: return launch_dlog_n<64>(a, stream);
    case 128: return launch_dlog_n<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
