// ssd_cumsum_passing.hip -- the two scalar-recurrence stages of the chunked SSD
// forward pass on gfx950: the per-chunk cumulative log decay (chunk_cumsum)
// and the inter-chunk state recurrence (state_passing).
//
// Source: "Transformers are SSMs" paper card (wikillm.com/papers/2405.21060),
// Method 5 / paper section 6: the cumulative log decay restarted in every
// chunk gives the 1-semiseparable mask and each chunk's total decay; the
// "Center Factors" step carries states across chunks with a scalar recurrence.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_passing.h"
#include "ssd_segsum.h"

namespace ssd {

// ----------------------------------------------------------------------------
// chunk_cumsum: grid (slot x, row y). Workgroup x writes the record of chunk
// slot x and of state-block slot x (chunk_record, block_record), reads the
// chunk's log_a rows (contiguous, [len][H]) into LDS, and its 16 waves take
// heads in turn and write the segment sums (wave_segsum). The Mamba-2 call
// stages dt' = softplus(dt + dt_bias) instead and also writes ck.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_cumsum_kernel(SegArgs sa, int H, int Q, int Gs,
                                                           int4* __restrict__ table, int4* __restrict__ btable,
                                                           float* __restrict__ cs, float* __restrict__ ck) {
  extern __shared__ float tile[];  // [Q][H + 1] log_a (or dt') of the chunk, token-major
  const int row = blockIdx.y;
  const long x = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (threadIdx.x == 0 && x < sa.blocks_per_row)
    btable[row * sa.blocks_per_row + x] = block_record(sa.cu, sa.S, row, x, Q, Gs, sa.slots_per_row);
  if (x >= sa.slots_per_row) return;

  const long slot = (long)row * sa.slots_per_row + x;
  const int4 rec = chunk_record(sa.cu, sa.S, row, x, sa.T, Q, sa.slots_per_row);
  if (threadIdx.x == 0) table[slot] = rec;
  const int tok0 = rec.y, len = rec.z;
  if (len <= 0) return;

  // The chunk's rows are contiguous: read them coalesced into LDS.
  const bool m2 = sa.dt != nullptr;
  const int HP = H + 1;
  const float* src = (m2 ? sa.dt : sa.la) + (long)tok0 * H;
  for (int idx = threadIdx.x; idx < len * H; idx += 1024) {
    float v = src[idx];
    if (m2) v = softplus_f32(v + (sa.dt_bias ? sa.dt_bias[idx % H] : 0.f));
    tile[(idx / H) * HP + idx % H] = v;
  }
  __syncthreads();

  for (int h = wave; h < H; h += 16) {
    const float A = m2 ? -expf(sa.A_log[h]) : 1.f;
    wave_segsum([&](int j) { return tile[j * HP + h]; }, len, Q, m2, A, cs + (slot * H + h) * (long)Q,
                m2 ? ck + (slot * H + h) * (long)Q : nullptr, nullptr, lane);
  }
}

hipError_t launch_chunk_cumsum(const FwdDims& d, const float* log_a, const int32_t* cu,
                               const Workspace& ws, hipStream_t stream, const Mamba2Args& m2) {
  const long gx = d.slots_per_row > d.blocks_per_row ? d.slots_per_row : d.blocks_per_row;
  const size_t lds = (size_t)d.Q * (d.H + 1) * sizeof(float);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_cumsum_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const SegArgs sa = seg_args(d, log_a, cu, m2);
  dim3 grid((unsigned)gx, (unsigned)d.batch);
  hipLaunchKernelGGL(chunk_cumsum_kernel, grid, dim3(1024), lds, stream, sa, d.H, d.Q, d.state_block, ws.table,
                     ws.btable, ws.cs, ws.ck);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// state_passing: the centre-factor recurrence over each sequence's state blocks
// (pass_states). One thread owns 4 consecutive (p, n) elements of one
// (sequence, head) and moves them with 16-byte loads; the block loop is
// unrolled so that the loads of sixteen blocks are in flight together.
// ----------------------------------------------------------------------------
// The chunk-scan stage's launch order (scan_unit): the last workgroup of the
// state-passing launch ranks the block slots by chunk count, most first, ties
// by slot (a counting sort over the 17 possible counts), and writes
// btable[rank].w = (slot + 1) | (nfull << 16), nfull = the number of slots with
// the largest count. Slot counts from 2^15 on keep the records' w = 0 (the
// plain XCD order). 256 threads.
__device__ void rank_blocks(int4* __restrict__ btable, long nblocks) {
  __shared__ int cnt[17], start[17], wcnt[4][17], top;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (nblocks >= 32768) return;
  auto count_of = [&](long m) { return min(max(btable[m].z, 0), 16); };
  if (tid < 17) cnt[tid] = 0;
  __syncthreads();
  for (long m = tid; m < nblocks; m += 256) atomicAdd(&cnt[count_of(m)], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0, t = -1;
    for (int v = 16; v >= 0; --v) {
      start[v] = acc;
      acc += cnt[v];
      if (t < 0 && cnt[v] > 0) t = v;
    }
    top = t;
  }
  __syncthreads();
  const int nfull = cnt[top];
  for (long c0 = 0; c0 < nblocks; c0 += 256) {
    const long m = c0 + tid;
    const int v = m < nblocks ? count_of(m) : -1;
    int below = 0;  // slots of this wave below this lane with the same count
#pragma unroll
    for (int b = 0; b <= 16; ++b) {
      const uint64_t bal = __ballot(v == b);
      if (v == b) below = __popcll(bal & ((1ull << lane) - 1));
      if (lane == 0) wcnt[wave][b] = __popcll(bal);
    }
    __syncthreads();
    if (v >= 0) {
      int pos = start[v] + below;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][v];
      btable[pos].w = (int)(m + 1) | (nfull << 16);
    }
    __syncthreads();
    if (tid < 17) start[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void state_passing_kernel(const float* __restrict__ states,
                                                            const float* __restrict__ bdecay,
                                                            void* __restrict__ start,
                                                            float* __restrict__ final_state,
                                                            const float* __restrict__ init,
                                                            const int32_t* __restrict__ cu,
                                                            long blocks_per_row, int H, int PN, int span,
                                                            int4* __restrict__ btable, long nblocks, int rank) {
  if (rank && blockIdx.x == gridDim.x - 1) {  // the extra workgroup: the chunk-scan order
    rank_blocks(btable, nblocks);
    return;
  }
  const int eblocks = (PN / kPassElems + 255) / 256;
  const long unit = blockIdx.x;
  const int e = (int)(unit % eblocks) * (256 * kPassElems) + threadIdx.x * kPassElems;
  const int h = (int)((unit / eblocks) % H);
  const int s = (int)(unit / ((long)eblocks * H));
  if (e >= PN) return;
  pass_states<OUT_BF16>(states, bdecay, start, final_state, init, cu, blocks_per_row, H, PN, span, s, h, e);
}

hipError_t launch_state_passing(const FwdDims& d, const int32_t* cu, const float* init, float* final_state,
                                const Workspace& ws, hipStream_t stream) {
  const int PN = d.P * d.N;
  const int nseq = cu ? d.num_seqs : d.batch;
  const long eblocks = (PN / kPassElems + 255) / 256;
  const int rank = ranked_blocks(d) ? 1 : 0;
  dim3 grid((unsigned)(eblocks * d.H * nseq + rank));  // + the workgroup that ranks the blocks
  const int span = d.state_block * d.Q;
  if (d.bf16) {
    hipLaunchKernelGGL(state_passing_kernel<true>, grid, dim3(256), 0, stream, ws.bstates, ws.bdecay,
                       ws.start_states, final_state, init, cu, d.blocks_per_row, d.H, PN, span, ws.btable,
                       (long)d.nblocks, rank);
  } else {
    hipLaunchKernelGGL(state_passing_kernel<false>, grid, dim3(256), 0, stream, ws.bstates, ws.bdecay,
                       ws.start_states, final_state, init, cu, d.blocks_per_row, d.H, PN, span, ws.btable,
                       (long)d.nblocks, rank);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// ssd_step: one decode step. One workgroup per (row, head); N/4 consecutive
// lanes share a state row p, each owning 4 consecutive n. The state is read
// and written once (fp32); y[p] = sum_n state'[p][n] C[n] is reduced across
// the lanes of the row. The state streams through with non-temporal loads and
// stores: a model's per-layer decode states together exceed the Infinity Cache,
// so each step's state comes from HBM, and streaming accesses move it at a
// higher rate there (a cached read and write of one resident state is faster
// only while that state stays in the cache). The Mamba-2 block's step (dt != null) discretises
// first, dt' = softplus(dt + dt_bias), a = exp(dt' A) with A = -exp(A_log),
// feeds x dt' into the state, and finishes y with the skip D x and the gate
// silu(z) (paper card Method 6 block sketch; Paper vs code items 3, 7).
// ----------------------------------------------------------------------------
// Sum over aligned groups of n consecutive lanes, n a power of two from 4 to
// 64; every lane of a group receives the sum (DPP within rows of 16 lanes,
// then lane swaps across rows).
__device__ __forceinline__ float lanes_sum(float v, int n) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(ctrl)::value,
                                                                 0xF, 0xF, false));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});                // quad_perm [1, 0, 3, 2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});                // quad_perm [2, 3, 0, 1]
  if (n > 4) v += dpp(v, std::integral_constant<int, 0x141>{});    // row_half_mirror
  if (n > 8) v += dpp(v, std::integral_constant<int, 0x140>{});    // row_mirror
  if (n > 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  if (n > 32) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  return v;
}

template <bool BF16>
__global__ __launch_bounds__(256) void ssd_step_kernel(float* __restrict__ state,
                                                       const void* __restrict__ x,
                                                       const float* __restrict__ la,
                                                       const void* __restrict__ Bv,
                                                       const void* __restrict__ Cv,
                                                       void* __restrict__ y, int H, int G, int P, int N,
                                                       const float* __restrict__ dt,
                                                       const float* __restrict__ dt_bias,
                                                       const float* __restrict__ A_log,
                                                       const float* __restrict__ Dskip,
                                                       const void* __restrict__ zv) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int g = h / (H / G);
  const int tpr = N >> 2;             // lanes per state row (4..64, power of two)
  const int c4 = threadIdx.x & (tpr - 1);
  const int p0 = threadIdx.x / tpr;
  const int rpp = 256 / tpr;          // rows per pass
  const long bh = (long)b * H + h;
  const long bg = (long)b * G + g;
  float* st = state + bh * (long)P * N;
  float a, xscale = 1.f, Dh = 0.f;
  if (dt) {
    const float dtp = softplus_f32(dt[bh] + (dt_bias ? dt_bias[h] : 0.f));
    a = fast_exp2(dtp * -expf(A_log[h]) * kLog2e);
    xscale = dtp;
    Dh = Dskip ? Dskip[h] : 0.f;
  } else {
    a = fast_exp2(la[bh] * kLog2e);
  }

  float bb[4], cc[4];
  if (BF16) {
    const u32x2 wb = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(Bv) + bg * N + 4 * c4);
    const u32x2 wc = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(Cv) + bg * N + 4 * c4);
    bb[0] = bf16_lo(wb.x); bb[1] = bf16_hi(wb.x); bb[2] = bf16_lo(wb.y); bb[3] = bf16_hi(wb.y);
    cc[0] = bf16_lo(wc.x); cc[1] = bf16_hi(wc.x); cc[2] = bf16_lo(wc.y); cc[3] = bf16_hi(wc.y);
  } else {
    const f32x4 fb = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(Bv) + bg * N + 4 * c4);
    const f32x4 fc = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(Cv) + bg * N + 4 * c4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { bb[i] = fb[i]; cc[i] = fc[i]; }
  }

  // Up to 8 state rows per thread per round: every row's load is issued
  // before the first is used, so each lane keeps 8 loads in flight; rows past
  // P are neither read nor written (their addresses are clamped to row P - 1).
  constexpr int kRows = 8;
  for (int pb = p0; pb < P; pb += kRows * rpp) {
    f32x4* sp[kRows];
    f32x4 s[kRows];
    float xr[kRows];
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int p = pb + k * rpp;
      sp[k] = reinterpret_cast<f32x4*>(st + (long)min(p, P - 1) * N + 4 * c4);
      if (p < P) s[k] = __builtin_nontemporal_load(sp[k]);
    }
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int p = min(pb + k * rpp, P - 1);
      xr[k] = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[bh * P + p])
                   : reinterpret_cast<const float*>(x)[bh * P + p];
    }
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int p = pb + k * rpp;
      if (p >= P) break;
      const float xp = xr[k];
      const float xs = xp * xscale;
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[k][i] = a * s[k][i] + xs * bb[i];
        part += s[k][i] * cc[i];
      }
      __builtin_nontemporal_store(s[k], sp[k]);
      part = lanes_sum(part, tpr);
      part += Dh * xp;
      if (zv) {
        const float zp = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(zv)[bh * P + p])
                              : reinterpret_cast<const float*>(zv)[bh * P + p];
        part *= silu_f32(zp);
      }
      if (c4 == 0) {
        if (BF16) reinterpret_cast<uint16_t*>(y)[bh * P + p] = f32_to_bf16(part);
        else reinterpret_cast<float*>(y)[bh * P + p] = part;
      }
    }
  }
}

hipError_t launch_ssd_step(int batch, int H, int G, int P, int N, int bf16, float* state,
                           const void* x, const float* log_a, const void* B, const void* C, void* y,
                           hipStream_t stream, const Mamba2Args& m2) {
  dim3 grid((unsigned)H, (unsigned)batch);
  if (bf16) {
    hipLaunchKernelGGL(ssd_step_kernel<true>, grid, dim3(256), 0, stream, state, x, log_a, B, C, y, H, G,
                       P, N, m2.dt, m2.dt_bias, m2.A_log, m2.D, m2.z);
  } else {
    hipLaunchKernelGGL(ssd_step_kernel<false>, grid, dim3(256), 0, stream, state, x, log_a, B, C, y, H,
                       G, P, N, m2.dt, m2.dt_bias, m2.A_log, m2.D, m2.z);
  }
  return hipGetLastError();
}

}  // namespace ssd
