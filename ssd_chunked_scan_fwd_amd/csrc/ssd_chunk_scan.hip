// ssd_chunk_scan.hip -- diagonal blocks and left factors of the chunked SSD
// forward pass on gfx950.
//
// For every chunk slot and head, with cs the log2-scaled cumulative decay:
//   Y[i][p] = exp2(cs_i) sum_n C[i][n] start[p][n]                   (left factor)
//           + sum_{j <= i} exp2(cs_i - cs_j) (sum_n C[i][n] B[j][n]) X[j][p]
//                                                                   (diagonal block)
// ("Transformers are SSMs" paper card, Method 5 / paper section 6, "Diagonal
// Blocks" and "Left Factors"; pseudocode lines "within_mask", "Y_within",
// "decay_from_start", "Y_carry"). The mask is applied before the exponential
// (paper card Pitfalls: "Mask before exp"), so no positive exponent is formed.
//
// bf16 path, one workgroup (4 waves) per (slot, head):
//  * S^T = B C^T is computed tile by tile on 16x16x32 bf16 MFMA. Its
//    accumulator layout (lane = query row i, registers = 4 key rows j) is, after
//    masking and decay, directly the A operand of the next MFMA Y += (L o S) X,
//    so S never goes through LDS. L o S is carried as a bf16 hi/lo pair (two
//    MFMAs on the same X fragment): one bf16 rounding of L o S alone would
//    double the output error of the pass.
//  * The carry C start^T goes into the same accumulator first and is scaled by
//    exp2(cs_i) per row; only the lower triangle of S is formed.
//  * B (token-major) and the start state are staged in LDS as they are; X is
//    staged transposed. C fragments are read straight from global memory.
//  * Query-row tiles are dealt to waves in a zig-zag so that the triangular work
//    is balanced.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

size_t chunk_scan_bf16_lds_bytes(int P, int N, int Q) {
  return (size_t)Q * (N + 8) * 2 + (size_t)P * (Q + 8) * 2 + (size_t)P * (N + 8) * 2 + (size_t)Q * 4;
}

template <int P, int N>
__global__ __launch_bounds__(256) void chunk_scan_bf16_kernel(const uint16_t* __restrict__ X,
                                                              const uint16_t* __restrict__ B,
                                                              const uint16_t* __restrict__ C,
                                                              const int4* __restrict__ table,
                                                              const float* __restrict__ cs,
                                                              const uint16_t* __restrict__ start,
                                                              uint16_t* __restrict__ Y, int H, int G,
                                                              int Q) {
  const long unit = blockIdx.x;
  const int h = (int)(unit % H);
  const long slot = unit / H;
  const SlotRec rec = load_slot(table, slot);
  const int len = rec.len;
  if (len <= 0) return;
  const int g = h / (H / G);

  constexpr int TP = P / 16;
  constexpr int NB = N / 32;
  constexpr int BP = N + 8;       // LDS pitch of B rows and start rows (elements)
  const int XP = Q + 8;           // LDS pitch of X^T rows

  extern __shared__ uint16_t lds[];
  uint16_t* bs = lds;                       // [Q][BP]  B rows of the chunk
  uint16_t* xt = bs + Q * BP;               // [P][XP]  X^T
  uint16_t* st = xt + P * XP;               // [P][BP]  start state (bf16)
  float* csl = reinterpret_cast<float*>(st + P * BP);  // [Q]

  const int tid = threadIdx.x;
  const long tok0 = rec.tok0;
  const float* csr = cs + (slot * H + h) * (long)Q;
  for (int i = tid; i < Q; i += 256) csl[i] = csr[i];

  // B rows (zero past the chunk's length)
  {
    constexpr int CB = N / 8;
    const uint16_t* src = B + (tok0 * G + g) * N;
    for (int idx = tid; idx < Q * CB; idx += 256) {
      const int j = idx / CB, c = idx % CB;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (j < len) v = *reinterpret_cast<const u32x4*>(src + (long)j * G * N + c * 8);
      *reinterpret_cast<u32x4*>(bs + j * BP + c * 8) = v;
    }
  }
  // X^T via 8x8 register transposes (zero past the chunk's length)
  {
    constexpr int CB = P / 8;
    const uint16_t* src = X + (tok0 * H + h) * P;
    const long ld = (long)H * P;
    const int nblk = (Q / 8) * CB;
    for (int blk = tid; blk < nblk; blk += 256) {
      const int cb = blk % CB, jb = blk / CB;
      u32x4 in[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int j = jb * 8 + r;
        in[r] = (j < len) ? *reinterpret_cast<const u32x4*>(src + (long)j * ld + cb * 8) : u32x4{0u, 0u, 0u, 0u};
      }
      u32x4 out[8];
      transpose8x8_b16(in, out);
#pragma unroll
      for (int q = 0; q < 8; ++q) *reinterpret_cast<u32x4*>(xt + (cb * 8 + q) * XP + jb * 8) = out[q];
    }
  }
  // start state [P][N]
  {
    constexpr int CB = N / 8;
    const uint16_t* src = start + (slot * H + h) * (long)(P * N);
    for (int idx = tid; idx < P * CB; idx += 256) {
      const int p = idx / CB, c = idx % CB;
      *reinterpret_cast<u32x4*>(st + p * BP + c * 8) = *reinterpret_cast<const u32x4*>(src + p * N + c * 8);
    }
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int nIt = Q / 16;
  const int rounds = (nIt + 3) / 4;
  for (int rr = 0; rr < rounds; ++rr) {
    const int it = (rr & 1) ? (4 * rr + 3 - wave) : (4 * rr + wave);
    if (it >= nIt || it * 16 >= len) continue;

    const int irow = it * 16 + l16;  // this lane's query row (A rows of C, S^T columns)
    u32x4 cf[NB];
    {
      const uint16_t* crow = C + ((tok0 + irow) * G + g) * N + 8 * g4;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        cf[nb] = (irow < len) ? *reinterpret_cast<const u32x4*>(crow + nb * 32) : u32x4{0u, 0u, 0u, 0u};
    }

    // Left factor: acc[i][p] = sum_n C[i][n] start[p][n], then scaled by exp2(cs_i).
    f32x4 acc[TP];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt) {
      acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 sf = *reinterpret_cast<const u32x4*>(st + (pt * 16 + l16) * BP + nb * 32 + 8 * g4);
        acc[pt] = mfma16x16x32(cf[nb], sf, acc[pt]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = fast_exp2(csl[it * 16 + 4 * g4 + r]);
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) acc[pt][r] *= e;
    }

    // Diagonal block over key blocks of 32 tokens j <= i. The masked, decayed
    // block M = L o S is split into bf16 high and low parts (M = hi + lo to
    // about 16 significant bits) and both are multiplied into X, so that M is
    // not limited to bf16 precision.
    const float cs_i = csl[irow];
    for (int kb = 0; kb <= (it >> 1); ++kb) {
      uint32_t mw[4], ml[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int jt = 2 * kb + half;
        if (jt > it) {
          mw[2 * half] = 0u;
          mw[2 * half + 1] = 0u;
          ml[2 * half] = 0u;
          ml[2 * half + 1] = 0u;
          continue;
        }
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 bf = *reinterpret_cast<const u32x4*>(bs + (jt * 16 + l16) * BP + nb * 32 + 8 * g4);
          s = mfma16x16x32(bf, cf[nb], s);
        }
        // s[r] = S[i = irow][j = jt*16 + 4*g4 + r]; mask first, then exp.
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jt * 16 + 4 * g4 + r;
          v[r] = (j <= irow) ? s[r] * fast_exp2(cs_i - csl[j]) : 0.f;
        }
        mw[2 * half] = pack_bf16x2(v[0], v[1]);
        mw[2 * half + 1] = pack_bf16x2(v[2], v[3]);
        ml[2 * half] = pack_bf16x2(v[0] - bf16_lo(mw[2 * half]), v[1] - bf16_hi(mw[2 * half]));
        ml[2 * half + 1] = pack_bf16x2(v[2] - bf16_lo(mw[2 * half + 1]), v[3] - bf16_hi(mw[2 * half + 1]));
      }
      const u32x4 af = u32x4{mw[0], mw[1], mw[2], mw[3]};
      const u32x4 al = u32x4{ml[0], ml[1], ml[2], ml[3]};
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        const uint16_t* xr = xt + (pt * 16 + l16) * XP + 32 * kb + 4 * g4;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(xr);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(xr + 16);
        const u32x4 xf = u32x4{lo.x, lo.y, hi.x, hi.y};
        acc[pt] = mfma16x16x32(af, xf, acc[pt]);
        acc[pt] = mfma16x16x32(al, xf, acc[pt]);
      }
    }

    // Store rows i = it*16 + 4*g4 + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = it * 16 + 4 * g4 + r;
      if (i < len) {
        uint16_t* yr = Y + ((tok0 + i) * H + h) * P + l16;
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) yr[pt * 16] = f32_to_bf16(acc[pt][r]);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// fp32 path (plain FMA, fp32 accumulation). Query rows in blocks of 32; for
// each key block j0 <= i0 the masked, decayed block of C B^T is formed in LDS
// and multiplied into X.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_scan_f32_kernel(const float* __restrict__ X,
                                                             const float* __restrict__ B,
                                                             const float* __restrict__ C,
                                                             const int4* __restrict__ table,
                                                             const float* __restrict__ cs,
                                                             const float* __restrict__ start,
                                                             float* __restrict__ Y, int H, int G, int P,
                                                             int N, int Q) {
  const long unit = blockIdx.x;
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
  float* csl = m + IB * IB;        // [Q]
  const float* csr = cs + (slot * H + h) * (long)Q;
  for (int i = threadIdx.x; i < Q; i += 256) csl[i] = csr[i];
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
          v = s * fast_exp2(csl[i0 + i] - csl[j0 + j]);
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
        if (i < ni) Y[((tok0 + i0 + i) * H + h) * P + p] = acc[k];
      }
    }
  }
}

// ----------------------------------------------------------------------------

template <int P, int N>
static hipError_t launch_scan_bf16(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                                   const Workspace& ws, hipStream_t stream) {
  const size_t lds = chunk_scan_bf16_lds_bytes(P, N, d.Q);
  auto kern = chunk_scan_bf16_kernel<P, N>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(d.nslots * d.H)), dim3(256), lds, stream,
                     reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B),
                     reinterpret_cast<const uint16_t*>(C), ws.table, ws.cs,
                     reinterpret_cast<const uint16_t*>(ws.start_states), reinterpret_cast<uint16_t*>(Y), d.H,
                     d.G, d.Q);
  return hipGetLastError();
}

template <int P>
static hipError_t dispatch_scan_n(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                                  const Workspace& ws, hipStream_t stream) {
  switch (d.N) {
    case 32: return launch_scan_bf16<P, 32>(d, X, B, C, Y, ws, stream);
    case 64: return launch_scan_bf16<P, 64>(d, X, B, C, Y, ws, stream);
    case 128: return launch_scan_bf16<P, 128>(d, X, B, C, Y, ws, stream);
    case 256: return launch_scan_bf16<P, 256>(d, X, B, C, Y, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_scan(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                             const Workspace& ws, hipStream_t stream) {
  if (!d.bf16) {
    const size_t lds = ((size_t)32 * (2 * d.N + d.P) + 32 * 32 + d.Q) * 4;
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_scan_f32_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(chunk_scan_f32_kernel, dim3((unsigned)(d.nslots * d.H)), dim3(256), lds, stream,
                       reinterpret_cast<const float*>(X), reinterpret_cast<const float*>(B),
                       reinterpret_cast<const float*>(C), ws.table, ws.cs,
                       reinterpret_cast<const float*>(ws.start_states), reinterpret_cast<float*>(Y), d.H, d.G,
                       d.P, d.N, d.Q);
    return hipGetLastError();
  }
  switch (d.P) {
    case 16: return dispatch_scan_n<16>(d, X, B, C, Y, ws, stream);
    case 32: return dispatch_scan_n<32>(d, X, B, C, Y, ws, stream);
    case 64: return dispatch_scan_n<64>(d, X, B, C, Y, ws, stream);
    case 128: return dispatch_scan_n<128>(d, X, B, C, Y, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
