// ssd_chunk_state.hip -- right factors of the chunked SSD forward pass on gfx950.
//
// For every chunk slot k and head h:
//     s_k[p][n] = sum_j exp2(cs_last - cs_j) X[j][p] B[j][n]
// the state at the chunk end from a zero start ("Transformers are SSMs" paper
// card, Method 5 / paper section 6, "Right Factors": one batched matrix
// product per chunk; pseudocode lines "decay_to_end" and "chunk_states").
//
// bf16 path: the contraction runs over tokens j, which are the slow dimension
// of X [T][H][P] and B [T][G][N]. Both operands are staged into LDS
// transposed (p-major and n-major) with an in-register 8x8 transpose, so that
// every MFMA operand is one 16-byte LDS read. The decay is folded into X
// before it is rounded to bf16. Products run on 16x16x32 bf16 MFMA with fp32
// accumulation; the state is written in fp32.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kSubTokens = 128;  // tokens staged per pass

// Stage rows [j0, j0 + nb) of a token-major bf16 matrix (row stride `ld`
// elements, `cols` columns starting at `src`) into dst[col][j] (pitch `pitch`),
// zero-filling tokens nb .. qb-1. When `scale` is not null, row j is
// multiplied by scale[j] before rounding back to bf16.
template <int COLS>
__device__ __forceinline__ void stage_transposed(uint16_t* __restrict__ dst, int pitch,
                                                 const uint16_t* __restrict__ src, long ld, int nb,
                                                 int qb, const float* scale) {
  constexpr int CB = COLS / 8;
  const int nblk = (qb / 8) * CB;
  for (int blk = threadIdx.x; blk < nblk; blk += 256) {
    const int cb = blk % CB;
    const int jb = blk / CB;
    u32x4 in[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int j = jb * 8 + r;
      if (j < nb) {
        u32x4 v = *reinterpret_cast<const u32x4*>(src + (long)j * ld + cb * 8);
        if (scale) {
          const float w = scale[j];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = pack_bf16x2(bf16_lo(v[c]) * w, bf16_hi(v[c]) * w);
        }
        in[r] = v;
      } else {
        in[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    u32x4 out[8];
    transpose8x8_b16(in, out);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<u32x4*>(dst + (cb * 8 + q) * pitch + jb * 8) = out[q];
  }
}

}  // namespace

template <int P, int N>
__global__ __launch_bounds__(256) void chunk_state_bf16_kernel(const uint16_t* __restrict__ X,
                                                               const uint16_t* __restrict__ B,
                                                               const int4* __restrict__ table,
                                                               const float* __restrict__ cs,
                                                               float* __restrict__ states, int H,
                                                               int G, int Q) {
  const long unit = blockIdx.x;
  const int h = (int)(unit % H);
  const long slot = unit / H;
  const SlotRec rec = load_slot(table, slot);
  if (rec.len <= 0) return;
  const int g = h / (H / G);

  constexpr int TP = P / 16, TN = N / 16;
  constexpr int WN = TN < 4 ? TN : 4;
  constexpr int WP = (4 / WN) < TP ? (4 / WN) : TP;
  constexpr int TPW = TP / WP, TNW = TN / WN;

  const int qb = Q < kSubTokens ? Q : kSubTokens;
  const int pitch = qb + 8;
  extern __shared__ uint16_t lds[];
  uint16_t* xt = lds;                  // [P][pitch]: X^T scaled by the decay to the chunk end
  uint16_t* bt = lds + P * pitch;      // [N][pitch]: B^T
  float* wsc = reinterpret_cast<float*>(bt + N * pitch);  // [qb] decay weights

  const float* csr = cs + (slot * H + h) * (long)Q;
  const float cs_last = csr[Q - 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wn = wave % WN, wp = wave / WN;
  const bool active = wp < WP;

  f32x4 acc[TPW][TNW];
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int b = 0; b < TNW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j0 = 0; j0 < rec.len; j0 += qb) {
    const int nb = min(qb, rec.len - j0);
    for (int j = tid; j < nb; j += 256) wsc[j] = fast_exp2(cs_last - csr[j0 + j]);
    __syncthreads();
    const long tok = (long)rec.tok0 + j0;
    stage_transposed<P>(xt, pitch, X + (tok * H + h) * P, (long)H * P, nb, qb, wsc);
    stage_transposed<N>(bt, pitch, B + (tok * G + g) * N, (long)G * N, nb, qb, nullptr);
    __syncthreads();
    if (active) {
      const int nkb = (nb + 31) / 32;
      for (int kb = 0; kb < nkb; ++kb) {
        u32x4 af[TPW], bfr[TNW];
#pragma unroll
        for (int a = 0; a < TPW; ++a)
          af[a] = *reinterpret_cast<const u32x4*>(xt + ((wp * TPW + a) * 16 + l16) * pitch + kb * 32 + 8 * g4);
#pragma unroll
        for (int b = 0; b < TNW; ++b)
          bfr[b] = *reinterpret_cast<const u32x4*>(bt + ((wn * TNW + b) * 16 + l16) * pitch + kb * 32 + 8 * g4);
#pragma unroll
        for (int a = 0; a < TPW; ++a)
#pragma unroll
          for (int b = 0; b < TNW; ++b) acc[a][b] = mfma16x16x32(af[a], bfr[b], acc[a][b]);
      }
    }
    __syncthreads();
  }

  if (!active) return;
  float* out = states + (slot * H + h) * (long)(P * N);
#pragma unroll
  for (int a = 0; a < TPW; ++a)
#pragma unroll
    for (int b = 0; b < TNW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = (wp * TPW + a) * 16 + 4 * g4 + r;
        const int n = (wn * TNW + b) * 16 + l16;
        out[p * N + n] = acc[a][b][r];
      }
}

// ----------------------------------------------------------------------------
// fp32 path (plain FMA, fp32 accumulation): tokens staged 32 at a time in LDS.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_state_f32_kernel(const float* __restrict__ X,
                                                              const float* __restrict__ B,
                                                              const int4* __restrict__ table,
                                                              const float* __restrict__ cs,
                                                              float* __restrict__ states, int H, int G,
                                                              int P, int N, int Q) {
  const long unit = blockIdx.x;
  const int h = (int)(unit % H);
  const long slot = unit / H;
  const SlotRec rec = load_slot(table, slot);
  if (rec.len <= 0) return;
  const int g = h / (H / G);
  constexpr int JB = 32;
  extern __shared__ float sm[];
  float* xs = sm;            // [JB][P], scaled by the decay to the chunk end
  float* bs = sm + JB * P;   // [JB][N]
  const float* csr = cs + (slot * H + h) * (long)Q;
  const float cs_last = csr[Q - 1];
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
        xs[idx] = j < nb ? X[((tok + j) * H + h) * P + p] * fast_exp2(cs_last - csr[j0 + j]) : 0.f;
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

template <int P, int N>
static hipError_t launch_state_bf16(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                    hipStream_t stream) {
  const int qb = d.Q < kSubTokens ? d.Q : kSubTokens;
  const size_t lds = (size_t)(P + N) * (qb + 8) * 2 + (size_t)qb * 4;
  auto kern = chunk_state_bf16_kernel<P, N>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(d.nslots * d.H)), dim3(256), lds, stream,
                     reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B), ws.table,
                     ws.cs, ws.chunk_states, d.H, d.G, d.Q);
  return hipGetLastError();
}

template <int P>
static hipError_t dispatch_state_n(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                   hipStream_t stream) {
  switch (d.N) {
    case 32: return launch_state_bf16<P, 32>(d, X, B, ws, stream);
    case 64: return launch_state_bf16<P, 64>(d, X, B, ws, stream);
    case 128: return launch_state_bf16<P, 128>(d, X, B, ws, stream);
    case 256: return launch_state_bf16<P, 256>(d, X, B, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_state(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                              hipStream_t stream) {
  if (!d.bf16) {
    const size_t lds = (size_t)32 * (d.P + d.N) * 4;
    hipLaunchKernelGGL(chunk_state_f32_kernel, dim3((unsigned)(d.nslots * d.H)), dim3(256), lds, stream,
                       reinterpret_cast<const float*>(X), reinterpret_cast<const float*>(B), ws.table, ws.cs,
                       ws.chunk_states, d.H, d.G, d.P, d.N, d.Q);
    return hipGetLastError();
  }
  switch (d.P) {
    case 16: return dispatch_state_n<16>(d, X, B, ws, stream);
    case 32: return dispatch_state_n<32>(d, X, B, ws, stream);
    case 64: return dispatch_state_n<64>(d, X, B, ws, stream);
    case 128: return dispatch_state_n<128>(d, X, B, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
