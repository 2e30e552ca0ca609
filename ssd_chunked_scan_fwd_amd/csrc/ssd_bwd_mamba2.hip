// ssd_bwd_mamba2.hip -- the chain rule of the Mamba-2 block's call around the
// backward pass of the recurrence.
//
// The call computes dt' = softplus(dt + dt_bias), A = -exp(A_log),
// log a = dt' A, v = SSM(a, B, C)(x dt') + D x and y = v silu(z) ("Transformers
// are SSMs" paper card, Method 6 block sketch; Paper vs code items 3, 7, 8).
// For a cotangent dY of y:
//   dz = dY v silu'(z),  silu'(g) = sig(g) (1 + g (1 - sig(g))),  dv = dY silu(z)
//   the recurrence's backward for input x~ = x dt' and cotangent dv gives
//   dx~, d log a, dB, dC and the initial-state gradient;
//   dx = dx~ dt' + D dv,  d dt = (sum_p dx~ x + A d log a) sig(dt + dt_bias),
//   dD = sum dv x,  d dt_bias = sum d dt,  d A_log = A sum dt' d log a.
// m2_prep_kernel forms x~, log a, dv and dz; m2_epilogue_kernel forms dx and
// d dt and per-(token block, head) partial sums; m2_reduce_kernel sums them.
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"
#include "ssd_segsum.h"

namespace ssd {

namespace {

constexpr int kM2Tokens = 64;  // tokens per workgroup of the prep and epilogue kernels

template <bool BF16>
struct Elem {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  // Four consecutive values as fp32.
  static __device__ __forceinline__ f32x4 load4(const T* p) {
    if constexpr (BF16) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      return f32x4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
    } else {
      return *reinterpret_cast<const f32x4*>(p);
    }
  }
  static __device__ __forceinline__ void store4(T* p, f32x4 v) {
    if constexpr (BF16) {
      *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
      *reinterpret_cast<f32x4*>(p) = v;
    }
  }
};

__device__ __forceinline__ float sigmoid_f32(float v) { return __builtin_amdgcn_rcpf(1.f + fast_exp2(-v * kLog2e)); }

// Workgroup (token block, head); P/4 threads per token, 4 channels each.
// Writes log a and x~ = x dt'; with a gate also dv = dY silu(z) and
// dz = dY v silu'(z) (v: the call's output before the gate).
template <bool BF16>
__global__ __launch_bounds__(256) void m2_prep_kernel(const typename Elem<BF16>::T* __restrict__ X,
                                                      const float* __restrict__ dt, const float* __restrict__ dt_bias,
                                                      const float* __restrict__ A_log,
                                                      const typename Elem<BF16>::T* __restrict__ z,
                                                      const typename Elem<BF16>::T* __restrict__ dY,
                                                      const typename Elem<BF16>::T* __restrict__ v,
                                                      float* __restrict__ la, typename Elem<BF16>::T* __restrict__ xs,
                                                      typename Elem<BF16>::T* __restrict__ dv,
                                                      typename Elem<BF16>::T* __restrict__ dz, long tokens, int H,
                                                      int P) {
  using E = Elem<BF16>;
  const int h = blockIdx.y;
  const int tpt = P / 4;                 // threads per token
  const int per = 256 / tpt;             // tokens per pass
  const int q = threadIdx.x % tpt, tl = threadIdx.x / tpt;
  const float A = -expf(A_log[h]);
  const float bias = dt_bias ? dt_bias[h] : 0.f;
  for (int k = tl; k < kM2Tokens; k += per) {
    const long t = (long)blockIdx.x * kM2Tokens + k;
    if (t >= tokens) break;
    const long th = t * H + h;
    const float dtp = softplus_f32(dt[th] + bias);
    if (q == 0) la[th] = dtp * A;
    const long o = th * P + 4 * q;
    const f32x4 x = E::load4(X + o);
    E::store4(xs + o, x * dtp);
    if (z) {
      const f32x4 g = E::load4(z + o), d = E::load4(dY + o), vv = E::load4(v + o);
      f32x4 s, ds;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sg = sigmoid_f32(g[r]);
        s[r] = g[r] * sg;
        ds[r] = sg * (1.f + g[r] * (1.f - sg));
      }
      E::store4(dv + o, d * s);
      E::store4(dz + o, d * vv * ds);
    }
  }
}

// Workgroup (token block, head): dx = dx~ dt' + D dv and d dt per token, and
// the block's sums of dv x, dt' d log a and d dt into part[block][h][3]. dv is
// formed here again in fp32 from dY and z (the rounded copy is the
// recurrence's cotangent only), so the skip term is not rounded twice.
template <bool BF16>
__global__ __launch_bounds__(256) void m2_epilogue_kernel(
    const typename Elem<BF16>::T* __restrict__ X, const float* __restrict__ dt, const float* __restrict__ dt_bias,
    const float* __restrict__ A_log, const float* __restrict__ D, const typename Elem<BF16>::T* __restrict__ dY,
    const typename Elem<BF16>::T* __restrict__ z, const typename Elem<BF16>::T* __restrict__ dxs,
    const float* __restrict__ dla, typename Elem<BF16>::T* __restrict__ dX, float* __restrict__ ddt,
    float* __restrict__ part, long tokens, int H, int P) {
  using E = Elem<BF16>;
  const int h = blockIdx.y;
  const int tpt = P / 4;
  const int per = 256 / tpt;
  const int q = threadIdx.x % tpt, tl = threadIdx.x / tpt;
  const float A = -expf(A_log[h]);
  const float bias = dt_bias ? dt_bias[h] : 0.f;
  const float Dh = D ? D[h] : 0.f;
  float sD = 0.f, sA = 0.f, sB = 0.f;
  for (int k = tl; k < kM2Tokens; k += per) {
    const long t = (long)blockIdx.x * kM2Tokens + k;
    if (t >= tokens) break;
    const long th = t * H + h;
    const float raw = dt[th] + bias;
    const float dtp = softplus_f32(raw);
    const long o = th * P + 4 * q;
    const f32x4 x = E::load4(X + o), g = E::load4(dxs + o);
    f32x4 d = E::load4(dY + o);
    if (z) {
      const f32x4 zz = E::load4(z + o);
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] *= zz[r] * sigmoid_f32(zz[r]);
    }
    E::store4(dX + o, g * dtp + d * Dh);
    float r = g[0] * x[0] + g[1] * x[1] + g[2] * x[2] + g[3] * x[3];
    sD += d[0] * x[0] + d[1] * x[1] + d[2] * x[2] + d[3] * x[3];
    for (int off = 1; off < tpt; off <<= 1) r += __shfl_xor(r, off);  // the token's P/4 lanes
    if (q == 0) {
      const float l = dla[th];
      const float g_dt = (r + A * l) * sigmoid_f32(raw);
      ddt[th] = g_dt;
      sA += dtp * l;
      sB += g_dt;
    }
  }
  __shared__ float red[3][256];
  red[0][threadIdx.x] = sD;
  red[1][threadIdx.x] = sA;
  red[2][threadIdx.x] = sB;
  __syncthreads();
  for (int n = 128; n > 0; n >>= 1) {
    if ((int)threadIdx.x < n)
#pragma unroll
      for (int j = 0; j < 3; ++j) red[j][threadIdx.x] += red[j][threadIdx.x + n];
    __syncthreads();
  }
  if (threadIdx.x < 3) part[((long)blockIdx.x * H + h) * 3 + threadIdx.x] = red[threadIdx.x][0];
}

// One workgroup per head: dD, dA_log = A sum dt' d log a, d dt_bias from the
// token blocks' partial sums.
__global__ __launch_bounds__(256) void m2_reduce_kernel(const float* __restrict__ part, const float* __restrict__ A_log,
                                                        float* __restrict__ dD, float* __restrict__ dA_log,
                                                        float* __restrict__ ddt_bias, int nblk, int H) {
  const int h = blockIdx.x;
  float s[3] = {0.f, 0.f, 0.f};
  for (int b = threadIdx.x; b < nblk; b += 256)
#pragma unroll
    for (int j = 0; j < 3; ++j) s[j] += part[((long)b * H + h) * 3 + j];
  __shared__ float red[3][256];
#pragma unroll
  for (int j = 0; j < 3; ++j) red[j][threadIdx.x] = s[j];
  __syncthreads();
  for (int n = 128; n > 0; n >>= 1) {
    if ((int)threadIdx.x < n)
#pragma unroll
      for (int j = 0; j < 3; ++j) red[j][threadIdx.x] += red[j][threadIdx.x + n];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (dD) dD[h] = red[0][0];
    dA_log[h] = -expf(A_log[h]) * red[1][0];
    if (ddt_bias) ddt_bias[h] = red[2][0];
  }
}

}  // namespace

long m2_token_blocks(long tokens) { return (tokens + kM2Tokens - 1) / kM2Tokens; }

hipError_t launch_m2_prep(const M2BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)m2_token_blocks(a.tokens), (unsigned)a.H);
  if (a.bf16) {
    using T = uint16_t;
    hipLaunchKernelGGL(m2_prep_kernel<true>, grid, dim3(256), 0, stream, static_cast<const T*>(a.X), a.dt, a.dt_bias,
                       a.A_log, static_cast<const T*>(a.z), static_cast<const T*>(a.dY), static_cast<const T*>(a.v),
                       a.la, static_cast<T*>(a.xs), static_cast<T*>(a.dv), static_cast<T*>(a.dz), a.tokens, a.H, a.P);
  } else {
    using T = float;
    hipLaunchKernelGGL(m2_prep_kernel<false>, grid, dim3(256), 0, stream, static_cast<const T*>(a.X), a.dt,
                       a.dt_bias, a.A_log, static_cast<const T*>(a.z), static_cast<const T*>(a.dY),
                       static_cast<const T*>(a.v), a.la, static_cast<T*>(a.xs), static_cast<T*>(a.dv),
                       static_cast<T*>(a.dz), a.tokens, a.H, a.P);
  }
  return hipGetLastError();
}

hipError_t launch_m2_epilogue(const M2BwdArgs& a, hipStream_t stream) {
  const long nblk = m2_token_blocks(a.tokens);
  const dim3 grid((unsigned)nblk, (unsigned)a.H);
  if (a.bf16) {
    using T = uint16_t;
    hipLaunchKernelGGL(m2_epilogue_kernel<true>, grid, dim3(256), 0, stream, static_cast<const T*>(a.X), a.dt,
                       a.dt_bias, a.A_log, a.D, static_cast<const T*>(a.dY), static_cast<const T*>(a.z),
                       static_cast<const T*>(a.dxs), a.dla, static_cast<T*>(a.dXo), a.ddt, a.part, a.tokens, a.H,
                       a.P);
  } else {
    using T = float;
    hipLaunchKernelGGL(m2_epilogue_kernel<false>, grid, dim3(256), 0, stream, static_cast<const T*>(a.X), a.dt,
                       a.dt_bias, a.A_log, a.D, static_cast<const T*>(a.dY), static_cast<const T*>(a.z),
                       static_cast<const T*>(a.dxs), a.dla, static_cast<T*>(a.dXo), a.ddt, a.part, a.tokens, a.H,
                       a.P);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(m2_reduce_kernel, dim3((unsigned)a.H), dim3(256), 0, stream, a.part, a.A_log, a.dD, a.dA_log,
                     a.ddt_bias, (int)nblk, a.H);
  return hipGetLastError();
}

}  // namespace ssd
