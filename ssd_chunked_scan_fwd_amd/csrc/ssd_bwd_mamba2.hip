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

constexpr int kM2Threads = 256;
constexpr int kM2Tokens = 16;  // tokens per workgroup of the prep and epilogue kernels

// Thread layout of the prep and epilogue kernels: each thread takes 8
// consecutive channels of one (token, head); the P/8 threads of a (token,
// head) are consecutive lanes, and a workgroup covers `hg` consecutive heads
// of `tpr` tokens per round. The token rows [H][P] are contiguous in memory,
// so every wave reads and writes one contiguous run of 16-byte pieces.
struct M2Map {
  int tpt, hg, tph, tpr;  // threads per (token, head), heads per workgroup, threads per token, tokens per round
};

__host__ __device__ inline M2Map m2_map(int H, int P) {
  M2Map m;
  m.tpt = P / 8;
  m.hg = H < kM2Threads / m.tpt ? H : kM2Threads / m.tpt;
  m.tph = m.hg * m.tpt;
  m.tpr = kM2Threads / m.tph;
  return m;
}

template <bool BF16>
struct Elem {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int kWords = BF16 ? 1 : 2;  // 16-byte pieces per eight values
  // Eight consecutive values, as loaded (zeros past the buffer range).
  struct Raw {
    u32x4 w[kWords];
  };
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off) {
    Raw v;
#pragma unroll
    for (int i = 0; i < kWords; ++i) v.w[i] = buf_load16(r, off == kOffNone ? kOffNone : off + 16 * i);
    return v;
  }
  static __device__ __forceinline__ void to_f32(const Raw& w, f32x4 v[2]) {
    if constexpr (BF16) {
      const u32x4 a = w.w[0];
      v[0] = f32x4{bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y)};
      v[1] = f32x4{bf16_lo(a.z), bf16_hi(a.z), bf16_lo(a.w), bf16_hi(a.w)};
    } else {
      v[0] = __builtin_bit_cast(f32x4, w.w[0]);
      v[1] = __builtin_bit_cast(f32x4, w.w[1]);
    }
  }
  // Stores at offsets past the range (kOffNone included) are dropped.
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, f32x4 a, f32x4 b) {
    if constexpr (BF16) {
      buf_store16(u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])},
                  r, off);
    } else {
      buf_store16(__builtin_bit_cast(u32x4, a), r, off);
      buf_store16(__builtin_bit_cast(u32x4, b), r, off == kOffNone ? kOffNone : off + 16);
    }
  }
};

// Token rows of one thread whose loads are issued together: the loop over a
// workgroup's rows runs in steps of kM2Rows rows, every load of a step before
// any use, so that each thread keeps kM2Rows x (streams) 16-byte loads in
// flight. Rows past the input's end read zeros through the buffer ranges.
constexpr int kM2Rows = 4;

// Buffer range of a workgroup's token rows of a [tokens][H][P] tensor (an
// empty range for an absent tensor).
template <typename T>
__device__ __forceinline__ rsrc_t rows_rsrc(const T* base, long t0, int ntok, int H, int P) {
  if (!base) return make_rsrc(nullptr, 0u);
  return make_rsrc(base + t0 * H * P, (uint32_t)((long)ntok * H * P * sizeof(T)));
}

__device__ __forceinline__ float sigmoid_f32(float v) { return __builtin_amdgcn_rcpf(1.f + fast_exp2(-v * kLog2e)); }

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of n consecutive lanes, n in {2, 4, 8, 16}; every
// lane of a group receives the group's sum (DPP within rows of 16 lanes).
__device__ __forceinline__ float group_sum(float v, int n) {
  v = dpp_add<0xB1>(v);                // quad_perm [1, 0, 3, 2]
  if (n > 2) v = dpp_add<0x4E>(v);     // quad_perm [2, 3, 0, 1]
  if (n > 4) v = dpp_add<0x141>(v);    // row_half_mirror
  if (n > 8) v = dpp_add<0x140>(v);    // row_mirror
  return v;
}

__device__ __forceinline__ float dot8(const f32x4 a[2], const f32x4 b[2]) {
  return a[0][0] * b[0][0] + a[0][1] * b[0][1] + a[0][2] * b[0][2] + a[0][3] * b[0][3] + a[1][0] * b[1][0] +
         a[1][1] * b[1][1] + a[1][2] * b[1][2] + a[1][3] * b[1][3];
}

// Workgroup (token block, head group). Writes log a and x~ = x dt'; with a
// gate also dv = dY silu(z) and dz = dY v silu'(z) (v: the call's output
// before the gate).
template <bool BF16>
__global__ __launch_bounds__(kM2Threads) void m2_prep_kernel(const typename Elem<BF16>::T* __restrict__ X,
                                                             const float* __restrict__ dt,
                                                             const float* __restrict__ dt_bias,
                                                             const float* __restrict__ A_log,
                                                             const typename Elem<BF16>::T* __restrict__ z,
                                                             const typename Elem<BF16>::T* __restrict__ dY,
                                                             const typename Elem<BF16>::T* __restrict__ v,
                                                             float* __restrict__ la,
                                                             typename Elem<BF16>::T* __restrict__ xs,
                                                             typename Elem<BF16>::T* __restrict__ dv,
                                                             typename Elem<BF16>::T* __restrict__ dz, long tokens,
                                                             int H, int P) {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Raw = typename E::Raw;
  const M2Map mp = m2_map(H, P);
  const int tid = threadIdx.x;
  const int r = tid / mp.tph, q = tid % mp.tpt;
  const int h = blockIdx.y * mp.hg + (tid % mp.tph) / mp.tpt;
  if (r >= mp.tpr || h >= H) return;  // no barrier below
  const float A = -expf(A_log[h]);
  const float bias = dt_bias ? dt_bias[h] : 0.f;
  const long t0 = (long)blockIdx.x * kM2Tokens;
  const int ntok = (int)(tokens - t0 < kM2Tokens ? tokens - t0 : kM2Tokens);
  const rsrc_t rx = rows_rsrc(X, t0, ntok, H, P), rxs = rows_rsrc<T>(xs, t0, ntok, H, P);
  const rsrc_t rz = rows_rsrc(z, t0, ntok, H, P), rd = rows_rsrc(dY, t0, ntok, H, P);
  const rsrc_t rv = rows_rsrc(v, t0, ntok, H, P);
  const rsrc_t rdv = rows_rsrc<T>(dv, t0, ntok, H, P), rdz = rows_rsrc<T>(dz, t0, ntok, H, P);
  const rsrc_t rdt = rows_rsrc(dt, t0, ntok, H, 1);
  for (int k0 = r; k0 < kM2Tokens; k0 += kM2Rows * mp.tpr) {
    uint32_t off[kM2Rows];
    float dtr[kM2Rows];
    Raw xr[kM2Rows], gr[kM2Rows], dr[kM2Rows], vr[kM2Rows];
#pragma unroll
    for (int j = 0; j < kM2Rows; ++j) {
      const int k = k0 + j * mp.tpr;
      const bool in = k < ntok;
      off[j] = in ? (uint32_t)(((k * H + h) * P + 8 * q) * sizeof(T)) : kOffNone;
      dtr[j] = buf_load_f32(rdt, in ? (uint32_t)((k * H + h) * 4) : kOffNone);
      xr[j] = E::load(rx, off[j]);
      if (z) {
        gr[j] = E::load(rz, off[j]);
        dr[j] = E::load(rd, off[j]);
        vr[j] = E::load(rv, off[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kM2Rows; ++j) {
      const int k = k0 + j * mp.tpr;
      const float dtp = softplus_f32(dtr[j] + bias);
      if (q == 0 && k < ntok) la[(t0 + k) * H + h] = dtp * A;
      f32x4 x[2];
      E::to_f32(xr[j], x);
      E::store(rxs, off[j], x[0] * dtp, x[1] * dtp);
      if (z) {
        f32x4 g[2], d[2], vv[2], sw[2], ds[2];
        E::to_f32(gr[j], g);
        E::to_f32(dr[j], d);
        E::to_f32(vr[j], vv);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float sg = sigmoid_f32(g[i][c]);
            sw[i][c] = g[i][c] * sg;
            ds[i][c] = sg * (1.f + g[i][c] * (1.f - sg));
          }
        E::store(rdv, off[j], d[0] * sw[0], d[1] * sw[1]);
        E::store(rdz, off[j], d[0] * vv[0] * ds[0], d[1] * vv[1] * ds[1]);
      }
    }
  }
}

// Workgroup (token block, head group): dx = dx~ dt' + D dv and d dt per
// token, and the block's sums of dv x, dt' d log a and d dt per head into
// part[block][h][3]. dv is formed here again in fp32 from dY and z (the
// rounded copy is the recurrence's cotangent only), so the skip term is not
// rounded twice.
template <bool BF16>
__global__ __launch_bounds__(kM2Threads) void m2_epilogue_kernel(
    const typename Elem<BF16>::T* __restrict__ X, const float* __restrict__ dt, const float* __restrict__ dt_bias,
    const float* __restrict__ A_log, const float* __restrict__ D, const typename Elem<BF16>::T* __restrict__ dY,
    const typename Elem<BF16>::T* __restrict__ z, const typename Elem<BF16>::T* __restrict__ dxs,
    const float* __restrict__ dla, typename Elem<BF16>::T* __restrict__ dX, float* __restrict__ ddt,
    float* __restrict__ part, long tokens, int H, int P) {
  using E = Elem<BF16>;
  using T = typename E::T;
  using Raw = typename E::Raw;
  const M2Map mp = m2_map(H, P);
  const int tid = threadIdx.x;
  const int r = tid / mp.tph, hl = (tid % mp.tph) / mp.tpt, q = tid % mp.tpt;
  const int h = blockIdx.y * mp.hg + hl;
  const bool act = r < mp.tpr && h < H;  // whole (token, head) lane groups
  float sD = 0.f, sA = 0.f, sB = 0.f;
  if (act) {
    const float A = -expf(A_log[h]);
    const float bias = dt_bias ? dt_bias[h] : 0.f;
    const float Dh = D ? D[h] : 0.f;
    const long t0 = (long)blockIdx.x * kM2Tokens;
    const int ntok = (int)(tokens - t0 < kM2Tokens ? tokens - t0 : kM2Tokens);
    const rsrc_t rx = rows_rsrc(X, t0, ntok, H, P), rg = rows_rsrc(dxs, t0, ntok, H, P);
    const rsrc_t rd = rows_rsrc(dY, t0, ntok, H, P), rz = rows_rsrc(z, t0, ntok, H, P);
    const rsrc_t rdx = rows_rsrc<T>(dX, t0, ntok, H, P);
    const rsrc_t rdt = rows_rsrc(dt, t0, ntok, H, 1), rla = rows_rsrc(dla, t0, ntok, H, 1);
    for (int k0 = r; k0 < kM2Tokens; k0 += kM2Rows * mp.tpr) {
      uint32_t off[kM2Rows];
      float dtr[kM2Rows], lr[kM2Rows];
      Raw xr[kM2Rows], gr[kM2Rows], dr[kM2Rows], zr[kM2Rows];
#pragma unroll
      for (int j = 0; j < kM2Rows; ++j) {
        const int k = k0 + j * mp.tpr;
        const bool in = k < ntok;
        const uint32_t th4 = in ? (uint32_t)((k * H + h) * 4) : kOffNone;
        off[j] = in ? (uint32_t)(((k * H + h) * P + 8 * q) * sizeof(T)) : kOffNone;
        dtr[j] = buf_load_f32(rdt, th4);
        lr[j] = buf_load_f32(rla, th4);
        xr[j] = E::load(rx, off[j]);
        gr[j] = E::load(rg, off[j]);
        dr[j] = E::load(rd, off[j]);
        if (z) zr[j] = E::load(rz, off[j]);
      }
#pragma unroll
      for (int j = 0; j < kM2Rows; ++j) {
        const int k = k0 + j * mp.tpr;
        const float raw = dtr[j] + bias;
        const float dtp = softplus_f32(raw);
        f32x4 x[2], g[2], d[2];
        E::to_f32(xr[j], x);
        E::to_f32(gr[j], g);
        E::to_f32(dr[j], d);
        if (z) {
          f32x4 zz[2];
          E::to_f32(zr[j], zz);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) d[i][c] *= zz[i][c] * sigmoid_f32(zz[i][c]);
        }
        E::store(rdx, off[j], g[0] * dtp + d[0] * Dh, g[1] * dtp + d[1] * Dh);
        float rr = dot8(g, x);
        sD += dot8(d, x);     // zero for rows past the end
        rr = group_sum(rr, mp.tpt);  // over the (token, head)'s lanes
        if (q == 0 && k < ntok) {
          const float l = lr[j];
          const float g_dt = (rr + A * l) * sigmoid_f32(raw);
          ddt[(t0 + k) * H + h] = g_dt;
          sA += dtp * l;
          sB += g_dt;
        }
      }
    }
  }
  sD = group_sum(sD, mp.tpt);
  // Per head: the token rows' sums through LDS, in a fixed order.
  __shared__ float red[kM2Threads / 2][3];
  if (act && q == 0) {
    const int e = r * mp.hg + hl;
    red[e][0] = sD;
    red[e][1] = sA;
    red[e][2] = sB;
  }
  __syncthreads();
  const int hh = blockIdx.y * mp.hg + tid;
  if (tid < mp.hg && hh < H) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f;
    for (int rr = 0; rr < mp.tpr; ++rr) {
      s0 += red[rr * mp.hg + tid][0];
      s1 += red[rr * mp.hg + tid][1];
      s2 += red[rr * mp.hg + tid][2];
    }
    float* out = part + ((long)blockIdx.x * H + hh) * 3;
    out[0] = s0;
    out[1] = s1;
    out[2] = s2;
  }
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

static dim3 m2_grid(const M2BwdArgs& a) {
  const M2Map mp = m2_map(a.H, a.P);
  return dim3((unsigned)m2_token_blocks(a.tokens), (unsigned)((a.H + mp.hg - 1) / mp.hg));
}

hipError_t launch_m2_prep(const M2BwdArgs& a, hipStream_t stream) {
  const dim3 grid = m2_grid(a);
  if (a.bf16) {
    using T = uint16_t;
    hipLaunchKernelGGL(m2_prep_kernel<true>, grid, dim3(kM2Threads), 0, stream, static_cast<const T*>(a.X), a.dt, a.dt_bias,
                       a.A_log, static_cast<const T*>(a.z), static_cast<const T*>(a.dY), static_cast<const T*>(a.v),
                       a.la, static_cast<T*>(a.xs), static_cast<T*>(a.dv), static_cast<T*>(a.dz), a.tokens, a.H, a.P);
  } else {
    using T = float;
    hipLaunchKernelGGL(m2_prep_kernel<false>, grid, dim3(kM2Threads), 0, stream, static_cast<const T*>(a.X), a.dt,
                       a.dt_bias, a.A_log, static_cast<const T*>(a.z), static_cast<const T*>(a.dY),
                       static_cast<const T*>(a.v), a.la, static_cast<T*>(a.xs), static_cast<T*>(a.dv),
                       static_cast<T*>(a.dz), a.tokens, a.H, a.P);
  }
  return hipGetLastError();
}

hipError_t launch_m2_epilogue(const M2BwdArgs& a, hipStream_t stream) {
  const long nblk = m2_token_blocks(a.tokens);
  const dim3 grid = m2_grid(a);
  if (a.bf16) {
    using T = uint16_t;
    hipLaunchKernelGGL(m2_epilogue_kernel<true>, grid, dim3(kM2Threads), 0, stream, static_cast<const T*>(a.X), a.dt,
                       a.dt_bias, a.A_log, a.D, static_cast<const T*>(a.dY), static_cast<const T*>(a.z),
                       static_cast<const T*>(a.dxs), a.dla, static_cast<T*>(a.dXo), a.ddt, a.part, a.tokens, a.H,
                       a.P);
  } else {
    using T = float;
    hipLaunchKernelGGL(m2_epilogue_kernel<false>, grid, dim3(kM2Threads), 0, stream, static_cast<const T*>(a.X), a.dt,
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
