// ssd_passing.h -- the centre-factor recurrence of one (sequence, head) and
// four consecutive state elements, shared by the state-passing stage and the
// chunk-state kernel that runs it after a grid-wide barrier.
//
// h = h0 (the sequence's initial state, or 0); for each state block m of the
// sequence: start_m = h; h = exp2(total_m) h + s_m ("Transformers are SSMs"
// paper card, Method 5 / paper section 6, "Centre Factors": the recurrence over
// chunk states, here over state blocks). The final h is the sequence's final
// state. Sequence s: packed rows own block slots floor(cu[s]/(Gs*Q)) + s ..;
// unpacked row s owns s*blocks_per_row ...
#pragma once

#include "ssd_device.h"

namespace ssd {

constexpr int kPassElems = 4;   // (p, n) elements per thread

template <bool OUT_BF16>
__device__ __forceinline__ void pass_states(const float* __restrict__ states, const float* __restrict__ bdecay,
                                            void* __restrict__ start, float* __restrict__ final_state,
                                            const float* __restrict__ init, const int32_t* __restrict__ cu,
                                            long blocks_per_row, int H, int PN, int span, int s, int h, int e) {
  long base;
  int nblk;
  if (cu) {
    const int b = cu[s], en = cu[s + 1];
    base = b / span + s;
    nblk = (en - b + span - 1) / span;
  } else {
    base = (long)s * blocks_per_row;
    nblk = (int)blocks_per_row;
  }
  f32x4 hc = {0.f, 0.f, 0.f, 0.f};
  if (init) hc = *reinterpret_cast<const f32x4*>(init + ((long)s * H + h) * PN + e);
  auto put = [&](long blk, f32x4 v) {
    const long off = (blk * H + h) * (long)PN + e;
    if (OUT_BF16) {
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(start) + off) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(start) + off) = v;
    }
  };
  constexpr int U = 16;  // blocks whose loads are in flight together
  int k = 0;
  for (; k + U <= nblk; k += U) {
    f32x4 sv[U];
    float dv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long blk = base + k + u;
      sv[u] = *reinterpret_cast<const f32x4*>(states + (blk * H + h) * (long)PN + e);
      dv[u] = bdecay[blk * H + h];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      put(base + k + u, hc);
      const float a = fast_exp2(dv[u]);
      hc = a * hc + sv[u];
    }
  }
  for (; k < nblk; ++k) {
    const long blk = base + k;
    const f32x4 sv = *reinterpret_cast<const f32x4*>(states + (blk * H + h) * (long)PN + e);
    const float a = fast_exp2(bdecay[blk * H + h]);
    put(blk, hc);
    hc = a * hc + sv;
  }
  if (final_state) *reinterpret_cast<f32x4*>(final_state + ((long)s * H + h) * PN + e) = hc;
}

}  // namespace ssd
