// ssd_api.cpp -- the C ABI declared in include/ssd.h.
//
// Every entry point validates its arguments on the host first (no HIP call
// before validation succeeds), carves the caller's workspace, and enqueues the
// stage kernels on the caller's stream. Nothing is allocated, nothing is
// synchronised, and no C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include <atomic>
#include <mutex>

#include "ssd.h"
#include "ssd_launch.h"

namespace {

constexpr int64_t kMaxElems = INT32_MAX;  // every tensor holds fewer than 2^31 elements

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

enum Stage { kCumsum = 1, kState = 2, kPassing = 4, kScan = 8, kAll = 15 };

// Shape, dtype and size checks shared by every forward entry point.
ssd_status check_shape(const ssd_shape* s, const int32_t* cu, int32_t chunk) {
  if (!s) return SSD_ERR_INVALID_ARGUMENT;
  if (s->batch < 1 || s->seqlen < 1 || s->nheads < 1 || s->ngroups < 1 || s->headdim < 1 || s->dstate < 1)
    return SSD_ERR_INVALID_ARGUMENT;
  if (s->nheads % s->ngroups) return SSD_ERR_INVALID_ARGUMENT;
  if (chunk < 1) return SSD_ERR_INVALID_ARGUMENT;
  if (s->batch > 65535) return SSD_ERR_UNSUPPORTED;
  if (cu) {
    if (s->batch != 1 || s->num_seqs < 1 || s->num_seqs > s->seqlen) return SSD_ERR_INVALID_ARGUMENT;
  } else if (s->num_seqs != 0) {
    return SSD_ERR_INVALID_ARGUMENT;
  }
  if (s->dtype != SSD_DTYPE_F32 && s->dtype != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
  if (!pow2_in(s->headdim, 16, 128) || !pow2_in(s->dstate, 16, 256) || !pow2_in(chunk, 16, 256))
    return SSD_ERR_UNSUPPORTED;
  if (s->dtype == SSD_DTYPE_BF16) {
    if (chunk < 32 || s->dstate < 32) return SSD_ERR_UNSUPPORTED;
    if (ssd::chunk_scan_bf16_lds_bytes(s->headdim, s->dstate, chunk) > ssd::kMaxLdsBytes ||
        ssd::chunk_state_bf16_lds_bytes(s->headdim, s->dstate, 16 * 256) > ssd::kMaxLdsBytes)
      return SSD_ERR_UNSUPPORTED;
    // one chunk's rows of X, Y, B or C are addressed as one buffer range of fewer than 2^31 bytes
    if ((int64_t)chunk * s->nheads * s->headdim * 2 > kMaxElems || (int64_t)chunk * s->ngroups * s->dstate * 2 > kMaxElems)
      return SSD_ERR_UNSUPPORTED;
  }
  const int64_t bt = (int64_t)s->batch * s->seqlen;
  if (bt * s->nheads * s->headdim > kMaxElems || bt * s->ngroups * s->dstate > kMaxElems)
    return SSD_ERR_UNSUPPORTED;
  // the cumsum stage holds one chunk of log_a, [chunk][nheads + 1] fp32, in LDS
  if ((int64_t)chunk * (s->nheads + 1) * 4 > (int64_t)ssd::kMaxLdsBytes) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

int32_t default_state_block(const ssd_shape* s, const int32_t* cu, int32_t chunk) {
  if (s->dtype != SSD_DTYPE_BF16) return 1;
  // Longer state blocks cut the right-factor and state traffic and the
  // chunk-state stage's per-block set-up; keep at least 384 (state block,
  // head) workgroups, about one and a half per CU (256 CUs). States of 64 KB
  // (headdim * dstate >= 16384) double that traffic, so they take blocks of up
  // to 16 chunks, the others up to 8. Measured forward calls (us) by block size
  // 2 / 4 / 8 / 16: b 2, T 2048, H 24, N 64, chunk 64: 35.9 / 32.6 / 40.6 / 66.0;
  // T 16384, H 32, N 128: 101.8 / 83.9 / 79.5 / 119.6; b 8, T 4096, H 32, N 256:
  // 440.7 / 349.5 / 288.9 / 260.3; packed T 32768, H 80: 595.7 / 473.5 / 425.5 / 464.3.
  const int64_t T = s->seqlen;
  const int64_t chunks = cu ? (T / chunk + s->num_seqs) : (int64_t)s->batch * ((T + chunk - 1) / chunk);
  const int64_t units = chunks * s->nheads;
  const int32_t cap = (int64_t)s->headdim * s->dstate >= 16384 ? 16 : 8;
  int32_t gs = 1;
  while (gs < cap && units / (2 * gs) >= 384) gs *= 2;
  return gs;
}

ssd_status check_state_block(const ssd_shape* s, int32_t state_block) {
  if (!pow2_in(state_block, 1, 16)) return SSD_ERR_UNSUPPORTED;
  if (s->dtype != SSD_DTYPE_BF16 && state_block != 1) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

ssd_status make_layout(const ssd_shape* s, const int32_t* cu, int32_t chunk, int32_t gs, ssd_layout* out) {
  ssd_layout L{};
  const int64_t T = s->seqlen;
  const int64_t span = (int64_t)chunk * gs;
  L.slots_per_row = cu ? (T / chunk + s->num_seqs) : ((T + chunk - 1) / chunk);
  L.nslots = (int64_t)s->batch * L.slots_per_row;
  L.blocks_per_row = cu ? (T / span + s->num_seqs) : ((L.slots_per_row + gs - 1) / gs);
  L.nblocks = (int64_t)s->batch * L.blocks_per_row;
  const int64_t H = s->nheads, PN = (int64_t)s->headdim * s->dstate;
  if (L.nblocks * H * PN > kMaxElems || L.nslots * H * chunk > kMaxElems) return SSD_ERR_UNSUPPORTED;
  const int64_t nseq = cu ? s->num_seqs : s->batch;
  if (nseq * H * PN > kMaxElems) return SSD_ERR_UNSUPPORTED;
  if (L.slots_per_row > INT32_MAX / 2 || L.nblocks * H > INT32_MAX) return SSD_ERR_UNSUPPORTED;
  const size_t esz = s->dtype == SSD_DTYPE_BF16 ? 2 : 4;
  size_t off = 0;
  L.table_offset = off;
  off = align256(off + (size_t)L.nslots * 16);
  L.block_table_offset = off;
  off = align256(off + (size_t)L.nblocks * 16);
  L.cumsum_offset = off;
  off = align256(off + (size_t)L.nslots * H * chunk * 4);
  L.key_cumsum_offset = off;
  off = align256(off + (size_t)L.nslots * H * chunk * 4);
  L.block_decay_offset = off;
  off = align256(off + (size_t)L.nblocks * H * 4);
  L.block_states_offset = off;
  off = align256(off + (size_t)L.nblocks * H * PN * 4);
  L.start_states_offset = off;
  off = align256(off + (size_t)L.nblocks * H * PN * esz);
  L.total_bytes = off;
  *out = L;
  return SSD_OK;
}

struct Prepared {
  ssd::FwdDims d;
  ssd::Workspace ws;
};

// Full validation of a forward-stage call; fills `pp` on success.
// `mamba2`: the key-side exponent gets its own workspace array (written by
// the discretising cumsum stage); plain calls read cs in its place.
ssd_status prepare(int stages, const void* X, const float* log_a, const void* B, const void* C,
                   const void* Y, const int32_t* cu, int32_t chunk, int32_t gs, const ssd_shape* s,
                   void* workspace, size_t workspace_bytes, Prepared* pp, bool mamba2 = false,
                   const float* initial_state = nullptr, const float* final_state = nullptr) {
  ssd_status st = check_shape(s, cu, chunk);
  if (st != SSD_OK) return st;
  if (gs <= 0) gs = default_state_block(s, cu, chunk);
  st = check_state_block(s, gs);
  if (st != SSD_OK) return st;
  if ((stages & kCumsum) && !log_a) return SSD_ERR_INVALID_ARGUMENT;
  if ((stages & (kState | kScan)) && (!X || !B)) return SSD_ERR_INVALID_ARGUMENT;
  if ((stages & kScan) && (!C || !Y)) return SSD_ERR_INVALID_ARGUMENT;
  // the state-passing stage moves states in 16-byte pieces
  if (((uintptr_t)initial_state | (uintptr_t)final_state) & 15) return SSD_ERR_INVALID_ARGUMENT;
  ssd_layout L;
  st = make_layout(s, cu, chunk, gs, &L);
  if (st != SSD_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255)) return SSD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.total_bytes) return SSD_ERR_WORKSPACE_TOO_SMALL;
  char* base = static_cast<char*>(workspace);
  pp->d = ssd::FwdDims{s->batch, s->seqlen, s->nheads, s->ngroups, s->headdim, s->dstate, chunk, gs,
                       cu ? s->num_seqs : 0, s->dtype == SSD_DTYPE_BF16 ? 1 : 0,
                       (long)L.slots_per_row, (long)L.nslots, (long)L.blocks_per_row, (long)L.nblocks};
  pp->ws = ssd::Workspace{reinterpret_cast<int4*>(base + L.table_offset),
                          reinterpret_cast<int4*>(base + L.block_table_offset),
                          reinterpret_cast<float*>(base + L.cumsum_offset),
                          reinterpret_cast<float*>(base + (mamba2 ? L.key_cumsum_offset : L.cumsum_offset)),
                          reinterpret_cast<float*>(base + L.block_decay_offset),
                          reinterpret_cast<float*>(base + L.block_states_offset),
                          static_cast<void*>(base + L.start_states_offset)};
  return SSD_OK;
}

ssd_status hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

// Whether the state chain may run as one cooperative launch (ssd_set_state_chain; off by
// default: on ROCm 7 the cooperative launch costs more than the launch it saves).
std::atomic<int> g_state_chain{0};

// The state chain: chunk_state (with the segment sums) and state_passing, as
// one cooperative launch when allowed and the grid fits, else two launches.
hipError_t run_state_chain(const Prepared& pp, const void* X, const void* B, const ssd::SegArgs& sa,
                           const int32_t* cu, const float* init, float* final_state, hipStream_t s) {
  bool launched = false;
  hipError_t e = hipSuccess;
  if (g_state_chain.load(std::memory_order_relaxed))
    e = ssd::launch_chunk_state_chain(pp.d, X, B, pp.ws, s, sa, init, final_state, &launched);
  if (e != hipSuccess || launched) return e;
  e = ssd::launch_chunk_state(pp.d, X, B, pp.ws, s, &sa);
  if (e == hipSuccess) e = ssd::launch_state_passing(pp.d, cu, init, final_state, pp.ws, s);
  return e;
}

// One forward pass (the state chain, then chunk_scan) on prepared dimensions and workspace.
hipError_t run_forward(const Prepared& pp, const void* X, const float* log_a, const void* B, const void* C,
                       const int32_t* cu, const float* init, void* Y, float* final_state, hipStream_t s) {
  const ssd::SegArgs sa = ssd::seg_args(pp.d, log_a, cu, ssd::Mamba2Args{});
  hipError_t e = run_state_chain(pp, X, B, sa, cu, init, final_state, s);
  if (e == hipSuccess) e = ssd::launch_chunk_scan(pp.d, X, B, C, Y, pp.ws, s);
  return e;
}

// Backward workspace (offsets 256-aligned): the padded reversed copies, the
// head broadcasts, fp32 per-head partials, and three forward workspaces: the
// reversed run's and the forward chunk-state run's (both one chunk per state
// block, kept for the log-decay gradient) and one shared by the two
// role-exchanged runs.
//
// bf16 shapes that the fused chunk kernel covers need only the reversed dY and
// C, the two state runs and, when a chunk's heads are split over several
// workgroups, fp32 partials of dB and dC per head slice.
struct BwdLayout {
  size_t cur, rev_dy, rev_x, dx_rev, rev_b, rev_c, bcast, part, la_rev, states_t, lam_first;
  size_t part_b, part_c, cstart_f, cstart_r;
  size_t fwd_a, fwd_f, fwd_s, total;
  size_t a_bytes, f_bytes, s_bytes;
  int Tr;          // tokens per row of the padded reversed layout (packed: an upper bound)
  bool fused;      // the fused chunk kernel computes dX, d log a, dB and dC
  int nsl;         // head slices per (chunk, group) in the fused kernel
  int gs;          // state block of the two state runs (fused path; 1 otherwise)
};

// The role-exchanged runs (dB, dC) have headdim N, dstate P and one group per head.
ssd_shape swapped_shape(const ssd_shape* s) {
  ssd_shape w = *s;
  w.ngroups = s->nheads;
  w.headdim = s->dstate;
  w.dstate = s->headdim;
  return w;
}

ssd_status make_bwd_layout(const ssd_shape* s, const int32_t* cu, int32_t chunk, int32_t gs, BwdLayout* out) {
  ssd_status st = check_shape(s, cu, chunk);
  if (st != SSD_OK) return st;
  if (gs <= 0) gs = default_state_block(s, cu, chunk);
  st = check_state_block(s, gs);
  if (st != SSD_OK) return st;
  const int64_t P = s->headdim, N = s->dstate, H = s->nheads, G = s->ngroups;
  const bool fused = ssd::bwd_chunk_supported((int)P, (int)N, chunk, s->dtype == SSD_DTYPE_BF16);
  const ssd_shape w = swapped_shape(s);
  if (!fused) {
    st = check_shape(&w, cu, chunk);  // dstate <= 128 and, for bf16, headdim >= 32
    if (st != SSD_OK) return st;
    if (P + N > 192 || chunk > 256) return SSD_ERR_UNSUPPORTED;  // the log-decay kernel's register rows
    if (ssd::dlog_chunk_lds_bytes((int)P, (int)N, chunk, s->dtype == SSD_DTYPE_BF16 ? 2 : 4) > ssd::kMaxLdsBytes)
      return SSD_ERR_UNSUPPORTED;
  }
  const int64_t T = s->seqlen;
  const int64_t Tr = cu ? T + (int64_t)s->num_seqs * (chunk - 1) : T + (chunk - T % chunk) % chunk;
  if ((int64_t)s->batch * Tr > INT32_MAX / 2) return SSD_ERR_UNSUPPORTED;
  ssd_shape sr = *s;
  sr.seqlen = (int32_t)Tr;
  ssd_shape wr = w;
  wr.seqlen = (int32_t)Tr;
  ssd_layout La, Lf, Ls1{}, Ls2{};
  // The fused path runs the state runs in state blocks and expands the block
  // states to chunk states; the general path runs them one chunk per block.
  const int run_gs = fused ? gs : 1;
  if ((st = check_shape(&sr, cu, chunk)) != SSD_OK) return st;
  if ((st = make_layout(&sr, cu, chunk, run_gs, &La)) != SSD_OK) return st;
  if ((st = make_layout(s, cu, chunk, run_gs, &Lf)) != SSD_OK) return st;
  if (!fused) {
    if ((st = make_layout(&wr, cu, chunk, default_state_block(&wr, cu, chunk), &Ls1)) != SSD_OK) return st;
    if ((st = make_layout(&w, cu, chunk, default_state_block(&w, cu, chunk), &Ls2)) != SSD_OK) return st;
  }
  const size_t esz = s->dtype == SSD_DTYPE_BF16 ? 2 : 4;
  const size_t tok = (size_t)s->batch * T, tokr = (size_t)s->batch * Tr;
  const size_t tmax = tok > tokr ? tok : tokr;
  const size_t nseq = cu ? s->num_seqs : s->batch;
  if ((int64_t)tmax * H * (P > N ? P : N) > kMaxElems) return SSD_ERR_UNSUPPORTED;
  BwdLayout L{};
  L.fused = fused;
  L.gs = run_gs;
  L.nsl = fused ? ssd::bwd_chunk_slices(Lf.nslots, (int)G, (int)H) : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  L.cur = take((nseq + 1) * 4);
  L.rev_dy = take(tokr * H * P * esz);
  L.rev_c = take(tokr * G * N * esz);
  L.la_rev = take(tokr * H * 4);
  L.lam_first = take(nseq * H * P * N * 4);
  if (fused) {
    if (run_gs > 1) {
      L.cstart_f = take((size_t)Lf.nslots * H * P * N * esz);
      L.cstart_r = take((size_t)La.nslots * H * P * N * esz);
    }
    if (L.nsl > 1) {
      if ((int64_t)L.nsl * tok * G * N > kMaxElems) return SSD_ERR_UNSUPPORTED;
      L.part_b = take((size_t)L.nsl * tok * G * N * 4);
      L.part_c = take((size_t)L.nsl * tok * G * N * 4);
    }
  } else {
    L.rev_x = take(tokr * H * P * esz);
    L.dx_rev = take(tokr * H * P * esz);
    L.rev_b = take(tokr * G * N * esz);
    L.bcast = take(tmax * H * N * esz);
    L.part = take(tmax * H * N * 4);
    L.states_t = take(nseq * H * P * N * 4);
  }
  L.a_bytes = La.total_bytes;
  L.f_bytes = Lf.total_bytes;
  L.s_bytes = Ls1.total_bytes > Ls2.total_bytes ? Ls1.total_bytes : Ls2.total_bytes;
  L.fwd_a = take(L.a_bytes);
  L.fwd_f = take(L.f_bytes);
  if (!fused) L.fwd_s = take(L.s_bytes);
  L.total = off;
  L.Tr = (int)Tr;
  *out = L;
  return SSD_OK;
}

// Shape checks of the decode steps.
ssd_status check_step(const ssd_shape* s) {
  if (s->batch < 1 || s->nheads < 1 || s->ngroups < 1 || s->headdim < 1 || s->dstate < 1)
    return SSD_ERR_INVALID_ARGUMENT;
  if (s->nheads % s->ngroups) return SSD_ERR_INVALID_ARGUMENT;
  if (s->dtype != SSD_DTYPE_F32 && s->dtype != SSD_DTYPE_BF16) return SSD_ERR_UNSUPPORTED;
  if (!pow2_in(s->headdim, 16, 128) || !pow2_in(s->dstate, 16, 256)) return SSD_ERR_UNSUPPORTED;
  if (s->batch > 65535 || (int64_t)s->batch * s->nheads * s->headdim * s->dstate > kMaxElems)
    return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}
}  // namespace

extern "C" {

int32_t ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(ssd_status status) {
  switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_INVALID_ARGUMENT: return "SSD_ERR_INVALID_ARGUMENT";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_WORKSPACE_TOO_SMALL: return "SSD_ERR_WORKSPACE_TOO_SMALL";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
  }
  return "SSD_ERR_UNKNOWN";
}

int32_t ssd_default_state_block(const ssd_shape* shape, int32_t chunk) {
  const int32_t dummy = 0;
  const int32_t* cu = (shape && shape->num_seqs > 0) ? &dummy : nullptr;
  if (check_shape(shape, cu, chunk) != SSD_OK) return 1;
  return default_state_block(shape, cu, chunk);
}

ssd_status ssd_fwd_layout(const ssd_shape* shape, int32_t chunk, int32_t state_block, ssd_layout* layout) {
  if (!layout) return SSD_ERR_INVALID_ARGUMENT;
  // The layout depends on whether rows are packed; num_seqs > 0 means packed.
  const int32_t dummy = 0;
  const int32_t* cu = (shape && shape->num_seqs > 0) ? &dummy : nullptr;
  ssd_status st = check_shape(shape, cu, chunk);
  if (st != SSD_OK) return st;
  if (state_block <= 0) state_block = default_state_block(shape, cu, chunk);
  st = check_state_block(shape, state_block);
  if (st != SSD_OK) return st;
  return make_layout(shape, cu, chunk, state_block, layout);
}

ssd_status ssd_fwd_workspace_bytes(const ssd_shape* shape, int32_t chunk, int32_t state_block, size_t* bytes) {
  if (!bytes) return SSD_ERR_INVALID_ARGUMENT;
  ssd_layout L;
  ssd_status st = ssd_fwd_layout(shape, chunk, state_block, &L);
  if (st != SSD_OK) return st;
  *bytes = L.total_bytes;
  return SSD_OK;
}

ssd_status ssd_chunk_cumsum(const float* log_a, const int32_t* cu_seqlens, int32_t chunk, int32_t state_block,
                            const ssd_shape* shape, void* workspace, size_t workspace_bytes, void* stream) {
  Prepared pp;
  ssd_status st = prepare(kCumsum, nullptr, log_a, nullptr, nullptr, nullptr, cu_seqlens, chunk, state_block,
                          shape, workspace, workspace_bytes, &pp);
  if (st != SSD_OK) return st;
  return hip_status(ssd::launch_chunk_cumsum(pp.d, log_a, cu_seqlens, pp.ws, (hipStream_t)stream));
}

ssd_status ssd_chunk_state(const void* X, const void* B, const int32_t* cu_seqlens, int32_t chunk,
                           int32_t state_block, const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Prepared pp;
  ssd_status st = prepare(kState, X, nullptr, B, nullptr, nullptr, cu_seqlens, chunk, state_block, shape,
                          workspace, workspace_bytes, &pp);
  if (st != SSD_OK) return st;
  return hip_status(ssd::launch_chunk_state(pp.d, X, B, pp.ws, (hipStream_t)stream));
}

ssd_status ssd_state_passing(const int32_t* cu_seqlens, const float* initial_state, int32_t chunk,
                             int32_t state_block, float* final_state, const ssd_shape* shape, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Prepared pp;
  ssd_status st = prepare(kPassing, nullptr, nullptr, nullptr, nullptr, nullptr, cu_seqlens, chunk, state_block,
                          shape, workspace, workspace_bytes, &pp, false, initial_state, final_state);
  if (st != SSD_OK) return st;
  return hip_status(
      ssd::launch_state_passing(pp.d, cu_seqlens, initial_state, final_state, pp.ws, (hipStream_t)stream));
}

ssd_status ssd_chunk_scan(const void* X, const void* B, const void* C, const int32_t* cu_seqlens, int32_t chunk,
                          int32_t state_block, void* Y, const ssd_shape* shape, void* workspace,
                          size_t workspace_bytes, void* stream) {
  Prepared pp;
  ssd_status st = prepare(kScan, X, nullptr, B, C, Y, cu_seqlens, chunk, state_block, shape, workspace,
                          workspace_bytes, &pp);
  if (st != SSD_OK) return st;
  return hip_status(ssd::launch_chunk_scan(pp.d, X, B, C, Y, pp.ws, (hipStream_t)stream));
}

ssd_status ssd_fwd_ex(const void* X, const float* log_a, const void* B, const void* C, const int32_t* cu_seqlens,
                      const float* initial_state, int32_t chunk, int32_t state_block, void* Y, float* final_state,
                      const ssd_shape* shape, void* workspace, size_t workspace_bytes, void* stream) {
  Prepared pp;
  ssd_status st = prepare(kAll, X, log_a, B, C, Y, cu_seqlens, chunk, state_block, shape, workspace,
                          workspace_bytes, &pp, false, initial_state, final_state);
  if (st != SSD_OK) return st;
  // chunk_state computes the records and segment sums itself.
  return hip_status(run_forward(pp, X, log_a, B, C, cu_seqlens, initial_state, Y, final_state,
                                (hipStream_t)stream));
}

ssd_status ssd_fwd(const void* X, const float* log_a, const void* B, const void* C, const int32_t* cu_seqlens,
                   int32_t chunk, void* Y, float* final_state, const ssd_shape* shape, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return ssd_fwd_ex(X, log_a, B, C, cu_seqlens, nullptr, chunk, 0, Y, final_state, shape, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"

// Scratch of ssd_fwd_noalloc: one array per GPU, allocated when the code
// object loads and held until the process ends. In host code `scratch` only
// names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, asked once per device with that device current and kept
// in g_scratch_ptr. Kernels receive that address, never the name.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

ssd_status ssd_fwd_noalloc(const void* X, const float* log_a, const void* B, const void* C,
                           const int32_t* cu_seqlens, int32_t chunk, void* Y, float* final_state,
                           const ssd_shape* shape, void* stream) {
  // Host-side checks first, as in ssd_fwd: a workspace of the scratch's size at
  // a stand-in address (never dereferenced) makes prepare() check the shape,
  // pointers and alignment, and report a layout larger than the scratch.
  Prepared pp;
  void* const probe = reinterpret_cast<void*>((uintptr_t)256);
  ssd_status st = prepare(kAll, X, log_a, B, C, Y, cu_seqlens, chunk, 0, shape, probe, SSD_NOALLOC_SCRATCH_BYTES,
                          &pp, false, nullptr, final_state);
  if (st != SSD_OK) return st;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return SSD_ERR_HIP;
  ssd_layout L;
  st = make_layout(shape, cu_seqlens, chunk, pp.d.state_block, &L);
  if (st != SSD_OK) return st;
  st = prepare(kAll, X, log_a, B, C, Y, cu_seqlens, chunk, pp.d.state_block, shape, ws, L.total_bytes, &pp, false,
               nullptr, final_state);
  if (st != SSD_OK) return st;
  return hip_status(run_forward(pp, X, log_a, B, C, cu_seqlens, nullptr, Y, final_state, (hipStream_t)stream));
}

ssd_status ssd_bwd_workspace_bytes(const ssd_shape* shape, int32_t chunk, int32_t state_block, size_t* bytes) {
  if (!bytes || !shape) return SSD_ERR_INVALID_ARGUMENT;
  const int32_t dummy = 0;
  const int32_t* cu = shape->num_seqs > 0 ? &dummy : nullptr;
  BwdLayout L;
  const ssd_status st = make_bwd_layout(shape, cu, chunk, state_block, &L);
  if (st != SSD_OK) return st;
  *bytes = L.total;
  return SSD_OK;
}

// The backward pass. fwd_run_done: the forward state run's block tables,
// segment sums and block-entering states are already in the workspace (the
// fused path skips that run); see ssd_bwd_mamba2.
static ssd_status bwd_run(const void* X, const float* log_a, const void* B, const void* C,
                          const int32_t* cu_seqlens, const float* initial_state, const void* dY,
                          const float* dfinal_state, int32_t chunk, int32_t state_block, void* dX, float* dlog_a,
                          void* dB, void* dC, float* dinitial_state, const ssd_shape* shape, void* workspace,
                          size_t workspace_bytes, void* stream, bool fwd_run_done) {
  if (!X || !log_a || !B || !C || !dY || !dX || !dlog_a || !dB || !dC || !shape) return SSD_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)initial_state | (uintptr_t)dfinal_state | (uintptr_t)dinitial_state) & 15)
    return SSD_ERR_INVALID_ARGUMENT;
  const ssd_shape* s = shape;
  BwdLayout L;
  ssd_status st = make_bwd_layout(s, cu_seqlens, chunk, state_block, &L);
  if (st != SSD_OK) return st;
  if (!workspace || ((uintptr_t)workspace & 255)) return SSD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.total) return SSD_ERR_WORKSPACE_TOO_SMALL;
  char* w = static_cast<char*>(workspace);
  const bool packed = cu_seqlens != nullptr;
  int32_t* cur = packed ? reinterpret_cast<int32_t*>(w + L.cur) : nullptr;
  const int rows = s->batch, T = s->seqlen, Tr = L.Tr, H = s->nheads, G = s->ngroups, P = s->headdim, N = s->dstate;
  const int S = packed ? s->num_seqs : 0;
  const long nseq = packed ? s->num_seqs : s->batch;
  const bool bf16 = s->dtype == SSD_DTYPE_BF16;
  const int esz = bf16 ? 2 : 4;
  hipStream_t hs = (hipStream_t)stream;
  void* rev_dy = w + L.rev_dy;
  void* rev_c = w + L.rev_c;
  float* la_rev = reinterpret_cast<float*>(w + L.la_rev);
  float* lam_first = reinterpret_cast<float*>(w + L.lam_first);
  ssd_shape sr = *s;
  sr.seqlen = Tr;
  if (L.fused) {
    // Two state runs with one chunk per state block, then one kernel for the
    // four gradients of every chunk.
    Prepared pa, pf;
    if ((st = prepare(kAll, dY, log_a, C, B, dX, cur, chunk, L.gs, &sr, w + L.fwd_a, L.a_bytes, &pa)) != SSD_OK)
      return st;
    if ((st = prepare(kAll, X, log_a, B, C, dX, cu_seqlens, chunk, L.gs, s, w + L.fwd_f, L.f_bytes, &pf)) != SSD_OK)
      return st;
    // States entering every chunk: the runs' own block states when a block is
    // one chunk, else expanded from them.
    void* rstart = L.gs > 1 ? w + L.cstart_r : pa.ws.start_states;
    void* fstart = L.gs > 1 ? w + L.cstart_f : pf.ws.start_states;
    hipError_t e = hipSuccess;
    if (packed) e = ssd::launch_padded_offsets(cu_seqlens, cur, S, chunk, hs);
    if (e == hipSuccess)
      e = ssd::launch_reverse_inputs(dY, rev_dy, P * esz, C, rev_c, N * esz, log_a, la_rev, cu_seqlens, cur, S, rows, T,
                                     Tr, H, G, hs);
    // Adjoint states: the reversed run over dY (x role) and C (B role) from the
    // final-state gradient; its chunk start states are the adjoints at the
    // forward chunk ends.
    if (e == hipSuccess) {
      const ssd::SegArgs sa = ssd::seg_args(pa.d, la_rev, cur, ssd::Mamba2Args{});
      e = run_state_chain(pa, rev_dy, rev_c, sa, cur, dfinal_state, dinitial_state ? lam_first : nullptr, hs);
    }
    if (e == hipSuccess && L.gs > 1) e = ssd::launch_chunk_starts(pa.d, rev_dy, rev_c, pa.ws, rstart, hs);
    // Forward chunk start states and segment sums.
    if (e == hipSuccess && !fwd_run_done) {
      const ssd::SegArgs sa = ssd::seg_args(pf.d, log_a, cu_seqlens, ssd::Mamba2Args{});
      e = run_state_chain(pf, X, B, sa, cu_seqlens, initial_state, nullptr, hs);
    }
    if (e == hipSuccess && L.gs > 1) e = ssd::launch_chunk_starts(pf.d, X, B, pf.ws, fstart, hs);
    if (e == hipSuccess) {
      ssd::BwdChunkArgs a{};
      a.X = X;
      a.dY = dY;
      a.B = B;
      a.C = C;
      a.la = log_a;
      a.fcs = pf.ws.cs;
      a.fstart = fstart;
      a.rstart = rstart;
      a.cu = cu_seqlens;
      a.cur = cur;
      a.S = S;
      a.T = T;
      a.spr = pf.d.slots_per_row;
      a.spr_r = pa.d.slots_per_row;
      a.nslots = pf.d.nslots;
      a.tokens = (long)rows * T;
      a.dX = dX;
      a.dla = dlog_a;
      a.dB = dB;
      a.dC = dC;
      a.part_b = L.nsl > 1 ? reinterpret_cast<float*>(w + L.part_b) : nullptr;
      a.part_c = L.nsl > 1 ? reinterpret_cast<float*>(w + L.part_c) : nullptr;
      a.H = H;
      a.G = G;
      a.P = P;
      a.N = N;
      a.Q = chunk;
      a.nsl = L.nsl;
      a.lam_first = lam_first;
      a.dinit = dinitial_state;  // formed in the launch that sums the head slices
      a.nseq = (int)nseq;
      e = ssd::launch_bwd_chunks(a, hs);
    }
    return hip_status(e);
  }
  // Dimensions of the four internal runs of the general path.
  const ssd_shape sw = swapped_shape(s);
  ssd_shape swr = sw;
  swr.seqlen = Tr;
  Prepared pa, pf, pbr, pbf;  // reversed dX run, forward state run, role-exchanged runs (reversed, forward)
  if ((st = prepare(kAll, X, log_a, B, C, dX, cur ? cur : nullptr, chunk, 1, &sr, w + L.fwd_a, L.a_bytes, &pa)) != SSD_OK)
    return st;
  if ((st = prepare(kAll, X, log_a, B, C, dX, cu_seqlens, chunk, 1, s, w + L.fwd_f, L.f_bytes, &pf)) != SSD_OK) return st;
  if ((st = prepare(kAll, X, log_a, B, C, dX, cur, chunk, 0, &swr, w + L.fwd_s, L.s_bytes, &pbr)) != SSD_OK) return st;
  if ((st = prepare(kAll, X, log_a, B, C, dX, cu_seqlens, chunk, 0, &sw, w + L.fwd_s, L.s_bytes, &pbf)) != SSD_OK)
    return st;
  pbr.d.y_f32 = pbf.d.y_f32 = 1;  // per-head partials in fp32, rounded once after the group sum
  void* rev_x = w + L.rev_x;
  void* dx_rev = w + L.dx_rev;
  void* rev_b = w + L.rev_b;
  void* bcast = w + L.bcast;
  float* part = reinterpret_cast<float*>(w + L.part);
  float* states_t = reinterpret_cast<float*>(w + L.states_t);

  hipError_t e = hipSuccess;
  if (packed) e = ssd::launch_padded_offsets(cu_seqlens, cur, S, chunk, hs);
  // The padded reversed copies and decays.
  if (e == hipSuccess) e = ssd::launch_gather_rows(dY, rev_dy, cu_seqlens, cur, S, rows, T, Tr, H, H, P * esz, 1, hs);
  if (e == hipSuccess) e = ssd::launch_gather_rows(X, rev_x, cu_seqlens, cur, S, rows, T, Tr, H, H, P * esz, 1, hs);
  if (e == hipSuccess) e = ssd::launch_gather_rows(B, rev_b, cu_seqlens, cur, S, rows, T, Tr, G, G, N * esz, 1, hs);
  if (e == hipSuccess) e = ssd::launch_gather_rows(C, rev_c, cu_seqlens, cur, S, rows, T, Tr, G, G, N * esz, 1, hs);
  if (e == hipSuccess) e = ssd::launch_reverse_log_decay(log_a, la_rev, cu_seqlens, cur, S, rows, T, Tr, H, hs);
  // dX = M^T dY: the reversed run with B and C exchanged, from the final-state
  // gradient; its chunk start states are the adjoints at the forward chunk ends.
  if (e == hipSuccess)
    e = run_forward(pa, rev_dy, la_rev, rev_c, rev_b, cur, dfinal_state, dx_rev, dinitial_state ? lam_first : nullptr,
                    hs);
  if (e == hipSuccess) e = ssd::launch_gather_rows(dx_rev, dX, cu_seqlens, cur, S, rows, T, Tr, H, H, P * esz, 2, hs);
  // The forward chunk start states (one chunk per state block) and segment sums.
  if (e == hipSuccess) {
    const ssd::SegArgs sa = ssd::seg_args(pf.d, log_a, cu_seqlens, ssd::Mamba2Args{});
    e = ssd::launch_chunk_state(pf.d, X, B, pf.ws, hs, &sa);
  }
  if (e == hipSuccess) e = ssd::launch_state_passing(pf.d, cu_seqlens, initial_state, nullptr, pf.ws, hs);
  // d log a by chunks, from both runs' chunk start states.
  if (e == hipSuccess) {
    ssd::DlogArgs da{X, dY, B, C, log_a, pf.ws.table, pf.ws.btable, pf.ws.cs, pf.ws.start_states, pa.ws.start_states,
                     cu_seqlens, cur, pf.d.slots_per_row, pa.d.slots_per_row, pf.d.nslots, dlog_a, H, G, P, N, chunk,
                     bf16 ? 1 : 0};
    e = ssd::launch_dlog_chunks(da, hs);
  }
  // dB: reversed run with x-role C (broadcast to heads), B-role dY, C-role x.
  if (e == hipSuccess) e = ssd::launch_gather_rows(C, bcast, cu_seqlens, cur, S, rows, T, Tr, G, H, N * esz, 1, hs);
  if (e == hipSuccess && dfinal_state) e = ssd::launch_transpose_states(dfinal_state, states_t, nseq * H, P, N, hs);
  if (e == hipSuccess)
    e = run_forward(pbr, bcast, la_rev, rev_dy, rev_x, cur, dfinal_state ? states_t : nullptr, part, nullptr, hs);
  if (e == hipSuccess) e = ssd::launch_group_sum(part, dB, cu_seqlens, cur, S, rows, T, Tr, H, G, N, bf16, true, hs);
  // dC: forward-time run with x-role B (broadcast to heads), B-role x, C-role dY.
  if (e == hipSuccess) e = ssd::launch_gather_rows(B, bcast, cu_seqlens, cur, S, rows, T, Tr, G, H, N * esz, 0, hs);
  if (e == hipSuccess && initial_state) e = ssd::launch_transpose_states(initial_state, states_t, nseq * H, P, N, hs);
  if (e == hipSuccess)
    e = run_forward(pbf, bcast, log_a, X, dY, cu_seqlens, initial_state ? states_t : nullptr, part, nullptr, hs);
  if (e == hipSuccess) e = ssd::launch_group_sum(part, dC, cu_seqlens, cur, S, rows, T, Tr, H, G, N, bf16, false, hs);
  // d h_init = a_first * (adjoint of the first state).
  if (e == hipSuccess && dinitial_state)
    e = ssd::launch_dinit(log_a, lam_first, dinitial_state, cu_seqlens, (int)nseq, T, H, P * N, hs);
  return hip_status(e);
}

ssd_status ssd_fwd_mamba2(const void* X, const float* dt, const float* dt_bias, const float* A_log,
                          const float* D, const void* z, const void* B, const void* C, const int32_t* cu_seqlens,
                          const float* initial_state, int32_t chunk, int32_t state_block, void* Y,
                          float* final_state, const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!dt || !A_log) return SSD_ERR_INVALID_ARGUMENT;
  Prepared pp;
  // log_a is not read on this path; dt stands in for the non-null check.
  ssd_status st = prepare(kAll, X, dt, B, C, Y, cu_seqlens, chunk, state_block, shape, workspace,
                          workspace_bytes, &pp, true, initial_state, final_state);
  if (st != SSD_OK) return st;
  ssd::Mamba2Args m2;
  m2.dt = dt;
  m2.dt_bias = dt_bias;
  m2.A_log = A_log;
  m2.D = D;
  m2.z = z;
  hipStream_t s = (hipStream_t)stream;
  const ssd::SegArgs sa = ssd::seg_args(pp.d, nullptr, cu_seqlens, m2);
  hipError_t e = run_state_chain(pp, X, B, sa, cu_seqlens, initial_state, final_state, s);
  if (e == hipSuccess) e = ssd::launch_chunk_scan(pp.d, X, B, C, Y, pp.ws, s, m2);
  return hip_status(e);
}

ssd_status ssd_step_mamba2(float* state, const void* x, const float* dt, const float* dt_bias, const float* A_log,
                           const float* D, const void* z, const void* B, const void* C, void* y,
                           const ssd_shape* shape, void* stream) {
  if (!shape || !state || !x || !dt || !A_log || !B || !C || !y) return SSD_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)state & 15) return SSD_ERR_INVALID_ARGUMENT;  // the state moves in 16-byte pieces
  const ssd_shape* s = shape;
  const ssd_status st = check_step(s);
  if (st != SSD_OK) return st;
  ssd::Mamba2Args m2;
  m2.dt = dt;
  m2.dt_bias = dt_bias;
  m2.A_log = A_log;
  m2.D = D;
  m2.z = z;
  return hip_status(ssd::launch_ssd_step(s->batch, s->nheads, s->ngroups, s->headdim, s->dstate,
                                         s->dtype == SSD_DTYPE_BF16 ? 1 : 0, state, x, nullptr, B, C, y,
                                         (hipStream_t)stream, m2));
}

int32_t ssd_set_state_chain(int32_t mode) { return g_state_chain.exchange(mode ? 1 : 0); }

ssd_status ssd_state_chain_cooperative(const ssd_shape* shape, int32_t chunk, int32_t state_block,
                                       int32_t* cooperative) {
  if (!cooperative) return SSD_ERR_INVALID_ARGUMENT;
  // packed shapes (num_seqs > 0) size their slots as a call with cu_seqlens does
  static const int32_t kPackedMarker = 0;
  const int32_t* cu = (shape && shape->num_seqs > 0) ? &kPackedMarker : nullptr;
  ssd_status st = check_shape(shape, cu, chunk);
  if (st != SSD_OK) return st;
  const int32_t gs = state_block > 0 ? state_block : default_state_block(shape, cu, chunk);
  st = check_state_block(shape, gs);
  if (st != SSD_OK) return st;
  ssd_layout L;
  st = make_layout(shape, cu, chunk, gs, &L);
  if (st != SSD_OK) return st;
  const ssd_shape* s = shape;
  const ssd::FwdDims d{s->batch, s->seqlen, s->nheads, s->ngroups, s->headdim, s->dstate, chunk, gs,
                       cu ? s->num_seqs : 0, s->dtype == SSD_DTYPE_BF16 ? 1 : 0,
                       (long)L.slots_per_row, (long)L.nslots, (long)L.blocks_per_row, (long)L.nblocks};
  bool coop = false;
  const hipError_t e = ssd::chunk_state_chain_cooperative(d, &coop);
  if (e != hipSuccess) return SSD_ERR_HIP;
  *cooperative = coop ? 1 : 0;
  return SSD_OK;
}

ssd_status ssd_chunk_scan_kernel(const ssd_shape* shape, int32_t chunk, int32_t state_block, int32_t* kernel) {
  if (!kernel) return SSD_ERR_INVALID_ARGUMENT;
  static const int32_t kPackedMarker = 0;
  const int32_t* cu = (shape && shape->num_seqs > 0) ? &kPackedMarker : nullptr;
  ssd_status st = check_shape(shape, cu, chunk);
  if (st != SSD_OK) return st;
  const int32_t gs = state_block > 0 ? state_block : default_state_block(shape, cu, chunk);
  st = check_state_block(shape, gs);
  if (st != SSD_OK) return st;
  ssd_layout L;
  st = make_layout(shape, cu, chunk, gs, &L);
  if (st != SSD_OK) return st;
  const ssd_shape* s = shape;
  const ssd::FwdDims d{s->batch, s->seqlen, s->nheads, s->ngroups, s->headdim, s->dstate, chunk, gs,
                       cu ? s->num_seqs : 0, s->dtype == SSD_DTYPE_BF16 ? 1 : 0,
                       (long)L.slots_per_row, (long)L.nslots, (long)L.blocks_per_row, (long)L.nblocks};
  *kernel = ssd::chunk_scan_kind(d);
  return SSD_OK;
}

ssd_status ssd_bwd(const void* X, const float* log_a, const void* B, const void* C, const int32_t* cu_seqlens,
                   const float* initial_state, const void* dY, const float* dfinal_state, int32_t chunk,
                   int32_t state_block, void* dX, float* dlog_a, void* dB, void* dC, float* dinitial_state,
                   const ssd_shape* shape, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_run(X, log_a, B, C, cu_seqlens, initial_state, dY, dfinal_state, chunk, state_block, dX, dlog_a, dB, dC,
                 dinitial_state, shape, workspace, workspace_bytes, stream, false);
}

// Workspace of ssd_bwd_mamba2: one region that the ungated forward run (for v)
// and then ssd_bwd use in turn, then v, log a, x dt', dv, the recurrence's
// gradients of x dt' and log a, and the per-(token block, head) partial sums.
struct M2BwdLayout {
  size_t region, v, la, xs, dv, dxs, dla, part, total;
};

static ssd_status m2_bwd_layout(const ssd_shape* s, int32_t chunk, int32_t gs, M2BwdLayout* out) {
  size_t bwd = 0, fwd = 0;
  ssd_status st = ssd_bwd_workspace_bytes(s, chunk, gs, &bwd);
  if (st != SSD_OK) return st;
  st = ssd_fwd_workspace_bytes(s, chunk, gs, &fwd);
  if (st != SSD_OK) return st;
  if (s->headdim % 8) return SSD_ERR_UNSUPPORTED;  // eight channels per thread
  const size_t esz = s->dtype == SSD_DTYPE_BF16 ? 2 : 4;
  const size_t tok = (size_t)s->batch * s->seqlen, H = s->nheads, P = s->headdim;
  M2BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  L.region = take(bwd > fwd ? bwd : fwd);
  L.v = take(tok * H * P * esz);
  L.la = take(tok * H * 4);
  L.xs = take(tok * H * P * esz);
  L.dv = take(tok * H * P * esz);
  L.dxs = take(tok * H * P * esz);
  L.dla = take(tok * H * 4);
  L.part = take((size_t)ssd::m2_token_blocks((long)tok) * H * 3 * 4);
  L.total = off;
  *out = L;
  return SSD_OK;
}

ssd_status ssd_bwd_mamba2_workspace_bytes(const ssd_shape* shape, int32_t chunk, int32_t state_block,
                                          size_t* bytes) {
  if (!shape || !bytes) return SSD_ERR_INVALID_ARGUMENT;
  M2BwdLayout L;
  const ssd_status st = m2_bwd_layout(shape, chunk, state_block, &L);
  if (st != SSD_OK) return st;
  *bytes = L.total;
  return SSD_OK;
}

ssd_status ssd_bwd_mamba2(const void* X, const float* dt, const float* dt_bias, const float* A_log, const float* D,
                          const void* z, const void* B, const void* C, const int32_t* cu_seqlens,
                          const float* initial_state, const void* dY, const float* dfinal_state, int32_t chunk,
                          int32_t state_block, void* dX, float* ddt, float* ddt_bias, float* dA_log, float* dD,
                          void* dz, void* dB, void* dC, float* dinitial_state, const ssd_shape* shape,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !dt || !A_log || !B || !C || !dY || !dX || !ddt || !dA_log || !dB || !dC || !shape)
    return SSD_ERR_INVALID_ARGUMENT;
  if ((D == nullptr) != (dD == nullptr) || (z == nullptr) != (dz == nullptr)) return SSD_ERR_INVALID_ARGUMENT;
  if (!workspace || ((uintptr_t)workspace & 255)) return SSD_ERR_INVALID_ARGUMENT;
  M2BwdLayout L;
  ssd_status st = m2_bwd_layout(shape, chunk, state_block, &L);
  if (st != SSD_OK) return st;
  if (workspace_bytes < L.total) return SSD_ERR_WORKSPACE_TOO_SMALL;
  char* w = static_cast<char*>(workspace);
  const size_t region_bytes = L.v - L.region;
  hipStream_t hs = (hipStream_t)stream;
  ssd::M2BwdArgs a{};
  a.X = X;
  a.dt = dt;
  a.dt_bias = dt_bias;
  a.A_log = A_log;
  a.D = D;
  a.z = z;
  a.dY = dY;
  a.v = w + L.v;
  a.la = reinterpret_cast<float*>(w + L.la);
  a.xs = w + L.xs;
  a.dv = w + L.dv;
  a.dz = dz;
  a.dv_in = z ? static_cast<const void*>(w + L.dv) : dY;
  a.dxs = w + L.dxs;
  a.dla = reinterpret_cast<float*>(w + L.dla);
  a.dXo = dX;
  a.ddt = ddt;
  a.ddt_bias = ddt_bias;
  a.dA_log = dA_log;
  a.dD = dD;
  a.part = reinterpret_cast<float*>(w + L.part);
  a.tokens = (long)shape->batch * shape->seqlen;
  a.H = shape->nheads;
  a.P = shape->headdim;
  a.bf16 = shape->dtype == SSD_DTYPE_BF16 ? 1 : 0;
  // v = SSM(x dt') + D x: the call itself without the gate, for dz. On the
  // fused backward path it runs in the backward's forward-run workspace, with
  // the backward's state block: its block tables, segment sums (of dt' A, the
  // backward's log a) and block-entering states are those of the backward's
  // forward state run, which is then skipped.
  bool fwd_run_done = false;
  if (z) {
    BwdLayout Lb;
    st = make_bwd_layout(shape, cu_seqlens, chunk, state_block, &Lb);
    if (st != SSD_OK) return st;
    if (Lb.fused) {
      st = ssd_fwd_mamba2(X, dt, dt_bias, A_log, D, nullptr, B, C, cu_seqlens, initial_state, chunk, Lb.gs, w + L.v,
                          nullptr, shape, w + L.region + Lb.fwd_f, Lb.f_bytes, stream);
      fwd_run_done = true;
    } else {
      st = ssd_fwd_mamba2(X, dt, dt_bias, A_log, D, nullptr, B, C, cu_seqlens, initial_state, chunk, state_block,
                          w + L.v, nullptr, shape, w + L.region, region_bytes, stream);
    }
    if (st != SSD_OK) return st;
  }
  hipError_t e = ssd::launch_m2_prep(a, hs);
  if (e != hipSuccess) return hip_status(e);
  st = bwd_run(w + L.xs, a.la, B, C, cu_seqlens, initial_state, a.dv_in, dfinal_state, chunk, state_block,
               w + L.dxs, reinterpret_cast<float*>(w + L.dla), dB, dC, dinitial_state, shape, w + L.region,
               region_bytes, stream, fwd_run_done);
  if (st != SSD_OK) return st;
  return hip_status(ssd::launch_m2_epilogue(a, hs));
}

ssd_status ssd_step(float* state, const void* x, const float* log_a, const void* B, const void* C, void* y,
                    const ssd_shape* shape, void* stream) {
  if (!shape || !state || !x || !log_a || !B || !C || !y) return SSD_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)state & 15) return SSD_ERR_INVALID_ARGUMENT;  // the state moves in 16-byte pieces
  const ssd_shape* s = shape;
  const ssd_status st = check_step(s);
  if (st != SSD_OK) return st;
  return hip_status(ssd::launch_ssd_step(s->batch, s->nheads, s->ngroups, s->headdim, s->dstate,
                                         s->dtype == SSD_DTYPE_BF16 ? 1 : 0, state, x, log_a, B, C, y,
                                         (hipStream_t)stream));
}

}  // extern "C"
