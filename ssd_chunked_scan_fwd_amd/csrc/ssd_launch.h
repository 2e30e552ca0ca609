// ssd_launch.h -- host-side launchers of the gfx950 SSD kernels (internal).
//
// Arguments have been validated by the C-ABI layer before any of these runs.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

struct FwdDims {
  int batch, T, H, G, P, N, Q;
  int state_block;        // Gs: chunks per state block
  int num_seqs;           // packed sequences (0 when unpacked)
  int bf16;               // 1: bf16 tensors, 0: fp32
  long slots_per_row;     // chunk slots per row
  long nslots;
  long blocks_per_row;    // state-block slots per row
  long nblocks;
  int y_f32 = 0;          // bf16 inputs only: write Y in fp32 (partials the backward pass sums)
};

// Whether block slots can differ in length (packed sequences, or rows that
// are not a whole number of state blocks): then the state-passing stage ranks
// them and the chunk-scan stage takes them in that order (scan_unit).
inline bool ranked_blocks(const FwdDims& d) {
  return d.nblocks < 32768 && (d.num_seqs > 0 || d.T % (d.state_block * d.Q) != 0);
}

struct Workspace {
  int4* table;            // [nslots] chunk records
  int4* btable;           // [nblocks] state-block records
  float* cs;              // [nslots][H][Q] cumulative log2 decay, restarted per chunk
  float* ck;              // [nslots][H][Q] exponent of the key-side weights: cs itself for plain
                          // calls, cs_j - log2(dt_j) for the Mamba-2 block's call
  float* bdecay;          // [nblocks][H] total log2 decay of each block
  float* bstates;         // [nblocks][H][P][N] right factors of each block
  void* start_states;     // [nblocks][H][P][N] state entering each block
};

// The Mamba-2 block's per-head parameters and gate (device pointers). With dt
// set, the cumsum stage takes raw step sizes instead of log a; D and z shape
// the chunk-scan output (null: no skip, no gate).
struct Mamba2Args {
  const float* dt = nullptr;       // [rows * T][H] raw step sizes
  const float* dt_bias = nullptr;  // [H] or null (zero)
  const float* A_log = nullptr;    // [H], A = -exp(A_log)
  const float* D = nullptr;        // [H] or null
  const void* z = nullptr;         // like X, or null
};

// Arguments of the segment sums: the log decay, or the Mamba-2 step sizes,
// and what locates chunk and block slots.
struct SegArgs {
  const float* la;       // [rows * T][H] log a (plain calls)
  const float* dt;       // [rows * T][H] raw step sizes (Mamba-2 calls), else null
  const float* dt_bias;  // [H] or null
  const float* A_log;    // [H]
  const int32_t* cu;     // packed sequence starts, or null
  int S, T;
  long slots_per_row, blocks_per_row;
};

inline SegArgs seg_args(const FwdDims& d, const float* log_a, const int32_t* cu, const Mamba2Args& m2) {
  return SegArgs{log_a, m2.dt, m2.dt_bias, m2.A_log, cu, d.num_seqs, d.T, d.slots_per_row, d.blocks_per_row};
}

hipError_t launch_chunk_cumsum(const FwdDims& d, const float* log_a, const int32_t* cu,
                               const Workspace& ws, hipStream_t stream, const Mamba2Args& m2 = Mamba2Args{});
// With `seg` given, chunk_state computes the records and segment sums itself
// (the fused form that ssd_fwd* run); without it, it reads them from the
// workspace as written by launch_chunk_cumsum.
hipError_t launch_chunk_state(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                              hipStream_t stream, const SegArgs* seg = nullptr);
hipError_t launch_state_passing(const FwdDims& d, const int32_t* cu, const float* init, float* final_state,
                                const Workspace& ws, hipStream_t stream);
// chunk_state (fused with the segment sums) and state_passing in one
// cooperative launch, when every workgroup of the grid can be resident and the
// stream is not being captured; *launched says whether it ran (else the caller
// runs the two launches).
hipError_t launch_chunk_state_chain(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                                    hipStream_t stream, const SegArgs& sa, const float* init, float* final_state,
                                    bool* launched);
// Whether launch_chunk_state_chain would launch the cooperative kernel for
// these dimensions on the current device (on a stream not being captured).
hipError_t chunk_state_chain_cooperative(const FwdDims& d, bool* cooperative);
// Which chunk_scan kernel a call takes (values of the public SSD_SCAN_* codes):
// fp32; bf16 one head per workgroup; two heads per workgroup walking whole
// chunks (eight waves, one workgroup per CU); two heads per workgroup walking
// chunks in halves of 64 tokens (four waves, two workgroups per CU; or, for
// dstate 256, eight waves, one per CU).
constexpr int kScanF32 = 0, kScanSingle = 1, kScanPair = 2, kScanHalfPair = 3, kScanHalfPairWide = 4;
int chunk_scan_kind(const FwdDims& d);
hipError_t launch_chunk_scan(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                             const Workspace& ws, hipStream_t stream, const Mamba2Args& m2 = Mamba2Args{});
hipError_t launch_ssd_step(int batch, int H, int G, int P, int N, int bf16, float* state,
                           const void* x, const float* log_a, const void* B, const void* C, void* y,
                           hipStream_t stream, const Mamba2Args& m2 = Mamba2Args{});

// Backward-pass helpers (ssd_bwd.hip). The reversed runs use a padded reversed
// layout: each sequence reversed in time behind (Q - len mod Q) mod Q zero
// tokens, so that its chunks line up with the forward chunks; cur[] holds the
// packed sequence starts of that layout (unpacked rows have Tr tokens each).
hipError_t launch_padded_offsets(const int32_t* cu, int32_t* cur, int S, int Q, hipStream_t stream);
// mode 0: same layout; 1: forward -> padded reversed; 2: padded reversed -> forward.
hipError_t launch_gather_rows(const void* in, void* out, const int32_t* cu, const int32_t* cur, int S, int rows, int T,
                              int Tr, int Hin, int Hout, int row_bytes, int mode, hipStream_t stream);
hipError_t launch_group_sum(const float* in, void* out, const int32_t* cu, const int32_t* cur, int S, int rows, int T,
                            int Tr, int H, int G, int D, bool bf16, bool from_reversed, hipStream_t stream);
hipError_t launch_reverse_log_decay(const float* la, float* out, const int32_t* cu, const int32_t* cur, int S,
                                    int rows, int T, int Tr, int H, hipStream_t stream);
hipError_t launch_transpose_states(const float* in, float* out, long nmat, int A, int Bd, hipStream_t stream);
// dY and C into the padded time-reversed layout and the shifted reversed log
// decay, in one launch (the fused backward's first step).
hipError_t launch_reverse_inputs(const void* dY, void* rev_dy, int dy_bytes, const void* C, void* rev_c, int c_bytes,
                                 const float* la, float* la_rev, const int32_t* cu, const int32_t* cur, int S, int rows,
                                 int T, int Tr, int H, int G, hipStream_t stream);
hipError_t launch_dinit(const float* la, const float* lam_first, float* dinit, const int32_t* cu, int nseq, int T,
                        int H, int PN, hipStream_t stream);

struct DlogArgs {
  const void *X, *dY, *B, *C;   // forward layout, dtype
  const float* la;
  const int4* ftable;           // forward run (one chunk per state block): chunk records,
  const int4* fbtable;          //   block records (written for every slot),
  const float* fcs;             //   segment sums,
  const void* fstart;           //   chunk start states
  const void* rstart;           // reversed run: chunk start states (padded reversed slots)
  const int32_t *cu, *cur;
  long spr, spr_r, nslots;      // chunk slots per row (forward, reversed), forward slots
  float* dla;
  int H, G, P, N, Q, bf16;
};
hipError_t launch_dlog_chunks(const DlogArgs& a, hipStream_t stream);
size_t dlog_chunk_lds_bytes(int P, int N, int Q, int esz);

// The fused backward chunk kernel (bf16; ssd_bwd_chunk.hip): dX, d log a and
// dB, dC of each chunk from the forward run's chunk-entering states (fstart)
// and the reversed run's (rstart), one chunk per state block in both.
struct BwdChunkArgs {
  const void *X, *dY, *B, *C;   // forward layout, bf16
  const float* la;
  const float* fcs;             // forward run: segment sums,
  const void* fstart;           //   chunk start states (bf16)
  const void* rstart;           // reversed run: chunk start states (bf16, padded reversed slots)
  const int32_t *cu, *cur;
  int S, T;                     // packed sequences, tokens per row
  long spr, spr_r, nslots, tokens;
  void* dX;
  float* dla;
  void *dB, *dC;                // bf16 [tokens][G][N]
  float *part_b, *part_c;       // fp32 [nsl][tokens][G][N] when nsl > 1
  // Initial-state gradient, formed in the same tail launch as the slice sums
  // when dinit is not null: dinit = exp(log a of each sequence's first token)
  // * lam_first, [nseq][H][P*N] fp32.
  const float* lam_first;
  float* dinit;
  int nseq;
  int H, G, P, N, Q, nsl;
};
bool bwd_chunk_supported(int P, int N, int Q, bool bf16);
int bwd_chunk_slices(long nslots, int G, int H);  // head slices per (chunk, group)
hipError_t launch_bwd_chunks(const BwdChunkArgs& a, hipStream_t stream);
// The bf16 state entering every chunk slot ([nslots][H][P][N]) from a run's
// block-entering states (start_states), for the shapes of the fused kernel.
hipError_t launch_chunk_starts(const FwdDims& d, const void* X, const void* B, const Workspace& ws, void* out,
                               hipStream_t stream);

// The chain rule of the Mamba-2 block's call around the recurrence's backward
// (ssd_bwd_mamba2.hip). Device pointers; `tokens` = rows * T.
struct M2BwdArgs {
  const void* X;
  const float *dt, *dt_bias, *A_log, *D;   // dt_bias and D may be null
  const void *z, *dY, *v;                 // z null: no gate (then v, dv, dz unused)
  float* la;                              // [tokens][H] log a (written by the prep kernel)
  void *xs, *dv, *dz;                     // x dt', dY silu(z), the gate's gradient
  const void* dv_in;                      // the recurrence's cotangent: dv, or dY without a gate
  const void* dxs;                        // gradient of x dt' from the recurrence's backward
  const float* dla;                       // gradient of log a
  void* dXo;
  float *ddt, *ddt_bias, *dA_log, *dD;    // ddt_bias and dD may be null
  float* part;                            // [token blocks][H][3]
  long tokens;
  int H, P, bf16;
};
long m2_token_blocks(long tokens);
hipError_t launch_m2_prep(const M2BwdArgs& a, hipStream_t stream);
hipError_t launch_m2_epilogue(const M2BwdArgs& a, hipStream_t stream);

// Bytes of dynamic LDS the bf16 kernels need (host-side checks).
size_t chunk_scan_bf16_lds_bytes(int P, int N, int Q);
size_t chunk_state_bf16_lds_bytes(int P, int N, int block_tokens);  // block_tokens: Gs*Q when fused, else 0
constexpr size_t kMaxLdsBytes = 160 * 1024;

}  // namespace ssd
