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
};

struct Workspace {
  int4* table;            // [nslots] chunk records
  int4* btable;           // [nblocks] state-block records
  float* cs;              // [nslots][H][Q]
  float* bdecay;          // [nblocks][H] total log2 decay of each block
  float* bstates;         // [nblocks][H][P][N] right factors of each block
  void* start_states;     // [nblocks][H][P][N] state entering each block
};

hipError_t launch_chunk_cumsum(const FwdDims& d, const float* log_a, const int32_t* cu,
                               const Workspace& ws, hipStream_t stream);
hipError_t launch_chunk_state(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                              hipStream_t stream);
hipError_t launch_state_passing(const FwdDims& d, const int32_t* cu, const float* init, float* final_state,
                                const Workspace& ws, hipStream_t stream);
hipError_t launch_chunk_scan(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                             const Workspace& ws, hipStream_t stream);
hipError_t launch_ssd_step(int batch, int H, int G, int P, int N, int bf16, float* state,
                           const void* x, const float* log_a, const void* B, const void* C, void* y,
                           hipStream_t stream);

// Bytes of dynamic LDS the bf16 kernels need (host-side checks).
size_t chunk_scan_bf16_lds_bytes(int P, int N, int Q);
size_t chunk_state_bf16_lds_bytes(int P, int N);
constexpr size_t kMaxLdsBytes = 160 * 1024;

}  // namespace ssd
