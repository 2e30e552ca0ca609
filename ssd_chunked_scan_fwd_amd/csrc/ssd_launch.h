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
  int num_seqs;           // packed sequences (0 when unpacked)
  int bf16;               // 1: bf16 tensors, 0: fp32
  long slots_per_row;
  long nslots;
};

struct Workspace {
  int4* table;
  float* cs;
  float* chunk_states;
  void* start_states;
};

hipError_t launch_chunk_cumsum(const FwdDims& d, const float* log_a, const int32_t* cu,
                               const Workspace& ws, hipStream_t stream);
hipError_t launch_chunk_state(const FwdDims& d, const void* X, const void* B, const Workspace& ws,
                              hipStream_t stream);
hipError_t launch_state_passing(const FwdDims& d, const int32_t* cu, float* final_state,
                                const Workspace& ws, hipStream_t stream);
hipError_t launch_chunk_scan(const FwdDims& d, const void* X, const void* B, const void* C, void* Y,
                             const Workspace& ws, hipStream_t stream);
hipError_t launch_ssd_step(int batch, int H, int G, int P, int N, int bf16, float* state,
                           const void* x, const float* log_a, const void* B, const void* C, void* y,
                           hipStream_t stream);

// Bytes of dynamic LDS the bf16 chunk-scan kernel needs (host-side check).
size_t chunk_scan_bf16_lds_bytes(int P, int N, int Q);
constexpr size_t kMaxLdsBytes = 160 * 1024;

}  // namespace ssd
