/*
 * ssd.h -- C ABI of the MI355X (gfx950) chunked SSD forward pass and decode step.
 *
 * The operator is the scalar-decay state space model of "Transformers are
 * SSMs" (paper card at wikillm.com/papers/2405.21060, Method 1 and Method 2,
 * paper sections 2-3 and 5.1):
 *
 *     h_t = a_t h_{t-1} + B_t x_t^T,   y_t = C_t^T h_t,   a_t = exp(log_a_t)
 *
 * with one decay per (token, head). The forward pass computes it with the
 * chunked SSD block decomposition (paper card Method 5, paper section 6): the
 * sequence is cut into chunks of `chunk` tokens; diagonal blocks use the
 * quadratic form inside a chunk, right factors give each chunk's end state from
 * a zero start, centre factors pass states across chunks with a scalar
 * recurrence, and left factors add the carried-in state to each output.
 *
 * Shapes (row-major, contiguous, no aliasing between any two arguments):
 *   X      [batch, seqlen, nheads, headdim]           dtype
 *   log_a  [batch, seqlen, nheads]                    fp32, finite, <= 0
 *   B, C   [batch, seqlen, ngroups, dstate]           dtype
 *   Y      [batch, seqlen, nheads, headdim]           dtype (written)
 *   final  [batch or num_seqs, nheads, headdim, dstate] fp32 (written),
 *          element (p, n) is h[n][p] of the state after the sequence's last token.
 * Head h reads B/C group h / (nheads / ngroups).
 *
 * Packed variable-length batches: pass cu_seqlens (device, int32, num_seqs+1
 * entries, strictly increasing from 0 to seqlen) with batch == 1. Every packed
 * sequence starts from a zero state, as if run alone (the pages' training on
 * variable-length sequences without padding; a reset is a_t = 0 at the start).
 *
 * Ownership and streams: every pointer is a caller-owned buffer; device
 * pointers for all tensors, host pointers for `shape` and `layout`. The
 * library allocates nothing, keeps no mutable global state, never
 * synchronises, and enqueues its kernels on `stream` (a hipStream_t; NULL is the
 * null stream). A call returns after enqueueing; errors of the kernels
 * themselves surface on the stream like any HIP error.
 *
 * Errors: arguments are checked on the host before any HIP call. On
 * SSD_ERR_INVALID_ARGUMENT, SSD_ERR_UNSUPPORTED or SSD_ERR_WORKSPACE_TOO_SMALL
 * nothing is enqueued and no output is touched. SSD_ERR_HIP reports a failed
 * launch (hipGetLastError). Device data (log_a values, cu_seqlens contents) is
 * not validated; log_a = -inf is not supported on the GPU.
 *
 * Supported sizes: headdim in {16, 32, 64, 128}; dstate in {16, 32, 64, 128,
 * 256}; chunk in {16, 32, 64, 128, 256}; for bf16, chunk >= 32 and dstate >= 32.
 * Other sizes return SSD_ERR_UNSUPPORTED. Every tensor must hold fewer than
 * 2^31 elements.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 1

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, H % G != 0, ... */
  SSD_ERR_UNSUPPORTED = 2,        /* a size or dtype outside the supported set        */
  SSD_ERR_WORKSPACE_TOO_SMALL = 3,
  SSD_ERR_HIP = 4                 /* a kernel launch failed                           */
} ssd_status;

typedef enum { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype;

typedef struct {
  int32_t batch;     /* b: rows; 1 when cu_seqlens is given                 */
  int32_t seqlen;    /* T: tokens per row (packed: total tokens)            */
  int32_t nheads;    /* H                                                   */
  int32_t ngroups;   /* G: B/C groups, H % G == 0                           */
  int32_t headdim;   /* P                                                   */
  int32_t dstate;    /* N                                                   */
  int32_t num_seqs;  /* S: packed sequences when cu_seqlens != NULL, else 0 */
  int32_t dtype;     /* ssd_dtype of X, B, C, Y (and x, B, C, y of a step)  */
} ssd_shape;

/*
 * Workspace of one forward call, carved from one caller buffer (offsets in
 * bytes from its start, each 256-byte aligned). nslots = batch * slots_per_row
 * chunk slots; a slot may be empty (packed rows leave gaps).
 *   table        int32 [nslots][4]: sequence, first token (flattened: row * seqlen + t),
 *                length, chunk index in sequence
 *   cumsum       fp32  [nslots][H][chunk]: log2(e) * cumulative log_a, restarted per chunk,
 *                positions past the chunk's length repeat its total
 *   chunk_states fp32  [nslots][H][P][N]: right factors, state at the chunk end from a zero start
 *   start_states dtype [nslots][H][P][N]: centre factors, state entering the chunk
 *                (bf16 for bf16 inputs, fp32 for fp32 inputs)
 * Packed rows: sequence s owns slots floor(cu[s]/chunk) + s + j for its chunks
 * j = 0 .. ceil(len_s/chunk) - 1. Unpacked rows: row r owns slots
 * r*slots_per_row + j with slots_per_row = ceil(seqlen/chunk).
 */
typedef struct {
  int64_t slots_per_row;
  int64_t nslots;
  size_t table_offset;
  size_t cumsum_offset;
  size_t chunk_states_offset;
  size_t start_states_offset;
  size_t total_bytes;
} ssd_layout;

/* Version of this ABI (SSD_ABI_VERSION). */
int32_t ssd_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* ssd_status_string(ssd_status status);

/* Workspace layout and size of ssd_fwd for this shape and chunk length. */
ssd_status ssd_fwd_layout(const ssd_shape* shape, int32_t chunk, ssd_layout* layout);
ssd_status ssd_fwd_workspace_bytes(const ssd_shape* shape, int32_t chunk, size_t* bytes);

/*
 * Forward pass: Y and final states from zero initial states.
 * Runs the four stages below in order on `stream`. final_state may be NULL.
 */
ssd_status ssd_fwd(const void* X, const float* log_a, const void* B, const void* C,
                   const int32_t* cu_seqlens, int32_t chunk, void* Y, float* final_state,
                   const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * The four stages of ssd_fwd, callable one by one (same arguments, same
 * workspace; each stage reads what the previous stages wrote).
 *
 * ssd_chunk_cumsum -- segment sums of log a: the cumulative log decay
 *   restarted in every chunk, from which the 1-semiseparable mask
 *   L[i][j] = exp(cs_i - cs_j) (i >= j) and the chunk totals follow (paper card
 *   Method 5 pseudocode "decay_cumsum" and "chunk_decay"; Pitfalls: mask before
 *   exp). Writes table and cumsum.
 * ssd_chunk_state -- right factors: s_k = sum_j exp(cs_last - cs_j) x_j B_j^T
 *   per chunk and head, one batched matrix product per chunk (paper section 6,
 *   "Right Factors"). Writes chunk_states.
 * ssd_state_passing -- centre factors: h = 0; for each chunk k of a sequence,
 *   start_k = h, h = exp(A_k) h + s_k with A_k the chunk's total log decay
 *   (paper section 6, "Center Factors"); writes start_states and, when
 *   final_state is not NULL, the state after each sequence.
 * ssd_chunk_scan -- diagonal blocks plus left factors: Y = (L o C B^T) X within
 *   the chunk plus exp(cs) C start^T for the carried-in state (paper section 6,
 *   "Diagonal Blocks" and "Left Factors"). Writes Y.
 */
ssd_status ssd_chunk_cumsum(const float* log_a, const int32_t* cu_seqlens, int32_t chunk,
                            const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                            void* stream);
ssd_status ssd_chunk_state(const void* X, const void* B, const int32_t* cu_seqlens, int32_t chunk,
                           const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                           void* stream);
ssd_status ssd_state_passing(const int32_t* cu_seqlens, int32_t chunk, float* final_state,
                             const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                             void* stream);
ssd_status ssd_chunk_scan(const void* X, const void* B, const void* C, const int32_t* cu_seqlens,
                          int32_t chunk, void* Y, const ssd_shape* shape, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for `batch` independent streams: the loop body of
 * the recurrence with a constant-size state (paper card Method 8 and its cost
 * table: about N^2 work per step; the page-1 summary: generation needs only a
 * constant-size state).
 *   state [batch, H, P, N] fp32, updated in place: s = exp(la) s + x B^T
 *   x [batch, H, P] dtype, log_a [batch, H] fp32, B, C [batch, G, N] dtype
 *   y [batch, H, P] dtype (written), read from the updated state.
 * shape->seqlen and shape->num_seqs are ignored.
 */
ssd_status ssd_step(float* state, const void* x, const float* log_a, const void* B, const void* C,
                    void* y, const ssd_shape* shape, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
