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
 * Alignment: initial_state and final_state must be 16-byte aligned (states
 * move in 16-byte pieces); other tensors need their element alignment, and
 * the workspace 256 bytes.
 *
 * Ownership and streams: every pointer is a caller-owned buffer; device
 * pointers for all tensors, host pointers for `shape` and `layout`. The
 * library allocates nothing, never synchronises, issues no memset, and
 * enqueues its kernels on `stream` (a hipStream_t; NULL is the null stream).
 * Its only global state is the process-wide mode of ssd_set_state_chain (an
 * atomic). A
 * call returns after enqueueing; errors of the kernels themselves surface on
 * the stream like any HIP error. A call may be captured into a HIP graph: its
 * replays compute what the call computes, from the buffers' contents at
 * replay time.
 *
 * Errors: arguments are checked on the host before any HIP call. On
 * SSD_ERR_INVALID_ARGUMENT, SSD_ERR_UNSUPPORTED or SSD_ERR_WORKSPACE_TOO_SMALL
 * nothing is enqueued and no output is touched. SSD_ERR_HIP reports a failed
 * launch (hipGetLastError). Device data (log_a values, cu_seqlens contents) is
 * not validated; log_a = -inf is not supported on the GPU.
 *
 * Supported sizes: headdim in {16, 32, 64, 128}; dstate in {16, 32, 64, 128,
 * 256}; chunk in {16, 32, 64, 128, 256}; state_block in {1, 2, 4, 8, 16}; for
 * bf16, chunk >= 32 and dstate >= 32 and the chunk tiles must fit the 160 KiB
 * LDS; for fp32, state_block = 1; chunk * (nheads + 1) * 4 bytes <= 160 KiB. Other sizes return SSD_ERR_UNSUPPORTED. Every
 * tensor must hold fewer than 2^31 elements.
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 6

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
 * Two-level chunking. Chunks of `chunk` tokens are the blocks of the
 * quadratic form. State blocks of `state_block` consecutive chunks of one
 * sequence are the units of the state recurrence: the right factor and the
 * centre factor are computed per state block, and the chunk-scan stage carries
 * the state through the chunks of each state block itself. state_block = 1 is
 * exactly the pages' schedule (one chunk state per chunk); larger values give
 * the same result up to rounding with less HBM traffic. fp32 tensors support
 * state_block = 1 only. ssd_fwd chooses state_block itself
 * (ssd_default_state_block); ssd_fwd_ex takes it as an argument.
 *
 * Workspace of one forward call, carved from one caller buffer (offsets in
 * bytes from its start, each 256-byte aligned). nslots = batch * slots_per_row
 * chunk slots and nblocks = batch * blocks_per_row state-block slots; a slot
 * may be empty (packed rows leave gaps).
 *   table        int32 [nslots][4]: sequence, first token (flattened: row * seqlen + t),
 *                length (0: empty slot), chunk index in sequence
 *   block_table  int32 [nblocks][4]: sequence, first chunk slot, number of chunks
 *                (0: empty slot), and a launch-order word: 0 as the records are
 *                written; when block slots differ in length (packed sequences, or
 *                rows not a whole number of state blocks) the state-passing stage
 *                sets record r's word to (slot + 1) | (nfull << 16), slot being the
 *                block with rank r by chunk count (most first) and nfull the number
 *                of slots with the largest count; ssd_chunk_scan then takes the
 *                blocks in that order (short sequence-end blocks last)
 *   cumsum       fp32  [nslots][H][chunk]: log2(e) * cumulative log_a, restarted per chunk,
 *                positions past the chunk's length repeat its total
 *   key_cumsum   fp32  [nslots][H][chunk]: ssd_fwd_mamba2 only, cumsum_j - log2(dt'_j), the
 *                exponent of the weight of key token j (its decay and its input scale);
 *                positions past the chunk's length repeat the chunk total
 *   block_decay  fp32  [nblocks][H]: log2(e) * total log_a of each state block
 *   block_states fp32  [nblocks][H][P][N]: right factors, state at the block end from a
 *                zero start
 *   start_states dtype [nblocks][H][P][N]: centre factors, state entering the block
 *                (bf16 for bf16 inputs, fp32 for fp32 inputs)
 * Packed rows: sequence s owns chunk slots floor(cu[s]/chunk) + s + j for its
 * chunks j = 0 .. ceil(len_s/chunk) - 1, and state-block slots
 * floor(cu[s]/(chunk*state_block)) + s + j. Unpacked rows: row r owns chunk
 * slots r*slots_per_row + j with slots_per_row = ceil(seqlen/chunk), and block
 * slots r*blocks_per_row + j with blocks_per_row = ceil(slots_per_row/state_block).
 */
typedef struct {
  int64_t slots_per_row;
  int64_t nslots;
  int64_t blocks_per_row;
  int64_t nblocks;
  size_t table_offset;
  size_t block_table_offset;
  size_t cumsum_offset;
  size_t key_cumsum_offset;
  size_t block_decay_offset;
  size_t block_states_offset;
  size_t start_states_offset;
  size_t total_bytes;
} ssd_layout;

/* Version of this ABI (SSD_ABI_VERSION). */
int32_t ssd_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* ssd_status_string(ssd_status status);

/* The state_block ssd_fwd uses for this shape and chunk length (1 for fp32). */
int32_t ssd_default_state_block(const ssd_shape* shape, int32_t chunk);

/* Workspace layout and size of a forward call for this shape, chunk length and
 * state block (state_block <= 0 selects ssd_default_state_block). */
ssd_status ssd_fwd_layout(const ssd_shape* shape, int32_t chunk, int32_t state_block, ssd_layout* layout);
ssd_status ssd_fwd_workspace_bytes(const ssd_shape* shape, int32_t chunk, int32_t state_block,
                                   size_t* bytes);

/*
 * How the forward and backward calls run the state chain (the right factors
 * and the centre-factor recurrence over state blocks; paper card Method 5,
 * "Right Factors" and "Centre Factors"):
 *   mode 0 (the default): two launches, chunk_state then state_passing;
 *   mode 1: one cooperative launch, with a grid-wide barrier between the right
 *          factors and the recurrence, when the whole grid can be resident on
 *          the device and `stream` is not being captured into a graph (bf16,
 *          headdim * dstate in {4096, 8192, 16384}, headdim >= 32,
 *          dstate >= 64); otherwise two launches. The cooperative launch
 *          itself costs more than the launch it saves on ROCm 7 (about
 *          74 us per call at T = 16384, H = 32), hence not the default.
 * Both give bit-identical results. Process-wide; returns the previous mode.
 * Cooperative launches are not for profiled runs: rocprofv3 has ended with a
 * segmentation fault in its exit path after a program that made them.
 */
int32_t ssd_set_state_chain(int32_t mode);

/*
 * Whether, in mode 1, a forward call with this shape, chunk length and state
 * block (<= 0: the default) would run its state chain as the cooperative
 * launch on the current device, given a stream that is not being captured:
 * *cooperative = 1 if so, 0 if it would take the two launches. Asks the
 * runtime for the kernel's occupancy on every call and keeps nothing.
 * Packed shapes (num_seqs > 0) are sized as calls with cu_seqlens. Returns
 * the forward call's shape errors, or SSD_ERR_HIP if the runtime query fails.
 */
ssd_status ssd_state_chain_cooperative(const ssd_shape* shape, int32_t chunk, int32_t state_block,
                                       int32_t* cooperative);

/*
 * Which chunk_scan kernel (diagonal blocks and left factors, paper card
 * Method 5 / paper section 6, "Diagonal Blocks" and "Left Factors") a forward
 * call with this shape, chunk length and state block (<= 0: the default)
 * runs. *kernel receives one of:
 *   SSD_SCAN_F32        fp32 inputs;
 *   SSD_SCAN_SINGLE     bf16, one head per workgroup (odd heads per group,
 *                       headdim 128, chunk 256, and at dstate 256 any chunk
 *                       other than 64 and 128);
 *   SSD_SCAN_PAIR       bf16, two heads of one group per workgroup walking
 *                       whole chunks, one workgroup per CU;
 *   SSD_SCAN_HALF_PAIR  bf16, two heads per workgroup walking each chunk in
 *                       halves of 64 tokens with the state carried between
 *                       them, two workgroups per CU (chunk 64 or 128, headdim
 *                       <= 64, dstate <= 128, and at least 512 (state block,
 *                       head pair) units);
 *   SSD_SCAN_HALF_PAIR_WIDE  the same walk for dstate 256 (headdim <= 64,
 *                       chunk 64 or 128), eight waves, one workgroup per CU.
 * All give results within the same tolerance of the exact recurrence; the
 * two pair kernels round differently (the second half of a chunk sees the
 * first through the bf16 state). Host-only: makes no HIP call and keeps
 * nothing. Packed shapes (num_seqs > 0) are sized as calls with cu_seqlens.
 * Returns the forward call's shape and state-block errors.
 */
#define SSD_SCAN_F32 0
#define SSD_SCAN_SINGLE 1
#define SSD_SCAN_PAIR 2
#define SSD_SCAN_HALF_PAIR 3
#define SSD_SCAN_HALF_PAIR_WIDE 4
ssd_status ssd_chunk_scan_kernel(const ssd_shape* shape, int32_t chunk, int32_t state_block, int32_t* kernel);

/*
 * Forward pass: Y and final states from zero initial states, with the default
 * state block. Computes what the four stages below compute, in two or three
 * launches on `stream` (the state chain, see ssd_set_state_chain, then the
 * chunk scan): the chunk-state work also writes the records and segment sums
 * that ssd_chunk_cumsum writes, for every slot that holds a chunk (table rows
 * of slots that hold no chunk are left as they were). final_state may be NULL.
 * The workspace must hold ssd_fwd_workspace_bytes(shape, chunk, 0).
 */
ssd_status ssd_fwd(const void* X, const float* log_a, const void* B, const void* C,
                   const int32_t* cu_seqlens, int32_t chunk, void* Y, float* final_state,
                   const ssd_shape* shape, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Forward pass with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): ssd_fwd with the library's own scratch as the
 * workspace. The scratch is one static device array of
 * SSD_NOALLOC_SCRATCH_BYTES per GPU, allocated when the library's code object
 * loads and held until the process ends; nothing is allocated or freed per
 * call. Calls whose ssd_fwd_workspace_bytes(shape, chunk, 0) exceeds it return
 * SSD_ERR_WORKSPACE_TOO_SMALL before any HIP call (the headline shape, 16384
 * tokens x 32 heads x 64 x 128, needs 27.4 MB; larger calls use ssd_fwd). Every
 * call on one GPU uses that GPU's array: calls that overlap on one GPU (two
 * streams, two host threads) race and must be serialised by the caller. Each
 * call writes every part of the scratch it reads, so nothing needs clearing.
 * Arguments, results and other errors are those of ssd_fwd (SSD_ERR_HIP also
 * when the scratch's address cannot be obtained).
 */
#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)
ssd_status ssd_fwd_noalloc(const void* X, const float* log_a, const void* B, const void* C,
                           const int32_t* cu_seqlens, int32_t chunk, void* Y, float* final_state,
                           const ssd_shape* shape, void* stream);

/*
 * Forward pass with an initial state and an explicit state block
 * (state_block <= 0: the default).
 *   initial_state  device, fp32 [batch or num_seqs, nheads, headdim, dstate]
 *                  (the layout of final_state), or NULL for zero states:
 *                  the state each row (packed: each sequence) starts from, h_0
 *                  with h_1 = a_1 h_0 + B_1 x_1^T. A prompt can then be run in
 *                  pieces, each piece starting from the previous piece's
 *                  final_state, and handed on to ssd_step.
 * The other arguments are those of ssd_fwd.
 */
ssd_status ssd_fwd_ex(const void* X, const float* log_a, const void* B, const void* C,
                      const int32_t* cu_seqlens, const float* initial_state, int32_t chunk,
                      int32_t state_block, void* Y, float* final_state, const ssd_shape* shape,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The four stages of ssd_fwd_ex, callable one by one (same arguments, same
 * workspace; each stage reads what the previous stages wrote). Run in order,
 * they give the same Y, final state and workspace contents as ssd_fwd_ex,
 * bit for bit.
 *
 * ssd_chunk_cumsum -- segment sums of log a: the cumulative log decay
 *   restarted in every chunk, from which the 1-semiseparable mask
 *   L[i][j] = exp(cs_i - cs_j) (i >= j) and the chunk totals follow (paper card
 *   Method 5, the within-chunk cumulative decay and the chunk totals; Pitfalls:
 *   the mask comes before the exponential). Writes table, block_table and
 *   cumsum.
 * ssd_chunk_state -- right factors: s_m = sum_j exp(total decay from j to the
 *   end of block m) x_j B_j^T per state block and head, batched matrix
 *   products over tokens (paper section 6, "Right Factors"). Writes
 *   block_states and block_decay.
 * ssd_state_passing -- centre factors: h = initial state (NULL: 0); for each
 *   state block m of a sequence, start_m = h, h = exp(A_m) h + s_m with A_m the
 *   block's total log decay (paper section 6, "Center Factors"); writes
 *   start_states and, when final_state is not NULL, the state after each
 *   sequence.
 * ssd_chunk_scan -- diagonal blocks plus left factors: Y = (L o C B^T) X within
 *   each chunk plus exp(cs) C h^T for the state h entering the chunk (paper
 *   section 6, "Diagonal Blocks" and "Left Factors"); inside a state block the
 *   stage advances h from chunk to chunk itself. Writes Y.
 */
ssd_status ssd_chunk_cumsum(const float* log_a, const int32_t* cu_seqlens, int32_t chunk,
                            int32_t state_block, const ssd_shape* shape, void* workspace,
                            size_t workspace_bytes, void* stream);
ssd_status ssd_chunk_state(const void* X, const void* B, const int32_t* cu_seqlens, int32_t chunk,
                           int32_t state_block, const ssd_shape* shape, void* workspace,
                           size_t workspace_bytes, void* stream);
ssd_status ssd_state_passing(const int32_t* cu_seqlens, const float* initial_state, int32_t chunk,
                             int32_t state_block, float* final_state, const ssd_shape* shape,
                             void* workspace, size_t workspace_bytes, void* stream);
ssd_status ssd_chunk_scan(const void* X, const void* B, const void* C, const int32_t* cu_seqlens,
                          int32_t chunk, int32_t state_block, void* Y, const ssd_shape* shape,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The Mamba-2 block's SSD call (paper card Method 6, the block sketch; Paper vs
 * code items 3, 7 and 8; Pitfalls, "Discretisation is missing from the
 * paper"). Instead of log a and a pre-scaled input, the block hands over raw
 * step sizes and per-head parameters, and the output is finished in the same
 * pass:
 *     dt'_t  = softplus(dt_t + dt_bias)          softplus(v) = log(1 + e^v)
 *     log a_t = dt'_t * A,   A = -exp(A_log)
 *     Y = SSM(a, B, C)(x * dt') + D * x           (the skip uses the unscaled x)
 *     Y = Y * silu(z),   silu(v) = v / (1 + e^-v) (when z is given)
 * final_state is the state of SSM(a, B, C)(x * dt'), as in ssd_fwd_ex, and
 * initial_state works as there.
 *   X        [batch, seqlen, nheads, headdim] dtype: the block's x, unscaled
 *   dt       [batch, seqlen, nheads] fp32: raw step sizes (before bias and softplus)
 *   dt_bias  [nheads] fp32, or NULL for zero
 *   A_log    [nheads] fp32
 *   D        [nheads] fp32, or NULL for no skip
 *   z        [batch, seqlen, nheads, headdim] dtype, or NULL for no gate
 * The other arguments are those of ssd_fwd_ex. The workspace layout is that of
 * ssd_fwd_layout, including key_cumsum. No separate stages are exposed for
 * this call. Errors as for ssd_fwd_ex; dt and A_log must not be NULL.
 */
ssd_status ssd_fwd_mamba2(const void* X, const float* dt, const float* dt_bias, const float* A_log,
                          const float* D, const void* z, const void* B, const void* C,
                          const int32_t* cu_seqlens, const float* initial_state, int32_t chunk,
                          int32_t state_block, void* Y, float* final_state, const ssd_shape* shape,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass: the gradients of L = <dY, Y> + <dfinal_state, final_state>
 * with respect to X, log_a, B, C and the initial state, for a forward pass
 * with the same arguments. The pages give no backward algorithm; this one is
 * the transpose of the forward terms (paper card Method 5 blocks; Method 3-4
 * duality):
 *   dX    = M^T dY with M = L o (C B^T): the same chunked algorithm run over
 *           each sequence reversed in time, with B and C exchanged and the log
 *           decays shifted by one token, starting from dfinal_state;
 *   dB, dC: the chunked algorithm with the roles of x, B, C and dY exchanged
 *           (state dimension P, head dimension N), per head, summed over the
 *           heads of each group;
 *   dlog_a[t] = a_t <lam_t, h_{t-1}>, the sum of dY_i . M_ij x_j over the
 *           pairs i >= t > j, computed chunk by chunk: the pairs inside the
 *           chunk in fp32, and the pairs that reach across its ends through
 *           the chunk's entering state (a forward run) and the adjoint at its
 *           end (the reversed run), with no cancellation between long sums;
 *   dinitial_state = a_first * (adjoint of the first state).
 * Arguments as for ssd_fwd_ex, plus
 *   dY             [batch, seqlen, nheads, headdim] dtype
 *   dfinal_state   fp32, final-state layout, or NULL (zero)
 * Outputs: dX (dtype, X's layout), dlog_a (fp32, log_a's layout), dB and dC
 * (dtype, B's layout), dinitial_state (fp32, may be NULL: not written).
 * Supported: the forward's sizes with dstate <= 128, headdim + dstate <= 192
 * and, for bf16, headdim >= 32 (the exchanged roles must themselves be
 * supported sizes), and the log-decay tiles within the LDS (fp32 with
 * headdim 64 and dstate 128 needs chunk <= 64). The forward outputs are not
 * needed: every term is recomputed from the inputs. The workspace holds
 * ssd_bwd_workspace_bytes(shape, chunk, state_block) bytes; dB and dC are
 * summed over heads in fp32 and rounded once.
 */
ssd_status ssd_bwd_workspace_bytes(const ssd_shape* shape, int32_t chunk, int32_t state_block, size_t* bytes);
ssd_status ssd_bwd(const void* X, const float* log_a, const void* B, const void* C, const int32_t* cu_seqlens,
                   const float* initial_state, const void* dY, const float* dfinal_state, int32_t chunk,
                   int32_t state_block, void* dX, float* dlog_a, void* dB, void* dC, float* dinitial_state,
                   const ssd_shape* shape, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of the Mamba-2 block's call (ssd_fwd_mamba2): the gradients of
 * L = <dY, y> + <dfinal_state, final_state> with respect to every input. The
 * chain rule runs through the gate, the skip and the discretisation (paper card
 * Method 6 block sketch; Paper vs code items 3, 7, 8) around ssd_bwd:
 *   dz = dY v silu'(z) with v the output before the gate, dv = dY silu(z);
 *   ssd_bwd of the recurrence on x dt' (rounded to the input dtype) and
 *   log a = dt' A with cotangent dv gives d(x dt'), d log a, dB, dC and the
 *   initial-state gradient;
 *   dX = d(x dt') dt' + D dv;  ddt = (sum_p d(x dt') x + A d log a) sig(dt + dt_bias);
 *   dD = sum dv x;  ddt_bias = sum_t ddt;  dA_log = A sum_t dt' d log a.
 * Inputs as for ssd_fwd_mamba2, plus dY [batch, seqlen, nheads, headdim]
 * (dtype) and dfinal_state (fp32, final-state layout, NULL for zero).
 * Outputs: dX, dz (dtype, X's layout; dz NULL exactly when z is NULL),
 * ddt [batch, seqlen, nheads] fp32, ddt_bias, dA_log, dD [nheads] fp32 (dD NULL
 * exactly when D is NULL; ddt_bias may be NULL), dB, dC (dtype, B's layout),
 * dinitial_state (fp32, optional). headdim must be a multiple of 8 (every
 * headdim ssd_fwd supports is) and the shape one that ssd_bwd supports. With a
 * gate the forward call runs once more (without the gate) for v, and where the
 * fused backward path applies that run's state tables serve ssd_bwd's forward
 * state run. The workspace must hold
 * ssd_bwd_mamba2_workspace_bytes(shape, chunk, state_block); it is all
 * overwritten. Same stream, alignment and error rules as ssd_bwd.
 */
ssd_status ssd_bwd_mamba2_workspace_bytes(const ssd_shape* shape, int32_t chunk, int32_t state_block,
                                          size_t* bytes);
ssd_status ssd_bwd_mamba2(const void* X, const float* dt, const float* dt_bias, const float* A_log, const float* D,
                          const void* z, const void* B, const void* C, const int32_t* cu_seqlens,
                          const float* initial_state, const void* dY, const float* dfinal_state, int32_t chunk,
                          int32_t state_block, void* dX, float* ddt, float* ddt_bias, float* dA_log, float* dD,
                          void* dz, void* dB, void* dC, float* dinitial_state, const ssd_shape* shape,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step for `batch` independent streams: the loop body of
 * the recurrence with a constant-size state (paper card Method 8 and its cost
 * table: about N^2 work per step; the page-1 summary: generation needs only a
 * constant-size state).
 *   state [batch, H, P, N] fp32, updated in place: s = exp(la) s + x B^T;
 *         16-byte aligned (SSD_ERR_INVALID_ARGUMENT otherwise)
 *   x [batch, H, P] dtype, log_a [batch, H] fp32, B, C [batch, G, N] dtype
 *   y [batch, H, P] dtype (written), read from the updated state.
 * shape->seqlen and shape->num_seqs are ignored.
 */
ssd_status ssd_step(float* state, const void* x, const float* log_a, const void* B, const void* C,
                    void* y, const ssd_shape* shape, void* stream);

/*
 * The Mamba-2 block's decode step (the loop body of ssd_fwd_mamba2):
 *   dt' = softplus(dt + dt_bias), state = exp(dt' A) state + (x dt') B^T,
 *   y = C^T state + D x, y = y * silu(z).
 *   state [batch, H, P, N] fp32 in place, 16-byte aligned; x, z [batch, H, P] dtype (z may be NULL);
 *   dt [batch, H] fp32 raw; dt_bias (may be NULL), A_log, D (may be NULL) [H] fp32;
 *   B, C [batch, G, N] dtype; y [batch, H, P] dtype (written).
 * A prompt run through ssd_fwd_mamba2 hands its final_state to this step.
 */
ssd_status ssd_step_mamba2(float* state, const void* x, const float* dt, const float* dt_bias,
                           const float* A_log, const float* D, const void* z, const void* B,
                           const void* C, void* y, const ssd_shape* shape, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
