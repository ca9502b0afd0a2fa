/*
 * replayssm.h -- C ABI of the batched SSM decode step served from a checkpoint
 * state plus a buffer of the last per-token records, for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (blog "ReplaySSM: an SSM decoder that writes its state once
 * every 16 tokens", sections "The identity" and "Output without a state"):
 * per head, the recurrent state S_t (d_v x d_k) of
 *     S_t = alpha_t S_{t-1} + x_t k_t^T,   o_t = S_t q_t
 * is kept as a checkpoint C plus the records (lam_j = log alpha_j, x_j, k_j)
 * of the tokens seen since C was written.  With w records buffered,
 *     S_t = gamma C + sum_j gamma_j x_j k_j^T + x_t k_t^T,
 * gamma and gamma_j being products of the alphas after the checkpoint and
 * after record j.  For Mamba-2 x_t = v_t.  For Gated DeltaNet (blog section
 * "The delta-rule wrinkle") x_t is the corrected value
 *     d_t = beta_t (v_t - alpha_t S_{t-1} k_t),
 * where S_{t-1} k_t and S_{t-1} q_t are both rebuilt from the checkpoint and
 * the records (vLLM pull request "[Kernel] ReplaySSM: cache SSM inputs for
 * faster Gated DeltaNet standard decode", reviewer comment on the
 * output-only route).
 *
 * A non-flush step reads C, computes o_t and appends one record.  A flush
 * step (every L-th token of a row, or when forced) folds the records and the
 * current token into C, writes C once and empties the buffer.
 *
 * Conventions for every function below:
 *   - Memory: the caller owns all device memory, including the block pool;
 *     the library allocates no device or pinned host memory.  Its only
 *     mutable global state is a mutex-guarded host cache of occupancy
 *     queries (resident workgroups per compute unit, per kernel and device:
 *     facts that do not change while the process runs), so it may be called
 *     from several host threads.
 *   - Device calls are asynchronous on `stream` (a hipStream_t; NULL means
 *     the default stream) and never synchronise the host.  All device
 *     pointers must stay valid until the work on `stream` has completed.
 *   - Errors: each function returns an rs_status.  Arguments are validated on
 *     the host before anything is launched; on error nothing is launched and
 *     rs_last_error() describes the problem.  Per-row metadata lives on the
 *     device, so its checks happen in the kernels: a tile whose block id or
 *     cursor is out of range is skipped (no reads, no writes) and counted in
 *     rs_batch.err_count when that pointer is non-NULL.
 *   - Pointer alignment: pool 256 bytes; q, k, v, out, log_decay, beta
 *     16 bytes; q/k/v strides must keep every (row, head) vector 16-byte
 *     aligned; block_table, write_pos, flush and reset masks 4 bytes (the
 *     byte arrays are read in aligned 32-bit words, never past the word that
 *     holds the last entry).
 *   - Sizes: n_rows <= 65535 per launch.  A layer's buffered records are
 *     staged in LDS and must fit one gfx950 workgroup's 160 KiB (every
 *     supported shape does, up to L = 64); a launch whose workgroups need
 *     more than 64 KiB also checks the device's own limit
 *     (hipDeviceAttributeMaxSharedMemoryPerBlock) and returns
 *     RS_EUNSUPPORTED if it is lower.
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RS_OK = 0,
    RS_EINVAL = -1,        /* bad argument: NULL/misaligned pointer, bad size or stride */
    RS_EUNSUPPORTED = -2,  /* valid request with no compiled kernel (shape or dtype)  */
    RS_EHIP = -3           /* the HIP runtime reported an error at launch             */
} rs_status;

/* RS_E4M3: OCP 8-bit floating point E4M3 (Open Compute Project "OCP 8-bit
 * Floating Point Specification (OFP8)"), valid only as a read_dtype. */
typedef enum { RS_F32 = 0, RS_F16 = 1, RS_BF16 = 2, RS_E4M3 = 3 } rs_dtype;

typedef enum {
    RS_MAMBA2 = 0,  /* S_t = alpha S_{t-1} + v k^T                       */
    RS_GDN = 1      /* Gated DeltaNet: S_t = alpha S_{t-1} + d k^T, d as above */
} rs_form;

/*
 * One SSM layer.  Supported (d_v, d_k): (16, 32), (64, 128), (128, 128).
 * L: buffer length in tokens, 1..64 (the pages' default is 16); a row holds
 *    at most L - 1 records, and its L-th token is a flush.
 * state_dtype:  RS_F32 or RS_F16 (checkpoint / conventional state).
 * record_dtype: RS_F32 or RS_F16 (buffered x and k; the log-decay is fp32).
 * io_dtype:     RS_F32, RS_F16 or RS_BF16 (q, k, v inputs).
 * spec_T:       0 for standard decoding.  T in {1, 2, 4, 8} (T <= L) makes a
 *               speculative layer (blog "Speculative decoding: rollback
 *               becomes a pointer"): its ring holds up to L committed records
 *               and each step verifies T draft tokens per row with
 *               replay_spec_verify; replay_decode_step rejects it.  An
 *               fp32 or fp16 checkpoint, or (Mamba-2) an fp32 recurrence
 *               copy with an RS_F16, RS_BF16 or RS_E4M3 read copy; keys per
 *               head or grouped (n_groups); (d_v, d_k) = (16, 32),
 *               (64, 128) or (128, 128) (an E4M3 read copy: not 16 x 32).
 * n_groups:     0 or n_heads for a key and a query per head.  A divisor
 *               G < n_heads shares one key and one query among each run of
 *               n_heads / G consecutive heads, the released grouped-key
 *               layout (blog "The identity", the paragraph on the released
 *               kernel: values and decays per value head, keys per group):
 *               q and k inputs are [n_rows][G][d_k] ([n_rows][T][G][d_k]
 *               for a speculative layer) and the ring keeps one key record
 *               per group, written by the group's first head.
 * state_rounding: RS_ROUND_NEAREST (nearest even) for every store.
 *               RS_ROUND_STOCHASTIC, with state_dtype RS_F16 only: every
 *               store of the fp16 checkpoint, state or recurrence copy (a
 *               flush, a token-less flush, a conventional step, the flush of
 *               a speculative verify; an E4M3 read copy is still rounded to
 *               nearest even, from the same unrounded values)
 *               rounds each value x up to the next fp16 neighbour exactly
 *               when the value's 16-bit random word r is below p 2^16,
 *               p = (|x| - lo) / (hi - lo) for the fp16 neighbours
 *               lo <= |x| < hi (so E[stored] = x for every fp32 value from
 *               2^-17 up, where p is a multiple of 2^-13 or finer; fp16
 *               values, |x| >= 65504 and non-finite values round to nearest
 *               even).  Words come from Philox4x64-10 (Salmon et al.,
 *               "Parallel random numbers: as easy as 1, 2, 3", SC 2011)
 *               under key (batch->sr_key0, batch->sr_key1): element e
 *               (row-major within its (row, head) tile t = row * n_heads +
 *               head) uses 16-bit word e mod 16 (the 64-bit outputs split
 *               least significant half-word first) of the block for counter
 *               (batch->sr_step, t, e / 16, 0).  Launches that store must
 *               not repeat an sr_step under one key.  The blog ("The
 *               precision argument, derived") keeps the recurrence copy in
 *               FP16 with stochastic rounding, so that rounding enters the
 *               recurrence unbiased and once per window.
 * gdn_route:    Gated DeltaNet only.  RS_GDN_OUTPUT_ONLY (the PR reviewer's
 *               form): S_{t-1} q and S_{t-1} k come from C q, C k and the
 *               scalars k_j . q, k_j . k of the buffered keys, and the state
 *               is never formed on a non-flush step.  RS_GDN_RECONSTRUCT
 *               (the PR's kernel, "Core concept": the state is rebuilt from
 *               the checkpoint and the buffer): every step rebuilds
 *               S_{t-1} = P C + sum_j p_j d_j k_j^T in registers and reads
 *               both products from it.  Both routes store the same records
 *               and checkpoints and agree in real arithmetic; the second
 *               does w d_v d_k more multiply-adds per tile per step.
 * read_dtype:   -1 (or state_dtype) for a single checkpoint; for a
 *               two-precision checkpoint (blog "The precision argument,
 *               derived") RS_F16, RS_BF16 or RS_E4M3 over an RS_F32
 *               recurrence copy (state_dtype), or RS_E4M3 over an RS_F16
 *               one (the pages' preferred pairing: an FP16 recurrence copy
 *               with stochastic rounding and a coarse read copy): the
 *               recurrence copy is read by flushes only; a second copy in
 *               read_dtype is what non-flush steps read.  A flush folds from
 *               the recurrence copy and rewrites both copies from the same
 *               unrounded values, so the read copy's rounding never enters
 *               the recurrence.  Mamba-2 form only (RS_EUNSUPPORTED for GDN:
 *               its buffered corrections would carry the read copy's error).
 *               Read copies round to nearest even.  An RS_E4M3 read copy
 *               scales each state row (the d_k entries of one output
 *               component) by its own power of two 2^e, e the smallest
 *               integer with max|row| * 2^-e <= 448 (and at least -100): it
 *               stores E4M3(row * 2^-e) and the fp32 scale 2^e.
 */
typedef struct {
    int32_t form;
    int32_t n_heads;
    int32_t d_v;
    int32_t d_k;
    int32_t L;
    int32_t state_dtype;
    int32_t record_dtype;
    int32_t io_dtype;
    int32_t read_dtype;
    int32_t spec_T;   /* 0: standard decoding; 1, 2, 4 or 8: speculative layer,
                         see replay_spec_verify */
    int32_t n_groups; /* 0 (= n_heads): one key and query per head; else the
                         number of key groups, see below */
    int32_t state_rounding; /* RS_ROUND_NEAREST or RS_ROUND_STOCHASTIC, see below */
    int32_t gdn_route;      /* RS_GDN_OUTPUT_ONLY or RS_GDN_RECONSTRUCT, see below */
} rs_layer;

/* Rounding of state stores (rs_layer.state_rounding). */
typedef enum { RS_ROUND_NEAREST = 0, RS_ROUND_STOCHASTIC = 1 } rs_rounding;

/* How a Gated DeltaNet non-flush step forms S_{t-1} q and S_{t-1} k
 * (rs_layer.gdn_route; must be RS_GDN_OUTPUT_ONLY for Mamba-2). */
typedef enum { RS_GDN_OUTPUT_ONLY = 0, RS_GDN_RECONSTRUCT = 1 } rs_gdn_route;

/*
 * Byte layout of one paged block = the whole per-request state of one layer
 * (vLLM pull request above, "Paged cache layout": checkpoint and record
 * buffers live in the request's paged block behind its block table).
 * Offsets are from the block start; every region starts 256-byte aligned.
 *   ckpt     [n_heads][d_v][d_k]    state_dtype, row-major per head
 *   rec_x    [n_heads][slots][d_v]  record_dtype
 *   rec_k    [n_groups][key_slots][d_k] record_dtype (n_groups =
 *                                   n_heads unless the layer groups its
 *                                   keys)
 *   rec_lam  [n_heads][slots]       fp32 log-decay
 *   ckpt_lo  [n_heads][d_v][d_k]    read_dtype (two-precision checkpoint only;
 *                                   ckpt_lo_off is 0 otherwise), each row of
 *                                   d_k elements in lane order: with n read
 *                                   and m recurrence-copy elements per 16
 *                                   bytes (m = 4 for fp32, 8 for fp16),
 *                                   stored position p (chunk c = p / n,
 *                                   e = p mod n) holds column
 *                                   m (c + (d_k / n) floor(e / m)) + e mod m,
 *                                   so that both copies are read and
 *                                   written with contiguous accesses
 *   ckpt_sc  [n_heads][d_v]         fp32 row scales of an RS_E4M3 read copy
 *                                   (ckpt_scale_off is 0 otherwise)
 * slots = L - 1 (a speculative layer: slots = L).  key_slots = slots, except
 * on a speculative layer with grouped keys (n_groups < n_heads): L + T, the
 * last T holding the drafts of a row that flushed in its verify until
 * replay_spec_commit moves the accepted ones to slots 0.. (the verify cannot
 * write them there itself: other heads of the group may still be reading the
 * committed keys).  block_bytes is a multiple of 256.
 */
typedef struct {
    int64_t ckpt_off;
    int64_t rec_x_off;
    int64_t rec_k_off;
    int64_t rec_lam_off;
    int64_t block_bytes;
    int32_t slots;
    int32_t key_slots;
    int64_t ckpt_lo_off;
    int64_t ckpt_scale_off;
} rs_block_layout;

/* Host, pure.  Fills *out for `layer`.  RS_EINVAL / RS_EUNSUPPORTED on a bad
 * or uncompiled layer (the same checks as the device calls). */
int rs_block_layout_get(const rs_layer* layer, rs_block_layout* out);

/*
 * One decode batch.  All arrays are device memory with n_rows entries.
 *   pool        n_blocks * block_bytes bytes (rs_block_layout_get).
 *   block_table row -> block id in [0, n_blocks); -1 marks a padding row,
 *               which is neither read nor written (its outputs are left as
 *               they were).
 *   write_pos   records held by the row, 0..L-1 (the write cursor of the
 *               vLLM pull request, "CUDA graphs and continuous batching"),
 *               optionally with RS_CURSOR_ZERO_CKPT set: the row's checkpoint
 *               is zero and its stored values are never used (a request that
 *               joined the batch and has not flushed yet; its block's
 *               checkpoint region may hold anything).  replay_decode_step and
 *               replay_flush treat the checkpoint as zero for such a row; its
 *               first flush writes the checkpoint, and next_write_pos carries
 *               the bit until then.  This replaces replay_state_reset for a
 *               joining row (one launch fewer).  The one-workgroup kernels
 *               read only the first 16 bytes of such a checkpoint (one cache
 *               line, so that no load sits under a branch); the persistent
 *               non-flush form streams it and discards it.
 *               Not for speculative layers (their counts must be 0..L) or
 *               conventional_decode_step (which reads no cursor).
 *   flush       nonzero: this step folds the row into its checkpoint.  A row
 *               at write_pos == L-1 flushes whatever its flag says.  May be
 *               NULL (no forced flushes).
 *   err_count   optional (may be NULL): incremented once per (row, head) tile
 *               skipped because its block id or cursor was out of range.
 *   next_write_pos  optional (may be NULL), replay_decode_step only: receives
 *               each non-padding row's cursor for the next step, 0 after a
 *               flush and write_pos + 1 otherwise (the host rule of
 *               rs_meta_advance), with RS_CURSOR_ZERO_CKPT kept on a row
 *               that did not flush.  Passing it as the next step's write_pos
 *               lets a caller skip the per-step host -> device copy while
 *               the batch is unchanged.  Must not alias write_pos.
 *   flush_hint  replay_decode_step only: what the caller knows of this
 *               step's flushing rows (rs_flush_hint).  RS_FLUSH_UNKNOWN (0)
 *               runs one kernel over all rows.
 *               Two-precision checkpoints: RS_FLUSH_NONE promises that no row
 *               flushes and runs a kernel built without the fold;
 *               RS_FLUSH_ALL promises that every non-padding row flushes;
 *               RS_FLUSH_MIXED runs the no-fold kernel over the rows that do
 *               not flush and then the full kernel over those that do.
 *               Mamba-2 with one fp32 checkpoint and a key per head
 *               (n_groups 0 or n_heads): RS_FLUSH_NONE runs a
 *               persistent kernel without the fold that streams the
 *               checkpoint tiles with the next tile's loads in flight and
 *               stores the outputs and records after the stream; the other
 *               hints are not used.  Other layers do not use the hint.
 *               Where a hint is used, a row that breaks its promise is
 *               skipped and counted in err_count (never computed wrongly).
 */
/* write_pos flag: the row's checkpoint is zero and is not read (above). */
#define RS_CURSOR_ZERO_CKPT (1 << 30)

typedef enum {
    RS_FLUSH_UNKNOWN = 0,
    RS_FLUSH_NONE = 1,
    RS_FLUSH_ALL = 2,
    RS_FLUSH_MIXED = 3
} rs_flush_hint;

typedef struct {
    int32_t n_rows;
    int32_t flush_hint;
    int64_t n_blocks;
    void* pool;
    const int32_t* block_table;
    const int32_t* write_pos;
    const uint8_t* flush;
    int32_t* err_count;
    int32_t* next_write_pos;
    uint64_t sr_key0, sr_key1;  /* stochastic rounding: Philox key          */
    uint64_t sr_step;           /* stochastic rounding: first counter word,
                                   a new value for every launch that stores */
} rs_batch;

/*
 * One token per row.  q, k: [n_rows][n_heads][d_k] ([n_rows][n_groups][d_k]
 * for a layer with grouped keys, the "head" stride then being the group
 * stride); v: [n_rows][n_heads][d_v]; all io_dtype, unit stride along the
 * last dimension, row and head strides in ELEMENTS (so strided views into a
 * wider projection output work).
 * log_decay: [n_rows][n_heads] fp32, lam = log alpha <= 0 (Mamba-2) or the
 * gate g (Gated DeltaNet); -inf is allowed and means alpha = 0.
 * beta: [n_rows][n_heads] fp32, Gated DeltaNet only (NULL for Mamba-2).
 * out:  [n_rows][n_heads][d_v] fp32, contiguous; written for non-padding rows.
 */
typedef struct {
    const void* q;
    const void* k;
    const void* v;
    int64_t q_row_stride, q_head_stride;
    int64_t k_row_stride, k_head_stride;
    int64_t v_row_stride, v_head_stride;
    const float* log_decay;
    const float* beta;
    float* out;
} rs_step_io;

/*
 * Checkpoint + buffer decode step (blog, "The identity" and "Output without a
 * state"; vLLM pull request, "Core concept").  One launch serves every row:
 *   non-flush row: out = S_t q_t rebuilt from the checkpoint and the w
 *                  buffered records; record w <- (lam, x, k) cast to
 *                  record_dtype (round to nearest even); checkpoint untouched.
 *   flush row:     out as above; checkpoint <- S_t (the records and the
 *                  current token folded in), stored once in state_dtype
 *                  (round to nearest even); no record is written.  The caller
 *                  then sets the row's write_pos to 0.
 * Buffer slots >= write_pos are never read.  With a two-precision checkpoint
 * a non-flush row reads only the read copy (its output differs from the
 * single-checkpoint output by G (C_lo - C) q, one rounding of the last
 * checkpoint); a flush row reads the recurrence copy and writes both.
 */
int replay_decode_step(const rs_layer* layer, const rs_batch* batch, const rs_step_io* io,
                       hipStream_t stream);

/*
 * Token-less flush: for every non-padding row whose flush flag is set, fold
 * its write_pos records into its checkpoint (S = gamma C + sum_j gamma_j x_j
 * k_j^T, blog "The identity" with h = write_pos; from and into the recurrence
 * copy, the read copy rewritten from the same values).  Rows whose flag is clear
 * are untouched.  This materialises the exact state at any step: before a row
 * is retired or preempted, or at a prefix-cache block boundary (vLLM pull
 * request, "What this PR adds", align mode).  batch->flush must not be NULL.
 * On a speculative layer (spec_T > 0) write_pos is the row's committed count
 * h (0..L) and its h committed records are folded; the caller then sets h to
 * 0 in the count array its next verify reads.
 */
int replay_flush(const rs_layer* layer, const rs_batch* batch, hipStream_t stream);

/*
 * Conventional decode step (blog, "Why a fixed-size state is not cheap to
 * decode"; "The delta-rule wrinkle" for Gated DeltaNet): the checkpoint
 * region of each block holds the full state S, which is read, updated and
 * written back on every step; out = S_t q_t.  write_pos and flush are
 * ignored (may be NULL); record_dtype is unused.  With a two-precision layer
 * it works on the recurrence copy alone and leaves the read copy untouched.
 */
int conventional_decode_step(const rs_layer* layer, const rs_batch* batch, const rs_step_io* io,
                             hipStream_t stream);

/*
 * Zero the checkpoint (both copies of a two-precision checkpoint) of every
 * non-padding row whose mask entry (device uint8 [n_rows]) is nonzero: the
 * state of a request that joins the batch.
 * Its write_pos must start at 0; stale records need no clearing because
 * slots at or beyond write_pos are never read (vLLM pull request, "CUDA
 * graphs and continuous batching").  Implemented as a kernel, not a memset,
 * so it may be captured in a HIP graph.
 */
int replay_state_reset(const rs_layer* layer, const rs_batch* batch, const uint8_t* mask,
                       hipStream_t stream);

/*
 * Host metadata for one step (vLLM pull request, "CUDA graphs and continuous
 * batching": the write position is the row's decode step counted from its
 * anchor, modulo L; a row flushes at position L-1 or when a flush is forced,
 * e.g. on the step that completes a prefix-cache block).  Host arrays of
 * n_rows:
 *   steps_since_anchor  in:  decode steps since the row's anchor; < 0 = pad row
 *   force_flush         in:  nonzero forces a flush this step (may be NULL)
 *   write_pos           out: steps_since_anchor mod L (0 for pad rows)
 *   flush               out: 1 if the row flushes this step (0 for pad rows)
 * The caller copies write_pos and flush to the device.  RS_EINVAL on NULL
 * output pointers, n_rows < 0 or L outside 1..64.
 */
int rs_meta_step(int32_t L, int32_t n_rows, const int32_t* steps_since_anchor,
                 const uint8_t* force_flush, int32_t* write_pos, uint8_t* flush);

/*
 * Host: advance the per-row anchors after a step: a row that flushed is
 * re-anchored (0), any other live row counts one more step; pad rows (< 0)
 * stay as they are.  Re-anchoring a resumed or re-joined row is the caller
 * setting its entry to 0 (after replay_flush or replay_state_reset).
 */
int rs_meta_advance(int32_t L, int32_t n_rows, int32_t* steps_since_anchor, const uint8_t* flush);

/*
 * Speculative decoding (blog "Speculative decoding: rollback becomes a
 * pointer"; NVIDIA technical blog "ReplaySSM: Rethinking state storage for
 * faster hybrid model decoding", "Benefit 2: Simplify rollback and speed up
 * verification").  A row of a speculative layer holds a checkpoint C and h
 * committed records (batch->write_pos = h, 0..L).  One verify step takes T
 * draft tokens per row, (lam_i, v_i, k_i, q_i), i = 1..T, and computes the
 * output every draft would have if drafts 1..i were accepted:
 *     o_i = D_i (G C q_i + sum_j g_j (k_j . q_i) v_j) + sum_{m<=i} W_im (k_m . q_i) v_m
 * with G, g_j the decay products of the committed records after the
 * checkpoint and after record j, D_i the product of the draft decays 1..i
 * and W_im the product of draft decays m+1..i (a causal mask).  The
 * checkpoint is read once for all T queries and no state is formed.  The T
 * drafts are stored as records behind the committed ones (slots h..h+T-1).
 * A row whose ring has no room for T more records (h + T > L), or whose flag
 * is set, flushes first: its h committed records (only those) are folded into
 * the checkpoint, which is written once, and the drafts are stored from slot
 * 0 (with grouped keys, the drafts' keys go to the staging slots L..L+T-1
 * until the commit; see key_slots).  This needs no acceptance count, so it
 * happens in the same launch.  With a two-precision checkpoint a row that
 * does not flush reads the read copy (and its row scales) for the C q_i
 * term, and a flushing row reads the recurrence copy, folds in fp32 and
 * rewrites both copies from the same unrounded values, as in
 * replay_decode_step.
 * After sampling, replay_spec_commit advances each row's committed count by
 * the number of drafts accepted; records past it are never read and get
 * overwritten.
 *
 * Gated DeltaNet (blog "The delta-rule wrinkle"): records hold corrected
 * values u, and a draft's u_i = beta_i (v_i - alpha_i S_{i-1} k_i) depends on
 * the drafts before it, a T x T triangular system.  With S_h the committed
 * state (checkpoint plus committed records, never formed) read at k_i and q_i:
 *     u_i = beta_i (v_i - D_i S_h k_i) - beta_i sum_{m<i} W_im (k_m . k_i) u_m
 *     o_i = D_i S_h q_i + sum_{m<=i} W_im (k_m . q_i) u_m
 * solved draft by draft; the drafts' u_i are stored as their records.
 * Heads of 16 x 32, 64 x 128 and 128 x 128, both forms.
 *
 * q, k: [n_rows][T][n_heads][d_k] ([n_rows][T][n_groups][d_k] with grouped
 * keys); v: [n_rows][T][n_heads][d_v], io_dtype,
 * unit stride along the last dimension, row / token / head strides in
 * elements; log_decay (and beta): [n_rows][T][n_heads] fp32 contiguous; out:
 * [n_rows][T][n_heads][d_v] fp32 contiguous.
 */
typedef struct {
    const void* q;
    const void* k;
    const void* v;
    int64_t q_row_stride, q_token_stride, q_head_stride;
    int64_t k_row_stride, k_token_stride, k_head_stride;
    int64_t v_row_stride, v_token_stride, v_head_stride;
    const float* log_decay;
    float* out;
    const float* beta;  /* Gated DeltaNet: [n_rows][T][n_heads] fp32 contiguous; NULL for Mamba-2 */
} rs_spec_io;

/*
 * Verify step of a speculative layer (layer->spec_T = T).  batch->write_pos:
 * committed records per row; batch->flush: may be NULL, a nonzero entry
 * forces the row to flush; batch->next_write_pos is not used.  Padding rows
 * (block id -1) are neither read nor written.  A row whose metadata is out of
 * range is skipped and counted in err_count.
 */
int replay_spec_verify(const rs_layer* layer, const rs_batch* batch, const rs_spec_io* io,
                       hipStream_t stream);

/*
 * Commit after a verify step, on the device: for every non-padding row,
 * h' = (flushed ? 0 : h) + accepted[row], where flushed is the verify's
 * decision for that row (its flag, or h + T > L); writes h' to
 * batch->next_write_pos and next_flush[row] = (h' + T > L).  Passing
 * (next_write_pos, next_flush) as the next verify's (write_pos, flush) keeps
 * the cursor on the device.  accepted: device int32 [n_rows], 0..T; a row
 * with another value commits nothing and is counted in err_count.  With
 * grouped keys, a row that flushed also has its accepted drafts' keys moved
 * from the staging slots L.. to slots 0.. of each group (see key_slots): the
 * verify of a flushing row leaves them there, so the commit must run before
 * the row's next verify or token-less flush, on the same stream.
 * batch->next_write_pos and next_flush must not alias write_pos / flush.
 */
int replay_spec_commit(const rs_layer* layer, const rs_batch* batch, const int32_t* accepted,
                       uint8_t* next_flush, hipStream_t stream);

/*
 * Host mirror of the speculative cursor, for callers that keep it on the
 * host.  rs_spec_meta_step: flush[r] = 1 if committed[r] + T > L or
 * force[r] != 0 (force may be NULL), 0 for padding rows (committed < 0).
 * rs_spec_meta_advance: committed[r] = (flush[r] ? 0 : committed[r]) +
 * accepted[r] for non-padding rows, in place.  RS_EINVAL on NULL arrays,
 * n_rows < 0, L outside 1..64, T outside 1..L, or an accepted count of a
 * non-padding row outside 0..T (checked for every row first: on error no
 * row is updated; the device commit skips and counts such a row).
 */
int rs_spec_meta_step(int32_t L, int32_t T, int32_t n_rows, const int32_t* committed,
                      const uint8_t* force, uint8_t* flush);
int rs_spec_meta_advance(int32_t L, int32_t T, int32_t n_rows, int32_t* committed,
                         const uint8_t* flush, const int32_t* accepted);

/* Host: RS_OK if a kernel is compiled for this layer, else the reason code. */
int rs_layer_supported(const rs_layer* layer);

/* Host: description of the last error raised on the calling thread ("" if none). */
const char* rs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
