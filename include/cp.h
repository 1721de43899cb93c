/*
 * cp.h -- C ABI of libcp: chunked prefill with past on MI355X (gfx950).
 *
 * One transformer layer's hot path for a chunk of C prompt tokens padded to
 * a fixed C, against an external KV cache:
 *
 *   cp_rope_chunk (Q)  -> cp_rope_chunk (K) -> [cp_kv_snapshot_padded_append]
 *   -> cp_attn_chunk_with_past -> cp_kv_append -> [cp_kv_rollback_padded_append]
 *   -> cp_select_row
 *
 * or, with fewer launches, cp_rope_qk_chunk -> [snapshot] -> cp_attn_chunk_with_past
 * with select_out set -> cp_kv_append -> [rollback];
 * or, for a global cache, cp_rope_qk_append_chunk (which also writes the chunk's
 * K/V rows past seen) -> cp_attn_chunk_with_past with CP_ATTN_ADVANCE_SEEN and
 * select_out set: two calls, two to three launches.
 *
 * Sources:
 *   [SKaiNET] SKaiNET-transformers PR #417, "functiongemma: chunk prefill-with-
 *             past graph gemma_prefill_with_past", section "Change (additive)":
 *             heads-first [heads, C, headDim] tensors, RoPE from per-position
 *             [C, headDim] cos/sin tables, attention over past + C keys with an
 *             additive per-head mask [1, nHeads, C, past+C] (0 attends, -1e30
 *             masks; it carries the causal band, the zero padding and the
 *             sliding window), K/V extended by the chunk, one selected row;
 *             section "Validation": select on row 51 of a 52-token chunk.
 *   [TICO]    Samsung/TICO issue #586, "Enable prefill-decode modeling",
 *             sections "Runtime behavior" and "Mask/cache layout used in the
 *             runtime": the KV cache is owned by the runtime, outside the
 *             graph; past tokens packed in the first past_len slots; the
 *             runtime writes the delta K/V into the external cache.
 *   [Kazeia]  Kazeia-engine docs, "Chantier 4 -- GDN chunkwise prefill":
 *             the gated delta rule of linear-attention layers and its chunkwise
 *             form (cp_gdn_chunk_prefill).
 *   [cactus]  cactus PR #716, "Pad the chunked-prefill tail for sliding-window
 *             models", section "Fix" and the review hardening: sliding caches
 *             evict chronologically; a padded append over-evicts up to
 *             pad_count of the oldest window rows; snapshot/rollback of a
 *             padded append leaves the cache byte-identical to an unpadded
 *             prefill; windows with window <= chunk + sink are rejected; bytes
 *             beyond the live length are a dead region no consumer reads.
 *
 * Conventions (all entry points):
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     allocates nothing, frees nothing, keeps no global mutable state and
 *     never synchronises the stream.  `stream` is a hipStream_t passed as an
 *     opaque pointer (NULL = the default stream); all work is enqueued on it.
 *   - Tensors are dense, row-major, last dimension contiguous.  Storage
 *     dtypes: CP_F32 (float) or CP_BF16 (bfloat16 bit patterns).
 *   - Empty work (a zero extent) is a no-op that returns CP_OK; the data
 *     pointers of empty tensors may then be NULL.
 *   - Return value: CP_OK (0) or a negative CP_ERR_* code.  Every error a
 *     host can detect (null pointers, bad shapes, dtypes, window guard,
 *     snapshot state, workspace size) is detected before anything is
 *     enqueued, so a failing call has no effect.  Values that live on the
 *     device (seen, n_valid) are checked by the kernels: they never read or
 *     write out of bounds, skip or clamp the offending sequence, and OR a
 *     CP_DEV_* bit into cache->status when that pointer is non-NULL.
 *   - Calls on one stream are ordered; calls that touch the same cache on
 *     different streams must be ordered by the caller.
 */
#ifndef CP_H
#define CP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *cp_stream_t; /* hipStream_t */

/* ---- status codes returned by every entry point ---- */
#define CP_OK 0
#define CP_ERR_ARG (-1)       /* null pointer or out-of-range scalar argument */
#define CP_ERR_SHAPE (-2)     /* unsupported or inconsistent shape (D odd, H % nKV, C > cap, ...) */
#define CP_ERR_DTYPE (-3)     /* dtype not CP_F32 / CP_BF16, or not supported by the call */
#define CP_ERR_WINDOW (-4)    /* ring with cap <= C + sink cannot take a padded append */
#define CP_ERR_STATE (-5)     /* rollback without a matching, armed snapshot */
#define CP_ERR_WORKSPACE (-6) /* workspace or snapshot buffer too small */
#define CP_ERR_HIP (-7)       /* the HIP runtime refused a launch */
#define CP_ERR_SCRATCH (-8)   /* the call needs more than the library's fixed scratch array */

/* ---- bits the kernels OR into cache->status (device int32) ---- */
#define CP_DEV_OVERFLOW 1 /* global append would pass cap: that sequence was not appended */
#define CP_DEV_NVALID 2   /* n_valid / n_rows outside [0, C]: clamped */
#define CP_DEV_MASK_LD 4  /* explicit mask narrower than live past + C: rows written as 0 */
#define CP_DEV_ROLLBACK 8 /* rollback on a sequence that did not take exactly C rows */
#define CP_DEV_SEEN 16    /* seen negative, or above cap for a global cache: sequence skipped */

/* ---- storage dtypes ---- */
#define CP_F32 0
#define CP_BF16 1

/*
 * External KV cache of one layer ([TICO] "Mask/cache layout"; [cactus] "Fix").
 *
 *   k, v    [B, nKV, cap, D] storage dtype.  Global cache (ring = 0): absolute
 *           position p lives in slot p, p < cap.  Sliding ring (ring = 1):
 *           `sink` pinned slots hold positions 0..sink-1; position p >= sink
 *           lives in slot sink + (p - sink) mod (cap - sink), so appending
 *           evicts the oldest non-sink row.  Slots that hold no live row are
 *           the dead region: never read, contents unspecified.
 *   seen    device int32 [B]: positions absorbed so far by each sequence.
 *           Live rows: global [0, seen); ring the sink rows below
 *           min(sink, seen) and positions [max(sink, seen - (cap - sink)), seen).
 *   status  device int32 or NULL: sticky CP_DEV_* error bits.
 *   sink    pinned rows (0 for none): positions below sink are attended
 *           regardless of the window.  A ring never evicts them; a global cache
 *           never evicts anything, so there it only widens what a windowed
 *           attention reads.
 */
typedef struct cp_cache {
  void *k;
  void *v;
  int32_t *seen;
  int32_t *status;
  int32_t B, nKV, cap, D;
  int32_t dtype;
  int32_t ring;
  int32_t sink;
  int32_t reserved; /* must be 0 */
} cp_cache;

/*
 * Snapshot of the rows a padded ring append would over-evict ([cactus]
 * "Fix": snapshot_cache_padded_append / rollback_cache_padded_append).
 * `buf` is a caller-owned device buffer of at least cp_snapshot_bytes()
 * bytes.  The other fields are filled by cp_kv_snapshot_padded_append and
 * consumed by cp_kv_rollback_padded_append; initialise them to zero.
 */
typedef struct cp_snapshot {
  void *buf;
  size_t bytes;
  const void *cache_k; /* identity of the cache the snapshot was taken from */
  int32_t C;
  int32_t armed; /* 1 between a snapshot and its rollback */
} cp_snapshot;

/*
 * Arguments of the chunk attention ([SKaiNET] "Change (additive)":
 * attnWithPastChunk).
 *
 *   q          [B, H, C, D]   queries, RoPE already applied
 *   k_new      [B, nKV, C, D] the chunk's keys, RoPE already applied
 *   v_new      [B, nKV, C, D] the chunk's values
 *   out        [B, H, C, D]   output, storage dtype; pad rows written as 0
 *   n_valid    device int32 [B] real rows per sequence (rows >= n_valid are
 *              padding), or NULL when all C rows are real
 *   mask       NULL: the mask is computed in the kernel from seen, n_valid,
 *              window and sink (causal inside the chunk, pad keys masked,
 *              sliding window of `window` positions counting the query).
 *              Otherwise an explicit fp32 additive mask: element (b, h, i, col)
 *              at mask[b*mask_batch_stride + h*mask_head_stride + i*mask_ld
 *              + col]; columns are the live past rows in chronological order
 *              then the C chunk rows; mask_ld >= live past + C (a sequence
 *              that violates this is flagged CP_DEV_MASK_LD and zeroed).
 *              A head stride of 0 broadcasts one mask over the heads.
 *   workspace  optional device scratch for the key-split path; size from
 *              cp_attn_workspace_bytes().  With less, the call runs unsplit.
 *   H          query heads (multiple of cache->nKV; head h reads KV head
 *              h / (H / nKV))
 *   C          chunk rows
 *   window     sliding window in positions (0 = none); in-kernel mask only
 *   scale      softmax scale (> 0) applied to q.k before the mask is added
 *   flags      CP_ATTN_* below
 *   select_out optional [B, H, D] storage dtype: also receives row
 *              max(n_valid[b], 1) - 1 of out for every (b, h) -- the last real
 *              row ([SKaiNET] "Validation": row 51 of a 52-token chunk), zeros
 *              for a sequence without real rows -- bit-identical to
 *              cp_select_row(out, n_valid, -1) for n_valid in [0, C] (n_valid
 *              NULL selects row C - 1).  Not written when C = 0.
 *   q_cos, q_sin  NULL: q is already rotated.  Otherwise q holds the chunk's queries
 *              BEFORE RoPE and the kernel rotates them as it loads them, with these
 *              fp32 [q_tables, C, D] tables (q_tables = 1 shares one table over the
 *              batch, q_tables = B gives each sequence its own) -- bit-identical to
 *              cp_rope_chunk(q) followed by the call with the rotated q ([SKaiNET]
 *              "Change (additive)": RoPE from per-position tables; here folded into
 *              the attention's load of Q, so the rotated queries never go to memory).
 *   max_seen   0, or an upper bound on every sequence's seen that the caller knows on
 *              the host (a serving scheduler holds the lengths; the device counters
 *              are not read back).  The host planner sizes the key splits from it
 *              instead of from the capacity, so that a past much shorter than the
 *              cache does not get more splits than it has key tiles.  It chooses the
 *              split count only: every sequence's keys are still divided on the device
 *              by its own live length, so a bound below some seen is not an error
 *              (the results are those of a call with that split count).  Negative:
 *              CP_ERR_ARG.
 *
 * The cache is read as it stands BEFORE the chunk is appended.
 */
typedef struct cp_attn_args {
  const void *q;
  const void *k_new;
  const void *v_new;
  void *out;
  const int32_t *n_valid;
  const float *mask;
  int64_t mask_ld;
  int64_t mask_head_stride;
  int64_t mask_batch_stride;
  void *workspace;
  size_t workspace_bytes;
  int32_t H;
  int32_t C;
  int32_t window;
  float scale;
  uint32_t flags;
  int32_t reserved; /* must be 0 */
  void *select_out;
  const float *q_cos;
  const float *q_sin;
  int32_t q_tables;
  int32_t max_seen;
} cp_attn_args;

#define CP_ATTN_NO_SPLIT 1u      /* one pass per query tile, no key split */
#define CP_ATTN_FORCE_GENERIC 2u /* use the vector-ALU kernel even for bf16 */
#define CP_ATTN_FULL_TILES 4u    /* visit every key tile and apply the mask on each, as the
                                    explicit-mask path does (same partition, same expressions) */
/* Force the number of key splits to n (1..64; needs the workspace for n) instead of
   the planner's choice.  Placed in bits 8..15 of flags. */
#define CP_ATTN_SPLITS(n) (((uint32_t)(n) & 0xffu) << 8)
/* After reading the cache, advance seen[b] by n_valid[b] as cp_kv_advance does (for a
   chunk whose rows cp_rope_qk_append_chunk already wrote): inside the split merge when
   the keys are split, else by one small launch after the attention. */
#define CP_ATTN_ADVANCE_SEEN 8u
/* Balance the work of a batch whose past lengths differ: a one-workgroup kernel reads the
   lengths on the device, cuts each sequence's keys into pieces by its own length (no
   piece shorter than the total over the workgroups the GPU holds at once), orders them
   longest first, and a merge combines the cut rows; the other rows are written directly
   (the bf16 matrix-core kernel's standard configuration, up to 1024 sequences; otherwise
   the flag is ignored).  Needs the workspace cp_attn_workspace_bytes() returns with it;
   with less the call runs unbalanced.  Three launches (plan, attention, merge). */
#define CP_ATTN_BALANCE 16u

/* ---- introspection ---- */

/* Text of a CP_OK / CP_ERR_* code. */
const char *cp_status_str(int status);

/* ABI version of this header (bumped on any layout change). */
int cp_abi_version(void);

/* sizeof of the ABI structs: which = 0 cp_cache, 1 cp_snapshot, 2 cp_attn_args. */
size_t cp_struct_size(int which);

/* ---- RoPE ---- */

/*
 * Rotary embedding from caller-supplied per-position tables ([SKaiNET]
 * "Change (additive)"; [TICO] "Runtime behavior": (cos_t, sin_t) at the
 * absolute position).  Half-split pairing, j < D/2:
 *   y[j]     = x[j]     * cos[j]     - x[j+D/2] * sin[j]
 *   y[j+D/2] = x[j+D/2] * cos[j+D/2] + x[j]     * sin[j+D/2]
 * evaluated in fp64 on the exact fp32 operands, rounded to fp32, then to
 * the storage dtype (bf16: round to nearest even).
 *
 *   x, y   [B, Hx, C, D] storage dtype; y may equal x (in place)
 *   cos, sin  fp32 [Bt, C, D]; Bt = 1 shares one table over the batch,
 *          Bt = B gives each sequence its own positions
 * Errors: CP_ERR_ARG (null, negative sizes, Bt not 1 or B),
 *         CP_ERR_SHAPE (D odd), CP_ERR_DTYPE.
 */
int cp_rope_chunk(const void *x, void *y, const float *cos, const float *sin, int B, int Hx,
                  int C, int D, int Bt, int dtype, cp_stream_t stream);

/*
 * The same rotation of a chunk's queries and keys in one launch: q, q_out
 * [B, H, C, D] and k, k_out [B, nKV, C, D] with the shared tables; results
 * bit-identical to two cp_rope_chunk calls.  q_out may equal q, k_out k.
 * Errors: as cp_rope_chunk (CP_ERR_ARG also for H or nKV < 0).
 */
int cp_rope_qk_chunk(const void *q, void *q_out, const void *k, void *k_out, const float *cos,
                     const float *sin, int B, int H, int nKV, int C, int D, int Bt, int dtype,
                     cp_stream_t stream);

/*
 * cp_rope_qk_chunk plus the append of the chunk into a GLOBAL cache, in one launch:
 * q -> q_out [B, H, C, D], k -> k_out [B, nKV, C, D] (B, nKV, D, dtype from the
 * cache), and rows [0, n_valid[b]) of k_out and of v [B, nKV, C, D] are written to
 * slots seen[b], seen[b] + 1, ... -- bytes identical to cp_kv_append(k_out, v).
 * seen is NOT advanced: the attention of the same chunk reads the past below seen
 * and the chunk's rows from k_out / v, so it never sees these slots; advance seen
 * afterwards with CP_ATTN_ADVANCE_SEEN on the attention call, or cp_kv_advance.
 * n_valid NULL appends all C rows.  Same device checks as cp_kv_append
 * (CP_DEV_OVERFLOW, CP_DEV_SEEN, CP_DEV_NVALID); a skipped sequence is also
 * skipped by the advance.
 * Errors: CP_ERR_ARG (ring cache: a ring append may evict rows the attention
 *         reads; null, negative sizes, Bt not 1 or B), CP_ERR_SHAPE (D odd,
 *         C > cap), CP_ERR_DTYPE.
 */
int cp_rope_qk_append_chunk(const cp_cache *cache, const void *q, void *q_out, const void *k,
                            void *k_out, const void *v, const float *cos, const float *sin, int H,
                            int C, int Bt, const int32_t *n_valid, cp_stream_t stream);

/* ---- KV cache ---- */

/*
 * Append rows [0, n_rows[b]) of the chunk's K/V at positions seen[b],
 * seen[b] + 1, ... and advance seen[b] by n_rows[b] ([SKaiNET] K/V extended
 * by the chunk; [TICO] runtime writes the delta K/V; [cactus] chronological
 * eviction for a ring).  n_rows == NULL appends all C rows (the static
 * padded append).  Bit-exact row copies.
 *
 *   k_new, v_new  [B, nKV, C, D] storage dtype (k_new already rotated)
 * Device checks: a global sequence with seen + n > cap is skipped
 * (CP_DEV_OVERFLOW); n outside [0, C] is clamped (CP_DEV_NVALID).
 * Errors: CP_ERR_ARG, CP_ERR_SHAPE, CP_ERR_DTYPE.
 */
int cp_kv_append(const cp_cache *cache, const void *k_new, const void *v_new, int C,
                 const int32_t *n_rows, cp_stream_t stream);

/*
 * The seen update of cp_kv_append alone: seen[b] += n_rows[b] (all C rows for
 * NULL), skipping the sequences cp_kv_append would skip, without setting
 * status bits (cp_rope_qk_append_chunk reported them when it wrote the rows).
 * Errors: as cp_kv_append.
 */
int cp_kv_advance(const cp_cache *cache, int C, const int32_t *n_rows, cp_stream_t stream);

/* Bytes a snapshot of a C-row padded append of `cache` needs (0 on bad args). */
size_t cp_snapshot_bytes(const cp_cache *cache, int C);

/*
 * Before a padded append of C rows (n_valid[b] real): save, per sequence,
 * the rows the padded append evicts but an exact append of n_valid rows
 * would keep -- positions [max(sink, seen+n_valid-R), max(sink, seen+C-R)),
 * R = cap - sink, at most C - n_valid rows -- and record seen and n_valid.
 * A global cache saves no rows (its pad rows land in the dead region).
 * Errors: CP_ERR_WINDOW for a ring with cap <= C + sink (nothing enqueued),
 *         CP_ERR_WORKSPACE if snap->bytes < cp_snapshot_bytes(), CP_ERR_ARG,
 *         CP_ERR_SHAPE.
 */
int cp_kv_snapshot_padded_append(const cp_cache *cache, int C, const int32_t *n_valid,
                                 cp_snapshot *snap, cp_stream_t stream);

/*
 * After the padded append: write the saved rows back to their slots and set
 * seen = seen_before + n_valid, so the live region is byte-identical to an
 * exact append of the n_valid real rows.  Pad rows left in slots that are
 * not live are dead region.  A sequence whose seen is not seen_before + C
 * is left alone and flagged CP_DEV_ROLLBACK.
 * Errors: CP_ERR_STATE (snapshot not armed, taken from another cache, or
 *         for another C), CP_ERR_ARG.
 */
int cp_kv_rollback_padded_append(const cp_cache *cache, cp_snapshot *snap, cp_stream_t stream);

/*
 * The padded ring append's two halves with fewer launches ([cactus] "Fix": the rows
 * a padded append over-evicts are saved before it and written back after it, so the
 * cache ends byte-identical to an unpadded prefill):
 *
 *   cp_rope_qk_snapshot_chunk -> cp_attn_chunk_with_past -> cp_kv_append_rollback
 *
 * does what cp_rope_qk_chunk -> cp_kv_snapshot_padded_append -> cp_attn_chunk_with_past
 * -> cp_kv_append (all C rows) -> cp_kv_rollback_padded_append does, with the same
 * bytes everywhere (rotated tensors, snapshot buffer, every cache slot, seen, status).
 *
 * cp_rope_qk_snapshot_chunk: cp_rope_qk_chunk (q, q_out [B, H, C, D]; k, k_out
 * [B, nKV, C, D]; H = 0 rotates the keys only) and cp_kv_snapshot_padded_append (same
 * snapshot layout and arming) in one launch.  B, nKV, D and the dtype come from the
 * cache.  Safe because nothing writes the cache between the snapshot and the append.
 * Errors: as the two calls (CP_ERR_WINDOW for a ring with cap <= C + sink,
 *         CP_ERR_WORKSPACE, CP_ERR_ARG, CP_ERR_SHAPE, CP_ERR_DTYPE); nothing is
 *         enqueued and the snapshot is not armed on error.
 */
int cp_rope_qk_snapshot_chunk(const cp_cache *cache, const void *q, void *q_out, const void *k,
                              void *k_out, const float *cos, const float *sin, int H, int C,
                              int Bt, const int32_t *n_valid, cp_snapshot *snap,
                              cp_stream_t stream);

/*
 * cp_kv_append of all C rows of k_new, v_new [B, nKV, C, D] followed by
 * cp_kv_rollback_padded_append, in one launch: the real rows land where the append
 * puts them; a pad row whose slot held an over-evicted row gets that row back from the
 * snapshot; the other pad rows land in the dead region as the append leaves them;
 * seen = seen_before + n_valid.  The pre-append seen is the snapshot's, so this must
 * follow the snapshot with no other change of the cache in between; if seen moved, the
 * rows are written for seen_before, seen is left alone and CP_DEV_ROLLBACK is set.
 * Disarms the snapshot.
 * Errors: CP_ERR_STATE (snapshot not armed, from another cache, or for another C),
 *         CP_ERR_ARG; nothing is enqueued on error.
 */
int cp_kv_append_rollback(const cp_cache *cache, const void *k_new, const void *v_new, int C,
                          cp_snapshot *snap, cp_stream_t stream);

/* ---- attention ---- */

/* Workspace bytes that let cp_attn_chunk_with_past split keys (0 if never). */
size_t cp_attn_workspace_bytes(const cp_cache *cache, const cp_attn_args *args);

/*
 * Grouped-query attention of the chunk over the live past plus the C chunk
 * keys, softmax(scale * q.k + mask) v, fp32 accumulation (bf16 matrix
 * cores for CP_BF16).  See cp_attn_args.
 * Kernels: bf16 with D in {64, 128, 256} (and 16-byte aligned tensors) runs on
 * the matrix cores; fp32, and bf16 with any other D up to 256, on the vector-ALU
 * kernel.
 * Errors: CP_ERR_ARG (also: only one of q_cos / q_sin, q_tables not 1 or B),
 *         CP_ERR_SHAPE (H % nKV, D > 256, odd D with q tables, C > cap for a
 *         global cache), CP_ERR_DTYPE, CP_ERR_HIP.
 */
int cp_attn_chunk_with_past(const cp_cache *cache, const cp_attn_args *args, cp_stream_t stream);

/*
 * For callers that cannot allocate device memory (code being captured into a HIP
 * graph whose owner forbids allocation, tight serving loops, harnesses that ban
 * hipMalloc): cp_attn_chunk_with_past with the key-split partials kept in a
 * device array that the library owns, instead of a caller workspace.  The array
 * holds CP_ATTN_SCRATCH_BYTES on each GPU the library runs on, from the first
 * call on that device (the current device, which must own `stream`) until the
 * process ends.  args->workspace and args->workspace_bytes are ignored; every
 * other argument, output and error is as for cp_attn_chunk_with_past, and the
 * outputs are bit-identical to it.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array and leaves its partials there:
 * calls that may overlap on one GPU (different streams, or different host
 * threads without ordering) race and must be ordered by the caller.  Nothing in
 * the array needs clearing between calls (each call writes every partial it
 * reads).
 * Errors: those of cp_attn_chunk_with_past; CP_ERR_SCRATCH (nothing enqueued)
 *         when the call's key splits need more than CP_ATTN_SCRATCH_BYTES
 *         (cp_attn_workspace_bytes() gives the need); CP_ERR_HIP if the
 *         array's device address cannot be obtained.
 */
#define CP_ATTN_SCRATCH_BYTES (64u << 20)
int cp_attn_chunk_with_past_noalloc(const cp_cache *cache, const cp_attn_args *args,
                                    cp_stream_t stream);

/*
 * Materialise the explicit mask from the in-kernel rule ([SKaiNET] mask
 * layout [B, H, C, ld]; 0 attends, -1e30 masks; columns past live + C are
 * masked).  n_valid may be NULL (all rows real).
 * Errors: CP_ERR_ARG, CP_ERR_SHAPE.
 */
int cp_build_mask(float *mask, int64_t ld, const cp_cache *cache, const int32_t *n_valid, int H,
                  int C, int window, cp_stream_t stream);

/* ---- row selection ---- */

/*
 * y[b, h, :] = x[b, h, idx[b] + offset, :] ([SKaiNET] one-hot selected row;
 * "Validation": row 51 = last real row).  Pass n_valid with offset -1 for
 * the last real row.  Rows outside [0, C) give zeros.
 *   x [B, H, C, D], y [B, H, D], idx device int32 [B].
 * Errors: CP_ERR_ARG, CP_ERR_DTYPE.
 */
int cp_select_row(const void *x, void *y, const int32_t *idx, int offset, int B, int H, int C,
                  int D, int dtype, cp_stream_t stream);

/* ---- gated delta rule (the linear-attention layers of hybrid models) ---- */

/*
 * Prefill of P tokens through the gated delta rule ([Kazeia] "Chantier 4 -- GDN
 * chunkwise prefill", sections "Le kernel actuel" and "P1 -- chunk f32"): per
 * (sequence, head) a state S of dk x dv; per token, in order,
 *   S <- exp(alpha_t) S;  delta = (v_t - S^T k_t) beta_t;  S <- S + k_t delta^T;
 *   out_t = S^T q_t
 * computed in chunks of 64 tokens ("Chunkwise (delta rule)"), fp32.
 *
 *   q, k       fp32 [B, H, P, dk] (as the layer produces them; commonly unit keys)
 *   v          fp32 [B, H, P, dv]
 *   beta       fp32 [B, H, P]   write strengths
 *   alpha      fp32 [B, H, P]   log of the gates (<= 0 for decaying gates)
 *   state      fp32 [B, H, dk, dv], in/out: the entry state, replaced by the state
 *              after the last token (the layer's "cache")
 *   out        fp32 [B, H, P, dv]
 *   workspace  device scratch of at least cp_gdn_workspace_bytes(); it holds the
 *              per-chunk products and is overwritten
 * dk and dv each 64 or 128; q, k, v and workspace 16-byte aligned.
 * Both launches go to `stream` in order; the call returns once they are queued.
 * Errors: CP_ERR_ARG (null, misaligned, negative sizes), CP_ERR_SHAPE (dk, dv; B * H * P beyond one launch grid),
 *         CP_ERR_WORKSPACE, CP_ERR_HIP.  P = 0 is a no-op (state untouched).
 */
size_t cp_gdn_workspace_bytes(int B, int H, int P, int dk, int dv);
int cp_gdn_chunk_prefill(const float *q, const float *k, const float *v, const float *beta,
                         const float *alpha, float *state, float *out, int B, int H, int P,
                         int dk, int dv, void *workspace, size_t workspace_bytes,
                         cp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CP_H */
