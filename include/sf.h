/*
 * sf.h - C-ABI of the Summaryformer per-block memory, native on MI355X (gfx950).
 *
 * The method is described on the model card titled "GTA world model: weights
 * and inference code" (Summaryformer).  Citations below name its sections:
 *   [record]   "A frame is a record": a frame's record is its H*W raw tokens
 *              followed by its X summary tokens (the record(t) equation).
 *   [attends]  "What a frame attends to": the four-item list of what frame
 *              t's tokens see.
 *   [buffer]   "One buffer, no mask": one preallocated K/V buffer per block,
 *              laid out Z0 | RAW | SUM; the eviction paragraph; the figure
 *              "The buffer one frame apart"; the parameter table; the single
 *              dense, unmasked read of the filled rows.
 *   [sampling] "The rest of the model", item "Sampling": a clean pass
 *              rewrites the frame's entry in memory.
 *   [limits]   "Limits": sessions end at the last frame id of the position
 *              table (4096 ids on the page).
 *   [sink]     "Running for a long time: the start image follows the window":
 *              Z0's stored keys are moved forward in time by one more RoPE
 *              rotation, in place, whenever the gap to the oldest frame in
 *              memory reaches 5; values are untouched.  With "Telling a summary
 *              from a pixel: level planes" (12 temporal planes per head) and
 *              the "Positions" item (a rotary table adapted from Wan2.1).
 *   [level]    "Telling a summary from a pixel: level planes": the two slowest of
 *              a head's temporal RoPE planes turn by under half a radian over 1024
 *              frames; summary tokens take an exact quarter turn on them, and the
 *              model refuses to build unless they are idle.
 *   [files]    "Files": the model's files include an optional recency bias on
 *              summary keys.
 *   [credits]  "Credits": that bias follows the Recency Forcing paper, which the
 *              page does not reproduce.
 *
 * Terms.  A session is one player's memory: n_blocks independent buffers,
 * one per transformer block, stepped together frame by frame.  R = hw + x
 * rows per record; capacity C = R*(y+2) + (w-y)*x rows per buffer:
 *   Z0        rows [0, R)                        record of frame 0 (start image)
 *   RAW s     rows [R*(1+s), R*(2+s))            s = t mod (y+1), frame t >= 1
 *   SUM u     rows [R*(y+2)+u*x, R*(y+2)+(u+1)*x) u = f mod (w-y), summary of frame f
 *
 * Memory.  The caller owns all device memory.  One session needs
 * sf_buffer_bytes(cfg) bytes of device memory, which it hands to
 * sf_buffer_create; the library never allocates device memory.  That memory
 * holds, for block b = 0..n_blocks-1, K_b then V_b, each [C][n_heads][head_dim]
 * row-major in the config's dtype (so byte offset of K_b is
 * b * 2 * C*n_heads*head_dim*elem, V_b follows K_b); after the last block
 * comes a scratch region that sf_attend uses for partial results of this
 * session (and, when the library applies the temporal band, room for one rotated
 * query; with the recency bias on, its table and the per-row biases of the
 * current frame).  The canonical K/V bytes are the first sf_kv_bytes(cfg) bytes.
 *
 * Tensors passed per call (device pointers, row-major, contiguous, 16-byte aligned:
 * the kernels move them in 16-byte vectors; a misaligned pointer is SF_E_ARG):
 *   q, k, v : [R][n_heads][head_dim] in the config dtype (fp32 or bf16)
 *   out     : [R][n_heads][head_dim] fp32
 *
 * Ordering and state.  All device work is enqueued on the given HIP stream
 * (NULL = the default stream) with no host synchronisation; host state
 * advances at enqueue.  All of one session's calls must use one stream (or
 * be ordered by the caller).  A handle is not thread-safe.  Every call that
 * returns an error leaves the host state unchanged and enqueues nothing,
 * except SF_E_HIP raised by a launch after an earlier launch of the same call
 * was enqueued: the host state is restored, but device contents of the rows
 * that call touches are then undefined.
 *
 * Dry-run handles.  sf_buffer_create with dev_mem == NULL and bytes == 0
 * makes a handle that validates and advances state exactly like a real one
 * but never touches a device; its device-pointer arguments may be NULL.
 *
 * Errors never throw; sf_last_error gives a message.
 */
#ifndef SF_H
#define SF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sf_status {
  SF_OK = 0,
  SF_E_ARG = -1,          /* bad argument: NULL pointer, bad index, bad config, short memory */
  SF_E_ORDER = -2,        /* call out of order for the session's frame sequence */
  SF_E_RANGE = -3,        /* frame id at or beyond max_frames */
  SF_E_STATE = -4,        /* handle not in a state that allows the call */
  SF_E_HIP = -5,          /* a HIP runtime call or kernel launch failed */
  SF_E_UNSUPPORTED = -6   /* valid but not implemented (e.g. head_dim other than 64/128) */
} sf_status;

typedef enum sf_dtype { SF_F32 = 0, SF_BF16 = 1 } sf_dtype;

/* [level], [sink] Who applies the temporal RoPE band (the first hd/2 - 2*floor(hd/6) planes
 * of a head; plane i = dims (2i, 2i+1) as (real, imaginary), turning rope_theta^(-2i /
 * (hd - 4*floor(hd/6))) rad per frame).
 *   SF_ROPE_CALLER         the caller's q and k arrive rotated; the library turns nothing
 *                          except Z0's keys in the sink (every temporal plane of every row).
 *   SF_ROPE_LEVEL_REPLACE  the library turns each record's keys by its frame id at the
 *   SF_ROPE_LEVEL_ADD      write, and each query by the current frame at the read; raw rows
 *                          (record rows < hw) on every temporal plane; summary rows on all
 *                          but the two slowest, which carry the level axis: REPLACE puts the
 *                          exact quarter turn (x, y) -> (-y, x) of the input there, ADD turns
 *                          by the time angle and then by the quarter turn.  The height and
 *                          width bands stay the caller's.  Under REPLACE the sink leaves the
 *                          level planes of Z0's summary rows alone (they hold no time).
 *                          Config check: both level planes turn by less than 0.5 rad over
 *                          1024 frames at rope_theta, else SF_E_UNSUPPORTED. */
typedef enum sf_rope_mode { SF_ROPE_CALLER = 0, SF_ROPE_LEVEL_REPLACE = 1, SF_ROPE_LEVEL_ADD = 2 } sf_rope_mode;

/* Shape of one session ([record], [buffer] parameter table). */
typedef struct sf_config {
  int32_t hw;         /* raw tokens per frame: one per latent grid cell (H*W), >= 1 */
  int32_t x;          /* summary tokens per frame (X), >= 1 */
  int32_t y;          /* frames kept whole before the current one (Y), >= 0 */
  int32_t w;          /* memory window in frames (W), > y */
  int32_t n_heads;    /* attention heads (K/V heads = Q heads), >= 1 */
  int32_t head_dim;   /* 64 or 128 */
  int32_t n_blocks;   /* transformer blocks, one buffer each, >= 1 */
  int32_t dtype;      /* sf_dtype of q, k, v and of the stored K/V */
  int64_t max_frames; /* frame ids must stay below this ([limits]); 0 = no cap */
  int32_t sink_gap;   /* [sink] 0 = off; else >= 2: when the oldest generated frame still in
                         memory is sink_gap frames past Z0's frame id, Z0's keys are rotated
                         forward to bring the gap back to 1 (the page uses 5) */
  float rope_theta;   /* [sink] base of the temporal RoPE band the stored keys carry (> 1;
                         the page's table follows Wan2.1: 10000); read only when sink_gap > 0
                         or rope_mode != SF_ROPE_CALLER */
  int32_t rope_mode;  /* [level] sf_rope_mode */
  int32_t recency_bias; /* [files], [credits] 0 = off, 1 = on: the read adds a per-head term,
                         set by sf_set_recency_bias, to the scaled scores of summary keys by the
                         age of their frame (starts at 0) */
} sf_config;

#define SF_MAX_SEGMENTS 4
#define SF_MAX_BATCH 64

/* Host-side snapshot of one session's slot map and fill state. */
typedef struct sf_view {
  int64_t t_cur;        /* newest frame id written; -1 before the first write */
  int64_t n_keys;       /* rows the next attend reads (sum of seg_len) */
  int64_t evicted_for;  /* frame id whose eviction step last ran; -1 if none */
  int32_t n_seg;        /* readable row segments, ascending, <= SF_MAX_SEGMENTS */
  int32_t raw_slot;     /* RAW slot of t_cur; -1 while t_cur <= 0 */
  int32_t blocks_written; /* blocks whose record for t_cur has been written */
  int32_t reserved;
  int64_t seg_begin[SF_MAX_SEGMENTS];
  int64_t seg_len[SF_MAX_SEGMENTS];
  int64_t* raw_frame;   /* in: caller array of y+1 entries or NULL; out: frame id per RAW slot (-1 empty) */
  int64_t* sum_frame;   /* in: caller array of w-y entries or NULL; out: frame id per SUM slot (-1 empty) */
  int64_t z0_frame;     /* [sink] frame id Z0's keys are rotated to (0 until the first rotation) */
} sf_view;

typedef struct sf_buffer sf_buffer;

/* Checks a config; SF_OK, SF_E_ARG (inconsistent) or SF_E_UNSUPPORTED. */
sf_status sf_config_check(const sf_config* cfg);

/* Device bytes one session needs (K/V of all blocks + attend scratch); 0 if cfg is invalid. */
size_t sf_buffer_bytes(const sf_config* cfg);

/* Canonical K/V bytes (a prefix of the session memory): n_blocks * 2 * C*n_heads*head_dim*elem. */
size_t sf_kv_bytes(const sf_config* cfg);

/* Byte offset of block b's K (which = 0) or V (which = 1) in the session memory; -1 if invalid. */
int64_t sf_kv_offset(const sf_config* cfg, int32_t block, int32_t which);

/* [buffer] One preallocated buffer per block.  Binds dev_mem (>= sf_buffer_bytes, 16-byte
 * aligned, owned by the caller, valid until destroy and until enqueued work ends) to a new
 * handle and enqueues a zero fill of the K/V bytes (and of the recency bias table, when the
 * config has one) on stream, so empty slots read as zero.  dev_mem == NULL with bytes == 0
 * makes a dry-run handle. */
sf_status sf_buffer_create(const sf_config* cfg, void* dev_mem, size_t bytes, void* hip_stream,
                           sf_buffer** out);

/* Frees the host handle only (the device memory stays the caller's). NULL is allowed. */
sf_status sf_buffer_destroy(sf_buffer* buf);

/* [buffer], [sampling] Copies record(t)'s K and V of one block into Z0 (t = 0) or RAW slot
 * t mod (y+1).  t must be t_cur (a rewrite: last write wins) or t_cur + 1 (an advance, allowed
 * once every block holds t_cur and the frame leaving that RAW slot has been evicted).  k and v
 * are device pointers to [R][n_heads][head_dim] in the config dtype (16-byte aligned).
 * [level] Under SF_ROPE_LEVEL_*, k arrives unrotated and is stored turned by frame id t (in
 * fp32, rounded to the storage type) in the same launch as the copy. */
sf_status sf_write_record(sf_buffer* buf, int32_t block, int64_t t, const void* k, const void* v,
                          void* hip_stream);

/* [buffer], [sampling] Zero-copy form of sf_write_record.  Sets *k_rows and *v_rows to the
 * device rows where record(t) of one block is stored (Z0 for t = 0, else RAW slot
 * t mod (y+1)), each [R][n_heads][head_dim] in the config dtype (NULL on a dry-run handle),
 * after the same checks as sf_write_record; nothing changes.  The caller fills those rows on
 * its own stream (its K/V projection can write there directly), then calls
 * sf_commit_record with the same block and t.  A rewrite (t == t_cur) may be filled in place
 * as long as no read of this block is in flight.  The rows are stored as given, so under
 * SF_ROPE_LEVEL_* (where the library turns keys at the write) both calls return
 * SF_E_UNSUPPORTED. */
sf_status sf_record_slot(sf_buffer* buf, int32_t block, int64_t t, void** k_rows, void** v_rows);

/* Records that record(t) of one block now sits in the rows sf_record_slot gave (same checks
 * as sf_write_record; no device work).  A later read of the block sees those rows as they are
 * when the read runs on its stream. */
sf_status sf_commit_record(sf_buffer* buf, int32_t block, int64_t t);

/* Host state of a session (slot map, per-block frame, Z0's frame id), for moving a session
 * between handles: the caller copies the device bytes itself (sf_buffer_bytes of them, or the
 * first sf_kv_bytes for K/V alone) and the host state with these.  sf_state_bytes gives the
 * size for a config (0 if invalid); sf_state_export writes it (SF_E_ARG if bytes is smaller);
 * sf_state_import checks it against the handle's config and for consistency and replaces the
 * handle's state (SF_E_ARG and no change if anything is off). */
size_t sf_state_bytes(const sf_config* cfg);
sf_status sf_state_export(const sf_buffer* buf, void* dst, size_t bytes);
sf_status sf_state_import(sf_buffer* buf, const void* src, size_t bytes);

/* [buffer] eviction paragraph.  Before frame t is written: copies K and V of the x summary rows
 * (record rows [hw, R)) of the frame leaving RAW slot t mod (y+1) into its SUM slot
 * f mod (w-y), in every block, in one launch.  The raw rows are not copied.  t must be
 * t_cur + 1 with every block holding t_cur.  A no-op when no generated frame leaves (t <= y+1);
 * repeating it for the same t is a no-op.
 * [sink] With sink_gap > 0, once this step's eviction is done: if the oldest generated frame
 * in memory is now sink_gap or more frames past Z0's frame id z, every block's Z0 keys (all R
 * rows, all heads; values untouched) are rotated in place by rotation(T), T = oldest - 1 - z,
 * on the temporal RoPE planes, and z advances by T.  Plane i (dims 2i, 2i+1 of a head, i below
 * hd/2 - 2*floor(hd/6)) turns by T * rope_theta^(-2i / (hd - 4*floor(hd/6))); the rotation is
 * done in fp32 and rounded to the storage type.  Under SF_ROPE_LEVEL_REPLACE the two slowest
 * planes of Z0's summary rows are left as they are. */
sf_status sf_evict(sf_buffer* buf, int64_t t, void* hip_stream);

/* [attends], [buffer] The dense read.  For each of n sessions (n <= SF_MAX_BATCH; equal
 * n_heads, head_dim and dtype; block < n_blocks in each): out[i] = softmax(scale * q K^T) V over
 * every filled row of that session's block buffer, per head, for all R query rows; no mask.
 * scale <= 0 means 1/sqrt(head_dim).  Each session's block must hold its t_cur, and the
 * eviction step of t_cur + 1 must not have run yet (it replaces a summary frame t_cur still
 * sees and may turn Z0): SF_E_STATE otherwise.  bf16 sessions: QK^T and PV on bf16 MFMA with fp32 accumulation, softmax in fp32,
 * probabilities rounded to bf16 before PV.  fp32 sessions: fp32 throughout.  One attention
 * launch per read path and per 16 sessions, plus a combine launch where the keys are split
 * (and, at bf16 head_dim 64, a tail launch for reads shorter than 64 keys).
 * [level] A session under SF_ROPE_LEVEL_* takes q unrotated: it is turned by that session's
 * t_cur (as sf_rope_rows does) into the session's own memory first, one launch per session.
 * [files], [credits] A session with recency_bias = 1 adds its bias (sf_set_recency_bias) to
 * the scores of summary keys; a batch is launched per read path (sessions with and without
 * the bias at bf16 head_dim 64 take different kernels). */
sf_status sf_attend(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q,
                    void* const* out, float scale, void* hip_stream);

/* Allocation-free form of sf_attend, for callers that cannot allocate device memory or hand
 * the library a workspace while they run: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, checks, kernels and results as sf_attend,
 * but the read's scratch (the partial results of reads split across workgroups, and the
 * turned query of a session under a rope mode) lives in a library-owned static device array
 * of SF_STATIC_SCRATCH_BYTES instead of the sessions' memory; each GPU the library runs on
 * holds its own copy until the process ends.  The call allocates nothing: the array's device
 * address is looked up (hipGetSymbolAddress) on the first call on each device, with that
 * device current.  A read whose scratch does not fit (the whole batch's, laid out one session
 * after another) returns SF_E_UNSUPPORTED and enqueues nothing; a served read (16 heads of 64,
 * 1,104 query rows, 6,528 keys) takes about 24.3 MB.  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other threads) race and give
 * undefined results; calls ordered on one stream are safe.  Nothing in the array needs to
 * start at zero: each call writes every slot it reads. */
#define SF_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
sf_status sf_attend_static_scratch(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q,
                                   void* const* out, float scale, void* hip_stream);

/* [files], [credits] The recency bias of a session configured with recency_bias = 1.
 * table: device pointer to [n_heads][w+1] fp32 (4-byte aligned, read by this call's launch
 * only; NULL allowed on a dry-run handle).  Entry [h][a] is added, in natural-log units, to
 * head h's scaled scores scale * <q, k> against every summary row (record rows [hw, R)) of
 * the generated frame a frames older than the current frame t_cur, wherever that row is:
 * the record of t_cur itself (a = 0), a RAW slot (a = 1..y) or a SUM slot (a = y+1..w).  Raw
 * rows and Z0's rows (the start image) get no bias.  Entries must not be NaN; -inf (or any
 * value below -1e30) drops those keys.  The table is copied into the session memory on the
 * stream (one launch) and holds for every later read until set again; before the first call
 * it is all zeros.  The per-row biases of the current frame are rebuilt on the read's
 * stream by the first read of each frame (one small launch).  Reads of such a session go
 * through the split-key attention kernel at every head_dim, and sf_step writes the record
 * before the read (no fused write).  SF_E_UNSUPPORTED when the config has recency_bias = 0;
 * SF_E_ARG for a NULL or misaligned table. */
sf_status sf_set_recency_bias(sf_buffer* buf, const float* table, void* hip_stream);

/* One block of one frame: sf_evict(t) if it is due and has not run, then sf_write_record,
 * then sf_attend of this session alone (q and k unrotated under SF_ROPE_LEVEL_*).  A rewrite
 * (t == t_cur) after sf_evict(t_cur + 1) is SF_E_STATE, as its read would be. */
sf_status sf_step(sf_buffer* buf, int32_t block, int64_t t, const void* q, const void* k,
                  const void* v, void* out, float scale, void* hip_stream);

/* [level], [positions] The rotation the library applies under cfg's rope mode (which must be
 * SF_ROPE_LEVEL_REPLACE or _ADD, else SF_E_ARG), for callers that read the memory with
 * their own attention: src [R][n_heads][head_dim] (a record's q or k rows, config dtype,
 * 16-byte aligned device pointer) turned by frame id t into dst (same shape; dst == src
 * turns in place; partial overlap is undefined).  One launch on the stream. */
sf_status sf_rope_rows(const sf_config* cfg, int64_t t, const void* src, void* dst, void* hip_stream);

/* Host snapshot of the slot map and fill state; no device work. */
sf_status sf_query(const sf_buffer* buf, sf_view* view);

/* The view a session has after stepping frames 0..t in order (every block written each
 * frame, evictions as due); t = -1 gives the empty state.  Pure host arithmetic. */
sf_status sf_plan(const sf_config* cfg, int64_t t, sf_view* view);

/* Static name of a status code. */
const char* sf_status_str(sf_status s);

/* Message of the last error on buf (NULL buf: of the calling thread's last failed call). */
const char* sf_last_error(const sf_buffer* buf);

/* Test hook: the next device launch made through buf fails with SF_E_HIP before launching. */
sf_status sf_debug_fail_next_launch(sf_buffer* buf);

/* Test hook, process-wide: how every later bf16 head_dim-64 read cuts its work into
 * workgroup ranges.  form 0: the library's choice (a table of ranges made by the host,
 * weighted by how fast each workgroup group runs, when the launch has at most 384 groups;
 * else computed by the kernel); 1: computed by the kernel from the unweighted formula, in
 * 32-bit arithmetic where it fits; 2: the same in 64-bit arithmetic, the form of the
 * largest launches.  Forms 1 and 2 give the same ranges, so their reads are bit-identical;
 * form 0's ranges differ, so its reads differ by rounding.  SF_E_ARG for another form. */
sf_status sf_debug_range_form(int32_t form);

/* Kernel timing (tracing).  While enabled on a handle, every kernel the library launches
 * for it is given two HIP events that its dispatch stamps with its own start and end (on
 * the caller's stream, through hipExtLaunchKernelGGL), so a duration covers the kernel
 * alone.  sf_kernel_times_read waits for those events, returns the summed milliseconds and
 * launch counts per kind since the last read, and starts a new period.  Kinds (ATTEND: the main attention kernel; TAIL: keys past the
 * last full 64-key tile of a bf16 head_dim-64 read; COMBINE: merging of split results; SINK:
 * the rotation of Z0's keys; ROPE: the rotation of a query before a read; BIAS: the copy of a
 * recency bias table and the rebuild of the per-row biases): */
enum { SF_K_FILL = 0, SF_K_WRITE = 1, SF_K_EVICT = 2, SF_K_ATTEND = 3, SF_K_COMBINE = 4, SF_K_TAIL = 5,
       SF_K_SINK = 6, SF_K_ROPE = 7, SF_K_BIAS = 8, SF_K_KINDS = 9 };
typedef struct sf_kernel_times {
  double ms[SF_K_KINDS];
  int64_t launches[SF_K_KINDS];
} sf_kernel_times;
/* on != 0 enables, 0 disables (pending events are dropped).  Dry-run handles: SF_E_STATE. */
sf_status sf_profile_enable(sf_buffer* buf, int32_t on);
sf_status sf_kernel_times_read(sf_buffer* buf, sf_kernel_times* out);

/* Measurement aid, not part of the method: copies `bytes` from src to dst (device pointers,
 * 16-byte aligned, bytes a multiple of 16384, regions not overlapping) through LDS with the
 * buffer-to-LDS transfer the head_dim-64 attention uses for its K/V tiles, on hip_stream
 * (NULL: the default stream), so that hardware traffic counters (FETCH_SIZE) can be
 * calibrated on that path against a copy of known size.  SF_E_ARG on a bad pointer or
 * size, SF_E_HIP on a launch failure; enqueues nothing on error. */
sf_status sf_debug_lds_copy(void* dst, const void* src, size_t bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SF_H */
