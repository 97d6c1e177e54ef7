/*
 * kvm.h -- C ABI of the MI355X (gfx950) Key-Value Means attention layer.
 *
 * The layer ([KVM abstract]; [KVM summary, Methodology]) is one softmax
 * attention over [compressed state || block-sliding window].  Tokens that
 * overflow the window are merged winner-take-all into a state of raw sums
 * and counts, or appended as new rows on a size schedule, and the state is
 * renormalised just in time when read ([KVM summary, Core mechanisms 1-5]).
 *
 * Conventions for every entry point
 *   - Plain C types only.  Device buffers are HIP device pointers; `stream`
 *     is a hipStream_t passed as void* (NULL = the null stream).
 *   - The caller owns every buffer, including the device workspace.  The
 *     library never allocates or frees device memory; it owns only the small
 *     host-side kvm_state object.  It never writes to its inputs.
 *   - All device work is queued on `stream`; no call synchronises the host
 *     with the device.  Results are visible after the caller synchronises.
 *   - Every call returns a kvm_status and never aborts or throws.  Arguments
 *     are checked before anything is queued: any status other than KVM_OK
 *     and KVM_E_HIP means nothing was queued and the state is unchanged.
 *     KVM_E_HIP (a failed HIP call) poisons the state: later calls on it
 *     return KVM_E_STATE.  kvm_last_error() gives a thread-local message.
 *   - One kvm_state must not be used by two calls at the same time.
 *   - NaN/Inf inputs are not checked; they propagate.
 *
 * Tensor layouts (row-major, contiguous):
 *   prefill  q, k, v, out: [B*H, n, head_dim] in cfg.dtype; gate_logits [B*H, n] float32
 *   decode   q, k, v, out: [B*H, head_dim]    in cfg.dtype; gate_logits [B*H]    float32
 *   q and k are passed UNROTATED: the library applies RoPE itself.
 *   Sequence index s = b*H + h.  All sequences share one position.
 */
#ifndef KVM_H
#define KVM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVM_OK = 0,
  KVM_E_INVALID_ARG = 1, /* bad config, null pointer, bad size */
  KVM_E_WORKSPACE = 2,   /* workspace too small or misaligned */
  KVM_E_CAPACITY = 3,    /* would go past cfg.max_tokens */
  KVM_E_STATE = 4,       /* call not valid in the state's current position, or state poisoned */
  KVM_E_HIP = 5          /* a HIP runtime call failed; the state is poisoned */
} kvm_status;

typedef enum { KVM_F32 = 0, KVM_BF16 = 1 } kvm_dtype;

/* State size schedules ([KVM summary, Core mechanisms 3]; [KVM summary,
 * Experimental results]: fixed-size state, power-law "sqrt" and saturating).
 * capacity(T) for T absorbed tokens, sinks included:
 *   FIXED       max_slots
 *   SQRT        ceil(alpha * sqrt(T))       (exact integer ceil-sqrt of alpha^2*T)
 *   SATURATING  min(max_slots, ceil(alpha * sqrt(T)))
 *   POWER       ceil(alpha * T^exponent)    (IEEE double pow; 0 < exponent <= 1) */
typedef enum { KVM_SCHED_FIXED = 0, KVM_SCHED_SQRT = 1, KVM_SCHED_SATURATING = 2, KVM_SCHED_POWER = 3 } kvm_sched;

/* Record, per absorbed token, the row it created or merged into and the kind
 * (sink / append / merge); read back with kvm_state_read. */
#define KVM_FLAG_TRACE 1u

/* Ablation variants ([KVM summary, Experimental results]: the ablation study
 * removes value-length normalisation, sink protection and the merge gate). */
#define KVM_FLAG_NO_VALUE_NORM 2u    /* read a row's value as its mean V/n instead of rho * V/|V| */
#define KVM_FLAG_NO_SINK_PROTECT 4u  /* sink rows are ordinary rows: surprise references and merge targets */
#define KVM_FLAG_NO_MERGE_GATE 8u    /* merged tokens are added with weight 1 (gate logits ignored) */

/* Serial prefill: kvm_prefill absorbs every chunk it needs before any
 * attention, then runs the attention of all its query chunks in one launch,
 * everything on the caller's stream (no library-owned stream).  Same results
 * bit for bit; by default the attention of chunks whose state is ready runs
 * on a second stream beside the rest of the absorption. */
#define KVM_FLAG_SERIAL_PREFILL 16u

typedef struct kvm_config {
  int32_t batch;          /* B >= 1 */
  int32_t heads;          /* H >= 1; heads are independent sequences */
  int32_t head_dim;       /* must be 64 */
  int32_t rope_dims;      /* must be 32: RoPE on dims [0,32), state keys keep dims [32,64) */
  int32_t chunk;          /* C in {32, 64, 128, 256} */
  int32_t window;         /* W: a positive multiple of C */
  int32_t n_sinks;        /* 0 <= n_sinks <= C: first tokens kept as protected rows */
  int32_t sched;          /* kvm_sched */
  int32_t max_slots;      /* FIXED / SATURATING ceiling (>= 1) */
  int32_t alpha;          /* SQRT / SATURATING integer growth constant (>= 1) */
  int64_t max_tokens;     /* largest position + 1 the state will ever see (sizes the workspace) */
  float rope_theta;       /* RoPE base (10000) */
  float ln_eps;           /* LayerNorm epsilon for state keys (1e-5) */
  float softmax_scale;    /* 0 => 1/sqrt(head_dim) */
  int32_t dtype;          /* kvm_dtype of q, k, v, out and of the stored read forms */
  uint32_t flags;         /* KVM_FLAG_TRACE | KVM_FLAG_NO_VALUE_NORM | KVM_FLAG_NO_SINK_PROTECT | KVM_FLAG_NO_MERGE_GATE
                             | KVM_FLAG_SERIAL_PREFILL */
  double exponent;        /* POWER: growth exponent in (0, 1]; ignored by the other schedules */
} kvm_config;

typedef struct kvm_state kvm_state;

/* A state in plain arrays: what kvm_state_read fills and kvm_state_load takes.
 * [KVM lay summary, "smart merge"]: the state is kept as raw (gated) sums and
 * counts per row, divided only when read; [KVM summary, Core mechanisms 1]: it
 * is a separate state beside the exact window, so a state plus the window's
 * tokens is everything a later call needs.
 * Any pointer may be NULL (skipped).  S_cap = kvm_state_info.max_rows,
 * R = window + chunk.  Row-indexed arrays hold S_cap rows per sequence; rows
 * beyond n_rows[s] are undefined.
 * ktype, the read-form key storage type, is float32 on the KVM_F32 path and
 * IEEE fp16 on the KVM_BF16 path: a LayerNorm output over 32 dims has
 * |k| <= sqrt(31), so fp16 keeps more precision than bf16 with no overflow.
 * Read-form values rho * u are stored in cfg.dtype (bf16 or f32): their range
 * is that of the input values. */
typedef struct kvm_state_view {
  int32_t* n_rows;        /* [B*H] host                rows of each sequence's state */
  float* key_sum;         /* [B*H, S_cap, 32] f32      raw gated key sums (live dims) */
  float* val_sum;         /* [B*H, S_cap, 64] f32      raw gated value sums */
  int32_t* count;         /* [B*H, S_cap] i32          tokens absorbed per row */
  float* rho;             /* [B*H, S_cap] f32          read radius fixed at row creation */
  void* key_read;         /* [B*H, S_cap, 32] ktype    read-form key, live dims (rotary dims are 0) */
  void* val_read;         /* [B*H, S_cap, 64] dtype    read-form value rho * u, u = V / |V| (V/n with KVM_FLAG_NO_VALUE_NORM) */
  int32_t* trace_slot;    /* [B*H, max_tokens] i32     row created/merged into, -1 if not absorbed */
  uint8_t* trace_kind;    /* [B*H, max_tokens] u8      0 sink, 1 append, 2 merge, 255 not absorbed */
  int64_t position;       /* tokens consumed (kvm_state_read with chunk -1 writes it; kvm_state_load reads it) */
  void* ring_k;           /* [B*H, R, 64] dtype        window keys, RoPE-rotated at their positions: position p in slot p mod R */
  void* ring_v;           /* [B*H, R, 64] dtype        window values, same slots */
  float* ring_l;          /* [B*H, R] f32              window gate logits, same slots */
} kvm_state_view;

typedef struct kvm_state_info {
  int64_t position;       /* tokens consumed so far */
  int64_t absorbed_chunks;/* chunks merged into the state so far */
  int32_t rows;           /* current rows per sequence (same for all: the schedule is data-independent) */
  int32_t max_rows;       /* S_cap: rows after the last chunk max_tokens can absorb */
  int64_t max_chunks;     /* chunks max_tokens can absorb */
  int32_t poisoned;       /* 1 after KVM_E_HIP */
  int32_t scan_groups;    /* workgroups that share one sequence's absorption scan (1, 2, 4 or 8) */
  int32_t per_sequence;   /* 1 while sequences are at different positions (position, absorbed_chunks, rows
                             are then -1; see kvm_state_positions) */
} kvm_state_info;

/* Device workspace size for cfg (bytes; the workspace must be 256-byte aligned).
 * The workspace holds the state of [KVM summary, Core mechanisms 1] (raw sums,
 * counts and radii per row [KVM lay summary, "smart merge"], sized by the
 * schedule of Core mechanisms 3 at max_tokens), its read-form row versions
 * (Core mechanisms 2), the last W + C tokens of the window, and RoPE tables
 * (Core mechanisms 4).  Host only: queues nothing.
 * Errors: KVM_E_INVALID_ARG. */
kvm_status kvm_workspace_bytes(const kvm_config* cfg, size_t* bytes);

/* Data-independent schedule ([KVM summary, Core mechanisms 3, 5]): for each of
 * the first n_chunks absorbed chunks, the sinks created, the rows appended and
 * the rows after the chunk.  Host only.  Output arrays hold n_chunks entries
 * (any may be NULL).  Errors: KVM_E_INVALID_ARG. */
kvm_status kvm_schedule(const kvm_config* cfg, int64_t n_chunks, int32_t* sinks, int32_t* appends,
                        int32_t* rows_after);

/* Bind a fresh, empty state (position 0: no tokens seen, no state rows, the
 * starting point of the chunk recurrence of [KVM summary, Core mechanisms 1])
 * to a caller-owned device workspace of at least kvm_workspace_bytes(cfg).
 * Queues the workspace initialisation (RoPE table, schedule table, counters)
 * on `stream`.
 * Errors: KVM_E_INVALID_ARG (config; null pointers), KVM_E_WORKSPACE (too
 * small / misaligned), KVM_E_HIP.  On success *out owns host memory that
 * kvm_state_destroy frees; the workspace stays the caller's. */
kvm_status kvm_state_create(const kvm_config* cfg, void* d_workspace, size_t workspace_bytes,
                            void* stream, kvm_state** out);

/* Free the host side of a state made by kvm_state_create (the host record of
 * the state of [KVM summary, Core mechanisms 1], its internal stream and
 * events).  Does not touch the workspace.  NULL is allowed.  Never fails. */
kvm_status kvm_state_destroy(kvm_state* st);

/* Chunk-parallel prefill of n_tokens tokens at the state's current position
 * ([KVM abstract]: chunk-wise parallelizable prefill; [KVM summary, Core
 * mechanisms 1-5]).  For each query chunk c, every chunk j <= c - W/C - 1 is
 * absorbed (sinks, appends, winner-take-all merges) and query t attends with
 * one softmax over the read form of that state (unrotated q against
 * LayerNorm-ed state keys whose rotary dims are zero; radius-scaled values)
 * and the window [max(0, cC - W), t] (rotated q against rotated k).
 * The position must be a multiple of chunk (else KVM_E_STATE);
 * position + n_tokens must not exceed max_tokens (else KVM_E_CAPACITY).
 * n_tokens == 0 is a no-op.  out may not alias q, k, v.
 * Stream order: the call's work starts after everything queued on `stream`
 * before it and everything queued after it starts after the call's work.
 * Inside, attention of query chunks whose state is ready runs on a second,
 * library-owned stream (created on first use, default priority) beside the
 * remaining absorption, joined back to `stream` with events.
 * Errors: KVM_E_INVALID_ARG, KVM_E_STATE, KVM_E_CAPACITY, KVM_E_HIP. */
kvm_status kvm_prefill(kvm_state* st, const void* q, const void* k, const void* v,
                       const float* gate_logits, void* out, int64_t n_tokens, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): one
 * prefill of n_tokens tokens from an empty state at position 0, the same
 * computation and results as kvm_state_create + kvm_prefill on a state with
 * this configuration (bit for bit), with the workspace in the library's static
 * device scratch instead of a caller buffer.  Nothing is allocated: no
 * hipMalloc/hipFree, no library stream or event, no host memory on success;
 * the scratch (KVM_NOALLOC_SCRATCH_BYTES, 128 MiB) is held by each GPU the
 * library runs on until the process ends.  Everything runs on `stream`.
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  The call clears what must start at
 * zero itself.  q, k, v, out [B*H, n_tokens, 64] in cfg.dtype, gate_logits
 * [B*H, n_tokens] f32, as for kvm_prefill; n_tokens <= cfg.max_tokens.
 * Errors: KVM_E_INVALID_ARG (config; KVM_FLAG_TRACE, which needs a state;
 * KVM_SCHED_POWER; tensors), KVM_E_WORKSPACE (the configuration's workspace,
 * kvm_workspace_bytes, exceeds the scratch), KVM_E_HIP.  Nothing is queued on
 * any error but KVM_E_HIP. */
#define KVM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
kvm_status kvm_prefill_noalloc(const kvm_config* cfg, const void* q, const void* k, const void* v,
                               const float* gate_logits, void* out, int64_t n_tokens, void* stream);

/* One decode step at position t = current position ([KVM summary, Problem
 * statement and Significance]: per-token decoding over a state smaller than
 * the context).  If t is a multiple of chunk and t >= W + C, chunk
 * (t - W - C)/C leaves the window and is absorbed first; then the single
 * query t attends over [state || window [cC - W, t]].  Position advances by 1.
 * Errors: KVM_E_INVALID_ARG, KVM_E_CAPACITY, KVM_E_STATE, KVM_E_HIP. */
kvm_status kvm_decode_step(kvm_state* st, const void* q, const void* k, const void* v,
                           const float* gate_logits, void* out, void* stream);

/* Device workspace for kvm_prefill_backward over up to cfg.max_tokens tokens
 * (bytes; 256-byte aligned): per-(query chunk, key) partial gradients, the
 * running gradients of every snapshot row's sums, per-query softmax
 * statistics.  Host only.  Errors: KVM_E_INVALID_ARG. */
kvm_status kvm_backward_workspace_bytes(const kvm_config* cfg, size_t* bytes);

/* Backward pass of the prefill ([KVM abstract]: the layer supports chunk-wise
 * parallelizable training): the gradient of sum(d_out * out) with respect to
 * q, k, v and the gate logits, where out is what kvm_prefill computed on this
 * state for positions [0, n_tokens) with these inputs.  The discrete choices
 * of the forward (the winner-take-all row of each merged token and the
 * appended tokens, [KVM summary, Core mechanisms 2-3]) are held fixed; the
 * gradient flows through the joint softmax, RoPE, the just-in-time read form
 * (LayerNorm of K/n, values at the read radius), the gated sums of the chunk
 * recurrence and the gate sigmoid.  Counts carry no gradient.
 * The state must have been created with KVM_FLAG_TRACE (the decisions are read
 * from the trace) and be at position n_tokens (prefill calls and decode steps
 * from position 0; q, k, v and gate_logits are the inputs of all of them).
 * q, k, v, d_out: [B*H, n_tokens, 64] in cfg.dtype; gate_logits [B*H, n_tokens]
 * f32; outputs d_q, d_k, d_v [B*H, n_tokens, 64] f32 and d_gate [B*H, n_tokens]
 * f32 (written, not accumulated).  The state is not modified.  Deterministic:
 * no float atomics; the same call gives the same bits.
 * Errors: KVM_E_INVALID_ARG (pointers, sizes, no trace), KVM_E_STATE (position
 * differs from n_tokens, poisoned state), KVM_E_WORKSPACE, KVM_E_HIP. */
kvm_status kvm_prefill_backward(kvm_state* st, const void* q, const void* k, const void* v, const float* gate_logits,
                                const void* d_out, float* d_q, float* d_k, float* d_v, float* d_gate,
                                int64_t n_tokens, void* d_workspace, size_t workspace_bytes, void* stream);

/* The projections of the block around the layer ([KVM abstract]: KVM is an
 * attention layer, fed queries, keys and values projected from the tokens and
 * projected back; [KVM summary, Core mechanisms 2]: the merge gate is a
 * data-dependent scalar, one more projection of the same input, one logit per
 * head).  Linear maps, weights stored [out features, in features] in
 * cfg.dtype, D = heads * 64; features of q, k, v are head-major (feature
 * h*64 + d is dimension d of head h) and head h of batch b is sequence b*H + h.
 *
 * kvm_project_in: x [B, n_tokens, D] -> q, k, v [B*H, n_tokens, 64] (cfg.dtype)
 * and gate_logits [B*H, n_tokens] f32, with w_in [3D + H, D] (rows: q
 * features, k features, v features, one gate row per head) and an optional
 * per-head gate bias b_gate [H] f32 (NULL = 0).  Outputs are the inputs
 * kvm_prefill takes.  fp32 accumulation.
 * Errors: KVM_E_INVALID_ARG (config, NULL or misaligned pointers, n_tokens < 0), KVM_E_HIP. */
kvm_status kvm_project_in(const kvm_config* cfg, const void* x, const void* w_in, const float* b_gate, void* q,
                          void* k, void* v, float* gate_logits, int64_t n_tokens, void* stream);

/* kvm_project_out: the layer output o [B*H, n_tokens, 64] -> y [B, n_tokens, D]
 * = concat_h(o_h) . w_out^T with w_out [D, D], cfg.dtype.  fp32 accumulation.
 * Errors: KVM_E_INVALID_ARG, KVM_E_HIP. */
kvm_status kvm_project_out(const kvm_config* cfg, const void* o, const void* w_out, void* y, int64_t n_tokens,
                           void* stream);

/* Export the state ([KVM lay summary, "smart merge"]: raw sums and counts,
 * divided only at read; [KVM summary, Core mechanisms 2]: the read form).
 *   chunk == -1: the current state.  Every field of `dst` may be requested;
 *     n_rows and position are host fields written at once; the other arrays
 *     may be host or device memory (copies queued on `stream`, unified
 *     addressing).  trace_* need KVM_FLAG_TRACE.  What this fills is what
 *     kvm_state_load takes to resume.
 *   0 <= chunk < absorbed_chunks: the state right after absorbed chunk
 *     `chunk`, i.e. the one query chunk chunk + W/C + 1 attends to.  The
 *     state keeps past snapshots only as read-form row versions, so only
 *     n_rows, count, rho, key_read and val_read can be given (device memory:
 *     a gather kernel writes them); requesting key_sum, val_sum, ring_* or
 *     trace_* for a past chunk is KVM_E_INVALID_ARG (position is untouched).
 * Errors: KVM_E_INVALID_ARG, KVM_E_STATE, KVM_E_HIP. */
kvm_status kvm_state_read(const kvm_state* st, int64_t chunk, kvm_state_view* dst, void* stream);

/* Resume from an exported state ([KVM summary, Core mechanisms 1]: the state
 * and the window are the whole carry of the chunk recurrence, so continuing
 * from them is the same as never having stopped).  `src` holds what
 * kvm_state_read(chunk -1) wrote for a state with the same configuration:
 * position; key_sum, val_sum, count, rho (required when the position has
 * absorbed chunks); ring_k, ring_v, ring_l (required when position > 0);
 * n_rows (host; optional, checked against the schedule when given);
 * trace_slot and trace_kind (optional; with KVM_FLAG_TRACE a NULL trace is
 * cleared to "not absorbed").  key_read and val_read are ignored: the read
 * form, the unit directions and the row versions are rebuilt from the raw
 * sums with the same arithmetic the absorption uses, so later calls give the
 * bits an uninterrupted state would.  Source arrays may be host or device
 * memory (copies queued on `stream`; the caller keeps them alive until the
 * stream reaches this call).  The state's previous contents are discarded.
 * Errors: KVM_E_INVALID_ARG (position outside [0, max_tokens], row counts
 * that differ from the schedule, a required array missing), KVM_E_STATE
 * (poisoned state), KVM_E_HIP. */
kvm_status kvm_state_load(kvm_state* st, const kvm_state_view* src, void* stream);

/* Queue a gather of the read form of the state right after absorbed chunk j,
 * i.e. the state that query chunk j + W/C + 1 attends to ([KVM summary, Core
 * mechanisms 2]: LayerNorm-ed keys, values at the read radius): key
 * [B*H, rows_j, 32] ktype, value rho * u [B*H, rows_j, 64] in cfg.dtype, radius
 * [B*H, rows_j] f32 (device memory; any pointer may be NULL).  The dense form
 * of kvm_state_read(j) without the S_cap row stride.
 * j must be < absorbed_chunks.  Errors: KVM_E_INVALID_ARG, KVM_E_STATE, KVM_E_HIP. */
kvm_status kvm_snapshot_read(const kvm_state* st, int64_t j, void* key_read, void* val_read, float* rho_read,
                             void* stream);

/* Sequences at their own positions (serving: requests of different lengths
 * that start and finish at different times in one batch; [KVM summary,
 * Significance]: the state makes per-token decoding over long contexts cheap;
 * [KVM abstract]: chunk-wise prefill).  The B*H sequences of a state are
 * independent slots; each keeps its own position, absorbed chunks and rows.
 * While sequences differ, kvm_prefill, kvm_decode_step, kvm_state_load and
 * kvm_prefill_backward return KVM_E_STATE; kvm_state_read reads each
 * sequence's rows (n_rows per sequence, position -1) and past snapshots up to
 * the fewest any sequence has absorbed.  When the positions meet again the
 * state is uniform again.
 *
 * kvm_prefill_ragged: sequence s takes n_tokens[s] (host array, 0 <= n <= n_max)
 * tokens at its own position, which must be a multiple of chunk when n > 0;
 * q, k, v, out are [B*H, n_max, 64] (row t of sequence s is its position
 * pos_s + t; rows past n_tokens[s] are ignored and not written), gate_logits
 * [B*H, n_max].  Same results as kvm_prefill of each sequence alone.
 * Everything runs on `stream` (absorption, then attention).
 * Errors: KVM_E_INVALID_ARG, KVM_E_STATE, KVM_E_CAPACITY, KVM_E_HIP. */
kvm_status kvm_prefill_ragged(kvm_state* st, const int64_t* n_tokens, const void* q, const void* k, const void* v,
                              const float* gate_logits, void* out, int64_t n_max, void* stream);

/* kvm_decode_step_ragged: one decode step for the sequences with active[s] != 0
 * (host array [B*H]), each at its own position (absorbing the chunk that leaves
 * its window when it reaches a chunk boundary).  q, k, v, out [B*H, 64];
 * rows of inactive sequences are ignored and their out rows not written.
 * Errors: KVM_E_INVALID_ARG, KVM_E_STATE, KVM_E_CAPACITY, KVM_E_HIP. */
kvm_status kvm_decode_step_ragged(kvm_state* st, const uint8_t* active, const void* q, const void* k, const void* v,
                                  const float* gate_logits, void* out, void* stream);

/* Return one sequence slot to position 0 with an empty state (its version
 * counter, exchange records and trace are cleared on `stream`), so that the
 * slot can take a new request while the others continue.
 * Errors: KVM_E_INVALID_ARG, KVM_E_STATE, KVM_E_HIP. */
kvm_status kvm_state_reset_sequence(kvm_state* st, int32_t seq, void* stream);

/* Each sequence's position (host array [B*H]).  Never fails on valid pointers. */
kvm_status kvm_state_positions(const kvm_state* st, int64_t* positions);

/* Host-side facts about the state: position, absorbed chunks and rows of the
 * chunk recurrence ([KVM summary, Core mechanisms 1, 3]).  Never fails on a
 * valid pointer. */
kvm_status kvm_state_get_info(const kvm_state* st, kvm_state_info* info);

/* Check that every absorption scan queued so far on this state finished its
 * work ([KVM summary, Core mechanisms 2-3]: every overflowed token is merged
 * or appended).  When a sequence's state rows are split over several
 * workgroups (a state with few sequences), the workgroups meet once per
 * absorbed chunk to combine their best-matching rows; a workgroup that waits
 * there for a few seconds gives up, so that no kernel can hang, and marks the
 * state.  This call copies that mark to the host and synchronises `stream`.
 * Errors: KVM_E_INVALID_ARG; KVM_E_STATE if the state is already poisoned;
 * KVM_E_HIP if a scan gave up (the state is then poisoned) or on a HIP failure. */
kvm_status kvm_state_check(kvm_state* st, void* stream);

/* Return the state to position 0 with an empty compressed state, the start of
 * the chunk recurrence ([KVM summary, Core mechanisms 1]); the RoPE and
 * schedule tables are kept.  Queues a counter reset on `stream`.  Reset also
 * clears the poison of an earlier KVM_E_HIP: it rewrites every counter and
 * exchange buffer the kernels read, and later calls rewrite the rest.
 * Errors: KVM_E_INVALID_ARG, KVM_E_HIP. */
kvm_status kvm_state_reset(kvm_state* st, void* stream);

/* Per-phase device times gathered with HIP events while profiling is enabled. */
typedef struct kvm_profile_times {
  double scan_ms;          int64_t scan_launches;          /* prefill absorption scan */
  double attn_ms;          int64_t attn_launches;          /* prefill attention over [state || window] */
  double ring_ms;          int64_t ring_launches;          /* ring refresh after prefill */
  double dec_absorb_ms;    int64_t dec_absorb_launches;    /* decode-time absorption */
  double dec_attn_ms;      int64_t dec_attn_launches;      /* decode step kernel: ring write + attention */
  double prep_ms;          int64_t prep_launches;          /* prefill RoPE prep of the call's keys */
} kvm_profile_times;

/* Phases for kvm_profile_enable's mask (fields of kvm_profile_times). */
#define KVM_PROFILE_SCAN 1
#define KVM_PROFILE_ATTN 2
#define KVM_PROFILE_RING 4
#define KVM_PROFILE_DEC_ABSORB 8
#define KVM_PROFILE_DEC_ATTN 16
#define KVM_PROFILE_PREP 32
#define KVM_PROFILE_ALL 63

/* Record a HIP event pair, on the stream the launch uses, around every later
 * kernel launch of the phases in `phases` (a KVM_PROFILE_* mask; 0 stops
 * recording).  Measurement only: the phases are the steps of [KVM summary,
 * Core mechanisms 1-5] (absorption, attention, window upkeep).
 * Errors: KVM_E_INVALID_ARG (NULL state, bits outside ALL). */
kvm_status kvm_profile_enable(kvm_state* st, int phases);

/* Wait for the recorded events (this one call synchronises the host with
 * them), add up the elapsed times per phase into *out, and clear the record.
 * Measurement only (phases as for kvm_profile_enable).
 * Errors: KVM_E_INVALID_ARG, KVM_E_HIP. */
kvm_status kvm_profile_read(kvm_state* st, kvm_profile_times* out);

/* Name of a status code, and the calling thread's message for the last failed
 * call.  Error reporting of this library; no passage of the method defines it. */
const char* kvm_status_str(kvm_status s);
const char* kvm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVM_H */
