/*
 * mk.h - C ABI of the MI355X persistent decode megakernel (libmk.so).
 *
 * One call of mk_decode_step runs one whole decode step of a transformer in
 * ONE kernel launch: every CU holds one resident workgroup that walks a
 * host-built list of tile-sized tasks, each a 32 x int32 descriptor over the
 * 16 opcodes below, with dependencies carried by counters in global memory
 * (persistent decode megakernel pages: page 1 "One kernel for the full decode
 * step", "The calling convention that makes it hand-writable" and
 * "Scheduling: mostly static, selectively dynamic"; page 4, the list of the
 * 16 task types and the description of the 32-int32 descriptor).
 *
 * Model family: a parallel-block MoE decoder,
 *     x += Attn(RMSNorm(x)) + MoE(RMSNorm(x))     (one shared norm),
 * or a sequential pre-norm dense decoder,
 *     x += Attn(RMSNorm1(x));  x += SwiGLU(RMSNorm2(x)),
 * both with grouped-query attention over a paged KV cache, rotate-half RoPE,
 * a final RMSNorm and an LM head.
 *
 * Conventions
 *  - Every function returns MK_OK (0) or a negative MK_E_* code; nothing
 *    throws across the ABI.  mk_strerror() names a code.
 *  - All device memory is owned by the caller: weights, the KV pool, the
 *    workspace, step inputs and logits.  The library allocates no device
 *    memory; mk_destroy frees only host state.
 *  - Pointers documented as "device" must be device-accessible addresses on
 *    the device that is current when mk_init is called.
 *  - bf16 = IEEE-754 binary16-brain (1 sign, 8 exponent, 7 mantissa bits),
 *    stored as 16-bit words.  All matrices are row-major [out][in].
 *  - A handle is not thread-safe.  Calls on one handle must be issued from
 *    one host thread, and its steps must be serialised on one stream.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ codes */
#define MK_OK 0
#define MK_E_INVAL (-1)       /* a bad argument (null pointer, size, range)  */
#define MK_E_UNSUPPORTED (-2) /* a shape this build does not handle          */
#define MK_E_NOMEM (-3)       /* workspace smaller than mk_workspace_size()  */
#define MK_E_HIP (-4)         /* a HIP runtime call failed                   */
#define MK_E_TIMEOUT (-5)     /* device watchdog: a counter wait timed out   */
#define MK_E_DEVICE (-6)      /* device-detected bad input (token, page id)  */
#define MK_E_STATE (-7)       /* call order (e.g. no schedule built yet)     */

/* ---------------------------------------------------------------- opcodes
 * The 16 task types (page 4, "16 task types" list; page 1, "The calling
 * convention that makes it hand-writable").                                */
enum mk_opcode {
  MK_OP_ADD_RMSNORM = 0,          /* residual add (+ MoE combine) and RMSNorm  */
  MK_OP_QKV_PROJ = 1,             /* QKV GEMV, RoPE, append K/V to the pages  */
  MK_OP_O_PROJ = 2,               /* output projection, split-K by KV group   */
  MK_OP_FFN_UPGATE_ACT = 3,       /* dense gate/up GEMV + SiLU-and-multiply   */
  MK_OP_FFN_DOWN = 4,             /* dense down projection                    */
  MK_OP_LM_HEAD = 5,              /* vocabulary GEMV into the caller's logits  */
  MK_OP_ATTN_DECODE = 6,          /* one split of attention (a static task;
                                     emitted with MK_SCHED_STATIC_ATTN)       */
  MK_OP_ATTN_COMBINE = 7,         /* log-sum-exp merge of the splits          */
  MK_OP_ATTN_DRAIN = 8,           /* claimer: drains the split queue          */
  MK_OP_ROUTER_GEMM = 9,          /* router logits                            */
  MK_OP_ROUTER_TOPK = 10,         /* top-k + softmax-renormalised gates       */
  MK_OP_ROUTE_FINALIZE = 11,      /* expert histogram, rows, claim queues     */
  MK_OP_MOE_GATHER = 12,          /* expert-sorted copy of the routed rows:
                                     never a task of its own here; the up-gate
                                     items read each routed row by token id  */
  MK_OP_MOE_UPGATE_ACT_DRAIN = 13,/* claimer: expert gate/up + SiLU-and-mul   */
  MK_OP_MOE_DOWN_DRAIN = 14,      /* claimer: expert down projection          */
  MK_OP_MOE_COMBINE = 15,         /* gate-weighted sum of the expert outputs:
                                     never a task of its own here; the next
                                     ADD_RMSNORM adds the expert rows in top-k
                                     order (a descriptor with opcode 12 or 15
                                     reports MK_E_INVAL)                     */
  MK_NUM_OPCODES = 16
};

/* ------------------------------------------------------------- descriptor
 * One task: 32 int32 (page 4: opcode, layer, output tile, split-K
 * coordinates, the counter waited on and the counter signalled).          */
typedef struct mk_task {
  int32_t op;          /* enum mk_opcode                                     */
  int32_t layer;       /* 0..n_layers-1; n_layers for the final norm / head  */
  int32_t wait_ctr;    /* counter index waited on, or -1                     */
  int32_t wait_target; /* value to reach; MK_WAIT_* for targets read at run time */
  int32_t signal_ctr;  /* counter index bumped on completion, or -1          */
  int32_t flags;       /* MK_F_* bits                                        */
  int32_t n0, n1;      /* output tile [n0, n1): rows, rotation pairs or items */
  int32_t k0, k1;      /* reduction range [k0, k1) (split-K coordinates)     */
  int32_t group;       /* KV group (attention, O_PROJ, combine)              */
  int32_t batch;       /* batch slot (ATTN_COMBINE, ATTN_DECODE)             */
  int32_t split;       /* split index (ATTN_DECODE)                          */
  int32_t queue;       /* queue-head counter index (claimers)                */
  int32_t aux[18];     /* opcode-specific words; aux[16] = workgroup the     *
                        * task runs on, aux[17] = its index in the list     *
                        * (both set by the schedule builder)                */
} mk_task;

#define MK_WAIT_NONE (-1)
#define MK_WAIT_SPLITS (-2)   /* target = number of splits of (batch, group) */

/* ------------------------------------------------------------------ model */
typedef struct mk_config {
  int32_t n_layers;        /* L                                              */
  int32_t d_model;         /* d, a multiple of 8                             */
  int32_t n_q_heads;       /* Hq                                             */
  int32_t n_kv_heads;      /* Hkv; Hq % Hkv == 0                             */
  int32_t head_dim;        /* hd: 64 or 128                                  */
  int32_t vocab;           /* V                                              */
  int32_t n_experts;       /* E; 0 selects the dense SwiGLU FFN              */
  int32_t top_k;           /* k (MoE)                                        */
  int32_t expert_inter;    /* I, per-expert SwiGLU width (MoE)               */
  int32_t ffn_inter;       /* F, dense SwiGLU width (dense)                  */
  int32_t parallel_block;  /* 1: parallel MoE block; 0: sequential pre-norm  */
  int32_t page_size;       /* tokens per KV page; must be 16                 */
  int32_t max_batch;       /* 1..8                                           */
  int32_t swa_window;      /* 0: all layers global; else window in tokens    */
  int32_t swa_period;      /* layer l is global iff l % period == period - 1 */
  float rope_theta;        /* RoPE base                                      */
  float rms_eps;           /* RMSNorm epsilon                                */
  int32_t expert_fp8;      /* 1: expert weights are FP8 (see mk_layer_weights);
                              MoE only, d and I <= 2048 and multiples of 16 */
} mk_config;

/* Per-layer weights, all device pointers to bf16, row-major [out][in].
 *   attn_norm [d]                    norm gain (the shared norm of the parallel
 *                                    block, or the pre-attention norm)
 *   ffn_norm  [d]                    pre-FFN norm gain (sequential only)
 *   w_qkv     [(Hq+2Hkv)*hd][d]      q heads, then k heads, then v heads;
 *                                    head h owns rows h*hd .. h*hd+hd-1
 *   w_o       [d][Hq*hd]
 *   w_router  [E][d]                 (MoE)
 *   w_upgate  [E][2I][d] (MoE) or [2F][d] (dense): gate rows, then up rows
 *   w_down    [E][d][I]  (MoE) or [d][F]  (dense)
 *   router_bias [E]                  optional (NULL: none), added to the
 *                                    router logits before the softmax and the
 *                                    top-k: it moves both the selection and
 *                                    the gate weights.  Real routing is
 *                                    concentrated on a few experts, and the
 *                                    pages report the megakernel's advantage
 *                                    growing there (page 1, "Benchmark
 *                                    results"); a bias reproduces that skew
 *                                    with synthetic weights.
 *   upgate_scale [E][2I], down_scale [E][d]   float32, with expert_fp8 only:
 *                                    w_upgate and w_down then hold OCP FP8
 *                                    E4M3 (e4m3fn) codes, one byte per weight
 *                                    in the same [out][in] order, and weight
 *                                    [r][k] = scale[r] * E4M3(code[r][k]).
 *                                    FP8 weight streaming is on the pages'
 *                                    roadmap (page 1, "Current limitations":
 *                                    no FP8/FP4 yet): it halves the bytes of
 *                                    the largest stream of a MoE step.    */
typedef struct mk_layer_weights {
  const void* attn_norm;
  const void* ffn_norm;
  const void* w_qkv;
  const void* w_o;
  const void* w_router;
  const void* w_upgate;
  const void* w_down;
  const void* router_bias;
  const void* upgate_scale;
  const void* down_scale;
} mk_layer_weights;

typedef struct mk_weights {
  const void* embed;        /* [V][d] bf16, device                           */
  const void* lm_head;      /* [V][d] bf16, device (== embed when tied)      */
  const void* final_norm;   /* [d] bf16, device                              */
  const mk_layer_weights* layers; /* host array of n_layers entries (copied) */
} mk_weights;

/* Paged KV cache: per layer, a K pool [num_pages][Hkv][hd/32][page_size][32]
 * and a V pool [num_pages][Hkv][hd][page_size], bf16 (device).  Within a page,
 * a K block holds the keys in 32-dimension slices (slice s of every key, then
 * slice s+1), and a V block one head dimension per row: the attention
 * products read each operand fragment as whole contiguous cache lines (a QK
 * k-step: 32 dims of 16 keys; PV: 8 consecutive keys of one dimension).
 * page_size must be 16.  The
 * kernel writes only the slot of each sequence's new token.  Slots of a
 * sequence's pages beyond its length are read (and given zero attention
 * weight), so pools must be initialised (e.g. zeroed): NaN there would
 * propagate.                                                              */
typedef struct mk_kv_pool {
  void* const* k;           /* host array of n_layers device pointers        */
  void* const* v;           /* host array of n_layers device pointers        */
  int32_t num_pages;
} mk_kv_pool;

/* ------------------------------------------------------------- schedule */
enum mk_wave_order {
  MK_ORDER_TUNED = 0,           /* QKV, router, attention, MoE, O-proj, norm */
  MK_ORDER_INTERLEAVED = 1,     /* attention and MoE claimers alternate       */
  MK_ORDER_ATTENTION_FIRST = 2, /* attention (with O-proj) before routing     */
  MK_ORDER_PARTITIONED = 3      /* a quarter of the workgroups (spread over all
                                   XCDs) run attention and O-proj, the rest the
                                   router and the MoE projections, so the two
                                   branches of the parallel block overlap      */
};

enum mk_launch_mode {
  MK_LAUNCH_PERSISTENT = 0,     /* one cooperative launch per step            */
  MK_LAUNCH_PER_OPCODE = 1      /* ablation: one launch per task wave         */
};

typedef struct mk_sched_opts {
  int32_t wave_order;       /* enum mk_wave_order                            */
  int32_t launch_mode;      /* enum mk_launch_mode                           */
  int32_t attn_split;       /* keys per attention split (multiple of page_size,
                               >= MK_MIN_SPLIT); 0 picks one from the shape  */
  int32_t n_workgroups;     /* 0: one per CU                                 */
  int32_t timeout_ms;       /* watchdog per wait; 0 = 2000 ms                */
  int32_t flags;            /* MK_SCHED_* bits; 0 in normal use              */
  int32_t moe_ug_pairs;     /* gate/up row pairs per MoE up-gate item
                               (1..512); 0 picks one from the shape and batch */
  int32_t moe_dn_rows;      /* output rows per MoE down item (1..d); 0 picks
                               one from the shape and batch                   */
} mk_sched_opts;

/* Test hook: prepend one task that waits on a counter no task signals, so
 * the device watchdog fires (MK_E_TIMEOUT after timeout_ms) and every
 * workgroup leaves the step through its normal exit.                      */
#define MK_SCHED_UNREACHABLE_WAIT 1
/* Record, per task, the 100 MHz device clock at task start, when its wait
 * was satisfied and at its end, into the MK_TAP_TRACE region.             */
#define MK_SCHED_TRACE 2
/* Emit ROUTER_TOPK as its own task instead of running it in the last router
 * tile to finish (one more counter hop per layer).                        */
#define MK_SCHED_SEPARATE_TOPK 4
/* With MK_SCHED_SEPARATE_TOPK: emit ROUTE_FINALIZE as a task of its own
 * after ROUTER_TOPK (one more hop) instead of running it inside the top-k
 * task.                                                                   */
#define MK_SCHED_SEPARATE_FINALIZE 64
/* Static attention: one ATTN_DECODE task per (sequence, KV group, split) of
 * the longest context the block tables allow, dealt round-robin like the
 * GEMM tiles, plus one ATTN_COMBINE task per (sequence, group); splits past
 * a sequence's live length return at once.  The default pulls splits from a
 * claim queue sized by the live lengths (page 1 "Scheduling: mostly static,
 * selectively dynamic": attention is one of the two dynamic task kinds).  */
#define MK_SCHED_STATIC_ATTN 128
/* Emit ATTN_COMBINE as its own task per (sequence, KV group) instead of
 * sharing it among the last attention splits of that group to finish (one
 * share of the group's query heads each; both give the same bits).        */
#define MK_SCHED_SEPARATE_COMBINE 8
/* Claimer c of a MoE up-gate or down queue owns item c in advance (one
 * fewer atomic per workgroup).  By default every MoE item is pulled from its
 * claim queue, so the workgroups that finish attention first take them.   */
#define MK_SCHED_STATIC_MOE 16
/* Tuned order only: every workgroup claims attention splits and then drains
 * the MoE up-gate queue before its O-proj tile.  By default, when a layer's
 * splits at the longest context fit in half the workgroups, that many
 * workgroups (spread evenly over the grid) own them and go from attention
 * straight to their O-proj tile, and only the others drain the up-gate
 * queue (page 1 "Scheduling: mostly static, selectively dynamic").        */
#define MK_SCHED_SHARED_ATTN 32

#define MK_MIN_SPLIT 64

/* ---------------------------------------------------------------- status */
typedef struct mk_status {
  int32_t code;             /* MK_OK or the first device error of the step   */
  int32_t task;             /* task index that failed                        */
  int32_t counter;          /* counter waited on                             */
  int32_t value;            /* its value when the watchdog fired              */
  int32_t target;           /* the target it waited for                      */
  int32_t workgroup;        /* workgroup that reported                       */
} mk_status;

typedef struct mk_handle mk_handle;

/* Bytes of device workspace needed for this model with block tables of
 * max_blocks_per_seq pages per sequence.  0 on an invalid config.
 * The pages give the engine as a shared library that a serving process loads
 * and drives (page 2, "// Getting started": the server is started with the
 * path of the built .so); the caller owns every device buffer, so it asks
 * here how much scratch memory to allocate (descriptors, counters, claim
 * queues, per-layer activations, attention partials, the error record).
 * max_blocks_per_seq is the width of the block tables: it bounds the longest
 * context, hence the attention partials and the task list, so it is fixed for
 * the life of the handle (it is an argument of mk_init, not of
 * mk_build_schedule).                                                     */
size_t mk_workspace_size(const mk_config* cfg, int32_t max_blocks_per_seq);

/* Validate the model, copy the weight and pool pointer tables, lay out the
 * caller's workspace (device, ws_bytes >= mk_workspace_size, 256-byte
 * aligned) and clear it.  The weights and KV pools are the caller's, read in
 * place and never copied: weights are immutable for the life of the handle
 * (page 3, the weight-prefetch paragraph: weights do not depend on the
 * step's activations, which is what lets tasks stream them before their
 * inputs are ready).  max_blocks_per_seq is fixed here (see
 * mk_workspace_size).  Synchronous.  On success *out owns host state only.
 * Errors: INVAL (null/odd shape), UNSUPPORTED, NOMEM, HIP.                */
int mk_init(const mk_config* cfg, const mk_weights* w, const mk_kv_pool* kv,
            void* workspace, size_t ws_bytes, int32_t max_blocks_per_seq,
            mk_handle** out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mk_init
 * without a caller workspace.  The handle's workspace is the library's own
 * file-scope device array of MK_NOALLOC_WS_BYTES, one per device (held from
 * the library's first use on a device until the process ends), and the
 * handle itself is the library's per-device one; no device or host memory is
 * allocated.  The layout leaves out the task-trace region (MK_SCHED_TRACE is
 * refused) and sizes the task list for at most one workgroup per CU.
 * A model and max_blocks_per_seq whose workspace does not fit return
 * MK_E_NOMEM (the 30B MoE at batch 1 and 8K context needs about 30 MB; batch
 * 8 at 16K does not fit and needs mk_init).  Each call on a device rebinds
 * and clears that device's array and handle: a handle returned earlier on the
 * same device then sees the new binding, and steps of two such handles must
 * not overlap (they would race on the one array).  mk_destroy on this handle
 * only forgets its schedule.  Other arguments and errors as mk_init.     */
#define MK_NOALLOC_WS_BYTES (48u << 20)
int mk_init_noalloc(const mk_config* cfg, const mk_weights* w, const mk_kv_pool* kv,
                    int32_t max_blocks_per_seq, mk_handle** out);

/* Build the task list for a batch of `batch_size` slots and upload it to the
 * workspace (the host builds named waves per layer and deals task k to
 * workgroup k mod N: page 1 "Scheduling: mostly static, selectively
 * dynamic"; page 3, the schedule paragraph).  The schedule is fixed for a
 * batch shape: call this again when the caller admits, evicts or resizes a
 * batch, with the decode loop stopped (page 3, the paragraph on the price of
 * a baked-in schedule).  Synchronous.  opt may be NULL for defaults.
 * Errors: INVAL, UNSUPPORTED, NOMEM, HIP.                                 */
int mk_build_schedule(mk_handle* h, int32_t batch_size, const mk_sched_opts* opt);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL = default).
 * All arrays are device pointers owned by the caller:
 *   token_ids    [B]              token fed to each slot
 *   positions    [B]              cache index of the new token (= tokens
 *                                 already cached); K/V are written there
 *   block_tables [B][max_blocks]  page ids of each slot, in order
 *   seq_lens     [B]              positions[b] + 1, or 0 for an empty slot
 *                                 (its logits row is zeroed)
 *   logits       [B][V] float32   output
 * Returns after the enqueue, with no host synchronisation.  Errors found on
 * the host return at once (INVAL, STATE); errors found on the device
 * (TIMEOUT, DEVICE) are latched and reported by mk_get_status.            */
int mk_decode_step(mk_handle* h, const int32_t* token_ids, const int32_t* positions,
                   const int32_t* block_tables, const int32_t* seq_lens, float* logits,
                   void* stream);

/* -------------------------------------------------------------- sampling
 * The pages' engine decodes with greedy or temperature sampling only (page 1,
 * "Current limitations").  mk_decode_step_sample runs the same step and
 * then picks each sequence's next token on the device, fused after LM_HEAD:
 * every LM_HEAD tile reduces its rows to a best (score, id) per sequence and
 * the last tile to finish reduces the tiles' bests, so no separate argmax
 * kernel and no host round trip are needed between steps.
 *   temperature == 0  greedy: the largest logit, ties to the lowest id;
 *   temperature  > 0  a draw from softmax(logits / temperature) by the
 *                     Gumbel-max method: the id maximising
 *                     logits[v] / temperature - ln(-ln u_v), with
 *                     u_v = (floor(h_v / 2^8) + 1/2) / 2^24 and
 *                     h_v = fmix32(fmix32(fmix32(fmix32(seed) ^ position)
 *                                  ^ slot) ^ v)
 *                     (fmix32: MurmurHash3's 32-bit finaliser; position =
 *                     positions[slot] of the step, the cache index of the
 *                     token that was fed).                                 */
#define MK_SAMPLE_ADVANCE 1   /* after the step, for every live slot b:
                                 token_ids[b] = next_tokens[b],
                                 positions[b] += 1, seq_lens[b] += 1 (the
                                 caller keeps pages for the new positions in
                                 the block tables), so steps can be enqueued
                                 back to back with no host work between    */
typedef struct mk_sampling {
  float temperature;        /* >= 0, finite                                  */
  uint32_t seed;            /* stream of the temperature draws               */
  int32_t flags;            /* MK_SAMPLE_* bits                              */
} mk_sampling;

/* mk_decode_step plus the next token of every slot, written to
 * next_tokens[B] (device, int32; -1 for an empty slot).  With
 * MK_SAMPLE_ADVANCE, token_ids, positions and seq_lens are updated in place
 * at the end of the step.  Errors as mk_decode_step; INVAL for a bad
 * sampling argument.                                                      */
int mk_decode_step_sample(mk_handle* h, int32_t* token_ids, int32_t* positions,
                          const int32_t* block_tables, int32_t* seq_lens, float* logits,
                          const mk_sampling* sampling, int32_t* next_tokens, void* stream);

/* Synchronise the handle's last stream, read and clear the device error
 * record.  st may be NULL.  Returns st->code.  A persistent kernel has no
 * kernel boundary at which a failure can surface (page 2, "// Overview":
 * blocks stay resident for the whole step and wait on counters), so a
 * failed wait or a bad input found on the device is latched in the
 * workspace, every workgroup leaves the step, and the host reads it here.
 * After MK_E_TIMEOUT the counters are cleared, so the next step starts
 * clean.                                                                  */
int mk_get_status(mk_handle* h, mk_status* st);

/* Byte offset and size, inside the workspace, of a per-layer debug tap
 * written by every step (see enum mk_tap).  Errors: INVAL, STATE.         */
enum mk_tap {
  MK_TAP_X = 0,             /* [L+1][B][d] f32 residual entering layer l (L: final) */
  MK_TAP_XN = 1,            /* [L+1][B][d] f32 normed input of layer l (L: final)    */
  MK_TAP_QKV = 2,           /* [L][B][(Hq+2Hkv)*hd] f32, q and k after RoPE          */
  MK_TAP_ATTN = 3,          /* [L][B][Hq*hd] f32 attention output (before W_o)       */
  MK_TAP_ROUTER_LOGITS = 4, /* [L][B][E] f32                                         */
  MK_TAP_TOPK_IDS = 5,      /* [L][B][k] int32, highest logit first                  */
  MK_TAP_TOPK_WEIGHTS = 6,  /* [L][B][k] f32                                         */
  MK_TAP_FFN_OUT = 7,       /* [L][B][d] f32 MoE (or dense FFN) output               */
  MK_TAP_ATTN_OUT = 8,      /* [L][B][d] f32 output projection (sum over groups)     */
  MK_TAP_TRACE = 9,         /* [n_tasks][16] u64: start, ready, marks[10] (0 staged, 1 computed,
                               2 stored, 3..9 opcode-specific), end, workgroup, opcode, 0
                               (MK_SCHED_TRACE; 100 MHz clock, 0 = mark not reached)          */
  MK_NUM_TAPS = 10
};
int mk_tap_offset(const mk_handle* h, int32_t tap, size_t* offset, size_t* bytes);

/* Host-only schedule planning (no GPU needed): fill up to `cap` tasks into
 * `out` for (cfg, batch_size, opt) on n_workgroups workgroups and report the
 * task and counter counts.  out may be NULL to query the counts.          */
int mk_plan_schedule(const mk_config* cfg, int32_t batch_size, int32_t max_blocks_per_seq,
                     const mk_sched_opts* opt, int32_t n_workgroups, mk_task* out,
                     int32_t cap, int32_t* n_tasks, int32_t* n_counters);

/* Host-only discrete-event check that a planned task list cannot deadlock:
 * n_workgroups in-order workers, claim queues sized from seq_lens[B] and
 * n_active_experts[L] (distinct routed experts per layer).  Returns MK_OK,
 * or MK_E_STATE with *stuck_task set to the first blocked task.           */
int mk_plan_simulate(const mk_config* cfg, int32_t batch_size, int32_t max_blocks_per_seq,
                     const mk_sched_opts* opt, int32_t n_workgroups, const int32_t* seq_lens,
                     const int32_t* n_active_experts, int32_t* stuck_task);

/* Free the handle's host state.  No device memory is touched or freed (the
 * caller owns it all); call it after the last step has completed.  Part of
 * the loaded-library life cycle (page 2, "// Getting started").          */
void mk_destroy(mk_handle* h);
/* A static string naming an MK_* code (never NULL).                       */
const char* mk_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
