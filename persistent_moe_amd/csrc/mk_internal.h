// mk_internal.h - layout shared by the host schedule builder (mk_host.cpp) and
// the persistent kernel (mk_kernel.hip): counter indices, task flags and the
// kernel argument block.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/mk.h"

// ---------------------------------------------------------------- task flags
enum {
  MK_F_EMBED = 1 << 0,      // ADD_RMSNORM: x = embedding row of the fed token
  MK_F_FINAL = 1 << 1,      // ADD_RMSNORM: final norm (gain = final_norm)
  MK_F_MID = 1 << 2,        // ADD_RMSNORM: sequential block, pre-FFN norm
  MK_F_FUSE_FINALIZE = 1 << 3,  // ROUTER_TOPK also runs ROUTE_FINALIZE
  MK_F_FUSE_TOPK = 1 << 4,  // ROUTER_GEMM: the last tile to finish runs top-k and
                            // ROUTE_FINALIZE and signals the layer's ROUTE counter
                            // (aux[0] = number of router tiles)
  MK_F_FUSE_COMBINE = 1 << 5   // ATTN_DRAIN: the last min(splits, ncomb) splits of a
                                // (sequence, group) to finish combine a share of its
                                // heads each and add their head count to COMB[group]
};

// descriptor words set by the schedule builder
enum {
  MK_AUX_WG = 16,      // aux[16]: workgroup the task runs on
  MK_AUX_INDEX = 17    // aux[17]: index of the task in the builder's list (trace row)
};

// ---------------------------------------------------------------- counters
// Global counters first, then one block of MK_CTR_* counters per layer
// (n_layers + 1 blocks; block n_layers holds the final norm counter).
enum {
  MK_CG_DONE = 0,     // workgroups finished with the step
  MK_CG_ABORT = 1,    // set when any wait timed out
  MK_CG_LM = 2,       // LM_HEAD tiles finished (sampling: the last one reduces)
  MK_CG_COUNT = 4
};
enum {
  MK_CTR_NORM = 0,    // ADD_RMSNORM of this layer done (target 1)
  MK_CTR_QKV = 1,     // QKV tiles done
  MK_CTR_ROUTER = 2,  // router tiles done
  MK_CTR_ROUTE = 3,   // top-k (+ finalize) done (target 1)
  MK_CTR_LAYER = 4,   // everything feeding the next norm
  MK_CTR_QATTN = 5,   // attention split queue head
  MK_CTR_QUG = 6,     // MoE up-gate queue head
  MK_CTR_QDN = 7,     // MoE down queue head
  MK_CTR_NORM2 = 8,   // sequential: pre-FFN norm done
  MK_CTR_OPROJ = 9,   // sequential: O-proj tiles done
  MK_CTR_FFNUG = 10,  // sequential: FFN gate/up tiles done
  MK_CTR_FIXED = 11   // then: COMB[Hkv], ATTN[B*Hkv], UG[B*k]
};

#define MK_CTR_PAD 64   // ints between consecutive counters (one 256-byte line each)

struct mk_ctr_layout {
  int32_t stride;     // counters per layer block
  int32_t comb;       // offset of COMB[g]
  int32_t attn;       // offset of ATTN[b*Hkv + g]
  int32_t ug;         // offset of UG[a]
  int32_t total;      // total counters
};

static inline mk_ctr_layout mk_make_ctr_layout(int32_t L, int32_t Hkv, int32_t B, int32_t topk) {
  mk_ctr_layout c;
  c.comb = MK_CTR_FIXED;
  c.attn = c.comb + Hkv;
  c.ug = c.attn + B * Hkv;
  int32_t s = c.ug + (topk > 0 ? B * topk : 1);
  c.stride = (s + 15) & ~15;
  c.total = MK_CG_COUNT + (L + 1) * c.stride;
  return c;
}

// ---------------------------------------------------------------- MoE routing
// Per layer (ints): [0] n_active, [1] up-gate items, [2] down items,
// [3] rows, then slot[BK] (row of each (token, k)), then one 16-int record
// per active expert: expert id, first row, rows, 0, token of each row (8).
static inline int32_t mk_moe_stride(int32_t bk) { return 4 + bk + 16 * bk; }

// ---------------------------------------------------------------- error record
// err[0] code, [1] task, [2] counter, [3] value, [4] target, [5] workgroup
#define MK_ERR_WORDS 8

// ---------------------------------------------------------------- kernel args
struct mk_layer_dev {
  const uint16_t* attn_norm;
  const uint16_t* ffn_norm;
  const uint16_t* w_qkv;
  const uint16_t* w_o;
  const uint16_t* w_router;
  const uint16_t* w_upgate;
  const uint16_t* w_down;
  const uint16_t* router_bias;   // [E] or null
  const float* upgate_scale;     // [E][2I] with FP8 experts, else null
  const float* down_scale;       // [E][d]  with FP8 experts, else null
  uint16_t* k;
  uint16_t* v;
};

struct mk_kargs {
  const mk_task* tasks;            // grouped by workgroup
  int32_t n_tasks;
  const int32_t* wg_range;        // [n_wg][2]: tasks [begin, end) this launch runs on each workgroup
  int32_t n_wg;                   // workgroups of the persistent grid
  int32_t* ctr;
  int32_t n_ctr;
  int32_t* err;
  const mk_layer_dev* layers;
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  const double* inv_freq;         // [hd/2] RoPE inverse frequencies
  // step inputs
  const int32_t* tokens;
  const int32_t* positions;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* logits;
  // sampling after LM_HEAD (next_tok null: none)
  int32_t* next_tok;              // [B] sampled token of each slot
  int32_t* lm_best;               // [n_lm_tiles][B][2]: best score (bits), id per tile
  float inv_temp;                 // 1 / temperature, 0 for greedy
  uint32_t sample_seed;
  int32_t advance;                // MK_SAMPLE_ADVANCE: update tokens, positions, seq_lens
  // shapes
  int32_t L, d, Hq, Hkv, hd, G, E, topk, I, F, V;
  int32_t parallel, page, swa_window, swa_period;
  int32_t expert_fp8;             // expert weights are E4M3 codes with per-row scales
  int32_t B, max_blocks, num_pages;
  float eps, attn_scale;
  int32_t attn_split, max_splits;
  int32_t ug_tiles, ug_pairs, dn_tiles, dn_rows;  // MoE tiling per expert
  int32_t n_qkv_tiles;
  int32_t ncomb;                  // fused combine: most workgroups sharing one (sequence, group)
  int32_t bk;                     // max rows of routed tokens (max_batch * top_k)
  int32_t moe_stride;
  mk_ctr_layout cl;
  uint64_t timeout_ticks;         // s_memrealtime ticks (100 MHz)
  // workspace regions
  float* x;        // [L+1][B][d]
  float* xn;       // [L+1][B][d]
  float* xmid;     // [L][B][d]   sequential
  float* xn2;      // [L][B][d]   sequential
  float* qkv;      // [L][B][qkv_rows]
  float* attn;     // [L][B][Hq*hd]
  float* opart;    // [L][Hkv][B][d]
  float* rlog;     // [L][B][E]
  int32_t* topi;   // [L][B][k]
  float* topw;     // [L][B][k]
  int32_t* moe;    // [L][moe_stride]
  float* H;        // [L][bk][I]   MoE
  float* Y;        // [L][bk][d]   MoE
  float* fh;       // [L][B][F]    dense
  float* fo;       // [L][B][d]    FFN (MoE or dense) output
  float* oout;     // [L][B][d]    O-projection output (sum over groups), tap
  float* part_ml;  // [2][B][Hq][max_splits][2]
  float* part_o;   // [2][B][Hq][max_splits][hd]
  uint64_t* trace; // [n_tasks][4] or null
};

// The library's per-device scratch array (mk_kernel.hip): its address on
// the current device (looked up once per device) and its size in bytes.
extern "C" int mk_scratch_region(void** ptr, size_t* bytes);

// host entry of the device code (mk_kernel.hip)
// wg_ranges: (1 + n_waves) blocks of [n_wg][2] (block 0: the whole step,
// block 1 + v: wave v, used by the one-launch-per-wave ablation)
extern "C" int mk_launch(const mk_kargs* args, int launch_mode, const int32_t* wg_ranges, int n_waves,
                         void* stream);
