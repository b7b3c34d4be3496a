// mk_host.cpp - C ABI of libmk.so: validation, workspace layout, the host
// schedule builder, a discrete-event deadlock check of a schedule, and the
// step launch.
//
// The schedule follows the persistent decode megakernel pages (page 1
// "Scheduling: mostly static, selectively dynamic"; page 3 on the tuned
// per-layer wave order QKV, router, attention, MoE projections, O-proj and
// RMSNorm): the host emits named waves per layer in a topological order and
// deals task k to workgroup k mod N.  Attention splits and MoE expert tiles,
// whose counts depend on live lengths and routing, are claimer tasks: claimer
// c of a wave owns item c of its queue and pulls any items beyond the number
// of claimers from an atomic queue head.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "mk_internal.h"

namespace {

constexpr int kMaxWorkgroups = 1024;
constexpr int kYsFloats = 8192;    // LDS capacity for scores / tile outputs (mk_kernel.hip)
constexpr int kXsFloats = 16384;   // LDS capacity for staged activations
constexpr int kMaxGemvK = 8192;    // GEMV reduction length: 16 register slots x 512 (half from 4 rows)

struct Layout {
  size_t off_tasks, off_ranges, off_ctr, off_err, off_layers, off_invf;
  size_t off_x, off_xn, off_xmid, off_xn2, off_qkv, off_attn, off_opart, off_rlog, off_topi, off_topw;
  size_t off_moe, off_H, off_Y, off_fh, off_fo, off_oout, off_pml, off_po, off_lmbest, off_trace;
  size_t total;
  int32_t max_tasks, n_ctr, max_splits, bk, moe_stride;
  int32_t nw_bound;   // schedules may use up to this many workgroups
  bool has_trace;     // the task-trace region exists
  mk_ctr_layout cl;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Elements of one staged GEMV input row in LDS: K rounded up to a power-of-two
// number of 512-element chunks (the register tile's K-chunks).
long staged_row(long K) {
  long ch = 1;
  while (ch * 512 < K) ch <<= 1;
  return ch * 512;
}

int validate_config(const mk_config* c) {
  if (!c) return MK_E_INVAL;
  if (c->n_layers <= 0 || c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->vocab <= 0)
    return MK_E_INVAL;
  if (c->n_q_heads % c->n_kv_heads != 0) return MK_E_INVAL;
  if (c->d_model % 8 != 0 || c->page_size <= 0) return MK_E_INVAL;
  if (c->page_size != 16) return MK_E_UNSUPPORTED;   // one 16-key MFMA tile per page
  if (c->n_layers > 128) return MK_E_UNSUPPORTED;    // the layer table is copied into LDS
  if (c->max_batch < 1 || c->max_batch > 8) return MK_E_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return MK_E_UNSUPPORTED;
  if (c->n_q_heads / c->n_kv_heads > 8) return MK_E_UNSUPPORTED;
  if (c->rms_eps < 0.f || !(c->rope_theta > 0.f)) return MK_E_INVAL;
  const bool moe = c->n_experts > 0;
  if (moe) {
    if (c->top_k < 1 || c->top_k > c->n_experts || c->n_experts > 256 || c->expert_inter <= 0)
      return MK_E_INVAL;
    if (c->expert_inter % 8 != 0) return MK_E_INVAL;
    if (c->max_batch * c->top_k > 64) return MK_E_UNSUPPORTED;
    if (!c->parallel_block) return MK_E_UNSUPPORTED;
  } else {
    if (c->ffn_inter <= 0 || c->ffn_inter % 8 != 0) return MK_E_INVAL;
    if (c->parallel_block) return MK_E_UNSUPPORTED;
    if ((size_t)c->max_batch * c->ffn_inter > (size_t)kXsFloats) return MK_E_UNSUPPORTED;
    if (c->ffn_inter > (c->max_batch >= 4 ? kMaxGemvK / 2 : kMaxGemvK)) return MK_E_UNSUPPORTED;
  }
  if ((size_t)c->max_batch * c->d_model > (size_t)kXsFloats) return MK_E_UNSUPPORTED;
  if (c->d_model > 4096) return MK_E_UNSUPPORTED;   // the norm task holds 4 chunks of 4 per thread
  if (moe && c->expert_inter > (c->max_batch >= 4 ? kMaxGemvK / 2 : kMaxGemvK)) return MK_E_UNSUPPORTED;
  if (c->top_k > 8 || c->n_kv_heads > 8) return MK_E_UNSUPPORTED;
  const int gd = c->n_q_heads / c->n_kv_heads * c->head_dim;
  if ((size_t)c->max_batch * gd > (size_t)kXsFloats) return MK_E_UNSUPPORTED;
  if (c->swa_window < 0 || c->swa_period < 0) return MK_E_INVAL;
  if (c->expert_fp8 != 0 && c->expert_fp8 != 1) return MK_E_INVAL;
  if (c->expert_fp8) {
    // FP8 expert GEMVs: K up to two 1024-element chunks (the staged row of
    // one batch row is then at most 2048 elements, 8 rows fit the staging
    // area), rows of whole 16-byte loads
    if (!moe) return MK_E_UNSUPPORTED;
    if (c->d_model > 2048 || c->expert_inter > 2048) return MK_E_UNSUPPORTED;
    if (c->d_model % 16 != 0 || c->expert_inter % 16 != 0) return MK_E_UNSUPPORTED;
  }
  // staged GEMV inputs (hi and lo bf16 rows, padded) must fit the LDS staging area
  {
    const long B = c->max_batch;
    long kmax = std::max<long>(staged_row(c->d_model), staged_row((long)gd));
    if (moe) kmax = std::max(kmax, staged_row(c->expert_inter));
    else kmax = std::max(kmax, staged_row(c->ffn_inter));
    if (c->expert_fp8) {   // the FP8 GEMVs stage whole 1024-element chunks
      kmax = std::max(kmax, 2 * staged_row((c->d_model + 1) / 2));
      kmax = std::max(kmax, 2 * staged_row((c->expert_inter + 1) / 2));
    }
    if (B * kmax > kXsFloats) return MK_E_UNSUPPORTED;
  }
  return MK_OK;
}

// Task-list capacity for schedules of up to nw workgroups.
int max_tasks_bound(const mk_config* c, int nw = kMaxWorkgroups) {
  const int per_layer = 8 * nw + 2 * c->max_batch * c->n_kv_heads + 64;
  return (c->n_layers + 1) * per_layer + nw;
}
int max_waves_bound(const mk_config* c) { return (c->n_layers + 1) * 12 + 4; }
// LM-head tiles: one per workgroup, or more when a tile would exceed the
// LDS rows of the sampling epilogue (kYsFloats / 8)
int max_lm_tiles(const mk_config* c, int nw = kMaxWorkgroups) { return nw + c->vocab / (kYsFloats / 8) + 1; }

// Workspace layout for schedules of up to nw_bound workgroups, with or
// without the task-trace region.
Layout make_layout(const mk_config* c, int32_t max_blocks, int nw_bound = kMaxWorkgroups, bool trace = true) {
  Layout L{};
  const int Lr = c->n_layers, B = c->max_batch, d = c->d_model, hd = c->head_dim;
  const int rows = (c->n_q_heads + 2 * c->n_kv_heads) * hd;
  const int adim = c->n_q_heads * hd;
  const int E = c->n_experts, K = c->top_k;
  L.bk = E > 0 ? B * K : 1;
  L.moe_stride = mk_moe_stride(L.bk);
  L.cl = mk_make_ctr_layout(Lr, c->n_kv_heads, B, E > 0 ? K : 0);
  L.n_ctr = L.cl.total;
  L.max_tasks = max_tasks_bound(c, nw_bound);
  L.nw_bound = nw_bound;
  L.has_trace = trace;
  const long max_ctx = (long)max_blocks * c->page_size;
  L.max_splits = (int)std::max<long>(1, (max_ctx + MK_MIN_SPLIT - 1) / MK_MIN_SPLIT);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes, 256); return r; };
  L.off_tasks = take((size_t)L.max_tasks * sizeof(mk_task));
  L.off_ranges = take((size_t)(1 + max_waves_bound(c)) * nw_bound * 2 * 4);
  L.off_ctr = take((size_t)L.n_ctr * MK_CTR_PAD * 4);
  L.off_err = take(MK_ERR_WORDS * 4);
  L.off_layers = take((size_t)Lr * sizeof(mk_layer_dev));
  L.off_invf = take((size_t)(hd / 2) * 8);
  L.off_x = take((size_t)(Lr + 1) * B * d * 4);
  L.off_xn = take((size_t)(Lr + 1) * B * d * 4);
  L.off_xmid = take(c->parallel_block ? 4 : (size_t)Lr * B * d * 4);
  L.off_xn2 = take(c->parallel_block ? 4 : (size_t)Lr * B * d * 4);
  L.off_qkv = take((size_t)Lr * B * rows * 4);
  L.off_attn = take((size_t)Lr * B * adim * 4);
  L.off_opart = take((size_t)Lr * c->n_kv_heads * B * d * 4);
  L.off_rlog = take(E > 0 ? (size_t)Lr * B * E * 4 : 4);
  L.off_topi = take(E > 0 ? (size_t)Lr * B * K * 4 : 4);
  L.off_topw = take(E > 0 ? (size_t)Lr * B * K * 4 : 4);
  L.off_moe = take(E > 0 ? (size_t)Lr * L.moe_stride * 4 : 4);
  L.off_H = take(E > 0 ? (size_t)Lr * L.bk * c->expert_inter * 4 : 4);
  L.off_Y = take(E > 0 ? (size_t)Lr * L.bk * d * 4 : 4);
  L.off_fh = take(E > 0 ? 4 : (size_t)Lr * B * c->ffn_inter * 4);
  L.off_fo = take((size_t)Lr * B * d * 4);
  L.off_oout = take((size_t)Lr * B * d * 4);
  L.off_pml = take((size_t)2 * B * c->n_q_heads * L.max_splits * 2 * 4);
  L.off_po = take((size_t)2 * B * c->n_q_heads * L.max_splits * hd * 4);
  L.off_lmbest = take((size_t)max_lm_tiles(c, nw_bound) * B * 2 * 4);
  L.off_trace = take(trace ? (size_t)L.max_tasks * 16 * 8 : 0);
  L.total = o;
  return L;
}

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

struct Plan;
void finalize_plan(Plan& p);

// ------------------------------------------------------------ plan builder
struct Plan {
  std::vector<mk_task> tasks;         // builder order; aux[16] = workgroup, aux[17] = index
  std::vector<int32_t> wave_bounds;   // starts of each named wave, then the end
  int nw = 0;                         // workgroups
  std::vector<mk_task> dev_tasks;     // tasks grouped by workgroup (builder order within one)
  std::vector<int32_t> ranges;        // (1 + waves) blocks of nw [begin, end) pairs into dev_tasks:
                                      // block 0 = the whole step, block 1 + v = wave v
  int n_ctr = 0;
  int attn_split = 0, max_splits = 0;
  int ug_tiles = 0, ug_pairs = 0, dn_tiles = 0, dn_rows = 0;
  int n_qkv = 0;
  int ncomb = 1;                      // fused combine: workgroups per (sequence, group)
  mk_ctr_layout cl{};
};

mk_task blank(int op, int layer) {
  mk_task t;
  std::memset(&t, 0, sizeof t);
  t.op = op;
  t.layer = layer;
  t.wait_ctr = -1;
  t.wait_target = 0;
  t.signal_ctr = -1;
  t.queue = -1;
  return t;
}

int ctr_of(const mk_ctr_layout& cl, int layer, int off) { return MK_CG_COUNT + layer * cl.stride + off; }

int build_plan(const mk_config* c, int B, int32_t max_blocks, const mk_sched_opts* opt, int NW, Plan* P) {
  if (B < 1 || B > c->max_batch || NW < 1 || NW > kMaxWorkgroups || max_blocks < 1) return MK_E_INVAL;
  mk_sched_opts o{};
  if (opt) o = *opt;
  if (o.wave_order < 0 || o.wave_order > 3 || o.launch_mode < 0 || o.launch_mode > 1) return MK_E_INVAL;
  const int Lr = c->n_layers, d = c->d_model, hd = c->head_dim, Hkv = c->n_kv_heads;
  const int G = c->n_q_heads / Hkv;
  const bool moe = c->n_experts > 0;
  const long max_ctx = (long)max_blocks * c->page_size;
  Plan& p = *P;
  p.cl = mk_make_ctr_layout(Lr, Hkv, c->max_batch, moe ? c->top_k : 0);
  p.n_ctr = p.cl.total;
  // workgroup sets of the partitioned order: blocks of 8 consecutive
  // workgroups (one per XCD, since workgroups are dealt round-robin over the
  // 8 XCDs), every 4th block runs attention and O-proj
  std::vector<int> setA, setM;
  for (int w = 0; w < NW; ++w) ((w / 8) % 4 == 0 ? setA : setM).push_back(w);
  // (too few workgroups for two sets: the tuned placement)
  const bool part = o.wave_order == MK_ORDER_PARTITIONED && moe && !setA.empty() && !setM.empty();
  const int n_attn_wg = part ? (int)setA.size() : NW;
  // attention split length: about one item per three attention workgroups
  // at the longest context.  Longer splits mean fewer partials to combine and
  // leave two thirds of the workgroups free for the MoE items; at 8K keys and
  // bs=1, 384-key splits measured 341 tok/s against 330 for one item per
  // workgroup (144 keys) and 310 for 128 keys.
  int S = o.attn_split;
  // scores of a split live in LDS as [G][S + 32] floats (a split that does
  // not start on a page boundary touches one extra 16-key tile, and the
  // PV pass rounds the tiles up to pairs)
  const int smax = std::min((kYsFloats / G - 32) / 16 * 16, 1024);
  if (S > 0) {
    if (S % c->page_size != 0 || S < MK_MIN_SPLIT || S > smax) return MK_E_INVAL;
  } else {
    const long per = std::max(1, n_attn_wg / 3);
    long want = (max_ctx * B * Hkv + per - 1) / per;
    want = std::max<long>(want, MK_MIN_SPLIT);
    want = (want + c->page_size - 1) / c->page_size * c->page_size;
    // a whole number of QK passes: the kernel's three compute waves take four
    // 16-key tiles each per pass (400 keys ran a third, almost empty pass and
    // measured 334 tok/s against 341 for 384; at the LDS cap, 960 keys ran
    // the 256K context at 216.7 tok/s against 212.3 for 992)
    constexpr long kPassKeys = 16 * 3 * 4;
    const long cap = smax >= kPassKeys ? smax / kPassKeys * kPassKeys : smax;
    if (want < cap && want > kPassKeys) want = (want + kPassKeys / 2) / kPassKeys * kPassKeys;
    S = (int)std::min<long>(want, cap);
    S = std::max(S, MK_MIN_SPLIT);
  }
  p.attn_split = S;
  p.max_splits = ceil_div(max_ctx, S);
  if (p.max_splits > 1024) return MK_E_UNSUPPORTED;
  // tilings
  int r_rows = 0, n_r = 0;
  if (moe) {
    r_rows = std::max(8, ceil_div(c->n_experts, 8));
    n_r = ceil_div(c->n_experts, r_rows);
  }
  // tuned order: the router tiles (head of the MoE chain) get workgroups of
  // their own, [0, n_r), and the QKV tiles are spread over the others
  const bool router_own = moe && o.wave_order == MK_ORDER_TUNED && NW > 2 * n_r;
  const int qkv_wg = router_own ? NW - n_r : NW;
  const int pairs_tot = (c->n_q_heads + 2 * Hkv) * hd / 2;
  const int qkv_pp = std::max(1, ceil_div(pairs_tot, qkv_wg));
  const int n_qkv = ceil_div(pairs_tot, qkv_pp);
  if (2 * qkv_pp > kYsFloats / 8) return MK_E_UNSUPPORTED;
  p.n_qkv = n_qkv;
  const int o_tiles_g = std::max(1, (part ? n_attn_wg : NW) / Hkv);
  const int o_rows = ceil_div(d, o_tiles_g);
  const int n_o_g = ceil_div(d, o_rows);
  // LM-head tiles land in LDS (8 rows per batch slot of kYsFloats) for the
  // sampling epilogue: at most kYsFloats / 8 rows each
  const int lm_rows = std::min(ceil_div(c->vocab, NW), kYsFloats / 8);
  const int n_lm = ceil_div(c->vocab, lm_rows);
  // Attention owners (tuned order): when a layer's attention items, at the
  // longest context the block tables allow, fit in half the workgroups,
  // only that many workgroups claim them (spread evenly over the grid) and
  // then go straight on to their O-proj tile, which is ready when the
  // attention ends; the other workgroups drain the up-gate queue meanwhile.
  // Shared, every workgroup would enter the up-gate drain after its split
  // and reach its O-proj tile only after that drain's round trips.
  const bool static_attn = (o.flags & MK_SCHED_STATIC_ATTN) != 0;
  const bool fuse_combine = !(o.flags & MK_SCHED_SEPARATE_COMBINE) && !static_attn;
  p.ncomb = std::max(1, std::min(G, (NW - 1) / std::max(1, B * Hkv) + 1));
  const bool owners_ok = moe && o.wave_order == MK_ORDER_TUNED && !part && fuse_combine &&
                         !(o.flags & MK_SCHED_SHARED_ATTN);
  auto vis_ctx = [&](int l) -> long {
    return (c->swa_window > 0 && c->swa_period > 0 && l % c->swa_period != c->swa_period - 1)
               ? std::min<long>(max_ctx, c->swa_window)
               : max_ctx;
  };
  // number of owners of layer l's attention items, or 0 (shared): between a
  // quarter and half of the workgroups.  The live items never outnumber the
  // owners, so owner i runs item i and nothing is pulled from the queue: a
  // fused combine that waits for the other splits of its group waits for
  // owners that need nothing from it.  Fewer owners would each take a large
  // share of the O-proj rows (the 4096-key window layers of the 256K model
  // have 20 splits: 410-row tiles, 202 tok/s against 221.9 shared).
  auto owners_of = [&](int l) -> int {
    if (!owners_ok) return 0;
    const long n = (long)B * Hkv * ceil_div(vis_ctx(l), S);
    return n >= NW / 4 && n <= NW / 2 ? (int)n : 0;
  };
  int owners_max = 0;
  for (int l = 0; l < Lr; ++l) owners_max = std::max(owners_max, owners_of(l));
  if (moe) {
    const int K = c->top_k, I = c->expert_inter;
    if (o.moe_ug_pairs < 0 || o.moe_ug_pairs > kYsFloats / 8 / 2 || o.moe_dn_rows < 0 || o.moe_dn_rows > d)
      return MK_E_INVAL;
    // Up-gate items: at most one per workgroup that drains the queue (all of
    // them, or those that do not own attention), the same number for each of
    // the k experts of one row.  bs=1, 30B model: shared attention, 24 pairs
    // (348 tok/s against 326 for 16 and 347 for 32); attention owners, 39
    // pairs for 164 drainers (374.9 against 369.9 for 48, and 361.9 for 32,
    // whose 192 items need a second round).  With more rows, larger items in
    // proportion to the distinct experts expected under uniform routing,
    // E (1 - (1 - k/E)^B), at 1.5 k per multiple, up to 4 (bs=8, about 52
    // experts: 96 pairs, 838 tok/s against 730 for 24 and 798 for 48; with
    // concentrated routing, about 21 experts, 1057 against 971).
    int ug_mult = 1;
    if (B > 1) {
      const double ex = c->n_experts * (1.0 - std::pow(1.0 - (double)K / c->n_experts, B));
      ug_mult = std::min(4, std::max(1, (int)std::lround(ex / (1.5 * K))));
    }
    const int ug_wg = NW - owners_max;
    p.ug_pairs = o.moe_ug_pairs > 0 ? o.moe_ug_pairs : ceil_div(I, std::max(1, ug_wg / K)) * ug_mult;
    p.ug_pairs = std::min(p.ug_pairs, kYsFloats / 8 / 2);
    p.ug_tiles = ceil_div(I, p.ug_pairs);
    // Down items: with attention owners, about one per up-gate drainer (the
    // drainers go from the up-gate drain straight to the down drain; the
    // owners have their O-proj tiles first), rounded up to whole rounds of
    // the GEMV's row groups (three compute waves of 16 weight slots; a row
    // of I weights takes 2^kl slots of 512 bf16 or 1024 FP8 weights).  30B
    // model: 120 rows (five rounds of 24; 136 items), 393.2 tok/s against
    // 386.7 for 144, 379.4 for 168, 384.6 for 96, 385.5 for 72 and 387.9 for
    // 48.  Shared attention: one per two workgroups (128 rows: 350 against
    // 341 for 64 and 318 for 256).
    if (owners_max) {
      const int chunk = c->expert_fp8 ? 1024 : 512;
      int kl = 0;
      while ((chunk << kl) < I) ++kl;
      const int round_rows = std::max(1, 3 * (16 >> kl));
      const int per_wg = std::max(1, ceil_div((long)K * d, ug_wg));
      p.dn_rows = ceil_div(per_wg, round_rows) * round_rows;
    } else {
      p.dn_rows = std::max(1, ceil_div((long)K * d, std::max(1, NW / 2)));
    }
    if (o.moe_dn_rows > 0) p.dn_rows = o.moe_dn_rows;
    p.dn_rows = std::min(p.dn_rows, d);
    // with several rows, 3/4 of that (bs=8: 96 rows, 846 tok/s against 836
    // for 128 and 816 for 64; concentrated routing 1084 against 1077)
    if (o.moe_dn_rows <= 0 && B > 1) p.dn_rows = std::max(16, p.dn_rows * 3 / 4 / 16 * 16);
    p.dn_tiles = ceil_div(d, p.dn_rows);
  }
  int ffn_pp = 0, n_fug = 0, ffn_rows = 0, n_fdn = 0;
  if (!moe) {
    ffn_pp = std::max(1, ceil_div(c->ffn_inter, NW));
    ffn_pp = std::min(ffn_pp, kYsFloats / 8 / 2);
    n_fug = ceil_div(c->ffn_inter, ffn_pp);
    ffn_rows = std::max(1, ceil_div(d, NW));
    n_fdn = ceil_div(d, ffn_rows);
  }
  const int n_claim = NW;
  std::vector<mk_task>& T = p.tasks;
  T.clear();
  p.wave_bounds.clear();
  p.nw = NW;
  // default placement: task k on workgroup k mod NW
  auto push_on = [&](mk_task t, int wg) {
    t.aux[MK_AUX_WG] = wg;
    t.aux[MK_AUX_INDEX] = (int32_t)T.size();
    T.push_back(t);
  };
  auto push = [&](const mk_task& t) { push_on(t, (int)(T.size() % NW)); };
  auto wave = [&]() { p.wave_bounds.push_back((int32_t)T.size()); };
  if (o.flags & MK_SCHED_UNREACHABLE_WAIT) {
    // waits on a global counter slot that nothing signals
    wave();
    mk_task t = blank(MK_OP_LM_HEAD, Lr);
    t.n0 = 0;
    t.n1 = std::min(c->vocab, 8);
    t.wait_ctr = MK_CG_COUNT - 1;
    t.wait_target = 1;
    push(t);
  }

  // claimers / tiles on a workgroup set, or round-robin over all (null)
  auto place = [&](const mk_task& t, const std::vector<int>* set, int i) {
    if (set) push_on(t, (*set)[i % set->size()]);
    else push(t);
  };
  const std::vector<int>* onA = part ? &setA : nullptr;
  const std::vector<int>* onM = part ? &setM : nullptr;
  // the fused combine of a (sequence, group) is shared by its last ncomb
  // splits (p.ncomb above), one share of the G heads each; all but the last
  // wait for the rest, so at most (ncomb - 1) * B * Hkv workgroups wait at
  // once, and one more must stay free to claim the remaining splits
  // owner workgroup i of n: owner i goes to XCD i mod 8 (workgroups are
  // dealt round-robin over the 8 XCDs), and the owners of one XCD are
  // spread evenly over its workgroups, counted from the end of the grid
  // (the router tiles sit on the first workgroups and the last ones hold no
  // QKV tile); with a grid that is not a multiple of 8, evenly over the grid
  auto owner_wg = [&](int i, int n) {
    if (NW % 8 != 0 || n > NW / 2) return NW - 1 - (int)((long)i * NW / n);
    const int x = i % 8, k = i / 8, per_x = NW / 8;
    const int c_x = (n - x + 7) / 8;   // owners on XCD x
    return NW - 1 - (x + 8 * (int)((long)k * per_x / c_x));
  };
  int layer_target_prev = 0;
  for (int l = 0; l <= Lr; ++l) {
    // ADD_RMSNORM entering layer l (l == Lr: the final norm), one task per
    // sequence: each row is an independent reduction, and one workgroup
    // summing the residual sources of every row in turn would put B memory
    // round trips on the critical path
    wave();
    for (int b = 0; b < B; ++b) {
      mk_task t = blank(MK_OP_ADD_RMSNORM, l);
      t.batch = b;
      if (l == 0) {
        t.flags |= MK_F_EMBED;
      } else {
        t.wait_ctr = ctr_of(p.cl, l - 1, MK_CTR_LAYER);
        t.wait_target = layer_target_prev;
      }
      if (l == Lr) t.flags |= MK_F_FINAL;
      t.signal_ctr = ctr_of(p.cl, l, MK_CTR_NORM);
      place(t, onA, b);
    }
    if (l == Lr) break;
    const int cNORM = ctr_of(p.cl, l, MK_CTR_NORM);
    auto emit_qkv = [&]() {
      wave();
      for (int i = 0; i < n_qkv; ++i) {
        mk_task t = blank(MK_OP_QKV_PROJ, l);
        t.n0 = i * qkv_pp;
        t.n1 = std::min(pairs_tot, t.n0 + qkv_pp);
        t.wait_ctr = cNORM;
        t.wait_target = B;
        t.signal_ctr = ctr_of(p.cl, l, MK_CTR_QKV);
        if (router_own) push_on(t, n_r + i);
        else push(t);
      }
    };
    auto emit_attn = [&]() {
      wave();
      if (static_attn) {
        // one task per (sequence, group, split) of the longest visible
        // context of this layer; splits past a live length return at once
        const long vis = (c->swa_window > 0 && c->swa_period > 0 && l % c->swa_period != c->swa_period - 1)
                             ? std::min<long>(max_ctx, c->swa_window)
                             : max_ctx;
        const int ns_max = ceil_div(vis, S);
        for (int b = 0; b < B; ++b)
          for (int g = 0; g < Hkv; ++g)
            for (int sp = 0; sp < ns_max; ++sp) {
              mk_task t = blank(MK_OP_ATTN_DECODE, l);
              t.batch = b;
              t.group = g;
              t.split = sp;
              t.wait_ctr = ctr_of(p.cl, l, MK_CTR_QKV);
              t.wait_target = n_qkv;
              t.signal_ctr = ctr_of(p.cl, l, p.cl.attn + b * Hkv + g);
              place(t, onA, b * Hkv * ns_max + g * ns_max + sp);
            }
        return;
      }
      const int own = owners_of(l);
      const int nc = own ? own : onA ? (int)onA->size() : n_claim;
      for (int i = 0; i < nc; ++i) {
        mk_task t = blank(MK_OP_ATTN_DRAIN, l);
        t.n0 = i;
        t.n1 = nc;
        t.wait_ctr = ctr_of(p.cl, l, MK_CTR_QKV);
        t.wait_target = n_qkv;
        t.queue = ctr_of(p.cl, l, MK_CTR_QATTN);
        if (fuse_combine) t.flags |= MK_F_FUSE_COMBINE;
        if (own) push_on(t, owner_wg(i, own));
        else place(t, onA, i);
      }
    };
    auto emit_combine = [&]() {
      if (fuse_combine) return;
      wave();
      for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g) {
          mk_task t = blank(MK_OP_ATTN_COMBINE, l);
          t.batch = b;
          t.group = g;
          t.wait_ctr = ctr_of(p.cl, l, p.cl.attn + b * Hkv + g);
          t.wait_target = MK_WAIT_SPLITS;
          t.signal_ctr = ctr_of(p.cl, l, p.cl.comb + g);
          push(t);
        }
    };
    // O-proj tiles of layer l: with attention owners, one per owner (the
    // owners reach them as their attention ends, and the up-gate drainers
    // go on to the down drain without one); else one per workgroup
    const int own_l = owners_of(l);
    const int o_rows_l = own_l ? ceil_div(d, std::max(1, own_l / Hkv)) : o_rows;
    const int n_o_g_l = own_l ? ceil_div(d, o_rows_l) : n_o_g;
    auto emit_oproj = [&](int signal) {
      wave();
      for (int g = 0; g < Hkv; ++g)
        for (int i = 0; i < n_o_g_l; ++i) {
          mk_task t = blank(MK_OP_O_PROJ, l);
          t.group = g;
          t.n0 = i * o_rows_l;
          t.n1 = std::min(d, t.n0 + o_rows_l);
          t.k0 = g * G * hd;
          t.k1 = t.k0 + G * hd;
          t.wait_ctr = ctr_of(p.cl, l, p.cl.comb + g);
          t.wait_target = B * G;   // every head of every sequence
          t.signal_ctr = signal;
          if (own_l) push_on(t, owner_wg(g * n_o_g_l + i, own_l));
          else place(t, onA, g * n_o_g + i);
        }
    };
    if (moe) {
      const int cROUTE = ctr_of(p.cl, l, MK_CTR_ROUTE);
      const int cLAYER = ctr_of(p.cl, l, MK_CTR_LAYER);
      const bool fuse_topk = !(o.flags & MK_SCHED_SEPARATE_TOPK);
      auto emit_router = [&]() {
        wave();
        for (int i = 0; i < n_r; ++i) {
          mk_task t = blank(MK_OP_ROUTER_GEMM, l);
          t.n0 = i * r_rows;
          t.n1 = std::min(c->n_experts, t.n0 + r_rows);
          t.wait_ctr = cNORM;
          t.wait_target = B;
          t.signal_ctr = ctr_of(p.cl, l, MK_CTR_ROUTER);
          if (fuse_topk) {
            t.flags |= MK_F_FUSE_TOPK;
            t.aux[0] = n_r;
          }
          if (router_own) push_on(t, i);
          else place(t, onM, i);
        }
        if (fuse_topk) return;
        wave();
        const bool sep_fin = (o.flags & MK_SCHED_SEPARATE_FINALIZE) != 0;
        mk_task t = blank(MK_OP_ROUTER_TOPK, l);
        if (!sep_fin) t.flags |= MK_F_FUSE_FINALIZE;
        t.wait_ctr = ctr_of(p.cl, l, MK_CTR_ROUTER);
        t.wait_target = n_r;
        // top-k alone adds one more to the router counter, which the
        // finalize task waits for
        t.signal_ctr = sep_fin ? ctr_of(p.cl, l, MK_CTR_ROUTER) : cROUTE;
        place(t, onM, 0);
        if (!sep_fin) return;
        wave();
        mk_task f = blank(MK_OP_ROUTE_FINALIZE, l);
        f.wait_ctr = ctr_of(p.cl, l, MK_CTR_ROUTER);
        f.wait_target = n_r + 1;
        f.signal_ctr = cROUTE;
        place(f, onM, 1);
      };
      const int n_moe_claim = onM ? (int)onM->size() : n_claim;
      const bool dyn_moe = (o.flags & MK_SCHED_STATIC_MOE) == 0;
      auto emit_ug = [&]() {
        wave();
        const int own = owners_of(l);
        std::vector<int> drainers;   // with attention owners: every other workgroup
        if (own) {
          std::vector<char> is_owner(NW, 0);
          for (int i = 0; i < own; ++i) is_owner[owner_wg(i, own)] = 1;
          for (int w = 0; w < NW; ++w)
            if (!is_owner[w]) drainers.push_back(w);
        }
        const int n = own ? (int)drainers.size() : n_moe_claim;
        for (int i = 0; i < n; ++i) {
          mk_task t = blank(MK_OP_MOE_UPGATE_ACT_DRAIN, l);
          t.n0 = dyn_moe ? INT32_MAX : i;
          t.n1 = dyn_moe ? 0 : n;
          t.wait_ctr = cROUTE;
          t.wait_target = 1;
          t.queue = ctr_of(p.cl, l, MK_CTR_QUG);
          if (own) push_on(t, drainers[i]);
          else place(t, onM, i);
        }
      };
      auto emit_dn = [&]() {
        wave();
        for (int i = 0; i < n_moe_claim; ++i) {
          mk_task t = blank(MK_OP_MOE_DOWN_DRAIN, l);
          t.n0 = dyn_moe ? INT32_MAX : i;
          t.n1 = dyn_moe ? 0 : n_moe_claim;
          t.wait_ctr = cROUTE;
          t.wait_target = 1;
          t.queue = ctr_of(p.cl, l, MK_CTR_QDN);
          t.signal_ctr = cLAYER;
          place(t, onM, i);
        }
      };
      switch (o.wave_order) {
        case MK_ORDER_ATTENTION_FIRST:
          emit_qkv(); emit_attn(); emit_combine(); emit_oproj(cLAYER);
          emit_router(); emit_ug(); emit_dn();
          break;
        case MK_ORDER_INTERLEAVED:
          emit_qkv(); emit_router(); emit_ug(); emit_attn(); emit_dn(); emit_combine(); emit_oproj(cLAYER);
          break;
        case MK_ORDER_PARTITIONED:   // per set: A = QKV, attention, O-proj; M = QKV, router, up-gate, down
          emit_qkv(); emit_router(); emit_attn(); emit_ug(); emit_combine(); emit_dn(); emit_oproj(cLAYER);
          break;
        default:  // tuned: router, QKV, attention, up-gate, O-proj, down, norm
          emit_router(); emit_qkv(); emit_attn(); emit_ug(); emit_combine(); emit_oproj(cLAYER); emit_dn();
          break;
      }
      layer_target_prev = n_moe_claim + Hkv * n_o_g_l;
    } else {
      const int cO = ctr_of(p.cl, l, MK_CTR_OPROJ);
      const int cN2 = ctr_of(p.cl, l, MK_CTR_NORM2);
      const int cFUG = ctr_of(p.cl, l, MK_CTR_FFNUG);
      emit_qkv(); emit_attn(); emit_combine(); emit_oproj(cO);
      wave();
      for (int b = 0; b < B; ++b) {
        mk_task t = blank(MK_OP_ADD_RMSNORM, l);
        t.flags |= MK_F_MID;
        t.batch = b;
        t.wait_ctr = cO;
        t.wait_target = Hkv * n_o_g;
        t.signal_ctr = cN2;
        push(t);
      }
      wave();
      for (int i = 0; i < n_fug; ++i) {
        mk_task t = blank(MK_OP_FFN_UPGATE_ACT, l);
        t.n0 = i * ffn_pp;
        t.n1 = std::min(c->ffn_inter, t.n0 + ffn_pp);
        t.wait_ctr = cN2;
        t.wait_target = B;
        t.signal_ctr = cFUG;
        push(t);
      }
      wave();
      for (int i = 0; i < n_fdn; ++i) {
        mk_task t = blank(MK_OP_FFN_DOWN, l);
        t.n0 = i * ffn_rows;
        t.n1 = std::min(d, t.n0 + ffn_rows);
        t.wait_ctr = cFUG;
        t.wait_target = n_fug;
        t.signal_ctr = ctr_of(p.cl, l, MK_CTR_LAYER);
        push(t);
      }
      layer_target_prev = n_fdn;
    }
  }
  wave();
  for (int i = 0; i < n_lm; ++i) {
    mk_task t = blank(MK_OP_LM_HEAD, Lr);
    t.n0 = i * lm_rows;
    t.n1 = std::min(c->vocab, t.n0 + lm_rows);
    t.wait_ctr = ctr_of(p.cl, Lr, MK_CTR_NORM);
    t.wait_target = B;
    t.aux[0] = n_lm;     // tiles (the last to finish reduces the sampling bests)
    t.aux[1] = i;        // this tile's slot in lm_best
    push(t);
  }
  p.wave_bounds.push_back((int32_t)T.size());
  if ((int)T.size() > max_tasks_bound(c)) return MK_E_NOMEM;
  if ((int)p.wave_bounds.size() - 1 > max_waves_bound(c)) return MK_E_NOMEM;
  finalize_plan(p);
  return MK_OK;
}

// Group the tasks by workgroup (keeping builder order within one) and record,
// for the whole step and for every wave, the range of each workgroup's tasks.
void finalize_plan(Plan& p) {
  const int NW = p.nw, n = (int)p.tasks.size();
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return p.tasks[x].aux[MK_AUX_WG] < p.tasks[y].aux[MK_AUX_WG]; });
  p.dev_tasks.resize(n);
  for (int i = 0; i < n; ++i) p.dev_tasks[i] = p.tasks[order[i]];
  const int nwaves = (int)p.wave_bounds.size() - 1;
  p.ranges.assign((size_t)(1 + nwaves) * NW * 2, 0);
  // first position of each workgroup in dev_tasks
  std::vector<int> start(NW + 1, 0);
  for (int i = 0; i < n; ++i) start[p.tasks[i].aux[MK_AUX_WG] + 1]++;
  for (int w = 0; w < NW; ++w) start[w + 1] += start[w];
  for (int w = 0; w < NW; ++w) {
    p.ranges[2 * w] = start[w];
    p.ranges[2 * w + 1] = start[w + 1];
    int pos = start[w];
    for (int v = 0; v < nwaves; ++v) {
      int32_t* r = &p.ranges[((size_t)(1 + v) * NW + w) * 2];
      while (pos < start[w + 1] && p.dev_tasks[pos].aux[MK_AUX_INDEX] < p.wave_bounds[v]) ++pos;
      r[0] = pos;
      while (pos < start[w + 1] && p.dev_tasks[pos].aux[MK_AUX_INDEX] < p.wave_bounds[v + 1]) ++pos;
      r[1] = pos;
    }
  }
}

// ------------------------------------------------------- deadlock checker
// Discrete-event model of the persistent kernel: NW in-order workers, task k
// on worker k mod NW; a task runs when its counter reaches its target; a
// claimer owns item c of its queue and then pulls items past the number of
// claimers one at a time.  Items of a down queue wait on their expert's
// up-gate counter.  Any state in which no worker can advance and some task is
// unfinished is a deadlock.
struct SimQueue {
  int n_items = 0, head = 0;
};

int simulate(const mk_config* c, int B, const Plan& p, int NW, const int32_t* seq_lens,
             const int32_t* n_active, int32_t* stuck) {
  const int Hkv = c->n_kv_heads, Lr = c->n_layers;
  std::vector<long> ctr(p.n_ctr, 0);
  auto vis = [&](int l, int sl) {
    if (c->swa_window > 0 && c->swa_period > 0 && l % c->swa_period != c->swa_period - 1)
      return std::min(sl, c->swa_window);
    return sl;
  };
  auto nspl = [&](int l, int b) {
    int sl = seq_lens[b];
    return sl <= 0 ? 0 : ceil_div(vis(l, sl), p.attn_split);
  };
  if (NW != p.nw) return MK_E_INVAL;
  // worker w walks dev_tasks [ranges[2w], ranges[2w+1])
  std::vector<int> cursor(NW), cend(NW);
  for (int w = 0; w < NW; ++w) {
    cursor[w] = p.ranges[2 * w];
    cend[w] = p.ranges[2 * w + 1];
  }
  // per-claimer state: -1 before the static item, then dynamic claiming
  std::vector<int> phase(NW, 0);
  std::vector<int> cur_item(NW, -1);
  // a fused-combine share waiting for the other splits of its (b, g):
  // counter, target, COMB counter, heads
  struct PendComb { int ctr = -1, target = 0, comb = 0, heads = 0; };
  std::vector<PendComb> pend(NW);
  const int G = c->n_q_heads / Hkv;
  std::vector<SimQueue> qa(Lr), qu(Lr), qd(Lr);
  for (int l = 0; l < Lr; ++l) {
    int na = 0;
    for (int b = 0; b < B; ++b) na += Hkv * nspl(l, b);
    qa[l].n_items = na;
    if (c->n_experts > 0) {
      qu[l].n_items = n_active[l] * p.ug_tiles;
      qd[l].n_items = n_active[l] * p.dn_tiles;
    }
  }
  const int n_tasks = (int)p.tasks.size();
  // attention item -> (b, g)
  auto attn_bg = [&](int l, int item, int* b_out, int* g_out) {
    for (int b = 0; b < B; ++b) {
      int ns = nspl(l, b), cnt = ns * Hkv;
      if (item < cnt) { *b_out = b; *g_out = item / ns; return; }
      item -= cnt;
    }
    *b_out = *g_out = 0;
  };
  for (long iter = 0;; ++iter) {
    bool progress = false, all_done = true;
    for (int w = 0; w < NW; ++w) {
      while (cursor[w] < cend[w]) {
        all_done = false;
        if (pend[w].ctr >= 0) {
          if (ctr[pend[w].ctr] < pend[w].target) break;
          ctr[pend[w].comb] += pend[w].heads;
          pend[w].ctr = -1;
          progress = true;
        }
        const mk_task& t = p.dev_tasks[cursor[w]];
        int target = t.wait_target;
        if (target == MK_WAIT_SPLITS) target = nspl(t.layer, t.batch);
        if (t.wait_ctr >= 0 && target > 0 && ctr[t.wait_ctr] < target) break;
        const bool claimer = t.op == MK_OP_ATTN_DRAIN || t.op == MK_OP_MOE_UPGATE_ACT_DRAIN ||
                             t.op == MK_OP_MOE_DOWN_DRAIN;
        if (claimer) {
          SimQueue& q = (t.op == MK_OP_ATTN_DRAIN) ? qa[t.layer]
                        : (t.op == MK_OP_MOE_UPGATE_ACT_DRAIN) ? qu[t.layer] : qd[t.layer];
          // pick the next item of this claimer
          if (cur_item[w] < 0) {
            if (phase[w] == 0) {
              phase[w] = 1;
              if (t.n0 < q.n_items) cur_item[w] = t.n0;
              if (t.op == MK_OP_ATTN_DRAIN && (t.flags & MK_F_FUSE_COMBINE) && t.n0 == 0)
                for (int b = 0; b < B; ++b)   // sequences without keys: nothing to combine
                  if (nspl(t.layer, b) == 0)
                    for (int g = 0; g < Hkv; ++g) ctr[ctr_of(p.cl, t.layer, p.cl.comb + g)] += G;
            }
            if (cur_item[w] < 0) {
              const int item = t.n1 + q.head;
              if (item < q.n_items) { q.head++; cur_item[w] = item; }
            }
          }
          if (cur_item[w] >= 0) {
            const int item = cur_item[w];
            if (t.op == MK_OP_MOE_DOWN_DRAIN) {
              const int ae = item / p.dn_tiles;
              if (ctr[ctr_of(p.cl, t.layer, p.cl.ug + ae)] < p.ug_tiles) break;
            }
            if (t.op == MK_OP_ATTN_DRAIN) {
              int b, g;
              attn_bg(t.layer, item, &b, &g);
              const int actr = ctr_of(p.cl, t.layer, p.cl.attn + b * Hkv + g);
              const long rank = ctr[actr]++;
              const int ns = nspl(t.layer, b), nc = std::min(ns, p.ncomb);
              if ((t.flags & MK_F_FUSE_COMBINE) && rank >= ns - nc) {   // one of the last nc splits
                const int cb = (int)(rank - (ns - nc));
                pend[w] = PendComb{actr, ns, ctr_of(p.cl, t.layer, p.cl.comb + g), (G - cb + nc - 1) / nc};
                cur_item[w] = -1;
                progress = true;
                continue;   // the share is added once every split is in
              }
            } else if (t.op == MK_OP_MOE_UPGATE_ACT_DRAIN) {
              ctr[ctr_of(p.cl, t.layer, p.cl.ug + item / p.ug_tiles)]++;
            }
            cur_item[w] = -1;
            progress = true;
            continue;   // look for another item
          }
          phase[w] = 0;
        }
        if (t.op == MK_OP_ATTN_DECODE) {
          // a split past the live length signals nothing
          if (t.split < nspl(t.layer, t.batch)) ctr[t.signal_ctr] += 1;
        } else if (t.signal_ctr >= 0) {
          ctr[t.signal_ctr] += (t.op == MK_OP_ATTN_COMBINE ? G : 1);
        }
        if ((t.flags & MK_F_FUSE_TOPK) && ctr[t.signal_ctr] == t.aux[0])
          ctr[ctr_of(p.cl, t.layer, MK_CTR_ROUTE)]++;   // the last router tile runs top-k
        cursor[w] += 1;
        progress = true;
      }
    }
    if (all_done) return MK_OK;
    if (!progress) {
      int first = n_tasks;
      for (int w = 0; w < NW; ++w)
        if (cursor[w] < cend[w]) first = std::min(first, (int)p.dev_tasks[cursor[w]].aux[MK_AUX_INDEX]);
      if (stuck) *stuck = first;
      return MK_E_STATE;
    }
    if (iter > 100000000L) return MK_E_STATE;
  }
}

int device_cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MK_E_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MK_E_HIP;
  *out = cus;
  return MK_OK;
}

}  // namespace

// ------------------------------------------------------------------ handle
struct mk_handle {
  mk_config cfg;
  Layout lay;
  char* ws;
  size_t ws_bytes;
  int32_t max_blocks;
  int32_t num_pages;
  mk_layer_dev layers[128];   // one per layer (n_layers <= 128)
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  Plan plan;
  bool have_plan;
  int batch;
  int n_wg;
  mk_sched_opts opts;
  hipStream_t last_stream;
  int device;
  bool in_scratch;            // bound to the library's per-device scratch array
};

namespace {
constexpr int kMaxDevices = 16;
// handles of mk_init_noalloc: one per device, like the scratch array they use
mk_handle g_noalloc_handle[kMaxDevices];

int check_init_args(const mk_config* cfg, const mk_weights* w, const mk_kv_pool* kv, int32_t max_blocks) {
  int rc = validate_config(cfg);
  if (rc != MK_OK) return rc;
  if (!w || !kv || max_blocks < 1) return MK_E_INVAL;
  if (!w->embed || !w->lm_head || !w->final_norm || !w->layers || !kv->k || !kv->v || kv->num_pages < 1)
    return MK_E_INVAL;
  const bool moe = cfg->n_experts > 0;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const mk_layer_weights& lw = w->layers[l];
    if (!lw.attn_norm || !lw.w_qkv || !lw.w_o || !lw.w_upgate || !lw.w_down || !kv->k[l] || !kv->v[l])
      return MK_E_INVAL;
    if (moe && !lw.w_router) return MK_E_INVAL;
    if (!moe && !lw.ffn_norm) return MK_E_INVAL;
    if (cfg->expert_fp8 && (!lw.upgate_scale || !lw.down_scale)) return MK_E_INVAL;
  }
  return MK_OK;
}

// Fill a handle over the workspace ws (device) and clear / upload it.
int bind_handle(mk_handle* h, const mk_config* cfg, const mk_weights* w, const mk_kv_pool* kv, char* ws,
                size_t ws_bytes, int32_t max_blocks, const Layout& lay, int device) {
  h->cfg = *cfg;
  h->lay = lay;
  h->ws = ws;
  h->ws_bytes = ws_bytes;
  h->max_blocks = max_blocks;
  h->num_pages = kv->num_pages;
  h->embed = static_cast<const uint16_t*>(w->embed);
  h->lm_head = static_cast<const uint16_t*>(w->lm_head);
  h->final_norm = static_cast<const uint16_t*>(w->final_norm);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const mk_layer_weights& lw = w->layers[l];
    mk_layer_dev& ld = h->layers[l];
    ld.attn_norm = static_cast<const uint16_t*>(lw.attn_norm);
    ld.ffn_norm = static_cast<const uint16_t*>(lw.ffn_norm);
    ld.w_qkv = static_cast<const uint16_t*>(lw.w_qkv);
    ld.w_o = static_cast<const uint16_t*>(lw.w_o);
    ld.w_router = static_cast<const uint16_t*>(lw.w_router);
    ld.w_upgate = static_cast<const uint16_t*>(lw.w_upgate);
    ld.w_down = static_cast<const uint16_t*>(lw.w_down);
    ld.router_bias = static_cast<const uint16_t*>(lw.router_bias);
    ld.upgate_scale = cfg->expert_fp8 ? static_cast<const float*>(lw.upgate_scale) : nullptr;
    ld.down_scale = cfg->expert_fp8 ? static_cast<const float*>(lw.down_scale) : nullptr;
    ld.k = static_cast<uint16_t*>(kv->k[l]);
    ld.v = static_cast<uint16_t*>(kv->v[l]);
  }
  h->have_plan = false;
  h->batch = 0;
  h->last_stream = nullptr;
  h->device = device;
  // RoPE inverse frequencies (head dim <= 128: at most 64 values)
  double invf[64];
  for (int i = 0; i < cfg->head_dim / 2; ++i)
    invf[i] = std::pow((double)cfg->rope_theta, -2.0 * i / (double)cfg->head_dim);
  if (hipMemset(h->ws, 0, lay.total) != hipSuccess ||
      hipMemcpy(h->ws + lay.off_layers, h->layers, (size_t)cfg->n_layers * sizeof(mk_layer_dev),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(h->ws + lay.off_invf, invf, (size_t)(cfg->head_dim / 2) * 8, hipMemcpyHostToDevice) != hipSuccess)
    return MK_E_HIP;
  return MK_OK;
}
}  // namespace

extern "C" {

size_t mk_workspace_size(const mk_config* cfg, int32_t max_blocks_per_seq) {
  if (validate_config(cfg) != MK_OK || max_blocks_per_seq < 1) return 0;
  return make_layout(cfg, max_blocks_per_seq).total;
}

int mk_init(const mk_config* cfg, const mk_weights* w, const mk_kv_pool* kv, void* workspace,
            size_t ws_bytes, int32_t max_blocks_per_seq, mk_handle** out) {
  if (!out) return MK_E_INVAL;
  *out = nullptr;
  int rc = check_init_args(cfg, w, kv, max_blocks_per_seq);
  if (rc != MK_OK) return rc;
  if (!workspace) return MK_E_INVAL;
  Layout lay = make_layout(cfg, max_blocks_per_seq);
  if (ws_bytes < lay.total) return MK_E_NOMEM;
  if (((uintptr_t)workspace) % 256 != 0) return MK_E_INVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MK_E_HIP;
  mk_handle* h = new (std::nothrow) mk_handle();
  if (!h) return MK_E_INVAL;
  h->in_scratch = false;
  rc = bind_handle(h, cfg, w, kv, static_cast<char*>(workspace), ws_bytes, max_blocks_per_seq, lay, dev);
  if (rc != MK_OK) {
    delete h;
    return rc;
  }
  *out = h;
  return MK_OK;
}

int mk_init_noalloc(const mk_config* cfg, const mk_weights* w, const mk_kv_pool* kv, int32_t max_blocks_per_seq,
                    mk_handle** out) {
  if (!out) return MK_E_INVAL;
  *out = nullptr;
  int rc = check_init_args(cfg, w, kv, max_blocks_per_seq);
  if (rc != MK_OK) return rc;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MK_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MK_E_UNSUPPORTED;
  rc = device_cu_count(&cus);
  if (rc != MK_OK) return rc;
  void* scratch = nullptr;
  size_t cap = 0;
  rc = mk_scratch_region(&scratch, &cap);   // this device's array (looked up once per device)
  if (rc != MK_OK) return rc;
  // schedules of at most one workgroup per CU, no task trace
  Layout lay = make_layout(cfg, max_blocks_per_seq, cus, false);
  if (lay.total > cap) return MK_E_NOMEM;
  mk_handle* h = &g_noalloc_handle[dev];
  h->in_scratch = true;
  rc = bind_handle(h, cfg, w, kv, static_cast<char*>(scratch), cap, max_blocks_per_seq, lay, dev);
  if (rc != MK_OK) return rc;
  *out = h;
  return MK_OK;
}

int mk_build_schedule(mk_handle* h, int32_t batch_size, const mk_sched_opts* opt) {
  if (!h) return MK_E_INVAL;
  mk_sched_opts o{};
  if (opt) o = *opt;
  int nw = o.n_workgroups;
  if (nw <= 0) {
    int rc = device_cu_count(&nw);
    if (rc != MK_OK) return rc;
  }
  if (nw > h->lay.nw_bound) return MK_E_UNSUPPORTED;
  if ((o.flags & MK_SCHED_TRACE) && !h->lay.has_trace) return MK_E_UNSUPPORTED;
  Plan p;
  int rc = build_plan(&h->cfg, batch_size, h->max_blocks, &o, nw, &p);
  if (rc != MK_OK) return rc;
  if ((int)p.tasks.size() > h->lay.max_tasks) return MK_E_NOMEM;
  if (p.max_splits > h->lay.max_splits) return MK_E_UNSUPPORTED;
  if (hipMemcpy(h->ws + h->lay.off_tasks, p.dev_tasks.data(), p.dev_tasks.size() * sizeof(mk_task),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(h->ws + h->lay.off_ranges, p.ranges.data(), p.ranges.size() * 4, hipMemcpyHostToDevice) !=
          hipSuccess ||
      hipMemset(h->ws + h->lay.off_ctr, 0, (size_t)h->lay.n_ctr * MK_CTR_PAD * 4) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess)
    return MK_E_HIP;
  h->plan = std::move(p);
  h->have_plan = true;
  h->batch = batch_size;
  h->n_wg = nw;
  h->opts = o;
  return MK_OK;
}

namespace {
int launch_step(mk_handle* h, const int32_t* token_ids, const int32_t* positions, const int32_t* block_tables,
                const int32_t* seq_lens, float* logits, const mk_sampling* smp, int32_t* next_tokens,
                void* stream) {
  if (!h) return MK_E_INVAL;
  if (!h->have_plan) return MK_E_STATE;
  if (!token_ids || !positions || !block_tables || !seq_lens || !logits) return MK_E_INVAL;
  if (smp) {
    if (!next_tokens || !(smp->temperature >= 0.f) || !std::isfinite(smp->temperature) ||
        (smp->flags & ~MK_SAMPLE_ADVANCE) != 0)
      return MK_E_INVAL;
  }
  const mk_config& c = h->cfg;
  const Layout& L = h->lay;
  mk_kargs a;
  std::memset(&a, 0, sizeof a);
  char* ws = h->ws;
  a.tasks = reinterpret_cast<const mk_task*>(ws + L.off_tasks);
  a.n_tasks = (int32_t)h->plan.tasks.size();
  a.n_wg = h->n_wg;
  a.ctr = reinterpret_cast<int32_t*>(ws + L.off_ctr);
  a.n_ctr = L.n_ctr;
  a.err = reinterpret_cast<int32_t*>(ws + L.off_err);
  a.layers = reinterpret_cast<const mk_layer_dev*>(ws + L.off_layers);
  a.embed = h->embed;
  a.lm_head = h->lm_head;
  a.final_norm = h->final_norm;
  a.inv_freq = reinterpret_cast<const double*>(ws + L.off_invf);
  a.tokens = token_ids;
  a.positions = positions;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.logits = logits;
  if (smp) {
    a.next_tok = next_tokens;
    a.lm_best = reinterpret_cast<int32_t*>(ws + L.off_lmbest);
    a.inv_temp = smp->temperature > 0.f ? (float)(1.0 / (double)smp->temperature) : 0.f;
    a.sample_seed = smp->seed;
    a.advance = (smp->flags & MK_SAMPLE_ADVANCE) ? 1 : 0;
  }
  a.L = c.n_layers; a.d = c.d_model; a.Hq = c.n_q_heads; a.Hkv = c.n_kv_heads; a.hd = c.head_dim;
  a.G = c.n_q_heads / c.n_kv_heads; a.E = c.n_experts; a.topk = c.top_k; a.I = c.expert_inter;
  a.F = c.ffn_inter; a.V = c.vocab; a.parallel = c.parallel_block; a.page = c.page_size;
  a.swa_window = c.swa_window; a.swa_period = c.swa_period;
  a.expert_fp8 = c.expert_fp8;
  a.B = h->batch; a.max_blocks = h->max_blocks; a.num_pages = h->num_pages;
  a.eps = c.rms_eps;
  a.attn_scale = (float)(1.0 / std::sqrt((double)c.head_dim));
  a.attn_split = h->plan.attn_split;
  a.max_splits = h->plan.max_splits;
  a.ug_tiles = h->plan.ug_tiles; a.ug_pairs = h->plan.ug_pairs;
  a.dn_tiles = h->plan.dn_tiles; a.dn_rows = h->plan.dn_rows;
  a.n_qkv_tiles = h->plan.n_qkv;
  a.ncomb = h->plan.ncomb;
  a.bk = L.bk;
  a.moe_stride = L.moe_stride;
  a.cl = h->plan.cl;
  const int tmo = h->opts.timeout_ms > 0 ? h->opts.timeout_ms : 2000;
  a.timeout_ticks = (uint64_t)tmo * 100000ull;   // 100 MHz constant clock
  a.x = reinterpret_cast<float*>(ws + L.off_x);
  a.xn = reinterpret_cast<float*>(ws + L.off_xn);
  a.xmid = reinterpret_cast<float*>(ws + L.off_xmid);
  a.xn2 = reinterpret_cast<float*>(ws + L.off_xn2);
  a.qkv = reinterpret_cast<float*>(ws + L.off_qkv);
  a.attn = reinterpret_cast<float*>(ws + L.off_attn);
  a.opart = reinterpret_cast<float*>(ws + L.off_opart);
  a.rlog = reinterpret_cast<float*>(ws + L.off_rlog);
  a.topi = reinterpret_cast<int32_t*>(ws + L.off_topi);
  a.topw = reinterpret_cast<float*>(ws + L.off_topw);
  a.moe = reinterpret_cast<int32_t*>(ws + L.off_moe);
  a.H = reinterpret_cast<float*>(ws + L.off_H);
  a.Y = reinterpret_cast<float*>(ws + L.off_Y);
  a.fh = reinterpret_cast<float*>(ws + L.off_fh);
  a.fo = reinterpret_cast<float*>(ws + L.off_fo);
  a.oout = reinterpret_cast<float*>(ws + L.off_oout);
  a.part_ml = reinterpret_cast<float*>(ws + L.off_pml);
  a.part_o = reinterpret_cast<float*>(ws + L.off_po);
  a.trace = (h->opts.flags & MK_SCHED_TRACE) ? reinterpret_cast<uint64_t*>(ws + L.off_trace) : nullptr;
  h->last_stream = reinterpret_cast<hipStream_t>(stream);
  a.wg_range = reinterpret_cast<const int32_t*>(ws + L.off_ranges);
  return mk_launch(&a, h->opts.launch_mode, a.wg_range, (int)h->plan.wave_bounds.size() - 1, stream);
}
}  // namespace

int mk_decode_step(mk_handle* h, const int32_t* token_ids, const int32_t* positions,
                   const int32_t* block_tables, const int32_t* seq_lens, float* logits, void* stream) {
  return launch_step(h, token_ids, positions, block_tables, seq_lens, logits, nullptr, nullptr, stream);
}

int mk_decode_step_sample(mk_handle* h, int32_t* token_ids, int32_t* positions, const int32_t* block_tables,
                          int32_t* seq_lens, float* logits, const mk_sampling* sampling, int32_t* next_tokens,
                          void* stream) {
  if (!sampling) return MK_E_INVAL;
  return launch_step(h, token_ids, positions, block_tables, seq_lens, logits, sampling, next_tokens, stream);
}

int mk_get_status(mk_handle* h, mk_status* st) {
  if (!h) return MK_E_INVAL;
  if (hipStreamSynchronize(h->last_stream) != hipSuccess) return MK_E_HIP;
  int32_t e[MK_ERR_WORDS];
  if (hipMemcpy(e, h->ws + h->lay.off_err, sizeof e, hipMemcpyDeviceToHost) != hipSuccess) return MK_E_HIP;
  if (e[0] != 0) {
    if (hipMemset(h->ws + h->lay.off_err, 0, sizeof e) != hipSuccess) return MK_E_HIP;
    // a timed-out step may leave counters behind; clear them for the next step
    if (e[0] == MK_E_TIMEOUT &&
        hipMemset(h->ws + h->lay.off_ctr, 0, (size_t)h->lay.n_ctr * MK_CTR_PAD * 4) != hipSuccess)
      return MK_E_HIP;
    if (hipDeviceSynchronize() != hipSuccess) return MK_E_HIP;
  }
  if (st) {
    st->code = e[0];
    st->task = e[1];
    st->counter = e[2];
    st->value = e[3];
    st->target = e[4];
    st->workgroup = e[5];
  }
  return e[0];
}

int mk_tap_offset(const mk_handle* h, int32_t tap, size_t* offset, size_t* bytes) {
  if (!h || !offset || !bytes) return MK_E_INVAL;
  const Layout& L = h->lay;
  const mk_config& c = h->cfg;
  const size_t Lr = c.n_layers, B = c.max_batch, d = c.d_model;
  switch (tap) {
    case MK_TAP_X: *offset = L.off_x; *bytes = (Lr + 1) * B * d * 4; break;
    case MK_TAP_XN: *offset = L.off_xn; *bytes = (Lr + 1) * B * d * 4; break;
    case MK_TAP_QKV: *offset = L.off_qkv; *bytes = Lr * B * (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim * 4; break;
    case MK_TAP_ATTN: *offset = L.off_attn; *bytes = Lr * B * c.n_q_heads * c.head_dim * 4; break;
    case MK_TAP_ROUTER_LOGITS: *offset = L.off_rlog; *bytes = c.n_experts > 0 ? Lr * B * c.n_experts * 4 : 0; break;
    case MK_TAP_TOPK_IDS: *offset = L.off_topi; *bytes = c.n_experts > 0 ? Lr * B * c.top_k * 4 : 0; break;
    case MK_TAP_TOPK_WEIGHTS: *offset = L.off_topw; *bytes = c.n_experts > 0 ? Lr * B * c.top_k * 4 : 0; break;
    case MK_TAP_FFN_OUT: *offset = L.off_fo; *bytes = Lr * B * d * 4; break;
    case MK_TAP_ATTN_OUT: *offset = L.off_oout; *bytes = Lr * B * d * 4; break;
    case MK_TAP_TRACE:
      *offset = L.off_trace;
      *bytes = L.has_trace ? (size_t)(h->have_plan ? h->plan.tasks.size() : 0) * 128 : 0;
      break;
    default: return MK_E_INVAL;
  }
  return MK_OK;
}

int mk_plan_schedule(const mk_config* cfg, int32_t batch_size, int32_t max_blocks_per_seq,
                     const mk_sched_opts* opt, int32_t n_workgroups, mk_task* out, int32_t cap,
                     int32_t* n_tasks, int32_t* n_counters) {
  int rc = validate_config(cfg);
  if (rc != MK_OK) return rc;
  Plan p;
  rc = build_plan(cfg, batch_size, max_blocks_per_seq, opt, n_workgroups, &p);
  if (rc != MK_OK) return rc;
  if (n_tasks) *n_tasks = (int32_t)p.tasks.size();
  if (n_counters) *n_counters = p.n_ctr;
  if (out) {
    if (cap < (int32_t)p.tasks.size()) return MK_E_NOMEM;
    std::memcpy(out, p.tasks.data(), p.tasks.size() * sizeof(mk_task));
  }
  return MK_OK;
}

int mk_plan_simulate(const mk_config* cfg, int32_t batch_size, int32_t max_blocks_per_seq,
                     const mk_sched_opts* opt, int32_t n_workgroups, const int32_t* seq_lens,
                     const int32_t* n_active_experts, int32_t* stuck_task) {
  int rc = validate_config(cfg);
  if (rc != MK_OK) return rc;
  if (!seq_lens || (cfg->n_experts > 0 && !n_active_experts)) return MK_E_INVAL;
  Plan p;
  rc = build_plan(cfg, batch_size, max_blocks_per_seq, opt, n_workgroups, &p);
  if (rc != MK_OK) return rc;
  return simulate(cfg, batch_size, p, n_workgroups, seq_lens, n_active_experts, stuck_task);
}

void mk_destroy(mk_handle* h) {
  if (!h) return;
  if (h->in_scratch) {   // a per-device handle of mk_init_noalloc: only forget the schedule
    h->have_plan = false;
    return;
  }
  delete h;
}

const char* mk_strerror(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_E_INVAL: return "invalid argument";
    case MK_E_UNSUPPORTED: return "unsupported shape";
    case MK_E_NOMEM: return "workspace too small";
    case MK_E_HIP: return "HIP runtime error";
    case MK_E_TIMEOUT: return "device watchdog: counter wait timed out";
    case MK_E_DEVICE: return "device-detected bad input";
    case MK_E_STATE: return "bad call order or blocked schedule";
    default: return "unknown error";
  }
}

}  // extern "C"
