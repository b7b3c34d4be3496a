// mk_kernel.hip - the persistent decode megakernel for gfx950 (MI355X).
//
// One launch runs one decode step.  The grid holds one workgroup per CU
// (256 threads = 4 wave64s, one per SIMD, 153,800 bytes of LDS so no second
// workgroup fits).  One wave per SIMD gives each wave the SIMD's whole
// register file (256 VGPRs + 256 AGPRs), so the compiler spills into AGPRs
// instead of scratch memory: a scratch reload is a vector-memory load, and
// it would wait behind every weight load the wave has in flight.
// workgroup w walks tasks w, w+N, w+2N, ... of the host-built list (task k on
// workgroup k mod N).  A task waits on one counter in global memory, runs one
// tile, and bumps one counter (persistent decode megakernel pages: page 1
// "One kernel for the full decode step", "The calling convention that makes
// it hand-writable", "Scheduling: mostly static, selectively dynamic"; page 2
// "Overview"; page 3 on counters that tasks bump and spin on).
//
// Memory ordering across the 8 XCDs (each with its own L2): every value that
// one workgroup writes and another reads during the step (activations,
// partials, routing tables, the new K/V slot) is stored and loaded with
// agent-coherent accesses (the sc1 cache policy, i.e. relaxed agent-scope
// atomics), so no L2 write-back or invalidate is ever needed.  A producer's
// waves wait for their stores to complete (s_waitcnt vmcnt(0)), meet at a
// workgroup barrier, and one lane bumps the counter with an agent-scope
// atomic; a consumer lane spins on agent-scope loads of the counter with
// s_sleep between polls, then a workgroup barrier releases its other waves.
// (Agent-scope release/acquire fences would write back / invalidate the
// whole L2 of the XCD on every task, which measured 2-30 us per task here.)
//
// Weights are immutable during a step, so every GEMV tile issues the loads of
// its first row groups into registers *before* it waits on its activation
// dependency (page 1, third gain of the megakernel: weights stream while the
// task's input is not ready yet): two groups (96 KB per CU) in the one- and
// two-row form, three (144 KB) in the MFMA form.  They are issued when the
// workgroup reaches the task, not earlier.  Attention splits and MoE expert
// tiles are pulled from claim queues whose head is an atomic counter (page 1,
// "Scheduling").

#include <hip/hip_runtime.h>
#include <mutex>
#include <type_traits>
#include <stdint.h>

#include "mk_internal.h"

#define MK_THREADS 256
#define MK_WAVES 4
#define XS_FLOATS 16384   // staged activations, 64 KB
#define YS_FLOATS 8192    // tile outputs / attention scores, 32 KB
#define RED_FLOATS 8192   // attention cross-wave reduction, 32 KB
#define NBMAX 8
#ifndef MK_WB
#define MK_WB 16          // 16-byte weight loads per lane per GEMV row group
#endif
#ifndef MK_NT
#define MK_NT 2           // GEMV row groups (register tiles) in flight per compute wave
#endif
#ifndef MK_STAGE_N
#define MK_STAGE_N 8      // 16-byte activation loads per lane in flight while staging
#endif
#ifndef MK_NTM
#define MK_NTM 3          // MFMA GEMV groups in flight per compute wave (bs=8: 854 tok/s against 846 for 2)
#endif
#define MK_CW 3           // compute waves: wave 0 is the control wave (spins, stages)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The argument block stays in the kernarg segment and is read with scalar
// loads through a pointer laundered once per work unit (KA::operator->).
// Reading it directly would let loop-invariant code motion hoist dozens of
// argument-derived values to the kernel entry, where they no longer fit in
// registers and are spilled; reading it from LDS or through a generic
// pointer would turn every field access into a vector-memory load that
// waits behind the wave's in-flight weight loads.
typedef __attribute__((address_space(4))) const mk_kargs kargs_c;
struct KA {
  kargs_c* p;
  __device__ __forceinline__ kargs_c* operator->() const { return p; }
};
__device__ __forceinline__ KA kargs() {
  kargs_c* p = (kargs_c*)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  return KA{p};
}

struct __attribute__((aligned(16))) Smem {
  float xs[XS_FLOATS];
  float ys[YS_FLOATS];
  float red[RED_FLOATS];
  int misc[192];
  uint32_t sortk[128];
  mk_task tq[2];      // this task's descriptor and the next one (prefetched)
  uint64_t t_ready;   // trace: when the task's first wait was satisfied
  uint64_t t_mark[10]; // trace: [0] staged, [1] computed, [2] stores acknowledged, [3..9] free marks
  int seen_idx;       // the counter of the last wg_wait this workgroup saw satisfied, and its target
  int seen_val;
};

// ------------------------------------------------------------------ helpers
// The thread index, opaque to the optimiser at each use: otherwise every
// value derived from it (LDS and global offsets of every op) is hoisted to
// the kernel entry and kept live for the whole step, where they no longer
// fit in registers and are spilled to scratch memory.
__device__ __forceinline__ int tid_v() {
  int t = __builtin_amdgcn_workitem_id_x();
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}
// Pointers read from the argument block are generic; a load through a
// generic pointer is a flat load, which the hardware counts as both a vector
// memory and an LDS access, so any later LDS read would have to wait for every
// weight load still in flight.  Global accesses are cast to address space 1.
#define GLOBAL __attribute__((address_space(1)))
typedef GLOBAL const u32x4 gc_u32x4;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef GLOBAL const u32x2 gc_u32x2;
// 4 bf16 (8 bytes) from global memory
__device__ __forceinline__ u32x2 ldg8(const uint16_t* p) { return *(gc_u32x2*)p; }
__device__ __forceinline__ u32x4 ldg_nt(const uint16_t* p) {
  return __builtin_nontemporal_load((gc_u32x4*)p);
}
// Cross-lane reductions.  HIP's __shfl_xor is a ds_bpermute through the LDS
// crossbar: with one wave per SIMD every dependent step would stall the wave
// for a whole LDS round trip.  Within a row of 16 lanes these use DPP
// (quad permutes, half-row and row mirrors: for a sum or max each step pairs
// every lane with one of the other half, like a butterfly); across rows the
// gfx950 permlane swaps (rows 2r <-> 2r+1, then halves) or v_readlane.
// All of them must be called with every lane of the wave active.
enum { DPP_QP_X1 = 0xB1, DPP_QP_X2 = 0x4E, DPP_ROW_ROR8 = 0x128, DPP_ROW_MIRROR = 0x140, DPP_HALF_MIRROR = 0x141 };
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
// sum / max over aligned groups of N lanes (N in 2, 4, 8, 16), in every lane
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v += dppf<DPP_QP_X1>(v);
  if (N >= 4) v += dppf<DPP_QP_X2>(v);
  if (N >= 8) v += dppf<DPP_HALF_MIRROR>(v);
  if (N >= 16) v += dppf<DPP_ROW_MIRROR>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if (N >= 2) v = fmaxf(v, dppf<DPP_QP_X1>(v));
  if (N >= 4) v = fmaxf(v, dppf<DPP_QP_X2>(v));
  if (N >= 8) v = fmaxf(v, dppf<DPP_HALF_MIRROR>(v));
  if (N >= 16) v = fmaxf(v, dppf<DPP_ROW_MIRROR>(v));
  return v;
}
template <int N>
__device__ __forceinline__ int group_min(int v) {
  if (N >= 2) v = min(v, dppi<DPP_QP_X1>(v));
  if (N >= 4) v = min(v, dppi<DPP_QP_X2>(v));
  if (N >= 8) v = min(v, dppi<DPP_HALF_MIRROR>(v));
  if (N >= 16) v = min(v, dppi<DPP_ROW_MIRROR>(v));
  return v;
}
// sum of the lanes l, l^16, l^32, l^48 (the same position in the 4 rows)
__device__ __forceinline__ float cross_row_sum(float v) {
  const unsigned u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const unsigned w = __float_as_uint(v);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// whole-wave sum / max / min, returned uniform
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ int wave_min(int v) {
  v = group_min<16>(v);
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), two values per word
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint16_t h0 = f_to_bf16(x0), h1 = f_to_bf16(x1);
  const uint16_t l0 = f_to_bf16(x0 - bf16_to_f(h0)), l1 = f_to_bf16(x1 - bf16_to_f(h1));
  hi = (uint32_t)h0 | ((uint32_t)h1 << 16);
  lo = (uint32_t)l0 | ((uint32_t)l1 << 16);
}

// A value known to be the same in every lane, moved to scalar registers.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ long uniform_long(long x) {
  const uint64_t v = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (long)(((uint64_t)hi << 32) | lo);
}

// Step metadata, copied into LDS at kernel start: every task reads some of it
// before it can issue its first load (weight pointers, lengths, positions),
// and an LDS read avoids a memory round trip on that path.
#define MK_LDS_LAYERS 128
__shared__ mk_layer_dev sh_layers[MK_LDS_LAYERS];
__shared__ int sh_seq_lens[NBMAX], sh_positions[NBMAX], sh_tokens[NBMAX];
// block tables too when they are small (batch x max_blocks <= MK_LDS_BT)
#define MK_LDS_BT 2048
__shared__ int sh_bt[MK_LDS_BT];
__shared__ double sh_invf[64];   // RoPE inverse frequencies (head dim <= 128)
#define LAYER_PTR(l, f) uniform_ptr(sh_layers[l].f)
__device__ __forceinline__ int seq_len_u(int b) { return __builtin_amdgcn_readfirstlane(sh_seq_lens[b]); }
__device__ __forceinline__ int position_u(int b) { return __builtin_amdgcn_readfirstlane(sh_positions[b]); }
__device__ __forceinline__ int token_u(int b) { return __builtin_amdgcn_readfirstlane(sh_tokens[b]); }

// Each counter owns a 256-byte line (MK_CTR_PAD ints), so that workgroups
// polling different counters do not share a line.
__device__ __forceinline__ int32_t* ctrp(const KA a, int idx) { return a->ctr + (long)idx * MK_CTR_PAD; }

__device__ __forceinline__ int ld_agent(const int32_t* p) {
  return __hip_atomic_load((GLOBAL const int32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Agent-coherent loads and stores of data shared between workgroups.
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load((GLOBAL const float*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ldc(const int32_t* p) {
  return __hip_atomic_load((GLOBAL const int32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store((GLOBAL float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(int32_t* p, int v) {
  __hip_atomic_store((GLOBAL int32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(uint16_t* p, uint16_t v) {
  __hip_atomic_store((GLOBAL uint16_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte agent-coherent load at base + byte_off; base must be the same in
// every lane (the lane's part goes in byte_off).  The base is moved to scalar
// registers here: a descriptor the compiler cannot prove uniform is applied
// one lane group at a time in a loop, and a load in such a loop waits for
// the previous one.
__device__ __forceinline__ u32x4 ldc16(const void* base, int byte_off) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(base)), (short)0,
                                                               0x7FFFFFFF, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ void stc16(void* base, int byte_off, u32x4 v) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), (short)0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ f32x4 as_f4(u32x4 v) {
  return (f32x4){__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
}
__device__ __forceinline__ u32x4 as_u4(f32x4 v) {
  return (u32x4){__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
}
// Wait until this wave's stores have completed.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __noinline__ void report(const KA a, int code, int task, int ctr, int val, int target) {
  if (atomicCAS(&a->err[0], 0, code) == 0) {
    a->err[1] = task;
    a->err[2] = ctr;
    a->err[3] = val;
    a->err[4] = target;
    a->err[5] = (int)blockIdx.x;
  }
}

// One lane spins until ctr[idx] >= target.  false if the watchdog fired or
// another workgroup aborted the step.
__device__ __forceinline__ bool spin_until(const KA a, int idx, int target, int task) {
  const int32_t* p = ctrp(a, idx);
  if (ld_agent(p) < target) {
    const uint64_t t0 = wall_clock64();
    int backoff = 1;
    for (;;) {
      // back off to at most ~0.4 us between polls: a poll is a memory
      // transaction on a line that up to every CU is reading
      for (int k = 0; k < backoff; ++k) __builtin_amdgcn_s_sleep(3);
      if (backoff < 8) backoff <<= 1;
      // the clock read and both loads are in flight together: a poll costs
      // one round trip
      const uint64_t now = wall_clock64();
      const int v = ld_agent(p), ab = ld_agent(ctrp(a, MK_CG_ABORT));
      if (v >= target) break;
      if (ab) return false;
      if (now - t0 > a->timeout_ticks) {
        report(a, MK_E_TIMEOUT, task, idx, ld_agent(p), target);
        __hip_atomic_store(ctrp(a, MK_CG_ABORT), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
  }
  return true;
}

// Workgroup-wide wait; every thread must call it.  Uses misc[0].  Counters
// only grow during a launch, so a wait on the counter this workgroup last saw
// satisfied, for no more than it saw, costs no poll (the down drain and the
// next norm wait on the routing counter the up-gate drain already saw).
__device__ __forceinline__ bool wg_wait(const KA a, Smem& sm, int idx, int target, int task) {
  if (tid_v() == 0) {
    int ok = 1;
    if (idx >= 0 && target > 0 && !(sm.seen_idx == idx && sm.seen_val >= target)) {
      ok = (int)spin_until(a, idx, target, task);
      if (ok) {
        sm.seen_idx = idx;
        sm.seen_val = target;
      }
    }
    sm.misc[0] = ok;
    if (a->trace && sm.t_ready == 0) sm.t_ready = wall_clock64();
  }
  __syncthreads();
  const bool ok = sm.misc[0] != 0;
  return ok;
}

__shared__ uint64_t sm_t_signal;   // trace: when wg_signal last bumped a counter
// trace: first time this task passes mark k (thread 0)
#define MK_MARK(k)                                                              \
  do {                                                                          \
    if (a->trace && tid_v() == 0 && sm.t_mark[k] == 0) sm.t_mark[k] = wall_clock64(); \
  } while (0)

// Workgroup-wide signal: every wave waits for its (agent-coherent) stores to
// complete, then one lane bumps the counter.
__device__ __forceinline__ void wg_signal(const KA a, int idx, int inc) {
  stores_done();
  __syncthreads();
  if (a->trace && tid_v() == 0) sm_t_signal = wall_clock64();
  if (tid_v() == 0 && idx >= 0)
    __hip_atomic_fetch_add(ctrp(a, idx), inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Claim the next item of a queue; every thread must call it.  Uses misc[1].
__device__ __forceinline__ int wg_claim(const KA a, Smem& sm, int qidx) {
  __syncthreads();
  if (tid_v() == 0) {
    // the abort flag and the claim travel together (one round trip); a claim
    // taken during an abort is discarded, and the step's counters are
    // cleared before the next one
    const int ab = ld_agent(ctrp(a, MK_CG_ABORT));
    const int c = __hip_atomic_fetch_add(ctrp(a, qidx), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.misc[1] = ab ? 0x3FFFFFFF : c;
  }
  __syncthreads();
  return sm.misc[1];
}

// Claimer item order: claimer c of a wave owns item c of the queue; items
// past the number of claimers are pulled one at a time from the atomic queue
// head.  Returns -1 when the queue is exhausted.  Every thread must call it.
// pre: a queue position claimed ahead (when the claimer started), or -1.
__device__ __forceinline__ int next_item(const KA a, Smem& sm, const mk_task& t, int n_items, int qidx, bool& first,
                                         int& pre) {
  if (first) {
    first = false;
    if (t.n0 < n_items) return t.n0;
  }
  if (n_items <= t.n1) return -1;
  int c;
  if (pre >= 0) {
    c = pre;
    pre = -1;
  } else {
    c = wg_claim(a, sm, qidx);
  }
  const int it = t.n1 + c;
  return it < n_items ? it : -1;
}

__device__ __forceinline__ int layer_ctr(const KA a, int layer, int off) {
  return MK_CG_COUNT + layer * a->cl.stride + off;
}

__device__ __forceinline__ int visible_keys(const KA a, int layer, int seq_len) {
  if (a->swa_window > 0 && a->swa_period > 0 && (layer % a->swa_period) != a->swa_period - 1)
    return seq_len < a->swa_window ? seq_len : a->swa_window;
  return seq_len;
}
// Live length of slot b, clamped to what its block table can hold (a longer
// length is reported by the layer-0 norm task).
__device__ __forceinline__ int live_len(const KA a, int b) {
  const int sl = seq_len_u(b);
  const int cap = a->max_blocks * a->page;
  return sl < cap ? sl : cap;
}
__device__ __forceinline__ int n_splits(const KA a, int layer, int b) {
  const int sl = live_len(a, b);
  if (sl <= 0) return 0;
  return (visible_keys(a, layer, sl) + a->attn_split - 1) / a->attn_split;
}

// --------------------------------------------------------- the GEMV pipeline
// y[b][r] = sum_k W[row(r)][k] * x[b][k] for the rows of one tile.  Every
// GEMV opcode runs through this one routine; they differ in the row mapping,
// where x comes from, and the epilogue (page 1: all GEMM opcodes share one
// pipeline).  Lane l reads 16-byte segments l, l+64, ... of each weight row,
// so one wave load moves 1 KB of contiguous weights.  Two register tiles
// (row groups) are in flight: the next one loads while the current one is
// multiplied and reduced.
enum { ROW_PLAIN = 0, ROW_ROPE_PAIRS = 1, ROW_GATE_UP = 2 };

struct GemvArgs {
  const uint16_t* base;
  long ldw;        // elements between rows
  int r0;          // first row (or pair) of the tile
  int nrows;       // tile rows (2 per pair for the paired modes)
  int K;           // reduction length (multiple of 8)
  int mode;        // ROW_*
  int half;        // ROW_ROPE_PAIRS: hd/2 (a power of two); ROW_GATE_UP: I (offset of the up rows)
  int hd;
  int xstride;     // elements between staged x rows in LDS (set by gemv_run)
  int nb;          // live batch rows
  int pm, hs;      // row mapping (set by make_uniform): pairs?, log2 of the pair block
  // output
  float* out;      // mode 0: out[b*ob + r]; null: LDS ys[r*NBMAX + b]
  long ob;
};

// Weight row of tile row r, one formula for the three modes: tile rows come
// singly (plain) or in pairs (paired modes, pm = 1); pair p = r0 + r/2 maps to
// rows p + (p / (hd/2) + upper) * half, which for RoPE pairs (half = hd/2) is
// head * hd + i (+ hd/2 for the upper row), and for gate/up pairs (the shift
// hs = 31 makes p / 2^hs zero) is p (+ I).
// Every field is the same in all lanes; say so, so that the row arithmetic
// runs on the scalar unit and buffer descriptors stay in scalar registers.
__device__ __forceinline__ void make_uniform(GemvArgs& g) {
  g.base = uniform_ptr(g.base);
  g.ldw = uniform_long(g.ldw);
  g.r0 = __builtin_amdgcn_readfirstlane(g.r0);
  g.nrows = __builtin_amdgcn_readfirstlane(g.nrows);
  g.K = __builtin_amdgcn_readfirstlane(g.K);
  g.mode = __builtin_amdgcn_readfirstlane(g.mode);
  g.half = __builtin_amdgcn_readfirstlane(g.half);
  g.hd = __builtin_amdgcn_readfirstlane(g.hd);
  g.xstride = __builtin_amdgcn_readfirstlane(g.xstride);
  g.nb = __builtin_amdgcn_readfirstlane(g.nb);
  g.out = uniform_ptr(g.out);
  g.ob = uniform_long(g.ob);
  g.pm = g.mode != ROW_PLAIN ? 1 : 0;
  g.hs = g.mode == ROW_ROPE_PAIRS ? 31 - __builtin_clz(g.half) : 31;
}

// The weight row of tile row r, and its element offset: a 32 x 32 -> 64-bit
// scalar multiply (row index and row pitch both fit in 32 bits).
__device__ __forceinline__ uint32_t gemv_row_index(const GemvArgs& g, int r) {
  const int p = g.r0 + (r >> g.pm), upper = r & g.pm;
  return (uint32_t)(p + ((p >> g.hs) + upper) * g.half);
}
__device__ __forceinline__ const uint16_t* gemv_row(const GemvArgs& g, int r) {
  return g.base + (uint64_t)gemv_row_index(g, r) * (uint32_t)g.ldw;
}

// Register tile of one row group: WB 16-byte weight loads per lane of each
// compute wave (MK_WB, halved for 4 or more batch rows, whose accumulators
// take the registers).  Slot u holds K-chunk (u mod kch) of tile row
// (u / kch), where a K-chunk is 512 elements (64 lanes x 8) and kch = 2^kl
// covers K; so a wave owns WB / kch consecutive rows per group.  kch is a
// runtime value, so one instance per batch width serves every GEMV shape:
// the step's hot code stays small enough for the instruction cache.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// a.bf16[0] * b.bf16[0] + a.bf16[1] * b.bf16[1] + c (fp32 accumulate)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// D = A B + C on the matrix cores: A 16 x 32 bf16 (lane l: row l mod 16, K
// elements 8 (l / 16) .. + 7), B 32 x 16 bf16 (lane l: column l mod 16, the
// same K elements), D 16 x 16 fp32 (lane l: rows 4 (l / 16) .. + 3, column
// l mod 16).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

template <int NB>
struct GemvTile {
  static constexpr int WB = NB >= 4 ? MK_WB / 2 : MK_WB;
  u32x4 w[WB];

  // first tile row of compute wave cw (1..MK_CW) in row group grp
  __device__ __forceinline__ static int row0(int grp, int cw, int kl) {
    return (grp * MK_CW + cw - 1) * (WB >> kl);
  }

  // One buffer descriptor per weight row (wave-uniform, scalar registers)
  // whose size is the row's K elements, or 0 for a row past the tile: the
  // hardware returns zeros for those loads, so nothing is masked.  voff is
  // the lane's byte offset (16 lane) in a K-chunk.
  __device__ __forceinline__ void load(const GemvArgs& g, int grp, int kl, int voff) {
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6);
    const int r0 = row0(grp, wave, kl), cm = (1 << kl) - 1;
#pragma unroll
    for (int u = 0; u < WB; ++u) {
      const int r = r0 + (u >> kl), c = u & cm;
      __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(gemv_row(g, r < g.nrows ? r : 0)), (short)0, r < g.nrows ? g.K * 2 : 0, 0x00020000);
      w[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + c * 1024, 0, 2 /* nontemporal */);
    }
  }

  // load() with the K-chunk count 2^KL known: the chunks of one row share
  // one buffer descriptor, so a row group costs one row-address computation
  // per row instead of one per 16-byte load.
  template <int KL>
  __device__ __forceinline__ void load_k(const GemvArgs& g, int grp, int voff) {
    constexpr int RPW = WB >> KL;
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6);
    const int r0 = row0(grp, wave, KL);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = r0 + j;
      __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(gemv_row(g, r < g.nrows ? r : 0)), (short)0, r < g.nrows ? g.K * 2 : 0, 0x00020000);
#pragma unroll
      for (int c = 0; c < (1 << KL); ++c)
        w[(j << KL) + c] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + c * 1024, 0, 2 /* nontemporal */);
    }
  }

  // x comes from LDS as two bf16 arrays (high part, remainder) of the staged
  // fp32 rows, each row padded with zeros to whole K-chunks; xh and xl point
  // at the lane's first element.  Each 16-byte weight slot costs 8 bf16 dot
  // products.
  __device__ __forceinline__ void compute(const GemvArgs& g, int grp, int kl, const uint16_t* xh, const uint16_t* xl,
                                          float* ys) {
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    const int r0 = row0(grp, wave, kl), cm = (1 << kl) - 1;
    if (r0 >= g.nrows) return;   // wave-uniform: no rows in this group
    float acc[WB][NB];
#pragma unroll
    for (int u = 0; u < WB; ++u) {
      const int e0 = 512 * (u & cm);
      const u32x4 v = w[u];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4 h = *reinterpret_cast<const u32x4*>(xh + b * g.xstride + e0);
        const u32x4 q = *reinterpret_cast<const u32x4*>(xl + b * g.xstride + e0);
        float s = dot2_bf16(v.x, h.x, 0.f);
        s = dot2_bf16(v.y, h.y, s);
        s = dot2_bf16(v.z, h.z, s);
        s = dot2_bf16(v.w, h.w, s);
        s = dot2_bf16(v.x, q.x, s);
        s = dot2_bf16(v.y, q.y, s);
        s = dot2_bf16(v.z, q.z, s);
        s = dot2_bf16(v.w, q.w, s);
        acc[u][b] = s;
      }
    }
    // add the K-chunks of each row: slots 2i and 2i+1 belong to one row
    // until kch chunks have been folded
#pragma unroll
    for (int step = 1; step < WB; step <<= 1) {
      if ((1 << kl) > step) {
#pragma unroll
        for (int i = 0; i < WB / (2 * step); ++i)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[i][b] = acc[2 * i][b] + acc[2 * i + 1][b];
      }
    }
    const int rpw = WB >> kl;
#pragma unroll
    for (int j = 0; j < WB; ++j) {
      if (j < rpw) {
        const int r = r0 + j;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float s = wave_sum(acc[j][b]);
          if (lane == 0 && r < g.nrows && b < g.nb) {
            if (g.out) stc(g.out + (long)b * g.ob + r, s);
            else ys[r * NBMAX + b] = s;
          }
        }
      }
    }
  }

  // One batch row with K <= 512 << KL: the lane's pieces of the 1 << KL
  // K-chunks of x are in registers (xrh / xrl, loaded once per task), so the
  // products wait on no LDS read.
  template <int KL>
  __device__ __forceinline__ void compute_r(const GemvArgs& g, int grp, const u32x4* xrh, const u32x4* xrl,
                                            float* ys) {
    static_assert(NB == 1, "register-resident x holds one batch row");
    constexpr int CM = (1 << KL) - 1, RPW = WB >> KL;
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    const int r0 = row0(grp, wave, KL);
    if (r0 >= g.nrows) return;   // wave-uniform: no rows in this group
    float acc[WB];
#pragma unroll
    for (int u = 0; u < WB; ++u) {
      const u32x4 v = w[u], h = xrh[u & CM], q = xrl[u & CM];
      float s = dot2_bf16(v.x, h.x, 0.f);
      s = dot2_bf16(v.y, h.y, s);
      s = dot2_bf16(v.z, h.z, s);
      s = dot2_bf16(v.w, h.w, s);
      s = dot2_bf16(v.x, q.x, s);
      s = dot2_bf16(v.y, q.y, s);
      s = dot2_bf16(v.z, q.z, s);
      s = dot2_bf16(v.w, q.w, s);
      acc[u] = s;
    }
    // add the K-chunks of each row pairwise, as compute() does
#pragma unroll
    for (int step = 1; step < (1 << KL); step <<= 1) {
#pragma unroll
      for (int i = 0; i < WB / (2 * step); ++i) acc[i] = acc[2 * i] + acc[2 * i + 1];
    }
    if constexpr (RPW == 4 || RPW == 8) {
      // transpose-reduce: halves, then quarter rows of the wave swap so that
      // each 16-lane row (RPW = 4) or 8-lane half row (RPW = 8) ends up
      // holding one tile row, then a sum within it
      float b[RPW / 2];
#pragma unroll
      for (int j = 0; j < RPW / 2; ++j) {   // rows j (lanes 0-31) and j + RPW/2 (lanes 32-63)
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[j]), __float_as_uint(acc[j + RPW / 2]),
                                                        false, false);
        b[j] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
      }
      float c[RPW / 4];
#pragma unroll
      for (int j = 0; j < RPW / 4; ++j) {   // 16-lane rows: j, j + RPW/4, j + RPW/2, j + 3 RPW/4
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(b[j]), __float_as_uint(b[j + RPW / 4]),
                                                        false, false);
        c[j] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
      }
      float v;
      int r;
      if constexpr (RPW == 4) {
        v = group_sum<16>(c[0]);
        r = r0 + (lane >> 4);
      } else {
        // lanes 0-7 of each 16-lane row keep c[0]'s row, lanes 8-15 c[1]'s
        const bool hi8 = (lane & 8) != 0;
        const float keep = hi8 ? c[1] : c[0], give = hi8 ? c[0] : c[1];
        v = group_sum<8>(keep + dppf<DPP_ROW_ROR8>(give));
        r = r0 + 2 * (lane >> 4) + (hi8 ? 1 : 0);
      }
      if ((lane & (16 / (RPW / 4) - 1)) == 0 && r < g.nrows && g.nb > 0) {
        if (g.out) stc(g.out + r, v);
        else ys[r * NBMAX] = v;
      }
    } else {
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        const int r = r0 + j;
        const float sv = wave_sum(acc[j]);
        if (lane == 0 && r < g.nrows && g.nb > 0) {
          if (g.out) stc(g.out + r, sv);
          else ys[r * NBMAX] = sv;
        }
      }
    }
  }
};

// Staging of the activation rows a tile multiplies: nb rows of K floats.
struct StageArgs {
  const float* base;
  long ld;
  bool use_tok;         // row of x for batch row j: tok[j] (else j)
  int tok[NBMAX];
  int nb;
  int K;
  int wait_idx;         // counter waited on before staging (-1: none)
  int wait_target;
  int task;
};

// Rows go to LDS with stride kp (K padded to the GEMV's whole K-chunks),
// zeros in the padding, as two bf16 arrays [nb][kp] (x = hi + lo) at the
// start of xs.  Thread th of nth takes 16-byte pieces th, th + nth, ...,
// MK_STAGE_N at a time.
__device__ __forceinline__ void stage_rows(Smem& sm, const StageArgs& s, int kp, int th, int nth) {
  const int kv = s.K >> 2, total = s.nb * kv;
  uint16_t* xh = reinterpret_cast<uint16_t*>(sm.xs);
  uint16_t* xl = xh + s.nb * kp;
  for (int i0 = 0; i0 < total; i0 += nth * MK_STAGE_N) {
    // every offset first, then every load back to back, then the
    // conversion: address arithmetic between the loads made the compiler
    // reuse a register of an outstanding load and wait for all of them,
    // which left one or two loads in flight (a 64 KB staging took 17 us)
    int off[MK_STAGE_N], dst[MK_STAGE_N];
#pragma unroll
    for (int u = 0; u < MK_STAGE_N; ++u) {
      const int i = i0 + u * nth + th;
      const int j = i / kv, c = i - j * kv;
      int row = j;
      if (s.use_tok) {
#pragma unroll
        for (int q = 0; q < NBMAX; ++q)
          if (q == j) row = s.tok[q];
      }
      const bool in = i < total;
      off[u] = in ? (int)(((long)row * s.ld + c * 4) * 4) : 0;   // a piece past the end reads piece 0
      dst[u] = in ? j * kp + c * 4 : -1;
    }
    u32x4 v[MK_STAGE_N];
#pragma unroll
    for (int u = 0; u < MK_STAGE_N; ++u) v[u] = ldc16(s.base, off[u]);
#pragma unroll
    for (int u = 0; u < MK_STAGE_N; ++u)
      if (dst[u] >= 0) {
        uint32_t h0, h1, l0, l1;
        split_bf16(__uint_as_float(v[u].x), __uint_as_float(v[u].y), h0, l0);
        split_bf16(__uint_as_float(v[u].z), __uint_as_float(v[u].w), h1, l1);
        *reinterpret_cast<uint2*>(xh + dst[u]) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(xl + dst[u]) = make_uint2(l0, l1);
      }
  }
  if (kp > s.K) {
    const int pw = (kp - s.K) >> 2;   // 4-element pieces of padding per row
    for (int i = th; i < s.nb * pw; i += nth) {
      const int j = i / pw, e = s.K + (i - j * pw) * 4;
      *reinterpret_cast<uint2*>(xh + j * kp + e) = make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(xl + j * kp + e) = make_uint2(0u, 0u);
    }
  }
}

// Wave 0 waits (lane 0 spins), then the activation rows are staged into LDS
// (stage_rows).  Rows that fit one round of wave 0's loads are staged by
// wave 0 alone: its own weight loads have landed by the time its spin sees
// the counter, so its staging loads queue behind nothing, and the compute
// waves only meet it at the barrier.  Larger stagings (several batch rows)
// are shared by all four waves after a second barrier: a compute wave's
// staging loads wait behind its weight loads, which it needs next anyway,
// and eight rows of 2048 take two rounds instead of eight.  Every thread
// must call it.
__device__ __forceinline__ bool wait_and_stage(const KA a, Smem& sm, const StageArgs& s, int kp) {
  const bool wide = s.nb * (s.K >> 2) > 64 * MK_STAGE_N;   // uniform
  const int tid = tid_v();
  if (tid < 64) {
    int ok = 1;
    if (tid == 0) {
      ok = (s.wait_idx < 0 || s.wait_target <= 0) ? 1 : (int)spin_until(a, s.wait_idx, s.wait_target, s.task);
      if (a->trace && sm.t_ready == 0) sm.t_ready = wall_clock64();
    }
    ok = __builtin_amdgcn_readfirstlane(ok);
    if (tid == 0) sm.misc[0] = ok;
    if (ok && !wide) stage_rows(sm, s, kp, tid, 64);
  }
  if (wide) {
    __syncthreads();
    if (sm.misc[0]) stage_rows(sm, s, kp, tid, MK_THREADS);
  }
  __syncthreads();
  if (a->trace && tid == 0 && sm.t_mark[0] == 0) sm.t_mark[0] = wall_clock64();
  return sm.misc[0] != 0;
}

template <int NB>
__device__ __forceinline__ bool gemv_run(const KA a, Smem& sm, const GemvArgs& g_in, const StageArgs& s) {
  GemvTile<NB> T[MK_NT];
  GemvArgs g = g_in;
  make_uniform(g);
  const int kch = (g.K + 511) >> 9;
  const int kl = kch <= 1 ? 0 : 32 - __builtin_clz(kch - 1);   // ceil(log2(kch)); K <= 512 * WB
  const int per = MK_CW * (GemvTile<NB>::WB >> kl);
  const int ng = (g.nrows + per - 1) / per;
  const bool cw = (tid_v() >> 6) != 0;
  // the first MK_NT row groups are in flight before the dependency resolves;
  // the control wave loads no weights, so its staging loads queue behind nothing
  const int voff = (tid_v() & 63) * 16;
  const bool xreg = NB == 1 && kl <= 2;   // x in registers, chunk count known (below)
  if (cw) {
    if (xreg) {
      auto pre = [&](auto klc) {
        constexpr int KL = decltype(klc)::value;
#pragma unroll
        for (int u = 0; u < MK_NT; ++u)
          if (u < ng) T[u].template load_k<KL>(g, u, voff);
      };
      if (kl == 0) pre(std::integral_constant<int, 0>{});
      else if (kl == 1) pre(std::integral_constant<int, 1>{});
      else pre(std::integral_constant<int, 2>{});
    } else {
#pragma unroll
      for (int u = 0; u < MK_NT; ++u)
        if (u < ng) T[u].load(g, u, kl, voff);
    }
  }
  const int kp = 512 << kl;   // staged row stride (elements): the K-chunks the tiles read
  if (!wait_and_stage(a, sm, s, kp)) return false;
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(sm.xs) + (tid_v() & 63) * 8;
  const uint16_t* xl = xh + s.nb * kp;
  GemvArgs gx = g;
  gx.xstride = kp;
  make_uniform(gx);
  // trace: wave 1 passes the staging barrier (mark 3), finishes its row
  // groups (mark 4); the epilogue end is mark 5
  if (a->trace && tid_v() == 64) sm.t_mark[3] = wall_clock64();
  if constexpr (NB == 1) {
    if (xreg) {
      if (cw) {
        u32x4 xrh[4], xrl[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          xrh[c] = c < (1 << kl) ? *reinterpret_cast<const u32x4*>(xh + 512 * c) : (u32x4){0u, 0u, 0u, 0u};
          xrl[c] = c < (1 << kl) ? *reinterpret_cast<const u32x4*>(xl + 512 * c) : (u32x4){0u, 0u, 0u, 0u};
        }
        auto run = [&](auto klc) {
          constexpr int KL = decltype(klc)::value;
          for (int grp = 0; grp < ng; grp += MK_NT) {
#pragma unroll
            for (int u = 0; u < MK_NT; ++u) {
              if (grp + u < ng) {
                T[u].template compute_r<KL>(gx, grp + u, xrh, xrl, sm.ys);
                if (grp + u + MK_NT < ng) T[u].template load_k<KL>(g, grp + u + MK_NT, voff);
              }
            }
          }
        };
        if (kl == 0) run(std::integral_constant<int, 0>{});
        else if (kl == 1) run(std::integral_constant<int, 1>{});
        else run(std::integral_constant<int, 2>{});
      }
      if (a->trace && tid_v() == 64) sm.t_mark[4] = wall_clock64();
      if (a->trace && tid_v() == 0 && sm.t_mark[1] == 0) sm.t_mark[1] = wall_clock64();
      return true;
    }
  }
  if (cw) {
    for (int grp = 0; grp < ng; grp += MK_NT) {
#pragma unroll
      for (int u = 0; u < MK_NT; ++u) {
        if (grp + u < ng) {
          T[u].compute(gx, grp + u, kl, xh, xl, sm.ys);
          if (grp + u + MK_NT < ng) T[u].load(g, grp + u + MK_NT, kl, voff);
        }
      }
    }
  }
  if (a->trace && tid_v() == 64) sm.t_mark[4] = wall_clock64();
  if (a->trace && tid_v() == 0 && sm.t_mark[1] == 0) sm.t_mark[1] = wall_clock64();
  return true;
}

// ------------------------------------------------- FP8 weights, one batch row
// Expert matrices stored as E4M3 codes (one byte per weight, [out][in]) with
// a float32 scale per row: row r computes scale[r] * sum_k E4M3(q[r][k]) x[k].
// The register tile and its loads are the bf16 tile's, byte for byte (16
// bytes per lane, 1 KB per wave load), but a slot now holds 16 weights, so a
// K-chunk is 1024 elements; each 16-byte slot is widened to bf16 pairs with
// v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3 value is a bf16 value) and
// multiplied into the hi and lo parts of x as in the bf16 form (24
// instructions per slot against 8, for half the bytes).  The row scales
// travel with the weights: lane j of the wave loads row j's scale just before
// the tile's weight loads, so the wait for the weights covers it.
template <int KL>
struct Fp8Tile {
  static constexpr int WB = MK_WB;           // 16-byte slots per lane per row group
  static constexpr int RPW = WB >> KL;       // rows per wave per row group
  u32x4 w[WB];
  float scv;                                 // lane j < RPW: the scale of the group's row j

  __device__ __forceinline__ static int row0(int grp, int cw) { return (grp * MK_CW + cw - 1) * RPW; }

  __device__ __forceinline__ void load(const GemvArgs& g, const float* scale, int grp, int voff) {
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    const int r0 = row0(grp, wave);
    {
      const int r = r0 + lane;
      const bool ok = lane < RPW && r < g.nrows;
      __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(scale), (short)0, 0x7FFFFFFF, 0x00020000);
      scv = ok ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(gemv_row_index(g, r) * 4u), 0, 0))
               : 0.f;
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = r0 + j;
      __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(gemv_row(g, r < g.nrows ? r : 0)), (short)0, r < g.nrows ? g.K : 0, 0x00020000);
#pragma unroll
      for (int c = 0; c < (1 << KL); ++c)
        w[(j << KL) + c] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + c * 1024, 0, 2 /* nontemporal */);
    }
  }

  // xrh / xrl: the lane's 16 elements of x per K-chunk c in [2c], [2c + 1]
  __device__ __forceinline__ void compute(const GemvArgs& g, int grp, const u32x4* xrh, const u32x4* xrl,
                                          float* ys) {
    constexpr int CM = (1 << KL) - 1;
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    const int r0 = row0(grp, wave);
    if (r0 >= g.nrows) return;   // wave-uniform: no rows in this group
    float acc[WB];
#pragma unroll
    for (int u = 0; u < WB; ++u) {
      const int c = u & CM;
      const u32x4 v = w[u];
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
      const u32x4 h0 = xrh[2 * c], h1 = xrh[2 * c + 1], q0 = xrl[2 * c], q1 = xrl[2 * c + 1];
      const uint32_t hw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // weights 4q, 4q + 1 and 4q + 2, 4q + 3 of the slot, as bf16 pairs
        const uint32_t a0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw[q], 1.0f, false));
        const uint32_t a1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vw[q], 1.0f, true));
        s = dot2_bf16(a0, hw[2 * q], s);
        s = dot2_bf16(a1, hw[2 * q + 1], s);
        s = dot2_bf16(a0, qw[2 * q], s);
        s = dot2_bf16(a1, qw[2 * q + 1], s);
      }
      acc[u] = s;
    }
    // add the K-chunks of each row pairwise
#pragma unroll
    for (int step = 1; step < (1 << KL); step <<= 1) {
#pragma unroll
      for (int i = 0; i < WB / (2 * step); ++i) acc[i] = acc[2 * i] + acc[2 * i + 1];
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = r0 + j;
      const float sv = wave_sum(acc[j]) * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scv), j));
      if (lane == 0 && r < g.nrows && g.nb > 0) {
        if (g.out) stc(g.out + r, sv);
        else ys[r * NBMAX] = sv;
      }
    }
  }
};

template <int KL>
__device__ __forceinline__ bool gemv_fp8_run(const KA a, Smem& sm, const GemvArgs& g_in, const StageArgs& s,
                                             const float* scale) {
  Fp8Tile<KL> T[MK_NT];
  GemvArgs g = g_in;
  make_uniform(g);
  scale = uniform_ptr(scale);
  constexpr int PER = MK_CW * Fp8Tile<KL>::RPW;
  const int ng = (g.nrows + PER - 1) / PER;
  const bool cw = (tid_v() >> 6) != 0;
  const int lane = tid_v() & 63;
  const int voff = lane * 16;
  if (cw) {
#pragma unroll
    for (int u = 0; u < MK_NT; ++u)
      if (u < ng) T[u].load(g, scale, u, voff);
  }
  constexpr int kp = 1024 << KL;   // staged row stride: whole 1024-element chunks
  if (!wait_and_stage(a, sm, s, kp)) return false;
  if (cw) {
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(sm.xs) + lane * 16;
    const uint16_t* xl = xh + s.nb * kp;
    u32x4 xrh[4], xrl[4];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool in = c < (1 << KL);
      xrh[2 * c] = in ? *reinterpret_cast<const u32x4*>(xh + 1024 * c) : (u32x4){0u, 0u, 0u, 0u};
      xrh[2 * c + 1] = in ? *reinterpret_cast<const u32x4*>(xh + 1024 * c + 8) : (u32x4){0u, 0u, 0u, 0u};
      xrl[2 * c] = in ? *reinterpret_cast<const u32x4*>(xl + 1024 * c) : (u32x4){0u, 0u, 0u, 0u};
      xrl[2 * c + 1] = in ? *reinterpret_cast<const u32x4*>(xl + 1024 * c + 8) : (u32x4){0u, 0u, 0u, 0u};
    }
    for (int grp = 0; grp < ng; grp += MK_NT) {
#pragma unroll
      for (int u = 0; u < MK_NT; ++u) {
        if (grp + u < ng) {
          T[u].compute(g, grp + u, xrh, xrl, sm.ys);
          if (grp + u + MK_NT < ng) T[u].load(g, scale, grp + u + MK_NT, voff);
        }
      }
    }
  }
  if (a->trace && tid_v() == 64) sm.t_mark[4] = wall_clock64();
  if (a->trace && tid_v() == 0 && sm.t_mark[1] == 0) sm.t_mark[1] = wall_clock64();
  return true;
}

// One FP8-weight GEMV tile with one batch row: K up to two 1024-element chunks.
__device__ __forceinline__ bool gemv_fp8_row1(const KA a, Smem& sm, const GemvArgs& g, const StageArgs& s,
                                              const float* scale) {
  if (g.K <= 1024) return gemv_fp8_run<0>(a, sm, g, s, scale);
  return gemv_fp8_run<1>(a, sm, g, s, scale);
}

// ------------------------------------------------ MFMA GEMV (3 to 8 batch rows)
// With several batch rows the dot-product form costs 8 instructions per
// 16-byte weight slot for every row, and two LDS reads of x per row: the
// multiply becomes VALU- and LDS-bound.  Here the weights are the A operand
// of v_mfma_f32_16x16x32_bf16 (16 weight rows x 32 K elements per K-step)
// and the staged rows of x the B operand (32 K x 16 columns: batch row n in
// column n, zeros in the columns past the batch), so a 16-byte weight slot
// costs two MFMAs (x = hi + lo, as in the dot-product form) for all the
// batch rows at once.  Lane l loads 8 consecutive K elements of weight row
// l mod 16 of the block (each wave load covers 16 rows x 64 bytes).  A group
// is one 16-row block per compute wave times a 512-element K chunk (16
// K-steps, 16 KB per wave); blocks go to the compute waves in turn, and a
// wave walks the K chunks of its block in order, accumulating in registers,
// before its next block.  Rows past the tile and K past the row read as
// zeros (out-of-range buffer offsets).
struct MfmaTile {
  static constexpr int WS = 16;   // K-steps (16-byte slots per lane) per group
  u32x4 w[WS];

  // 16-row block and K chunk of group grp for compute wave cw (1..MK_CW)
  __device__ __forceinline__ static void where(int grp, int cw, int kch, int& blk, int& ch) {
    const int bt = grp / kch;
    ch = grp - bt * kch;
    blk = bt * MK_CW + cw - 1;
  }

  __device__ __forceinline__ void load(const GemvArgs& g, int grp, int kch, int nblk) {
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    int blk, ch;
    where(grp, wave, kch, blk, ch);
    if (blk >= nblk) return;   // wave-uniform: no block for this wave
    const int r = blk * 16 + (lane & 15);
    const bool rv = r < g.nrows;
    // element offset of the lane's weight row from the matrix base
    const uint32_t roff = rv ? (uint32_t)(gemv_row(g, r) - g.base) : 0u;
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(g.base), (short)0, 0x7FFFFFFF, 0x00020000);
    const int k0 = ch * 512 + 8 * (lane >> 4);
#pragma unroll
    for (int u = 0; u < WS; ++u) {
      const int k = k0 + 32 * u;
      const uint32_t off = (rv && k < g.K) ? (roff + (uint32_t)k) * 2u : 0x80000000u;
      w[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 2 /* nontemporal */);
    }
  }

  // xh / xl: the staged hi / lo bf16 rows (row n at n * g.xstride)
  __device__ __forceinline__ void compute(const GemvArgs& g, int grp, int kch, int nblk, const uint16_t* xh,
                                          const uint16_t* xl, f32x4& acc, float* ys) {
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    int blk, ch;
    where(grp, wave, kch, blk, ch);
    if (blk >= nblk) return;
    const int n = lane & 15;
    const bool nv = n < g.nb;
    const int xo = n * g.xstride + ch * 512 + 8 * (lane >> 4);
#pragma unroll
    for (int u = 0; u < WS; ++u) {
      const u32x4 bh = nv ? *reinterpret_cast<const u32x4*>(xh + xo + 32 * u) : (u32x4){0u, 0u, 0u, 0u};
      const u32x4 bl = nv ? *reinterpret_cast<const u32x4*>(xl + xo + 32 * u) : (u32x4){0u, 0u, 0u, 0u};
      acc = mfma_bf16(w[u], bh, acc);
      acc = mfma_bf16(w[u], bl, acc);
    }
    if (ch == kch - 1) {
      // lane l holds rows 4 (l / 16) .. + 3 of the block, batch column l mod 16
      if (nv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = blk * 16 + 4 * (lane >> 4) + i;
          if (r < g.nrows) {
            if (g.out) stc(g.out + (long)n * g.ob + r, acc[i]);
            else ys[r * NBMAX + n] = acc[i];
          }
        }
      }
      acc = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }
};

__device__ __forceinline__ bool gemv_run_mfma(const KA a, Smem& sm, const GemvArgs& g_in, const StageArgs& s) {
  MfmaTile T[MK_NTM];
  GemvArgs g = g_in;
  make_uniform(g);
  const int kch = (g.K + 511) >> 9;
  const int kl = kch <= 1 ? 0 : 32 - __builtin_clz(kch - 1);
  const int nblk = (g.nrows + 15) >> 4;
  const int ng = ((nblk + MK_CW - 1) / MK_CW) * kch;
  const bool cw = (tid_v() >> 6) != 0;
  // the first MK_NTM groups are in flight before the dependency resolves
  if (cw) {
#pragma unroll
    for (int u = 0; u < MK_NTM; ++u)
      if (u < ng) T[u].load(g, u, kch, nblk);
  }
  const int kp = 512 << kl;   // staged row stride (elements)
  if (!wait_and_stage(a, sm, s, kp)) return false;
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(sm.xs);
  const uint16_t* xl = xh + s.nb * kp;
  GemvArgs gx = g;
  gx.xstride = kp;
  make_uniform(gx);
  if (a->trace && tid_v() == 64) sm.t_mark[3] = wall_clock64();
  if (cw) {
    f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int grp = 0; grp < ng; grp += MK_NTM) {
#pragma unroll
      for (int u = 0; u < MK_NTM; ++u) {
        if (grp + u < ng) {
          T[u].compute(gx, grp + u, kch, nblk, xh, xl, acc, sm.ys);
          if (grp + u + MK_NTM < ng) T[u].load(g, grp + u + MK_NTM, kch, nblk);
        }
      }
    }
  }
  if (a->trace && tid_v() == 64) sm.t_mark[4] = wall_clock64();
  if (a->trace && tid_v() == 0 && sm.t_mark[1] == 0) sm.t_mark[1] = wall_clock64();
  return true;
}

// ------------------------------------- MFMA GEMV on FP8 weights (2 to 8 rows)
// The FP8 counterpart of MfmaTile: lane l loads 16 consecutive codes (16
// bytes) of weight row l mod 16, K elements 16 (l / 16) .. +15 of a
// 64-element K block, so one wave load covers 16 rows x 64 codes.  The codes
// are widened to bf16 (v_cvt_scalef32_pk_bf16_fp8, exact) and feed two
// v_mfma_f32_16x16x32_bf16 K-steps: the first takes elements 0..7 of every
// lane's piece, the second 8..15.  A K-step sums over its 32 K indices in any
// order, so the B operand only has to hold x at the same indices: lane
// (column n, quarter q) reads x[n][64 u + 16 q + 8 h .. + 7] for step h.  A
// group is one 16-row block per compute wave times a 1024-element K chunk (16
// slots, 16 KB per wave, as in the bf16 tile).  The row scales of a block are
// loaded with its last K chunk (lane l: the scales of its four output rows)
// and multiply the accumulated sums.
struct MfmaFp8Tile {
  static constexpr int WS = 16;   // 16-byte slots (64-element K blocks) per lane per group
  u32x4 w[WS];
  f32x4 sc;                       // last K chunk of a block: the scales of the lane's four rows

  __device__ __forceinline__ static void where(int grp, int cw, int kch, int& blk, int& ch) {
    const int bt = grp / kch;
    ch = grp - bt * kch;
    blk = bt * MK_CW + cw - 1;
  }

  __device__ __forceinline__ void load(const GemvArgs& g, const float* scale, int grp, int kch, int nblk) {
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    int blk, ch;
    where(grp, wave, kch, blk, ch);
    if (blk >= nblk) return;   // wave-uniform: no block for this wave
    if (ch == kch - 1) {
      __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(scale), (short)0, 0x7FFFFFFF, 0x00020000);
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = blk * 16 + 4 * (lane >> 4) + i;
        v[i] = r < g.nrows
                   ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(gemv_row_index(g, r) * 4u), 0, 0))
                   : 0.f;
      }
      sc = (f32x4){v[0], v[1], v[2], v[3]};
    }
    const int r = blk * 16 + (lane & 15);
    const bool rv = r < g.nrows;
    // byte offset of the lane's weight row from the matrix base (ldw counts 16-bit units)
    const uint32_t roff = rv ? (uint32_t)(gemv_row(g, r) - g.base) * 2u : 0u;
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(g.base), (short)0, 0x7FFFFFFF, 0x00020000);
    const int k0 = ch * 1024 + 16 * (lane >> 4);
#pragma unroll
    for (int u = 0; u < WS; ++u) {
      const int k = k0 + 64 * u;
      const uint32_t off = (rv && k < g.K) ? roff + (uint32_t)k : 0x80000000u;
      w[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 2 /* nontemporal */);
    }
  }

  __device__ __forceinline__ void compute(const GemvArgs& g, int grp, int kch, int nblk, const uint16_t* xh,
                                          const uint16_t* xl, f32x4& acc, float* ys) {
    const int wave = __builtin_amdgcn_readfirstlane(tid_v() >> 6), lane = tid_v() & 63;
    int blk, ch;
    where(grp, wave, kch, blk, ch);
    if (blk >= nblk) return;
    const int n = lane & 15;
    const bool nv = n < g.nb;
    const int xo = n * g.xstride + ch * 1024 + 16 * (lane >> 4);
#pragma unroll
    for (int u = 0; u < WS; ++u) {
      const u32x4 v = w[u];
      const u32x4 a0 = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true))};
      const u32x4 a1 = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.z, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.z, 1.0f, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.w, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.w, 1.0f, true))};
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 bh0 = nv ? *reinterpret_cast<const u32x4*>(xh + xo + 64 * u) : z;
      const u32x4 bl0 = nv ? *reinterpret_cast<const u32x4*>(xl + xo + 64 * u) : z;
      const u32x4 bh1 = nv ? *reinterpret_cast<const u32x4*>(xh + xo + 64 * u + 8) : z;
      const u32x4 bl1 = nv ? *reinterpret_cast<const u32x4*>(xl + xo + 64 * u + 8) : z;
      acc = mfma_bf16(a0, bh0, acc);
      acc = mfma_bf16(a0, bl0, acc);
      acc = mfma_bf16(a1, bh1, acc);
      acc = mfma_bf16(a1, bl1, acc);
    }
    if (ch == kch - 1) {
      // lane l holds rows 4 (l / 16) .. + 3 of the block, batch column l mod 16
      if (nv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = blk * 16 + 4 * (lane >> 4) + i;
          if (r < g.nrows) {
            const float v = acc[i] * sc[i];
            if (g.out) stc(g.out + (long)n * g.ob + r, v);
            else ys[r * NBMAX + n] = v;
          }
        }
      }
      acc = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  }
};

__device__ __forceinline__ bool gemv_fp8_mfma(const KA a, Smem& sm, const GemvArgs& g_in, const StageArgs& s,
                                              const float* scale) {
  MfmaFp8Tile T[MK_NTM];
  GemvArgs g = g_in;
  make_uniform(g);
  scale = uniform_ptr(scale);
  const int kch = (g.K + 1023) >> 10;
  const int kl = kch <= 1 ? 0 : 32 - __builtin_clz(kch - 1);
  const int nblk = (g.nrows + 15) >> 4;
  const int ng = ((nblk + MK_CW - 1) / MK_CW) * kch;
  const bool cw = (tid_v() >> 6) != 0;
  if (cw) {
#pragma unroll
    for (int u = 0; u < MK_NTM; ++u)
      if (u < ng) T[u].load(g, scale, u, kch, nblk);
  }
  const int kp = 1024 << kl;   // staged row stride: whole 1024-element chunks
  if (!wait_and_stage(a, sm, s, kp)) return false;
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(sm.xs);
  const uint16_t* xl = xh + s.nb * kp;
  GemvArgs gx = g;
  gx.xstride = kp;
  make_uniform(gx);
  if (a->trace && tid_v() == 64) sm.t_mark[3] = wall_clock64();
  if (cw) {
    f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int grp = 0; grp < ng; grp += MK_NTM) {
#pragma unroll
      for (int u = 0; u < MK_NTM; ++u) {
        if (grp + u < ng) {
          T[u].compute(gx, grp + u, kch, nblk, xh, xl, acc, sm.ys);
          if (grp + u + MK_NTM < ng) T[u].load(g, scale, grp + u + MK_NTM, kch, nblk);
        }
      }
    }
  }
  if (a->trace && tid_v() == 64) sm.t_mark[4] = wall_clock64();
  if (a->trace && tid_v() == 0 && sm.t_mark[1] == 0) sm.t_mark[1] = wall_clock64();
  return true;
}

// One FP8-weight GEMV tile: the register dot-product form for one batch row,
// the MFMA form for more.
__device__ __forceinline__ bool gemv_fp8(const KA a, Smem& sm, const GemvArgs& g, const StageArgs& s,
                                         const float* scale) {
  if (g.nb <= 1) return gemv_fp8_row1(a, sm, g, s, scale);
  return gemv_fp8_mfma(a, sm, g, s, scale);
}

// Runs one GEMV tile: prefetch, wait, stage x, multiply.  false if the step
// was aborted while waiting.
__device__ __forceinline__ bool gemv(const KA a, Smem& sm, const GemvArgs& g, const StageArgs& s) {
  if (g.nb <= 1) return gemv_run<1>(a, sm, g, s);
  if (g.nb <= 2) return gemv_run<2>(a, sm, g, s);
  return gemv_run_mfma(a, sm, g, s);
}

// ------------------------------------------------------------- ADD_RMSNORM
// x_l = x_{l-1} + sum_g O-proj partial_g + sum_j w_j Y_j (parallel block), or
// the embedding row at layer 0; xn_l = x_l / sqrt(mean(x_l^2) + eps) * gain,
// for the batch row t.batch (one task per sequence).  Each thread takes up to
// NCH 4-element chunks of the row; the ~Hkv + k + 1 source loads of all its
// chunks are issued together, so the row costs one round trip.  x is kept in
// LDS between the two passes.  NCH is 2 for d <= 2048 and 4 up to 4096: with
// arrays for four chunks the compiler cannot keep every source load of the
// chunks in registers at once and waits for the first chunks' loads before
// issuing the next ones (two round trips instead of one at d = 2048).
// The MoE combine (the gate-weighted sum of the routed expert outputs, in
// top-k order) is folded into this task.
template <int NCH>   // 4-element chunks per thread (d <= NCH * 4 * 256)
__device__ __forceinline__ bool op_add_rmsnorm(const KA a, Smem& sm, const mk_task& t, int ti) {
  const int l = t.layer, d = a->d, B = a->B, nv = d >> 2, K = a->topk;
  const int b0 = t.batch, b1 = t.batch + 1;   // the row of this task
  const int tid = tid_v(), wave = tid >> 6, lane = tid & 63;
  const bool mid = t.flags & MK_F_MID;
  const bool fin = t.flags & MK_F_FINAL;
  const bool emb = t.flags & MK_F_EMBED;
  const bool moe_in = !emb && !mid && a->parallel && a->E > 0;
  const int lp = l - 1;
  const int lx = mid ? l : lp;     // layer whose attention output is added
  const uint16_t* gain = fin ? a->final_norm : (mid ? LAYER_PTR(l, ffn_norm) : LAYER_PTR(l, attn_norm));
  // gains do not depend on anything: in flight during the wait
  u32x2 gg[NCH];
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int c = tid + q * MK_THREADS;
    gg[q] = c < nv ? ldg8(gain + c * 4) : (u32x2){0u, 0u};
  }
  // gate weights and rows of the routed outputs of the previous layer: final
  // once its routing counter is set, which is long before this layer's
  // counter completes, so they are read while waiting
  int* srow = sm.misc + 64;                              // [B*K]
  float* sw = reinterpret_cast<float*>(sm.misc + 128);   // [B*K]
  if (moe_in) {
    if (!wg_wait(a, sm, layer_ctr(a, lp, MK_CTR_ROUTE), 1, ti)) return false;
    const int32_t* slot = a->moe + (long)lp * a->moe_stride + 4;
    if (tid < K) {
      srow[b0 * K + tid] = ldc(slot + b0 * K + tid);
      sw[b0 * K + tid] = ldc(a->topw + ((long)lp * B + b0) * K + tid);
    }
  }
  if (!wg_wait(a, sm, t.wait_ctr, t.wait_target, ti)) return false;
  float* xdst = mid ? a->xmid + (long)l * B * d : a->x + (long)l * B * d;
  float* xndst = mid ? a->xn2 + (long)l * B * d : a->xn + (long)l * B * d;
  float* red = sm.red;      // [MK_WAVES][NBMAX] partial sums of squares
  float* xv = sm.xs;        // [B][d] the new residual rows
#pragma unroll 1
  for (int b = b0; b < b1; ++b) {
    const bool live = seq_len_u(b) > 0;
    int tok = 0;
    if (emb && live) {
      tok = token_u(b);
      if (tok < 0 || tok >= a->V) {
        if (tid == 0) report(a, MK_E_DEVICE, ti, -1, tok, a->V);
        tok = 0;
      }
      if (tid == 0 && seq_len_u(b) > a->max_blocks * a->page)
        report(a, MK_E_DEVICE, ti, -5, seq_len_u(b), a->max_blocks * a->page);
    }
    // every source chunk of this thread is loaded before any is used
    f32x4 acc[NCH];
    if (!live) {
#pragma unroll
      for (int q = 0; q < NCH; ++q) acc[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
    } else if (emb) {
#pragma unroll
      for (int q = 0; q < NCH; ++q) {
        const int c = tid + q * MK_THREADS;
        const u32x2 e = c < nv ? ldg8(a->embed + (long)tok * d + c * 4) : (u32x2){0u, 0u};
        acc[q] = (f32x4){bf_lo(e.x), bf_hi(e.x), bf_lo(e.y), bf_hi(e.y)};
      }
    } else if (mid || moe_in) {
      // Every load of the chunks is issued before any is used, and none sits
      // in a branch: a load under a runtime condition (g < Hkv, j < k, the
      // chunk inside the row) got its own basic block, the compiler merged
      // the matching add into it and waited right after the load.  Slots
      // past Hkv or k load a duplicate of the last partial or row and are
      // dropped by a select; lanes past the row load chunk 0.  The expert
      // rows come from LDS and are read before the first load.
      const int hkv = a->Hkv;
      int yrow[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) yrow[j] = moe_in ? __builtin_amdgcn_readfirstlane(srow[b * K + min(j, K - 1)]) : 0;
      u32x4 og[NCH][8], ym[NCH][8], xq[NCH];
#pragma unroll
      for (int q = 0; q < NCH; ++q) {
        const int c = tid + q * MK_THREADS, off = c < nv ? c * 16 : 0;
#pragma unroll
        for (int g = 0; g < 8; ++g) og[q][g] = ldc16(a->opart + (((long)lx * hkv + min(g, hkv - 1)) * B + b) * d, off);
        if (moe_in) {
#pragma unroll
          for (int j = 0; j < 8; ++j) ym[q][j] = ldc16(a->Y + ((long)lp * a->bk + yrow[j]) * d, off);
        }
        xq[q] = ldc16(a->x + ((long)lx * B + b) * d, off);
      }
#pragma unroll
      for (int q = 0; q < NCH; ++q) {
        const int c = tid + q * MK_THREADS, off = c * 16;
        f32x4 o = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const f32x4 v = as_f4(og[q][g]);
          o += g < hkv ? v : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        acc[q] = as_f4(xq[q]) + o;
        f32x4 m = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (moe_in) {
#pragma unroll
          for (int j = 0; j < 8; ++j) m += (j < K ? sw[b * K + j] : 0.f) * as_f4(ym[q][j]);
          acc[q] += m;
        }
        if (c < nv) {
          stc16(a->oout + ((long)lx * B + b) * d, off, as_u4(o));
          if (moe_in) stc16(a->fo + ((long)lp * B + b) * d, off, as_u4(m));
        } else {
          acc[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      }
    } else {
      // sequential block: x_l = x_mid + FFN output (every load first, none in
      // a branch, as above)
      u32x4 xm[NCH], fq[NCH];
#pragma unroll
      for (int q = 0; q < NCH; ++q) {
        const int c = tid + q * MK_THREADS, off = c < nv ? c * 16 : 0;
        xm[q] = ldc16(a->xmid + ((long)lp * B + b) * d, off);
        fq[q] = ldc16(a->fo + ((long)lp * B + b) * d, off);
      }
#pragma unroll
      for (int q = 0; q < NCH; ++q) {
        const int c = tid + q * MK_THREADS;
        acc[q] = c < nv ? as_f4(xm[q]) + as_f4(fq[q]) : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int c = tid + q * MK_THREADS;
      if (c < nv) {
        stc16(xdst + (long)b * d, c * 16, as_u4(acc[q]));
        *reinterpret_cast<f32x4*>(xv + b * d + c * 4) = acc[q];
        ss += acc[q].x * acc[q].x + acc[q].y * acc[q].y + acc[q].z * acc[q].z + acc[q].w * acc[q].w;
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave * NBMAX + b] = ss;
  }
  __syncthreads();
#pragma unroll 1
  for (int b = b0; b < b1; ++b) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < MK_WAVES; ++w) tot += red[w * NBMAX + b];
    const float r = 1.0f / sqrtf(tot / (float)d + a->eps);
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int c = tid + q * MK_THREADS;
      if (c < nv) {
        const f32x4 gv = (f32x4){bf_lo(gg[q].x), bf_hi(gg[q].x), bf_lo(gg[q].y), bf_hi(gg[q].y)};
        const f32x4 xb = *reinterpret_cast<const f32x4*>(xv + b * d + c * 4);
        stc16(xndst + (long)b * d, c * 16, as_u4(xb * r * gv));
      }
    }
  }
  wg_signal(a, t.signal_ctr, 1);
  return true;
}

// ------------------------------------------------------------ epilogues
// QKV_PROJ: tile = rotation pairs [n0, n1) over all heads (pair p of head h
// is rows h*hd + p and h*hd + p + hd/2).  RoPE (rotate-half, angle
// pos * theta^(-2i/hd) in double) on q and k; k and v rounded to bf16 and
// written to the sequence's page at its position (V pages are transposed).
__device__ __forceinline__ void epi_qkv(const KA a, Smem& sm, const mk_task& t, int ti) {
  const int l = t.layer, hd = a->hd, half = hd / 2, B = a->B;
  const int np = t.n1 - t.n0;
  const int rows = (a->Hq + 2 * a->Hkv) * hd;
  uint16_t* kpool = LAYER_PTR(l, k);
  uint16_t* vpool = LAYER_PTR(l, v);
  for (int idx = tid_v(); idx < np * B; idx += MK_THREADS) {
    const int p = idx / B, b = idx - p * B;
    if (sh_seq_lens[b] <= 0) continue;
    const int gp = t.n0 + p, head = gp / half, i = gp - head * half;
    float ya = sm.ys[(2 * p) * NBMAX + b], yb = sm.ys[(2 * p + 1) * NBMAX + b];
    const int pos = sh_positions[b];
    if (head < a->Hq + a->Hkv) {
      // cos/sin of pos * theta^(-2i/hd) (the inverse frequencies are in
      // LDS), evaluated in double here rather than read from a table of
      // angles (a load would cost a memory round trip)
      double sn, cs;
      sincos((double)pos * sh_invf[i], &sn, &cs);
      const float c = (float)cs, s_ = (float)sn;
      const float ra = ya * c - yb * s_;
      const float rb = yb * c + ya * s_;
      ya = ra;
      yb = rb;
    }
    float* qo = a->qkv + ((long)l * B + b) * rows;
    stc(qo + head * hd + i, ya);
    stc(qo + head * hd + i + half, yb);
    if (head >= a->Hq) {
      const bool isk = head < a->Hq + a->Hkv;
      const int kvh = isk ? head - a->Hq : head - a->Hq - a->Hkv;
      const int blk = pos / a->page;
      const bool bt_lds = a->B * a->max_blocks <= MK_LDS_BT;   // the step's block table is in LDS
      const int page = (blk >= 0 && blk < a->max_blocks)
                           ? (bt_lds ? sh_bt[b * a->max_blocks + blk] : a->block_tables[b * a->max_blocks + blk])
                           : -1;
      if (page < 0 || page >= a->num_pages || pos < 0) {
        report(a, MK_E_DEVICE, ti, -2, page, a->num_pages);
        continue;
      }
      if (isk) {   // K page [hd/32][16 keys][32 dims]
        uint16_t* dst = kpool + ((long)page * a->Hkv + kvh) * 16 * hd + (pos & 15) * 32;
        const int e1 = i + half;
        stc(dst + (i >> 5) * 512 + (i & 31), f_to_bf16(ya));
        stc(dst + (e1 >> 5) * 512 + (e1 & 31), f_to_bf16(yb));
      } else {     // V page [hd][16 keys]
        uint16_t* dst = vpool + ((long)page * a->Hkv + kvh) * hd * 16 + (pos & 15);
        stc(dst + i * 16, f_to_bf16(ya));
        stc(dst + (i + half) * 16, f_to_bf16(yb));
      }
    }
  }
}

// SiLU-and-multiply epilogue of the gate/up tiles: out[j][p] = silu(g) * u
// from the paired tile rows 2p (gate) and 2p+1 (up).
__device__ __forceinline__ void epi_swiglu(Smem& sm, int np, int nb, float* out, long ob) {
  for (int idx = tid_v(); idx < np * nb; idx += MK_THREADS) {
    const int p = idx / nb, j = idx - p * nb;
    const float gv = sm.ys[(2 * p) * NBMAX + j], uv = sm.ys[(2 * p + 1) * NBMAX + j];
    stc(out + (long)j * ob + p, silu(gv) * uv);
  }
}

// ------------------------------------------------------------- LM_HEAD
// The tile's logits (rows [n0, n1) of every slot, in LDS ys[r][b]) go to the
// caller's buffer.  When the step samples, each slot's candidate of the tile
// is the row with the largest score -- the logit (greedy), or logit / T plus
// Gumbel noise -- ties to the lowest id; the tile writes its candidates to
// lm_best, and the last tile to finish reduces all tiles' candidates into
// next_tok (one decision per slot, in the same order-free way: largest score,
// then lowest id).
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}
// the larger of two (score, id) candidates; equal scores go to the lower id
__device__ __forceinline__ void best_of(float& s, int& id, float s2, int id2) {
  if (s2 > s || (s2 == s && id2 < id)) { s = s2; id = id2; }
}
// wave-wide best candidate, returned uniform
__device__ __forceinline__ void wave_best(float& s, int& id) {
  const float m = wave_max(s);
  id = wave_min(s == m ? id : 0x7FFFFFFF);
  s = m;
}
__device__ __forceinline__ void epi_lm_head(const KA a, Smem& sm, const mk_task& t) {
  const int nr = t.n1 - t.n0, B = a->B, V = a->V;
  const int tid = tid_v(), wave = tid >> 6, lane = tid & 63;
  for (int idx = tid; idx < nr * B; idx += MK_THREADS) {
    const int b = idx / nr, r = idx - b * nr;
    stc(a->logits + (long)b * V + t.n0 + r, sm.ys[r * NBMAX + b]);
  }
  if (!a->next_tok) return;
  const float it = a->inv_temp;
  float* cs = sm.red;                               // [MK_WAVES][NBMAX] scores
  int* ci = reinterpret_cast<int*>(sm.red) + 64;    // [MK_WAVES][NBMAX] ids
  for (int b = 0; b < B; ++b) {
    uint32_t key = 0;
    if (it > 0.f) {
      key = fmix32(fmix32(fmix32(a->sample_seed) ^ (uint32_t)position_u(b)) ^ (uint32_t)b);
    }
    float bs = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int r = tid; r < nr; r += MK_THREADS) {
      float sc = sm.ys[r * NBMAX + b];
      if (it > 0.f) {
        // u = (h / 2^8 + 1/2) / 2^24 is exact in fp32 and lies in (0, 1)
        const uint32_t h = fmix32(key ^ (uint32_t)(t.n0 + r));
        const float u = ((float)(h >> 8) + 0.5f) * 5.9604644775390625e-8f;
        sc = sc * it - logf(-logf(u));
      }
      best_of(bs, bi, sc, t.n0 + r);
    }
    wave_best(bs, bi);
    if (lane == 0) {
      cs[wave * NBMAX + b] = bs;
      ci[wave * NBMAX + b] = bi;
    }
  }
  __syncthreads();
  if (tid < B) {
    float bs = cs[tid];
    int bi = ci[tid];
#pragma unroll
    for (int w = 1; w < MK_WAVES; ++w) best_of(bs, bi, cs[w * NBMAX + tid], ci[w * NBMAX + tid]);
    int32_t* slot = a->lm_best + ((long)t.aux[1] * B + tid) * 2;
    stc(slot, __float_as_int(bs));
    stc(slot + 1, bi);
  }
  stores_done();
  __syncthreads();
  if (tid == 0)
    sm.misc[3] = __hip_atomic_fetch_add(ctrp(a, MK_CG_LM), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 t.aux[0] - 1;
  __syncthreads();
  if (!sm.misc[3]) return;
  // the last tile: one wave per slot reduces every tile's candidate
  const int n_tiles = t.aux[0];
  for (int b = wave; b < B; b += MK_WAVES) {
    float bs = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int k = lane; k < n_tiles; k += 64) {
      const int32_t* slot = a->lm_best + ((long)k * B + b) * 2;
      best_of(bs, bi, __int_as_float(ldc(slot)), ldc(slot + 1));
    }
    wave_best(bs, bi);
    if (lane == 0) stc(a->next_tok + b, seq_len_u(b) > 0 ? bi : -1);
  }
  stores_done();
}

// ---------------------------------------------------------- ROUTER_TOPK
// Per token: top-k router logits (ties to the lower expert id); gate weights
// are the softmax probabilities of the selected experts renormalised to sum
// to 1, i.e. exp(r_j - r_max) / sum over the selected.  One wave per token;
// leaves the selected ids in misc[64 + b*k + j] for ROUTE_FINALIZE.
__device__ __forceinline__ void router_topk(const KA a, Smem& sm, int l) {
  const int B = a->B, E = a->E, K = a->topk;
  const int wave = tid_v() >> 6, lane = tid_v() & 63;
  const uint16_t* bias = LAYER_PTR(l, router_bias);   // optional [E] logit bias
  for (int b = wave; b < B; b += MK_WAVES) {
    // the logits and the bias are loaded together, unconditionally (a lane
    // past E reads expert E - 1 and is masked by a select): loads under a
    // per-lane condition were each followed by a wait
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ldc(a->rlog + ((long)l * B + b) * E + min(lane + 64 * u, E - 1));
    if (bias) {
      // the bias is part of the logits (selection and gate weights); the
      // router-logit tap keeps the projection alone
      uint16_t bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) bb[u] = ((GLOBAL const uint16_t*)bias)[min(lane + 64 * u, E - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] += bf16_to_f(bb[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = lane + 64 * u < E ? v[u] : -INFINITY;
    float top0 = 0.f, wsum = 0.f;
    float myw = 0.f;
    int myid = 0;
    for (int j = 0; j < K; ++j) {
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane + 64 * u;
        if (e < E && (v[u] > bv || (v[u] == bv && e < be))) { bv = v[u]; be = e; }
      }
      // the largest logit, then the lowest id among the lanes holding it
      const float mx = wave_max(bv);
      const int win = wave_min(bv == mx ? be : 0x7FFFFFFF);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (lane + 64 * u == win) v[u] = -INFINITY;
      if (j == 0) top0 = mx;
      const float ew = expf(mx - top0);
      wsum += ew;
      if (lane == j) { myw = ew; myid = win; }
    }
    if (lane < K) {
      stc(a->topi + ((long)l * B + b) * K + lane, myid);
      stc(a->topw + ((long)l * B + b) * K + lane, myw / wsum);
      sm.misc[64 + b * K + lane] = seq_len_u(b) > 0 ? myid : -1;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------- ROUTE_FINALIZE
// From the B*k routed (token, slot) pairs: sort by (expert, token slot) in
// one wave, each key placed at its rank (the number of smaller keys, counted
// from a copy in LDS); row r of the sorted order is the r-th routed row.  Writes the active expert list (ascending ids), each expert's
// first row, the token of each row, the row of each (token, slot), and the
// lengths of the up-gate and down claim queues.  Uses misc[64..] ids.
__device__ __forceinline__ void route_finalize(const KA a, Smem& sm, int l) {
  if ((tid_v() >> 6) != 0) return;
  const int lane = tid_v() & 63, K = a->topk, BK = a->B * K;
  int32_t* meta = a->moe + (long)l * a->moe_stride;
  int32_t* slot = meta + 4;
  int32_t* rec = slot + a->bk;            // [bk][16]: e, r0, nr, 0, token of each row
  uint32_t key = 0xFFFFFFFFu;
  if (lane < BK) {
    const int id = sm.misc[64 + lane];
    if (id >= 0) key = ((uint32_t)id << 8) | (uint32_t)lane;
  }
  // LDS accesses of one wave complete in program order, so the lanes see
  // each other's stores without a barrier
  uint32_t* kin = sm.sortk;          // [64] keys in (token, slot) order
  uint32_t* kso = sm.sortk + 64;     // [64] keys in sorted order
  kin[lane] = key;
  int rank = 0;
#pragma unroll 16
  for (int j = 0; j < 64; ++j) rank += kin[j] < key ? 1 : 0;
  if (key != 0xFFFFFFFFu) kso[rank] = key;
  const int nvalid = __popcll(__ballot(key != 0xFFFFFFFFu));
  key = lane < nvalid ? kso[lane] : 0xFFFFFFFFu;
  const bool valid = key != 0xFFFFFFFFu;
  const uint32_t prev = kso[lane > 0 ? lane - 1 : 0];
  const int e = (int)(key >> 8), src = (int)(key & 0xFF);
  const bool start = valid && (lane == 0 || (prev >> 8) != (key >> 8));
  const uint64_t vmask = __ballot(valid);
  const uint64_t smask = __ballot(start);
  const int nrows = __popcll(vmask), nact = __popcll(smask);
  const uint64_t le = (lane == 63) ? ~0ull : ((2ull << lane) - 1ull);
  const int aidx = __popcll(smask & le) - 1;
  if (valid) {
    const int r0 = 63 - __clzll(smask & le);           // first row of this expert
    stc(slot + src, lane);
    stc(rec + aidx * 16 + 4 + (lane - r0), src / K);  // token of this row
    if (start) {
      const uint64_t after = smask & ~le;
      const int next = after ? __ffsll((long long)after) - 1 : nrows;
      stc(rec + aidx * 16 + 0, e);
      stc(rec + aidx * 16 + 1, lane);
      stc(rec + aidx * 16 + 2, next - lane);
    }
  }
  if (lane == 0) {
    stc(meta + 0, nact);
    stc(meta + 1, nact * a->ug_tiles);
    stc(meta + 2, nact * a->dn_tiles);
    stc(meta + 3, nrows);
  }
}

// ---------------------------------------------------------- attention split
// Keys [p0, p1) of sequence b, KV group g: scores s_j = q_h . K_j / sqrt(hd)
// for the G query heads of the group, then m = max s, p = exp(s - m),
// l = sum p, o = sum p V_j (the split partials the combine merges).
//
// Both products run on the matrix cores (v_mfma_f32_16x16x32_bf16; one
// 16-row tile holds the group's <= 8 heads, the other rows are zero).  K and
// V are bf16 already; the fp32 operands q and p are split into a bf16 high
// part and a bf16 remainder, and each product is the sum of two MFMAs, so
// the result keeps about 16 mantissa bits of q and p (fp32 accumulation).  A
// key tile is one 16-key page.  QK: A = q (bf16), B = K^T: lane l holds key
// (l mod 16), dims 32s + 8(l/16) .. +7; a K page is stored as [hd/32][16
// keys][32 dims], so the 64 lanes of one k-step read 1 KB contiguous.
// PV: A = P (bf16, from LDS), B = V: lane l holds dim (l mod 16) of 8
// consecutive keys, a 16-byte piece of the transposed V page.  Result tiles:
// lane l holds rows (heads) 4(l/16) .. +3 of column (key or dim) l mod 16.
// Compute waves take key tiles (QK) and dim tiles (PV) in turn.  The K and V
// fragments of the first tiles are loaded before the wait on the QKV tiles
// (cached keys are immutable); the key appended this step is re-read with a
// coherent load after the wait.  q goes through LDS, staged by wave 0.

constexpr int ATT_PT = 4;   // K tiles in flight per compute wave
constexpr int ATT_PV = 6;   // V k-steps (32 keys) in flight per compute wave

template <int HD>
__device__ __forceinline__ bool attn_split(const KA a, Smem& sm, int l, int b, int g, int s, int p0, int p1, int ti,
                                           int wait_idx, int wait_target) {
  constexpr int KS = HD / 32;                       // QK k-steps per key tile
  constexpr int NDT = HD / 16;                      // PV dim tiles
  constexpr int DTW = (NDT + MK_CW - 1) / MK_CW;    // dim tiles per compute wave
  const int G = a->G, Hkv = a->Hkv;
  const int SP = a->attn_split + 32;                // LDS row stride of scores and P
  const int tid = tid_v(), wave = tid >> 6, lane = tid & 63;
  const int cw = wave - 1;                          // compute wave index (wave 0: -1)
  const int c16 = lane & 15, q4 = lane >> 4;
  const int tb0 = p0 & ~15;                         // first key of the first tile
  const int nt = (p1 - tb0 + 15) >> 4;              // key tiles
  const int nks = (nt + 1) >> 1;                    // PV k-steps
  const int nti = cw >= 0 && cw < nt ? (nt - cw + MK_CW - 1) / MK_CW : 0;   // key tiles of this wave
  const uint16_t* Kp = LAYER_PTR(l, k);
  const uint16_t* Vp = LAYER_PTR(l, v);
  const int32_t* bt = a->block_tables + (long)b * a->max_blocks + (tb0 >> 4);
  const bool bt_lds = a->B * a->max_blocks <= MK_LDS_BT;
  const int* btl = sh_bt + b * a->max_blocks + (tb0 >> 4);
  const int newest = position_u(b);
  // The key appended this step is not read from its page, whose store may
  // not be visible yet: its score and its share of P V are computed from the
  // QKV output (rounded to bf16 like the page copy), outside the MFMA loops,
  // and its page slot only ever meets p = 0 there.
  const bool has_new = newest >= p0 && newest < p1;
  const int kk_new = newest - tb0;
  float* fresh = reinterpret_cast<float*>(sm.misc + 16);   // [8..15]: its p per head
  const float* qkv_b = a->qkv + ((long)l * a->B + b) * (a->Hq + 2 * Hkv) * HD;
  // the split's page ids in LDS (loaded by wave 0 while it waits for q),
  // for the K and V loads inside the passes
  int* spg = reinterpret_cast<int*>(sm.xs + G * HD);
  auto page_of = [&](int t) -> int {
    int pg = spg[t];
    if (pg < 0 || pg >= a->num_pages) {
      report(a, MK_E_DEVICE, ti, -3, pg, a->num_pages);
      pg = 0;
    }
    return pg;
  };
  // element offset of this lane's piece of key tile t (dims 8(l/16) of the row)
  auto k_off = [&](int t) -> int { return (page_of(t) * Hkv + g) * 16 * HD + c16 * 32 + 8 * q4; };
  // element offset of this lane's V piece of k-step ks in dim tile 0, or -1
  // (dim tile dt adds 256 dt)
  auto v_off = [&](int ks) -> int {
    const int tt = 2 * ks + (lane >> 5);
    if (tt >= nt) return -1;
    return ((page_of(tt) * Hkv + g) * HD + c16) * 16 + 8 * (q4 & 1);
  };
  u32x4 kf[ATT_PT][KS], vf[ATT_PV][DTW];
  if (a->trace && tid == 64 && sm.t_mark[8] == 0) sm.t_mark[8] = wall_clock64();   // compute wave enters
  if (cw >= 0) {
    // every page id first (one round trip), then every K and V load.  From
    // memory the ids are loaded unconditionally (a slot past the split reads
    // the split's last tile, and a select drops it): under per-lane
    // conditions each load was followed by a wait, ten round trips per split
    int kpg[ATT_PT], vpg[ATT_PV];
    if (bt_lds) {
#pragma unroll
      for (int u = 0; u < ATT_PT; ++u) kpg[u] = u < nti ? btl[cw + MK_CW * u] : 0;
#pragma unroll
      for (int u = 0; u < ATT_PV; ++u) {
        const int tt = 2 * u + (lane >> 5);
        vpg[u] = (u < nks && tt < nt) ? btl[tt] : -1;
      }
    } else {
      int kr[ATT_PT], vr[ATT_PV];
#pragma unroll
      for (int u = 0; u < ATT_PT; ++u) kr[u] = bt[min(cw + MK_CW * u, nt - 1)];
#pragma unroll
      for (int u = 0; u < ATT_PV; ++u) vr[u] = bt[min(2 * u + (lane >> 5), nt - 1)];
#pragma unroll
      for (int u = 0; u < ATT_PT; ++u) kpg[u] = u < nti ? kr[u] : 0;
#pragma unroll
      for (int u = 0; u < ATT_PV; ++u) {
        const int tt = 2 * u + (lane >> 5);
        vpg[u] = (u < nks && tt < nt) ? vr[u] : -1;
      }
    }
    if (a->trace && tid == 64 && sm.t_mark[9] == 0) sm.t_mark[9] = kpg[0] + vpg[0] >= -2 ? wall_clock64() : 1;
    // Every load of the K and V windows is issued unconditionally (a slot
    // past the split reads the start of the pool, whose values are finite,
    // and is masked where it is used), so the compiler can count the loads
    // in flight and each MFMA waits only for its own operands.
#pragma unroll
    for (int u = 0; u < ATT_PT; ++u) {
      int pg = kpg[u];
      if (u < nti && (pg < 0 || pg >= a->num_pages)) {
        report(a, MK_E_DEVICE, ti, -3, pg, a->num_pages);
        pg = 0;
      }
      const int o = u < nti ? (pg * Hkv + g) * 16 * HD + c16 * 32 + 8 * q4 : 0;
#pragma unroll
      for (int k = 0; k < KS; ++k) kf[u][k] = ldg_nt(Kp + o + 512 * k);
    }
#pragma unroll
    for (int u = 0; u < ATT_PV; ++u) {
      int pg = vpg[u];
      if (pg >= a->num_pages || (pg < 0 && u < nks && 2 * u + (lane >> 5) < nt)) {
        report(a, MK_E_DEVICE, ti, -3, pg, a->num_pages);
        pg = 0;
      }
      const int o = pg >= 0 ? ((pg * Hkv + g) * HD + c16) * 16 + 8 * (q4 & 1) : -1;
#pragma unroll
      for (int j = 0; j < DTW; ++j) {
        const int dt = cw + MK_CW * j;
        vf[u][j] = ldg_nt(Vp + ((o >= 0 && dt < NDT) ? o + 256 * dt : 0));
      }
    }
    if (a->trace && tid == 64 && sm.t_mark[5] == 0) sm.t_mark[5] = wall_clock64();   // loads issued
  }
  MK_MARK(3);
  // wait for the QKV tiles, then wave 0 stages q of the group's heads
  float* qs = sm.xs;   // [G][HD]
  if (tid < 64) {
    // page ids of the split's key tiles (at most 2 per lane for a split of
    // up to 1024 keys + 2 tiles), in flight during the wait
    int pid[2];
    if (bt_lds) {
#pragma unroll
      for (int u = 0; u < 2; ++u) pid[u] = lane + 64 * u < nt ? btl[lane + 64 * u] : 0;
    } else {
      int r[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) r[u] = bt[min(lane + 64 * u, nt - 1)];
#pragma unroll
      for (int u = 0; u < 2; ++u) pid[u] = lane + 64 * u < nt ? r[u] : 0;
    }
    int ok = 1;
    if (lane == 0) {
      ok = (wait_idx < 0 || wait_target <= 0) ? 1 : (int)spin_until(a, wait_idx, wait_target, ti);
      if (a->trace && sm.t_ready == 0) sm.t_ready = wall_clock64();
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (lane + 64 * u < nt) spg[lane + 64 * u] = pid[u];
    ok = __builtin_amdgcn_readfirstlane(ok);
    if (lane == 0) sm.misc[0] = ok;
    if (ok) {
      // q of the group's heads (G <= 8: at most HD / 32 pieces per lane) and
      // the new key are loaded together, so staging costs one round trip; a
      // piece past the group's q reads its first piece and is not stored
      const float* qb = qkv_b + (long)(g * G) * HD;
      constexpr int QN = 8 * HD / 4 / 64;
      const int nq = G * HD / 4;
      u32x4 qv[QN];
#pragma unroll
      for (int u = 0; u < QN; ++u) {
        const int i = lane + 64 * u;
        qv[u] = ldc16(qb, (i < nq ? i : 0) * 16);
      }
      constexpr int DL = HD / 64;   // new-key dims per lane
      float kn[DL];
      if (has_new) {
#pragma unroll
        for (int e = 0; e < DL; ++e) kn[e] = ldc(qkv_b + (long)(a->Hq + g) * HD + lane + 64 * e);
      }
#pragma unroll
      for (int u = 0; u < QN; ++u) {
        const int i = lane + 64 * u;
        if (i < nq) *reinterpret_cast<u32x4*>(qs + i * 4) = qv[u];
      }
      if (has_new) {
        // scores of the new key: q . k with k rounded to bf16 like its page copy
#pragma unroll
        for (int e = 0; e < DL; ++e) kn[e] = bf16_to_f(f_to_bf16(kn[e]));
        for (int h = 0; h < G; ++h) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < DL; ++e) t += qs[h * HD + lane + 64 * e] * kn[e];
          t = wave_sum(t);
          if (lane == 0) sm.ys[h * SP + kk_new] = t * a->attn_scale;   // its slot of the score row
        }
      }
    }
  }
  __syncthreads();
  MK_MARK(4);
  if (!sm.misc[0]) return false;
  // V of the new key (bf16-rounded) for the lanes' output dims, in flight
  // until after the P V pass
  float vnew[DTW];
#pragma unroll
  for (int j = 0; j < DTW; ++j) {
    const int dt = cw + MK_CW * j;
    vnew[j] = (has_new && cw >= 0 && dt < NDT)
                  ? bf16_to_f(f_to_bf16(ldc(qkv_b + (long)(a->Hq + Hkv + g) * HD + 16 * dt + c16)))
                  : 0.f;
  }
  float* sc = sm.ys;                                       // [G][SP] scores
  uint16_t* pbh = reinterpret_cast<uint16_t*>(sm.red);     // [G][SP] p, bf16 high part
  uint16_t* pbl = pbh + G * SP;                            // [G][SP] p, bf16 remainder
  // pass 1: scores of this wave's key tiles
  if (cw >= 0) {
    u32x4 qh[KS], ql[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (c16 < G) {
        const f32x4* qp = reinterpret_cast<const f32x4*>(qs + c16 * HD + 32 * k + 8 * q4);
        const f32x4 x0 = qp[0], x1 = qp[1];
        uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
        split_bf16(x0.x, x0.y, h0, l0);
        split_bf16(x0.z, x0.w, h1, l1);
        split_bf16(x1.x, x1.y, h2, l2);
        split_bf16(x1.z, x1.w, h3, l3);
        qh[k] = (u32x4){h0, h1, h2, h3};
        ql[k] = (u32x4){l0, l1, l2, l3};
      } else {
        qh[k] = (u32x4){0u, 0u, 0u, 0u};
        ql[k] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
    for (int i0 = 0; i0 < nti; i0 += ATT_PT) {
#pragma unroll
      for (int u = 0; u < ATT_PT; ++u) {
        const int i = i0 + u;
        const int t = cw + MK_CW * i;
        const int kk = 16 * t + c16, kabs = tb0 + kk;
        f32x4 c = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          c = mfma_bf16(qh[k], kf[u][k], c);
          c = mfma_bf16(ql[k], kf[u][k], c);
        }
        const bool valid = kabs >= p0 && kabs < p1;
        const bool mine = i < nti && !(has_new && kk == kk_new);   // the new key's score comes from wave 0
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 4 * q4 + r;
          if (h < G && mine) sc[h * SP + kk] = valid ? c[r] * a->attn_scale : -INFINITY;
        }
        const int o = i + ATT_PT < nti ? k_off(t + MK_CW * ATT_PT) : 0;
#pragma unroll
        for (int k = 0; k < KS; ++k) kf[u][k] = ldg_nt(Kp + o + 512 * k);
      }
    }
  }
  __syncthreads();
  if (a->trace && tid == 0 && sm.t_mark[0] == 0) sm.t_mark[0] = wall_clock64();
  // pass 2: per-head max, exponentials (as bf16 for the PV product) and sum
  float* ml = a->part_ml + ((((long)(l & 1) * a->B + b) * a->Hq + g * G) * a->max_splits) * 2;
  // Each wave takes two heads at once (h and h + 4) and four keys per lane
  // per pass, so the LDS reads of a pass are issued together; p = 2^((s - m)
  // log2 e) on the hardware exp2.  The new key's p is kept in fp32 for its
  // own P V term and zeroed in the MFMA operands.
  const int nk = 16 * nt, nk2 = 32 * nks;
  constexpr float L2E = 1.4426950408889634f;
  for (int h0 = wave; h0 < G; h0 += 2 * MK_WAVES) {
    const int h1 = h0 + MK_WAVES;
    const bool two = h1 < G;
    const int hb = two ? h1 : h0;
    float m0 = -INFINITY, m1 = -INFINITY;
    for (int base = 0; base < nk; base += 256) {
      float v0[4], v1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = base + lane + 64 * u;
        v0[u] = kk < nk ? sc[h0 * SP + kk] : -INFINITY;
        v1[u] = kk < nk ? sc[hb * SP + kk] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        m0 = fmaxf(m0, v0[u]);
        m1 = fmaxf(m1, v1[u]);
      }
    }
    m0 = wave_max(m0);
    m1 = wave_max(m1);
    float s0 = 0.f, s1 = 0.f;
    for (int base = 0; base < nk2; base += 256) {
      float v0[4], v1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = base + lane + 64 * u;
        v0[u] = kk < nk ? sc[h0 * SP + kk] : -INFINITY;
        v1[u] = kk < nk ? sc[hb * SP + kk] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = base + lane + 64 * u;
        if (kk < nk2) {
          const bool isnew = has_new && kk == kk_new;
          const float pa = __builtin_amdgcn_exp2f((v0[u] - m0) * L2E);
          const float pb = __builtin_amdgcn_exp2f((v1[u] - m1) * L2E);
          const uint16_t ha = f_to_bf16(pa), hbv = f_to_bf16(pb);
          const uint16_t la = f_to_bf16(pa - bf16_to_f(ha)), lb = f_to_bf16(pb - bf16_to_f(hbv));
          pbh[h0 * SP + kk] = isnew ? (uint16_t)0 : ha;
          pbl[h0 * SP + kk] = isnew ? (uint16_t)0 : la;
          if (two) {
            pbh[h1 * SP + kk] = isnew ? (uint16_t)0 : hbv;
            pbl[h1 * SP + kk] = isnew ? (uint16_t)0 : lb;
          }
          if (isnew) {
            fresh[8 + h0] = pa;
            if (two) fresh[8 + h1] = pb;
          }
          s0 += pa;
          s1 += pb;
        }
      }
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if (lane == 0) {
      stc(ml + ((long)h0 * a->max_splits + s) * 2 + 0, m0);
      stc(ml + ((long)h0 * a->max_splits + s) * 2 + 1, s0);
      if (two) {
        stc(ml + ((long)h1 * a->max_splits + s) * 2 + 0, m1);
        stc(ml + ((long)h1 * a->max_splits + s) * 2 + 1, s1);
      }
    }
  }
  __syncthreads();
  MK_MARK(6);
  // pass 3: o = P V over this wave's dim tiles
  float* po = a->part_o + ((((long)(l & 1) * a->B + b) * a->Hq + g * G) * a->max_splits) * HD;
  if (cw >= 0) {
    f32x4 o[DTW];
#pragma unroll
    for (int j = 0; j < DTW; ++j) o[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int ks0 = 0; ks0 < nks; ks0 += ATT_PV) {
#pragma unroll
      for (int u = 0; u < ATT_PV; ++u) {
        const int ks = ks0 + u;
        // keys outside [p0, p1), the new key and k-steps past the split have
        // p = 0 here; their V values are finite pool contents (earlier keys
        // of the sequence, an older value of the slot, or the initialised
        // pool).  A dim tile past the head (the last wave's third) is
        // computed on such values and never stored.
        const int po_ = c16 * SP + 32 * ks + 8 * q4;
        const bool pk = ks < nks && c16 < G;
        const u32x4 ph = pk ? *reinterpret_cast<const u32x4*>(pbh + po_) : (u32x4){0u, 0u, 0u, 0u};
        const u32x4 pl = pk ? *reinterpret_cast<const u32x4*>(pbl + po_) : (u32x4){0u, 0u, 0u, 0u};
        const int onext = ks + ATT_PV < nks ? v_off(ks + ATT_PV) : -1;
#pragma unroll
        for (int j = 0; j < DTW; ++j) {
          const int dt = cw + MK_CW * j;
          const u32x4 v = vf[u][j];
          o[j] = mfma_bf16(ph, v, o[j]);
          o[j] = mfma_bf16(pl, v, o[j]);
          vf[u][j] = ldg_nt(Vp + ((onext >= 0 && dt < NDT) ? onext + 256 * dt : 0));
        }
      }
    }
    if (a->trace && tid == 64 && sm.t_mark[1] == 0) sm.t_mark[1] = wall_clock64();
#pragma unroll
    for (int j = 0; j < DTW; ++j) {
      const int dt = cw + MK_CW * j;
      if (dt < NDT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = 4 * q4 + r;
          if (h < G) {
            const float ov = has_new ? o[j][r] + fresh[8 + h] * vnew[j] : o[j][r];
            stc(po + ((long)h * a->max_splits + s) * HD + 16 * dt + c16, ov);
          }
        }
      }
    }
  }
  MK_MARK(7);
  return true;
}

__device__ __forceinline__ bool attn_item(const KA a, Smem& sm, int l, int b, int g, int s, int ti, int wait_idx,
                          int wait_target) {
  const int sl = live_len(a, b);
  const int kv = visible_keys(a, l, sl);
  const int start = sl - kv;
  const int p0 = start + s * a->attn_split;
  const int p1 = min(p0 + a->attn_split, sl);
  if (a->hd == 128) return attn_split<128>(a, sm, l, b, g, s, p0, p1, ti, wait_idx, wait_target);
  return attn_split<64>(a, sm, l, b, g, s, p0, p1, ti, wait_idx, wait_target);
}

// ATTN_COMBINE for (sequence b, group g), heads c, c + nc, ... of the group
// (combiner c of nc): M = max_s m_s; o = sum_s e^(m_s - M) o_s / sum_s
// e^(m_s - M) l_s.  Thread (sg, cq) owns 4 dims (chunk cq) and the splits
// s = sg, sg + SG, ... (SG = 256 / (hd/4) split groups), so all threads load
// partials for one head and up to CB splits each cost one round trip.  The
// order of every sum is fixed by the head alone (split groups are added in
// order), so a head's result has the same bits whichever combiner and share
// count produced it.  Heads of the share are done one after another.
template <int HD>
__device__ __forceinline__ void attn_combine_hd(const KA a, Smem& sm, int l, int b, int g, int c, int nc) {
  const int G = a->G;
  constexpr int q4 = HD / 4;                // float4 chunks per head
  constexpr int SG = MK_THREADS / q4;       // split groups
  constexpr int CB = 16;                    // splits per thread per round trip
  const int ns = n_splits(a, l, b);
  const int tid = tid_v(), wave = tid >> 6, lane = tid & 63;
  float* out = a->attn + ((long)l * a->B + b) * a->Hq * HD;
  const long hstride = (long)a->max_splits;
  const float* ml0 = a->part_ml + ((((long)(l & 1) * a->B + b) * a->Hq + g * G) * hstride) * 2;
  const float* po0 = a->part_o + ((((long)(l & 1) * a->B + b) * a->Hq + g * G) * hstride) * HD;
  const int nh = (G - c + nc - 1) / nc;     // heads of this share
  const int sg = tid / q4, cq = tid - sg * q4;
  float* wts = sm.ys;                       // [nh][max_splits]
  float* den = sm.red;                      // [nh]
  f32x4* part = reinterpret_cast<f32x4*>(sm.red + 64);   // [SG][q4] partial numerators
  for (int hh = wave; hh < nh; hh += MK_WAVES) {
    const float* ml = ml0 + (long)(c + nc * hh) * hstride * 2;
    float m[16], lsum[16];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int sp = lane + 64 * u;
      m[u] = sp < ns ? ldc(ml + sp * 2) : -INFINITY;
      lsum[u] = sp < ns ? ldc(ml + sp * 2 + 1) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) mx = fmaxf(mx, m[u]);
    mx = wave_max(mx);
    float dsum = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int sp = lane + 64 * u;
      if (sp < ns) {
        const float w = expf(m[u] - mx);
        wts[hh * hstride + sp] = w;
        dsum += w * lsum[u];
      }
    }
    dsum = wave_sum(dsum);
    if (lane == 0) den[hh] = dsum;
  }
  __syncthreads();
  for (int hs = 0; hs < nh; ++hs) {
    const int h = c + nc * hs;
    const int obase = (int)((h * hstride * HD + cq * 4) * 4);   // byte offset of split 0
    f32x4 num = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += SG * CB) {
      f32x4 pv[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int sp = s0 + sg + SG * u;
        pv[u] = sp < ns ? as_f4(ldc16(po0, obase + sp * HD * 4)) : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int sp = s0 + sg + SG * u;
        if (sp < ns) num += wts[hs * hstride + sp] * pv[u];
      }
    }
    part[sg * q4 + cq] = num;
    __syncthreads();
    if (sg == 0) {
      f32x4 tot = part[cq];
#pragma unroll
      for (int k = 1; k < SG; ++k) tot += part[k * q4 + cq];
      const f32x4 r = ns > 0 ? tot / den[hs] : (f32x4){0.f, 0.f, 0.f, 0.f};
      stc16(out, ((g * G + h) * HD + cq * 4) * 4, as_u4(r));
    }
    __syncthreads();
  }
}
__device__ __forceinline__ void attn_combine(const KA a, Smem& sm, int l, int b, int g, int c, int nc) {
  if (a->hd == 128) attn_combine_hd<128>(a, sm, l, b, g, c, nc);
  else attn_combine_hd<64>(a, sm, l, b, g, c, nc);
}

// ATTN_COMBINE as its own task: waits for every split of (b, g), combines
// all its heads and adds the head count to COMB[g].
__device__ __forceinline__ bool op_attn_combine(const KA a, Smem& sm, const mk_task& t, int ti) {
  if (!wg_wait(a, sm, t.wait_ctr, n_splits(a, t.layer, t.batch), ti)) return false;
  attn_combine(a, sm, t.layer, t.batch, t.group, 0, 1);
  wg_signal(a, t.signal_ctr, a->G);
  return true;
}

// ------------------------------------------------------------------ kernel
// The persistent loop walks work units: a static task is one unit; a
// claimer task yields one unit per queue item it owns or claims.  Every GEMV
// opcode only fills a GemvArgs/StageArgs pair before the single GEMV site
// below and then runs its epilogue, so the whole step is one function with
// no calls (a call would save and restore ~100 callee-saved VGPRs per wave
// on every task).
enum { U_NONE = 0, U_GEMV = 1 };

__device__ __forceinline__ bool is_claimer(int op) {
  return op == MK_OP_ATTN_DRAIN || op == MK_OP_MOE_UPGATE_ACT_DRAIN || op == MK_OP_MOE_DOWN_DRAIN;
}

// One 16-byte piece (lane 0..7) of task descriptor k.
__device__ __forceinline__ u32x4 load_task_piece(const mk_task* tasks, int k, int lane) {
  return *((GLOBAL const u32x4*)(tasks + k) + lane);
}

// The whole step.  FP8E: the expert matrices are E4M3 codes with row scales.
// Instantiated as two kernels, so that the bf16 kernel carries no FP8 code:
// with both expert forms in the one function, register allocation over the
// whole step cost the bf16 step about 2% (345 against 352 tok/s at bs=1).
template <bool FP8E>
__device__ __forceinline__ void mk_step(mk_kargs a_arg, int final_launch) {
  __shared__ Smem sm;
  const int tid = tid_v();
  // this workgroup's tasks: [k, kend) of the grouped list
  const int kbeg = ((GLOBAL const int32_t*)a_arg.wg_range)[2 * blockIdx.x];
  const int kend = ((GLOBAL const int32_t*)a_arg.wg_range)[2 * blockIdx.x + 1];
  int k = kbeg;
  bool claiming = false, first = false, aborted = false;
  int preclaim = -1;   // a MoE queue position claimed when the claimer started
  int n_items = 0, qidx = -1, attn_wait = -1, ti = 0;
  uint64_t t_start = 0;
  mk_task t;
  // Descriptors go through LDS: lanes 0..7 of wave 1 load the next one while
  // the current task runs (wave 1 is a compute wave: its first weight load is
  // issued after this and waits longer anyway), and store it at the top of
  // the next pass of the loop.
  int cur = 0;
  bool pending = false;
  u32x4 pre = (u32x4){0u, 0u, 0u, 0u};
  if (tid >= 64 && tid < 72 && k < kend)
    reinterpret_cast<u32x4*>(&sm.tq[0])[tid - 64] = load_task_piece(a_arg.tasks, k, tid - 64);
  if (tid == 0) sm.seen_idx = -1;
  {   // step metadata into LDS (visible after the loop's first barrier);
      // eight loads per thread are in flight at once
    auto copy_in = [&](int* dst, GLOBAL const int* src, int n) {
      for (int i0 = 0; i0 < n; i0 += 8 * MK_THREADS) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[min(i0 + u * MK_THREADS + tid, n - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * MK_THREADS + tid < n) dst[i0 + u * MK_THREADS + tid] = v[u];
      }
    };
    copy_in(reinterpret_cast<int*>(sh_layers), (GLOBAL const int*)a_arg.layers,
            a_arg.L * (int)(sizeof(mk_layer_dev) / 4));
    const int nbt = a_arg.B * a_arg.max_blocks;
    if (nbt <= MK_LDS_BT) copy_in(sh_bt, (GLOBAL const int*)a_arg.block_tables, nbt);
    if (tid < a_arg.B) {
      sh_seq_lens[tid] = ((GLOBAL const int*)a_arg.seq_lens)[tid];
      sh_positions[tid] = ((GLOBAL const int*)a_arg.positions)[tid];
      sh_tokens[tid] = ((GLOBAL const int*)a_arg.tokens)[tid];
    }
    if (tid < a_arg.hd / 2) sh_invf[tid] = ((GLOBAL const double*)a_arg.inv_freq)[tid];
  }
  for (;;) {
    if (pending) {
      if (tid >= 64 && tid < 72) reinterpret_cast<u32x4*>(&sm.tq[cur ^ 1])[tid - 64] = pre;
      pending = false;
    }
    __syncthreads();
    const KA a = kargs();
    int item = -1;
    if (!claiming) {
      if (k >= kend) break;
      if (k > kbeg) cur ^= 1;
      {   // the descriptor is the same for every lane: keep it in scalar registers
        const int* src = reinterpret_cast<const int*>(&sm.tq[cur]);
        int* dst = reinterpret_cast<int*>(&t);
#pragma unroll
        for (int q = 0; q < 32; ++q) dst[q] = __builtin_amdgcn_readfirstlane(src[q]);
      }
      ti = t.aux[MK_AUX_INDEX];
      if (k + 1 < kend) {
        if (tid >= 64 && tid < 72) pre = load_task_piece(a->tasks, k + 1, tid - 64);
        pending = true;
      }
      ++k;
      if (a->trace && tid == 0) {
        t_start = wall_clock64();
        sm.t_ready = 0;
        for (int q = 0; q < 10; ++q) sm.t_mark[q] = 0;
        sm_t_signal = 0;
      }
      if (is_claimer(t.op)) {
        const int l = t.layer;
        preclaim = -1;
        if (aborted) {
          n_items = 0;
        } else if (t.op == MK_OP_ATTN_DRAIN) {
          n_items = 0;
          for (int b = 0; b < a->B; ++b) n_items += n_splits(a, l, b) * a->Hkv;
          qidx = layer_ctr(a, l, MK_CTR_QATTN);
          attn_wait = t.wait_ctr;       // waited for inside the first item
          if ((t.flags & MK_F_FUSE_COMBINE) && t.n0 == 0 && tid == 0) {
            // a sequence without keys (empty slot) has no split to combine it
            for (int b = 0; b < a->B; ++b)
              if (n_splits(a, l, b) == 0)
                for (int g = 0; g < a->Hkv; ++g)
                  __hip_atomic_fetch_add(ctrp(a, layer_ctr(a, l, a->cl.comb + g)), a->G, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          if (!wg_wait(a, sm, t.wait_ctr, t.wait_target, ti)) {
            aborted = true;
            n_items = 0;
          } else {
            // the item count and every active expert's record, into LDS once
            // for all the items this workgroup will take (red is free
            // during the MoE drains)
            const int32_t* meta = a->moe + (long)l * a->moe_stride;
            int* recs = reinterpret_cast<int*>(sm.red);
            const int nrec = min(a->bk, RED_FLOATS / 16) * 16;
            qidx = layer_ctr(a, l, t.op == MK_OP_MOE_UPGATE_ACT_DRAIN ? MK_CTR_QUG : MK_CTR_QDN);
            for (int i0 = 0; i0 < nrec; i0 += 4 * MK_THREADS) {   // four loads per thread in flight
              int v[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) v[u] = ldc(meta + 4 + a->bk + min(i0 + u * MK_THREADS + tid, nrec - 1));
#pragma unroll
              for (int u = 0; u < 4; ++u)
                if (i0 + u * MK_THREADS + tid < nrec) recs[i0 + u * MK_THREADS + tid] = v[u];
            }
            if (tid == 0) {
              sm.misc[2] = ldc(meta + (t.op == MK_OP_MOE_UPGATE_ACT_DRAIN ? 1 : 2));
              // a claimer with no item of its own claims its first queue
              // position now, in the same round trip as the records
              sm.misc[3] = t.n0 == INT32_MAX
                               ? __hip_atomic_fetch_add(ctrp(a, qidx), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : -1;
            }
            __syncthreads();
            n_items = __builtin_amdgcn_readfirstlane(sm.misc[2]);
            preclaim = __builtin_amdgcn_readfirstlane(sm.misc[3]);
          }
          qidx = layer_ctr(a, l, t.op == MK_OP_MOE_UPGATE_ACT_DRAIN ? MK_CTR_QUG : MK_CTR_QDN);
        }
        claiming = true;
        first = true;
      }
    }
    if (claiming) {
      item = next_item(a, sm, t, n_items, qidx, first, preclaim);
      if (item < 0) {
        claiming = false;
        wg_signal(a, aborted ? -1 : t.signal_ctr, 1);
        goto task_done;
      }
    }
    if (aborted) goto unit_done;
    {
      const int l = t.layer, B = a->B;
      GemvArgs g;
      StageArgs st;
      int kind = U_NONE;
      int epi_ae = 0, epi_r0 = 0, epi_nr = 0, epi_p0 = 0, epi_np = 0;
      const float* fp8_scale = nullptr;   // FP8 expert tile: its row scales
      g.mode = ROW_PLAIN; g.half = 0; g.hd = a->hd; g.nb = B; g.out = nullptr; g.ob = 0;
      g.r0 = t.n0; g.nrows = t.n1 - t.n0;
      st.use_tok = false; st.nb = B; st.wait_idx = t.wait_ctr; st.wait_target = t.wait_target;
      st.task = ti;
      switch (t.op) {
        case MK_OP_QKV_PROJ:
          kind = U_GEMV;
          g.base = LAYER_PTR(l, w_qkv); g.ldw = a->d; g.K = a->d; g.nrows = 2 * (t.n1 - t.n0);
          g.mode = ROW_ROPE_PAIRS; g.half = a->hd / 2;
          st.base = a->xn + (long)l * B * a->d; st.ld = a->d; st.K = a->d;
          break;
        case MK_OP_ROUTER_GEMM:
          kind = U_GEMV;
          g.base = LAYER_PTR(l, w_router); g.ldw = a->d; g.K = a->d;
          g.out = a->rlog + (long)l * B * a->E + t.n0; g.ob = a->E;
          st.base = a->xn + (long)l * B * a->d; st.ld = a->d; st.K = a->d;
          break;
        case MK_OP_O_PROJ: {
          kind = U_GEMV;
          const int gd = a->G * a->hd, grp = t.group;
          g.base = LAYER_PTR(l, w_o) + (long)grp * gd; g.ldw = (long)a->Hq * a->hd; g.K = gd;
          g.out = a->opart + (((long)l * a->Hkv + grp) * B) * a->d + t.n0; g.ob = a->d;
          st.base = a->attn + (long)l * B * a->Hq * a->hd + (long)grp * gd; st.ld = (long)a->Hq * a->hd; st.K = gd;
          break;
        }
        case MK_OP_FFN_UPGATE_ACT:
          kind = U_GEMV;
          g.base = LAYER_PTR(l, w_upgate); g.ldw = a->d; g.K = a->d; g.nrows = 2 * (t.n1 - t.n0);
          g.mode = ROW_GATE_UP; g.half = a->F;
          st.base = (a->parallel ? a->xn : a->xn2) + (long)l * B * a->d; st.ld = a->d; st.K = a->d;
          epi_p0 = t.n0; epi_np = t.n1 - t.n0;
          break;
        case MK_OP_FFN_DOWN:
          kind = U_GEMV;
          g.base = LAYER_PTR(l, w_down); g.ldw = a->F; g.K = a->F;
          g.out = a->fo + (long)l * B * a->d + t.n0; g.ob = a->d;
          st.base = a->fh + (long)l * B * a->F; st.ld = a->F; st.K = a->F;
          break;
        case MK_OP_LM_HEAD:
          // the tile's logits land in LDS for the epilogue (logits out and
          // the tile's sampling candidates)
          kind = U_GEMV;
          g.base = a->lm_head; g.ldw = a->d; g.K = a->d;
          st.base = a->xn + (long)a->L * B * a->d; st.ld = a->d; st.K = a->d;
          break;
        case MK_OP_MOE_UPGATE_ACT_DRAIN: {
          // item = (active expert, tile of ug_pairs gate/up pairs) over that expert's rows
          kind = U_GEMV;
          epi_ae = item / a->ug_tiles;
          const int tt = item - epi_ae * a->ug_tiles;
          const u32x4* rec = reinterpret_cast<const u32x4*>(sm.red) + epi_ae * 4;   // this expert's record
          const u32x4 r0v = rec[0], r1v = rec[1], r2v = rec[2];
          const int e = __builtin_amdgcn_readfirstlane((int)r0v.x);
          epi_r0 = __builtin_amdgcn_readfirstlane((int)r0v.y);
          epi_nr = __builtin_amdgcn_readfirstlane((int)r0v.z);
          st.use_tok = true;
          st.tok[0] = __builtin_amdgcn_readfirstlane((int)r1v.x);
          st.tok[1] = __builtin_amdgcn_readfirstlane((int)r1v.y);
          st.tok[2] = __builtin_amdgcn_readfirstlane((int)r1v.z);
          st.tok[3] = __builtin_amdgcn_readfirstlane((int)r1v.w);
          st.tok[4] = __builtin_amdgcn_readfirstlane((int)r2v.x);
          st.tok[5] = __builtin_amdgcn_readfirstlane((int)r2v.y);
          st.tok[6] = __builtin_amdgcn_readfirstlane((int)r2v.z);
          st.tok[7] = __builtin_amdgcn_readfirstlane((int)r2v.w);
          epi_p0 = tt * a->ug_pairs;
          epi_np = min(a->ug_pairs, a->I - epi_p0);
          if (FP8E) {   // one byte per weight: the row pitch in 16-bit units is d / 2
            g.base = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(LAYER_PTR(l, w_upgate)) +
                                                       (long)e * 2 * a->I * a->d);
            g.ldw = a->d / 2;
            fp8_scale = LAYER_PTR(l, upgate_scale) + (long)e * 2 * a->I;
          } else {
            g.base = LAYER_PTR(l, w_upgate) + (long)e * 2 * a->I * a->d; g.ldw = a->d;
          }
          g.r0 = epi_p0;
          g.nrows = 2 * epi_np; g.K = a->d; g.mode = ROW_GATE_UP; g.half = a->I; g.nb = epi_nr;
          st.base = a->xn + (long)l * B * a->d; st.ld = a->d; st.nb = epi_nr;
          st.K = a->d; st.wait_idx = -1;
          break;
        }
        case MK_OP_MOE_DOWN_DRAIN: {
          // item = (active expert, tile of dn_rows output rows); waits on the
          // expert's up-gate tiles after its weights are in flight
          kind = U_GEMV;
          const int ae = item / a->dn_tiles, tt = item - ae * a->dn_tiles;
          const u32x4 r0v = reinterpret_cast<const u32x4*>(sm.red)[ae * 4];   // this expert's record
          const int e = __builtin_amdgcn_readfirstlane((int)r0v.x);
          const int r0 = __builtin_amdgcn_readfirstlane((int)r0v.y);
          const int nr = __builtin_amdgcn_readfirstlane((int)r0v.z);
          const int n0 = tt * a->dn_rows;
          if (FP8E) {
            g.base = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(LAYER_PTR(l, w_down)) +
                                                       (long)e * a->d * a->I);
            g.ldw = a->I / 2;
            fp8_scale = LAYER_PTR(l, down_scale) + (long)e * a->d;
          } else {
            g.base = LAYER_PTR(l, w_down) + (long)e * a->d * a->I; g.ldw = a->I;
          }
          g.r0 = n0;
          g.nrows = min(a->dn_rows, a->d - n0); g.K = a->I; g.nb = nr;
          g.out = a->Y + ((long)l * a->bk + r0) * a->d + n0; g.ob = a->d;
          st.base = a->H + ((long)l * a->bk + r0) * a->I; st.ld = a->I; st.nb = nr; st.K = a->I;
          st.wait_idx = layer_ctr(a, l, a->cl.ug + ae); st.wait_target = a->ug_tiles;
          break;
        }
        default:
          break;
      }
      if (kind == U_GEMV) {
        if (!((FP8E && fp8_scale) ? gemv_fp8(a, sm, g, st, fp8_scale) : gemv(a, sm, g, st))) {
          aborted = true;
          goto unit_done;
        }
        switch (t.op) {
          case MK_OP_QKV_PROJ:
            __syncthreads();
            epi_qkv(a, sm, t, ti);
            if (a->trace && tid_v() == 64) sm.t_mark[5] = wall_clock64();
            wg_signal(a, t.signal_ctr, 1);
            break;
          case MK_OP_FFN_UPGATE_ACT:
            __syncthreads();
            epi_swiglu(sm, epi_np, B, a->fh + (long)l * B * a->F + epi_p0, a->F);
            wg_signal(a, t.signal_ctr, 1);
            break;
          case MK_OP_MOE_UPGATE_ACT_DRAIN:
            __syncthreads();
            epi_swiglu(sm, epi_np, epi_nr, a->H + ((long)l * a->bk + epi_r0) * a->I + epi_p0, a->I);
            wg_signal(a, layer_ctr(a, l, a->cl.ug + epi_ae), 1);
            break;
          case MK_OP_MOE_DOWN_DRAIN:
            break;   // the claimer signals once its queue is drained
          case MK_OP_LM_HEAD:
            __syncthreads();
            epi_lm_head(a, sm, t);
            break;
          case MK_OP_ROUTER_GEMM:
            if (t.flags & MK_F_FUSE_TOPK) {
              // the last router tile to finish runs top-k and ROUTE_FINALIZE
              stores_done();
              __syncthreads();
              if (tid == 0)
                sm.misc[3] = __hip_atomic_fetch_add(ctrp(a, t.signal_ctr), 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT) == t.aux[0] - 1;
              __syncthreads();
              if (sm.misc[3]) {
                router_topk(a, sm, l);
                route_finalize(a, sm, l);
                wg_signal(a, layer_ctr(a, l, MK_CTR_ROUTE), 1);
              }
            } else {
              wg_signal(a, t.signal_ctr, 1);
            }
            break;
          default:
            wg_signal(a, t.signal_ctr, 1);
            break;
        }
        goto unit_done;
      }
      switch (t.op) {
        case MK_OP_ADD_RMSNORM:
          if (!(a->d <= 2 * 4 * MK_THREADS ? op_add_rmsnorm<2>(a, sm, t, ti) : op_add_rmsnorm<4>(a, sm, t, ti)))
            aborted = true;
          break;
        case MK_OP_ROUTER_TOPK:
          if (wg_wait(a, sm, t.wait_ctr, t.wait_target, ti)) {
            router_topk(a, sm, l);
            if (t.flags & MK_F_FUSE_FINALIZE) route_finalize(a, sm, l);
            wg_signal(a, t.signal_ctr, 1);
          } else {
            aborted = true;
          }
          break;
        case MK_OP_ROUTE_FINALIZE:
          if (wg_wait(a, sm, t.wait_ctr, t.wait_target, ti)) {
            for (int i = tid; i < B * a->topk; i += MK_THREADS) {
              const int b = i / a->topk;
              sm.misc[64 + i] = sh_seq_lens[b] > 0 ? ldc(a->topi + ((long)l * B) * a->topk + i) : -1;
            }
            __syncthreads();
            route_finalize(a, sm, l);
            wg_signal(a, t.signal_ctr, 1);
          } else {
            aborted = true;
          }
          break;
        case MK_OP_ATTN_DRAIN: {
          int it = item, b = 0, gq = 0, sp = -1;
          for (; b < B; ++b) {
            const int ns = n_splits(a, l, b);
            const int cnt = ns * a->Hkv;
            if (it < cnt) { gq = it / ns; sp = it - gq * ns; break; }
            it -= cnt;
          }
          if (sp >= 0) {
            if (!attn_item(a, sm, l, b, gq, sp, ti, attn_wait, t.wait_target)) {
              aborted = true;
              break;
            }
            attn_wait = -1;   // satisfied for every later item
            const int actr = layer_ctr(a, l, a->cl.attn + b * a->Hkv + gq);
            if (t.flags & MK_F_FUSE_COMBINE) {
              // the last nc splits of (b, gq) to finish combine them, one
              // share of the heads each: those that finish early wait for
              // the rest (at most ncomb - 1 per (b, g), fewer than the
              // workgroups, so some workgroup is always free to claim)
              stores_done();
              __syncthreads();
              if (tid == 0)
                sm.misc[3] = __hip_atomic_fetch_add(ctrp(a, actr), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __syncthreads();
              const int ns = n_splits(a, l, b);
              const int nc = min(ns, a->ncomb);
              const int rank = __builtin_amdgcn_readfirstlane(sm.misc[3]);
              if (rank >= ns - nc) {
                const int cb = rank - (ns - nc);
                if (rank < ns - 1 && !wg_wait(a, sm, actr, ns, ti)) {
                  aborted = true;
                  break;
                }
                attn_combine(a, sm, l, b, gq, cb, nc);
                wg_signal(a, layer_ctr(a, l, a->cl.comb + gq), (a->G - cb + nc - 1) / nc);
              }
            } else {
              wg_signal(a, actr, 1);
            }
          }
          break;
        }
        case MK_OP_ATTN_DECODE:
          // a static split: one (sequence, group, split) of the longest
          // context; one past the live length has nothing to do and
          // signals nothing (the combine waits for the live splits only)
          if (t.split < n_splits(a, l, t.batch)) {
            if (!attn_item(a, sm, l, t.batch, t.group, t.split, ti, t.wait_ctr, t.wait_target)) {
              aborted = true;
              break;
            }
            wg_signal(a, t.signal_ctr, 1);
          }
          break;
        case MK_OP_ATTN_COMBINE:
          if (!op_attn_combine(a, sm, t, ti)) aborted = true;
          break;
        default:
          if (tid == 0) report(a, MK_E_INVAL, ti, -4, t.op, MK_NUM_OPCODES);
          break;
      }
    }
  unit_done:
    if (claiming) continue;
  task_done:
    if (a->trace && tid == 0) {
      GLOBAL uint64_t* tr = (GLOBAL uint64_t*)(a->trace + (long)ti * 16);
      tr[0] = t_start;
      tr[1] = sm.t_ready ? sm.t_ready : t_start;
      if (sm_t_signal) sm.t_mark[2] = sm_t_signal;
      for (int q = 0; q < 10; ++q) tr[2 + q] = sm.t_mark[q];
      tr[12] = wall_clock64();
      tr[13] = blockIdx.x;
      tr[14] = t.op;
      tr[15] = 0;
    }
  }
  // The last workgroup out clears the counters for the next launch.
  __syncthreads();
  const KA a = kargs();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(ctrp(a, MK_CG_DONE), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.misc[2] = (old == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (sm.misc[2]) {
    if (final_launch) {
      for (int i = tid; i < a->n_ctr; i += MK_THREADS) stc(ctrp(a, i), 0);
      // every workgroup has read the step inputs by now: advance the slots
      if (a->next_tok && a->advance && tid < a->B) {
        const int nt = ldc(a->next_tok + tid);
        if (sh_seq_lens[tid] > 0 && nt >= 0) {
          stc(const_cast<int32_t*>(a->tokens) + tid, nt);
          stc(const_cast<int32_t*>(a->positions) + tid, sh_positions[tid] + 1);
          stc(const_cast<int32_t*>(a->seq_lens) + tid, sh_seq_lens[tid] + 1);
        }
      }
    } else if (tid == 0) {
      stc(ctrp(a, MK_CG_DONE), 0);
    }
  }
}

extern "C" __global__ void __launch_bounds__(MK_THREADS, 1) mk_persistent(mk_kargs a_arg, int final_launch) {
  mk_step<false>(a_arg, final_launch);
}
extern "C" __global__ void __launch_bounds__(MK_THREADS, 1) mk_persistent_fp8(mk_kargs a_arg, int final_launch) {
  mk_step<true>(a_arg, final_launch);
}

// ------------------------------------------------------- per-device scratch
// The workspace of the handle made by mk_init_noalloc: a file-scope device
// array, of which every device the library runs on holds its own copy until
// the process ends.  On the host the array's name stands for a host-side
// placeholder, not device memory, so host code never passes it: the array's
// address on each device is looked up once, with that device current, and
// kept; every later use (kernel arguments, clears, copies) goes through that
// address.
static __device__ __align__(256) char scratch[MK_NOALLOC_WS_BYTES];

namespace {
constexpr int kScratchDevices = 16;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

extern "C" int mk_scratch_region(void** ptr, size_t* bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MK_E_HIP;
  if (dev < 0 || dev >= kScratchDevices) return MK_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MK_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = MK_NOALLOC_WS_BYTES;
  return MK_OK;
}

// ------------------------------------------------------------------ launch
extern "C" int mk_launch(const mk_kargs* args, int launch_mode, const int32_t* wg_ranges, int n_waves,
                         void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  mk_kargs k = *args;
  const dim3 grid((unsigned)k.n_wg), block(MK_THREADS);
  const void* kernel = k.expert_fp8 ? reinterpret_cast<const void*>(mk_persistent_fp8)
                                    : reinterpret_cast<const void*>(mk_persistent);
  if (launch_mode == MK_LAUNCH_PERSISTENT) {
    k.wg_range = wg_ranges;
    int fin = 1;
    void* kp[] = {&k, &fin};
    hipError_t e = hipLaunchCooperativeKernel(kernel, grid, block, kp, 0, st);
    return e == hipSuccess ? MK_OK : MK_E_HIP;
  }
  // ablation: one launch per task wave; the kernel boundary orders the waves
  for (int w = 0; w < n_waves; ++w) {
    k.wg_range = wg_ranges + (size_t)(1 + w) * k.n_wg * 2;
    int fin = (w == n_waves - 1) ? 1 : 0;
    void* kp[] = {&k, &fin};
    hipError_t e = hipLaunchKernel(kernel, grid, block, kp, 0, st);
    if (e != hipSuccess) return MK_E_HIP;
  }
  return MK_OK;
}
