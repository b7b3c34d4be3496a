"""GPU harness: seeded inputs in HBM and decode steps through libmk.so.

PyTorch is used for device memory, the input generator and streams only;
every step of the decode path runs in the HIP library (``mk_decode_step``).
The harness owns the continuous-batching bookkeeping of the caller side:
positions, sequence lengths, block tables, and refilling a slot with a new
sequence (its pre-filled KV written into its pages) when the workload swaps
one in.
"""
from __future__ import annotations

import ctypes
import time
from typing import Dict, List, Optional

import numpy as np
import torch

from . import mk
from . import workloads as W


def _log(verbose, *a):
    if verbose:
        print("[runner]", *a, flush=True)


class DecodeEngine:
    """Weights, KV pool, workspace and the library handle for one workload."""

    def __init__(self, wl: W.Workload, device: str = "cuda", steps: Optional[int] = None,
                 opts: Optional[mk.mk_sched_opts] = None, verbose: bool = False, page_slack: int = 0):
        if not torch.cuda.is_available():
            raise RuntimeError("DecodeEngine needs a GPU")
        mk.load()  # fail loudly before allocating anything
        self.wl = wl
        self.cfg = wl.model
        self.dev = torch.device(device)
        self.steps = wl.steps if steps is None else steps
        self.verbose = verbose
        cfg, B = self.cfg, wl.batch
        self.plan = W.plan_batch(wl.with_(page_slack=page_slack), self.steps)
        self.pages = W.page_table(self.plan, self.steps)
        self.max_blocks = self.plan.max_blocks
        t0 = time.time()
        self._gen_weights()
        torch.cuda.synchronize()
        _log(verbose, "weights %.1f GB in %.1fs" % (self.weight_bytes() / 1e9, time.time() - t0))
        t0 = time.time()
        # K pages hold 32-dim slices of every key in turn, V pages one head
        # dimension per row
        kshape = (self.plan.num_pages, cfg.n_kv_heads, cfg.head_dim // 32, cfg.page_size, 32)
        vshape = (self.plan.num_pages, cfg.n_kv_heads, cfg.head_dim, cfg.page_size)
        self.kpool = [torch.zeros(kshape, dtype=torch.bfloat16, device=self.dev) for _ in range(cfg.n_layers)]
        self.vpool = [torch.zeros(vshape, dtype=torch.bfloat16, device=self.dev) for _ in range(cfg.n_layers)]
        # slot state
        self.slot_seq: List[W.SequenceSlot] = []
        self.slot_len: List[int] = []
        self.slot_tok: List[int] = []
        for b in range(B):
            _, seq = self.plan.slots[b][0]
            self._admit(b, seq, first=True)
        torch.cuda.synchronize()
        _log(verbose, "kv prefill in %.1fs" % (time.time() - t0))
        self.block_tables = torch.zeros((B, self.max_blocks), dtype=torch.int32, device=self.dev)
        self._refresh_block_tables()
        self.logits = torch.zeros((B, cfg.vocab), dtype=torch.float32, device=self.dev)
        # library state
        self.mkcfg = mk.make_config(cfg, B)
        ws = mk.mk_workspace_size(self.mkcfg, self.max_blocks)
        if ws == 0:
            raise mk.MkError(mk.MK_E_INVAL, "mk_workspace_size")
        self.workspace = torch.empty(ws + 256, dtype=torch.uint8, device=self.dev)
        base = self.workspace.data_ptr()
        self.ws_off = (-base) % 256
        self.ws_ptr = base + self.ws_off
        self.ws_bytes = ws
        self._make_tables()
        self.h = mk.mk_init(self.mkcfg, self._w, self._kv, self.ws_ptr, ws, self.max_blocks)
        self.opts = opts if opts is not None else mk.make_opts()
        mk.mk_build_schedule(self.h, B, self.opts)
        self.step_index = 0

    # ------------------------------------------------------------ inputs
    def _gen_weights(self):
        cfg, seed, dev = self.cfg, self.wl.seed, self.dev
        d, V = cfg.d_model, cfg.vocab

        def gen(name, shape, layer=-1):
            t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
            mean, std = W.tensor_dist(name)
            return W.fill_normal_(t, W.tensor_key(seed, name, layer), mean, std)

        self.embed = gen("embed", (V, d))
        self.lm_head = self.embed if cfg.tied_embeddings else gen("lm_head", (V, d))
        self.final_norm = gen("final_norm", (d,))
        shapes = W.weight_shapes(cfg)
        self.layers: List[Dict[str, torch.Tensor]] = []
        for l in range(cfg.n_layers):
            lw = {}
            for name, shp in shapes.items():
                if cfg.is_moe and name in ("w_upgate", "w_down"):
                    t = torch.empty((cfg.n_experts,) + shp, dtype=torch.bfloat16, device=dev)
                    keys = [W.tensor_key(seed, name, l, e) for e in range(cfg.n_experts)]
                    mean, std = W.tensor_dist(name)
                    W.fill_normal_keyed_(t, keys, mean, std)
                    if cfg.expert_fp8:   # E4M3 codes and per-row scales; the bf16 values are dropped
                        lw[name], lw[name + "_scale"] = W.quantize_e4m3_rows(t)
                        del t
                    else:
                        lw[name] = t
                else:
                    lw[name] = gen(name, shp, l)
            rb = W.router_bias(seed, cfg, l)
            if rb is not None:
                lw["router_bias"] = rb.to(dev)
            self.layers.append(lw)
            if self.verbose and (l % 8 == 7 or l == cfg.n_layers - 1):
                torch.cuda.synchronize()
                _log(True, "generated layer", l)

    def router_bias_f64(self, layer: int):
        """Layer ``layer``'s router bias as float64 values (or None)."""
        lw = self.layers[layer]
        return lw["router_bias"].float().cpu().numpy().astype(np.float64) if "router_bias" in lw else None

    def weight_bytes(self) -> int:
        ts = [self.embed, self.final_norm] + ([] if self.cfg.tied_embeddings else [self.lm_head])
        for lw in self.layers:
            ts += list(lw.values())
        return sum(t.numel() * t.element_size() for t in ts)

    def _admit(self, b: int, seq: W.SequenceSlot, first: bool = False):
        """Put ``seq`` into slot b: write its pre-filled KV into its pages."""
        cfg = self.cfg
        pages = torch.as_tensor(self.pages[seq.seq_id], dtype=torch.long, device=self.dev)
        ps = cfg.page_size
        n_full = -(-seq.ctx // ps)
        for l in range(cfg.n_layers):
            for which, pool in (("k", self.kpool[l]), ("v", self.vpool[l])):
                if seq.ctx == 0:
                    continue
                kv = W.gen_kv(self.wl.seed, cfg, seq.seq_id, l, which, 0, seq.ctx, device=self.dev)
                pad = n_full * ps - seq.ctx
                if pad:
                    kv = torch.cat([kv, torch.zeros((pad,) + kv.shape[1:], dtype=kv.dtype, device=self.dev)])
                kv = kv.view(n_full, ps, cfg.n_kv_heads, cfg.head_dim)
                if which == "k":   # [page][head][slice][key][32]
                    kv = kv.view(n_full, ps, cfg.n_kv_heads, cfg.head_dim // 32, 32).permute(0, 2, 3, 1, 4)
                else:              # [page][head][dim][key]
                    kv = kv.permute(0, 2, 3, 1)
                pool[pages[:n_full]] = kv
        if first:
            self.slot_seq.append(seq)
            self.slot_len.append(seq.ctx)
            self.slot_tok.append(seq.token)
        else:
            self.slot_seq[b] = seq
            self.slot_len[b] = seq.ctx
            self.slot_tok[b] = seq.token

    def _refresh_block_tables(self):
        bt = np.zeros((self.wl.batch, self.max_blocks), dtype=np.int32)
        for b, seq in enumerate(self.slot_seq):
            pg = self.pages[seq.seq_id]
            bt[b, :len(pg)] = pg
        self.block_tables.copy_(torch.from_numpy(bt))

    def _make_tables(self):
        cfg = self.cfg
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
        arr = (mk.mk_layer_weights * cfg.n_layers)()
        for l, lw in enumerate(self.layers):
            arr[l].attn_norm = lw["attn_norm"].data_ptr()
            arr[l].ffn_norm = lw["ffn_norm"].data_ptr() if "ffn_norm" in lw else None
            arr[l].w_qkv = lw["w_qkv"].data_ptr()
            arr[l].w_o = lw["w_o"].data_ptr()
            arr[l].w_router = lw["w_router"].data_ptr() if "w_router" in lw else None
            arr[l].w_upgate = lw["w_upgate"].data_ptr()
            arr[l].w_down = lw["w_down"].data_ptr()
            arr[l].router_bias = lw["router_bias"].data_ptr() if "router_bias" in lw else None
            arr[l].upgate_scale = lw["w_upgate_scale"].data_ptr() if "w_upgate_scale" in lw else None
            arr[l].down_scale = lw["w_down_scale"].data_ptr() if "w_down_scale" in lw else None
        self._layer_arr = arr
        self._w = mk.mk_weights(embed=self.embed.data_ptr(), lm_head=self.lm_head.data_ptr(),
                                final_norm=self.final_norm.data_ptr(), layers=arr)
        kp = (ctypes.c_void_p * cfg.n_layers)(*[t.data_ptr() for t in self.kpool])
        vp = (ctypes.c_void_p * cfg.n_layers)(*[t.data_ptr() for t in self.vpool])
        self._kp, self._vp = kp, vp
        self._kv = mk.mk_kv_pool(k=kp, v=vp, num_pages=self.plan.num_pages)

    # ------------------------------------------------------------ stepping
    def apply_swaps(self, step: int) -> List[int]:
        """Refill slots whose sequence changes at ``step``; returns those slots."""
        changed = []
        for b in range(self.wl.batch):
            for first, seq in self.plan.slots[b][1:]:
                if first == step:
                    self._admit(b, seq)
                    changed.append(b)
        if changed:
            self._refresh_block_tables()
        return changed

    def step_inputs(self, tokens: Optional[List[int]] = None):
        B = self.wl.batch
        toks = self.slot_tok if tokens is None else tokens
        t = torch.tensor(toks, dtype=torch.int32, device=self.dev)
        pos = torch.tensor(self.slot_len, dtype=torch.int32, device=self.dev)
        sl = torch.tensor([n + 1 for n in self.slot_len], dtype=torch.int32, device=self.dev)
        return t, pos, sl

    def decode(self, tokens: Optional[List[int]] = None, stream=None, inputs=None) -> torch.Tensor:
        """One decode step; returns the [B, V] logits (device).  Advances the
        slots by one token; the next fed token defaults to the argmax."""
        t, pos, sl = inputs if inputs is not None else self.step_inputs(tokens)
        s = stream if stream is not None else torch.cuda.current_stream()
        mk.mk_decode_step(self.h, t.data_ptr(), pos.data_ptr(), self.block_tables.data_ptr(), sl.data_ptr(),
                          self.logits.data_ptr(), s.cuda_stream)
        self._inputs_keepalive = (t, pos, sl)
        return self.logits

    def advance(self, next_tokens: List[int]):
        for b in range(self.wl.batch):
            self.slot_len[b] += 1
            self.slot_tok[b] = int(next_tokens[b])
        self.step_index += 1

    def status(self) -> mk.mk_status:
        return mk.mk_get_status(self.h)

    def tap(self, name: str) -> torch.Tensor:
        """A per-layer debug tap of the last step, viewed in the workspace."""
        off, nb = mk.mk_tap_offset(self.h, name)
        raw = self.workspace[self.ws_off + off:self.ws_off + off + nb]
        dt = {"topk_ids": torch.int32, "trace": torch.int64}.get(name, torch.float32)
        return raw.view(dt)

    def close(self):
        if getattr(self, "h", None) is not None:
            mk.mk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
