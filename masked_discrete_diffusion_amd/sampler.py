"""The sampling loop over the C ABI: device buffers and the order of calls.

Per sampling step k (page 3, section 3.2):

    mdm_kv_append(D_{k-1})                  rows decoded at step k-1 enter the cache
    mdm_step_attention(D_{k-1}, C_k, R)     step-causal attention over the query set
    mdm_subset_logits_confidence(h of C_k)  logits, confidence and argmax for C_k only
    mdm_unmask_select(C_k)                  unmask (pre-generated order or confidence)

With a pre-generated order (one bf16 layer) each step is instead one
mdm_order_step, which gives the same results in fewer launches: the rows
decoded at step k are unmasked and committed to the cache by step k itself
(not after the last step), and are the D rows of step k + 1.

With upper layers (layer l >= 2 projects layer l-1's outputs), every step
runs mdm_layer_project + mdm_layer_attention per upper layer after the first
attention, and the logits read the last layer's output.

The prompt is appended before step 1.  PyTorch only provides device memory
and streams; every step of the path runs in the library's kernels.  All
shapes are fixed by the workload's plan, so one whole generation can be
captured as a single HIP graph and replayed.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib as L


@dataclass
class StepPlan:
    n_d: int            # rows entering the cache (decoded at the previous step)
    d_buf: int          # which D buffer holds them
    c_kind: str         # "order" | "block" | "rem"
    c_off: int          # column offset into order/block positions, or rem buffer index
    n_c: int            # positions decoded this step
    n_sel: int          # positions unmasked this step
    mode: int           # L.MDM_SELECT_ORDER | L.MDM_SELECT_CONFIDENCE
    out_buf: int        # D buffer the selection writes
    rem_out: int        # rem buffer the selection writes (-1: none)


def make_plan(wl) -> list:
    cfg = wl.cfg
    plan = []
    n_d, d_buf = 0, 0
    if cfg.schedule == "semi_ar":
        rem = 0
        for k, st in enumerate(wl.semi_ar):
            out_buf = k % 2
            rem_out = k % 2 if st.n_cand > st.n_select else -1
            if st.sub == 0:
                c_kind, c_off = "block", st.block * cfg.block
            else:
                c_kind, c_off = "rem", rem
            plan.append(StepPlan(n_d, d_buf, c_kind, c_off, st.n_cand, st.n_select,
                                 L.MDM_SELECT_CONFIDENCE, out_buf, rem_out))
            n_d, d_buf, rem = st.n_select, out_buf, rem_out
    else:
        off = 0
        for k, n in enumerate(wl.counts.tolist()):
            out_buf = k % 2
            plan.append(StepPlan(n_d, d_buf, "order", off, n, n, L.MDM_SELECT_ORDER, out_buf, -1))
            off += n
            n_d, d_buf = n, out_buf
    return plan


def _to_device_table(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class SparseStepRunner:
    """Device state of one workload: tables, caches, workspace, loop buffers."""

    def __init__(self, wl, device: str = "cuda", accurate_conf: Optional[bool] = None,
                 precision: Optional[str] = None, fused: bool = True, n_registers: Optional[int] = None,
                 max_decode: Optional[int] = None, out_rows: Optional[int] = None, n_out: Optional[int] = None):
        """n_registers, max_decode, out_rows (query rows per sequence of the
        output buffers) and n_out (number of output buffers) override the
        values the workload's plan implies (the ablation loops use them)."""
        cfg = wl.cfg
        self.wl, self.cfg = wl, cfg
        self.device = torch.device(device)
        self.precision = precision or cfg.precision
        if self.precision != cfg.precision:
            raise ValueError("table storage precision is fixed by the workload")
        if accurate_conf is None:
            accurate_conf = cfg.schedule == "semi_ar"
        self.plan = make_plan(wl)
        if max_decode is None:
            max_decode = max(p.n_c for p in self.plan)
        max_sel = max(p.n_sel for p in self.plan)
        self.n_registers = cfg.n_registers if n_registers is None else n_registers
        self.mc = L.MdmConfig(batch=cfg.batch, n_heads=cfg.n_heads, n_kv_heads=cfg.n_kv_heads,
                              head_dim=cfg.head_dim, vocab=cfg.vocab, seq_len=cfg.seq_len,
                              n_registers=self.n_registers, max_decode=max_decode,
                              precision=L.MDM_BF16 if self.precision == "bf16" else L.MDM_FP32,
                              accurate_conf=int(bool(accurate_conf)), rope_theta=cfg.rope_theta)
        dev = self.device
        self.tq = _to_device_table(wl.tq, dev)
        self.tk = _to_device_table(wl.tk, dev)
        self.tv = _to_device_table(wl.tv, dev)
        self.w = _to_device_table(wl.w_vocab, dev)
        self.slots = L.mdm_cache_slots(self.mc)
        edt = torch.int16 if self.precision == "bf16" else torch.float32
        kv_elems = cfg.batch * cfg.n_kv_heads * self.slots * cfg.head_dim
        self.k_cache = torch.zeros(kv_elems, dtype=edt, device=dev)
        self.v_cache = torch.zeros(kv_elems, dtype=edt, device=dev)
        self.cache_pos = torch.zeros(cfg.batch * self.slots, dtype=torch.int32, device=dev)
        self.cache_tok = torch.zeros(cfg.batch * self.slots, dtype=torch.int32, device=dev)
        self.ws_bytes = L.mdm_workspace_bytes(self.mc)
        self.workspace = torch.zeros(self.ws_bytes // 4 + 64, dtype=torch.int32, device=dev)
        self.bufs = L.MdmBuffers(tq=self.tq.data_ptr(), tk=self.tk.data_ptr(), tv=self.tv.data_ptr(),
                                 w_vocab=self.w.data_ptr(), k_cache=self.k_cache.data_ptr(),
                                 v_cache=self.v_cache.data_ptr(), cache_pos=self.cache_pos.data_ptr(),
                                 cache_tok=self.cache_tok.data_ptr(), workspace=self.workspace.data_ptr(),
                                 workspace_bytes=self.ws_bytes)
        self.stream = torch.cuda.current_stream(dev)
        self.ctx = L.mdm_sparse_step_init(self.mc, self.bufs, self.stream.cuda_stream)

        B = cfg.batch
        i32 = dict(dtype=torch.int32, device=dev)
        self.prompt_tok = torch.from_numpy(wl.prompt_ids.astype(np.int32)).to(dev)
        self.prompt_pos = torch.from_numpy(np.ascontiguousarray(wl.prompt_pos, dtype=np.int32)).to(dev)
        self.order = (torch.from_numpy(wl.order.astype(np.int32)).to(dev) if wl.order is not None
                      else torch.zeros(B, 1, **i32))
        self.block_pos = torch.from_numpy(np.ascontiguousarray(wl.gen_pos, dtype=np.int32)).to(dev)
        self.max_decode = max_decode
        self.d_tok = [torch.zeros(B * max(max_sel, max_decode), **i32) for _ in range(2)]
        self.d_pos = [torch.zeros(B * max(max_sel, max_decode), **i32) for _ in range(2)]
        self.rem = [torch.zeros(B * max_decode, **i32) for _ in range(2)]
        self.layers = cfg.layers
        # A pre-generated order on one bf16 layer runs each step as one fused
        # mdm_order_step (the decoded rows enter the cache at the end of their
        # own step instead of at the start of the next).
        self.fused = (fused and self.precision == "bf16" and self.layers == 1
                      and all(p.mode == L.MDM_SELECT_ORDER for p in self.plan))
        rows = max(p.n_d + p.n_c for p in self.plan)
        if self.layers > 1:
            rows = max(rows, cfg.prompt_len)          # the prefill's first-layer rows feed layer 2
        self.n_q_max = rows + self.n_registers if out_rows is None else out_rows
        # layer outputs: layer l writes outs[(l - 1) % 2]; the logits read the last one
        if n_out is None:
            n_out = 1 if self.layers == 1 else 2
        self.outs = [torch.zeros(B * self.n_q_max * cfg.hidden, dtype=torch.float32, device=dev)
                     for _ in range(n_out)]
        self.out = self.outs[(self.layers - 1) % n_out]
        if self.layers > 1:
            w = np.stack(wl.layer_w)                  # [L-1][(H + 2 H_kv) d][H d] bf16 bits
            self.w_upper = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(dev)
            self.k_upper = torch.zeros((self.layers - 1) * kv_elems, dtype=edt, device=dev)
            self.v_upper = torch.zeros((self.layers - 1) * kv_elems, dtype=edt, device=dev)
            self.uws_bytes = L.mdm_upper_workspace_bytes(self.mc)
            self.upper_ws = torch.zeros(self.uws_bytes // 4 + 64, dtype=torch.int32, device=dev)
            self.up = L.MdmUpperLayers(n_layers=self.layers, w_upper=self.w_upper.data_ptr(),
                                       k_cache_upper=self.k_upper.data_ptr(), v_cache_upper=self.v_upper.data_ptr(),
                                       workspace=self.upper_ws.data_ptr(), workspace_bytes=self.uws_bytes)
            L.mdm_attach_upper_layers(self.ctx, self.up)
        self.conf = torch.zeros(B * max_decode, dtype=torch.float32, device=dev)
        self.token = torch.zeros(B * max_decode, **i32)
        seq0 = np.full((B, cfg.seq_len), cfg.vocab, dtype=np.int32)
        np.put_along_axis(seq0, wl.prompt_pos.astype(np.int64), wl.prompt_ids, axis=1)
        self.seq0 = torch.from_numpy(seq0).to(dev)
        self.seq_tokens = self.seq0.clone()

    def close(self):
        if self.ctx is not None:
            L.mdm_sparse_step_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_stream(self, stream: torch.cuda.Stream):
        self.stream = stream
        L.mdm_set_stream(self.ctx, stream.cuda_stream)

    # -- one generation ---------------------------------------------------------
    def _c_src(self, st: StepPlan):
        cfg = self.cfg
        if st.c_kind == "order":
            return self.order.data_ptr() + 4 * st.c_off, self.order.shape[1]
        if st.c_kind == "block":
            return self.block_pos.data_ptr() + 4 * st.c_off, cfg.gen_len
        return self.rem[st.c_off].data_ptr(), st.n_c

    def prefill(self):
        cfg = self.cfg
        P = cfg.prompt_len
        L.mdm_sparse_step_reset(self.ctx)
        L.mdm_kv_append(self.ctx, self.prompt_tok, self.prompt_pos, P, P)
        if self.layers > 1:
            # every upper layer caches the prompt: the first layer's outputs of
            # the prompt rows (they see the prompt only) feed layer 2, and so on
            L.mdm_step_attention(self.ctx, self.prompt_tok, self.prompt_pos, P, P, None, 0, 0, self.outs[0])
            self._upper(P, self.prompt_pos, P, None, 0, 0, prefill=True)

    def _upper(self, n_d, d_pos, d_stride, c_ptr, c_stride, n_c, prefill=False):
        for layer in range(2, self.layers + 1):
            src, dst = self.outs[(layer - 2) % 2], self.outs[(layer - 1) % 2]
            L.mdm_layer_project(self.ctx, layer, src, 0, d_pos, d_stride, n_d, c_ptr, c_stride, n_c)
            if not (prefill and layer == self.layers):
                L.mdm_layer_attention(self.ctx, layer, n_d, n_c, dst)

    def step(self, k: int, logits: Optional[torch.Tensor] = None):
        st = self.plan[k]
        cfg = self.cfg
        ctx = self.ctx
        c_ptr, c_stride = self._c_src(st)
        if self.fused:
            # the rows decoded here are committed here, except after the last step
            L.mdm_order_step(ctx, st.n_d, c_ptr, c_stride, st.n_c, k + 1 < len(self.plan), self.outs[0],
                             self.conf, self.token, self.seq_tokens, logits)
            return
        if st.n_d:
            L.mdm_kv_append(ctx, self.d_tok[st.d_buf], self.d_pos[st.d_buf], st.n_d, st.n_d)
        L.mdm_step_attention(ctx, self.d_tok[st.d_buf], self.d_pos[st.d_buf], st.n_d, st.n_d,
                             c_ptr, c_stride, st.n_c, self.outs[0])
        if self.layers > 1:
            self._upper(st.n_d, self.d_pos[st.d_buf], st.n_d, c_ptr, c_stride, st.n_c)
        n_q = st.n_d + st.n_c + cfg.n_registers
        h_ptr = self.out.data_ptr() + 4 * st.n_d * cfg.hidden
        L.mdm_subset_logits_confidence(ctx, h_ptr, n_q * cfg.hidden, st.n_c, self.conf, self.token, logits)
        rem = self.rem[st.rem_out] if st.rem_out >= 0 else None
        L.mdm_unmask_select(ctx, c_ptr, c_stride, self.conf, self.token, st.n_c, st.n_sel, st.mode,
                            self.d_tok[st.out_buf], self.d_pos[st.out_buf], rem, self.seq_tokens)

    def generate(self, n_steps: Optional[int] = None):
        """Enqueue one whole generation (no host synchronisation)."""
        self.prefill()
        for k in range(len(self.plan) if n_steps is None else n_steps):
            self.step(k)

    def generate_recorded(self, n_steps: Optional[int] = None, keep_o=(), keep_logits=(), trace: bool = False):
        """Eager generation that copies each step's decisions back to the host.
        With trace, every step also records the decisions' certificate rows
        (mdm_set_decision_trace); the decision counters of the generation are
        left in self.decision_counts."""
        cfg = self.cfg
        B = cfg.batch
        tbuf = None
        if trace:
            max_decode = max(p.n_c for p in self.plan)
            tbuf = torch.zeros(B * max_decode * 8, dtype=torch.float32, device=self.device)
            L.mdm_set_decision_trace(self.ctx, tbuf)
        L.mdm_decision_counts(self.ctx)                 # clear
        self.seq_tokens.copy_(self.seq0)
        self.prefill()
        recs = []
        n_steps = len(self.plan) if n_steps is None else n_steps
        for k in range(n_steps):
            st = self.plan[k]
            lg = None
            if k in keep_logits:
                lg = torch.empty(B * st.n_c * cfg.vocab, dtype=torch.float32, device=self.device)
            self.step(k, lg)
            torch.cuda.synchronize(self.device)
            n_q = st.n_d + st.n_c + cfg.n_registers
            token = self.token[:B * st.n_c].view(B, st.n_c).cpu().numpy().copy()
            if self.fused:
                # order mode unmasks every candidate, in candidate order
                sel_pos = self.order[:, st.c_off:st.c_off + st.n_c].cpu().numpy().copy()
                sel_tok = token.copy()
            else:
                sel_pos = self.d_pos[st.out_buf][:B * st.n_sel].view(B, st.n_sel).cpu().numpy().copy()
                sel_tok = self.d_tok[st.out_buf][:B * st.n_sel].view(B, st.n_sel).cpu().numpy().copy()
            rec = dict(
                k=k,
                conf=self.conf[:B * st.n_c].view(B, st.n_c).cpu().numpy().copy(),
                token=token,
                sel_pos=sel_pos,
                sel_tok=sel_tok,
            )
            if k in keep_o:
                rec["o"] = self.out[:B * n_q * cfg.hidden].view(B, n_q, cfg.hidden).cpu().numpy().copy()
            if lg is not None:
                rec["logits"] = lg.view(B, st.n_c, cfg.vocab).cpu().numpy()
            if tbuf is not None:
                rec["trace"] = tbuf[:B * st.n_c * 8].view(B, st.n_c, 8).cpu().numpy().copy()
            recs.append(rec)
        if tbuf is not None:
            L.mdm_set_decision_trace(self.ctx, None)
        L.mdm_device_status(self.ctx)
        self.decision_counts = L.mdm_decision_counts(self.ctx)
        return recs, self.seq_tokens.cpu().numpy().copy()

    def capture_graph(self, n_steps: Optional[int] = None) -> torch.cuda.CUDAGraph:
        """Capture one whole generation (prefill + steps) as a HIP graph."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        old = self.stream
        self.set_stream(s)
        try:
            with torch.cuda.graph(g, stream=s):
                self.generate(n_steps)
        finally:
            self.set_stream(old)
        torch.cuda.current_stream(self.device).wait_stream(s)
        return g
