"""The speed-up switches of page 1's ablation (Table 6): cache the prompt, cache
the decoded tokens ("res"), truncate the masked tokens ("truncate res"), each
on or off, on the same kernels as the sparse loop.

One model throughout: one attention layer under the step-causal rule (clean
rows - the prompt and the decoded tokens - see the clean rows present; the
masked rows and the registers see everything present).  Under that rule
keeping a clean row's key and value equals recomputing them, so the switches
change only the work of a step:

* cache prompt off: every step appends the prompt again (its keys and values
  recomputed) and runs its rows through the attention;
* cache res off: every step appends every decoded token again and runs it
  through the attention (on: only the rows decoded at the previous step,
  which then stay in the cache);
* truncate off: every still-masked position is present as the mask token and
  there are no registers (they stand in only for truncated tokens); each step
  appends the masked rows after the clean ones, attends with them and drops
  them again; the vocabulary head runs on every generated row that passes
  through the network and is not being cached (the dense MDM's L x V
  logits), not only on the rows decoded this step.

With truncation on, the decoded rows' context is the sparse loop's; with it
off, it is every masked position without registers (the oracle's
forward_untruncated).  The rows decoded at a step are those of the workload's
pre-generated order either way.

bidirectional=True (all switches off) is the plain dense MDM instead: every
row of the sequence sees every other row (the step-causal rule dropped); its
decoded rows see the same keys as with truncation off, so it makes the same
decisions.

Per step the calls are, in order: mdm_cache_rewind / mdm_kv_append for the
clean rows of the step, mdm_step_attention (clean rows, and with truncation
the decoded rows and registers), without truncation mdm_kv_append of the
masked rows + mdm_step_attention of them + mdm_cache_rewind,
mdm_subset_logits_confidence over the decoded rows (and, without truncation,
over the other rows the head runs on, in chunks of at most max_decode rows),
mdm_unmask_select.  Row lists are kept as [prompt | generated positions in
unmasking order]; torch copies the decided tokens into it (marshalling only).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib as L
from .sampler import SparseStepRunner


@dataclass(frozen=True)
class Switches:
    cache_prompt: bool = True
    cache_res: bool = True
    truncate: bool = True
    bidirectional: bool = False      # all off, and every row sees every row

    def __post_init__(self):
        if self.bidirectional and (self.cache_prompt or self.cache_res or self.truncate):
            raise ValueError("the bidirectional dense step has every switch off")

    @property
    def name(self) -> str:
        if self.bidirectional:
            return "dense_bidirectional"
        on = [n for n, v in (("cache_prompt", self.cache_prompt), ("cache_res", self.cache_res),
                             ("truncate", self.truncate)) if v]
        return "+".join(on) if on else "none"


# page 1, Table 6: its rows in order, then the plain dense MDM
TABLE6 = [Switches(False, False, False), Switches(True, False, False), Switches(False, True, False),
          Switches(False, False, True), Switches(True, True, False), Switches(True, False, True),
          Switches(True, True, True)]
ALL_SWITCHES = TABLE6 + [Switches(False, False, False, bidirectional=True)]


def switch_work(cfg, counts, sw: Switches):
    """Algorithmic FLOP of one generation under a setting: 4 d FLOP per
    visible (query, key) pair per query head (clean rows see the prompt and
    the decoded tokens; the other rows everything present), 2 hidden FLOP per
    vocabulary column per row the head runs on.  Returns (attention, head)."""
    P, Lg, R = cfg.prompt_len, cfg.gen_len, cfg.n_registers
    pairs = rows = 0
    c0 = 0
    for k, n_c in enumerate(counts):
        n_dprev = counts[k - 1] if k else 0
        if sw.bidirectional:
            pairs += (P + Lg) * (P + Lg)
            rows += Lg
        else:
            n_new = {(True, True): n_dprev, (True, False): c0, (False, True): n_dprev + P,
                     (False, False): P + c0}[(sw.cache_prompt, sw.cache_res)]
            pairs += n_new * (P + c0)
            if sw.truncate:
                pairs += (n_c + R) * (P + c0 + n_c + R)
                rows += n_c
            else:
                pairs += (Lg - c0) * (P + Lg)
                rows += (Lg - c0) + (0 if sw.cache_res else c0)
        c0 += n_c
    att = 4.0 * cfg.head_dim * pairs * cfg.n_heads * cfg.batch
    head = 2.0 * cfg.hidden * cfg.vocab * rows * cfg.batch
    return att, head


class AblationRunner(SparseStepRunner):
    """One workload (pre-generated order, one layer) under the given switches."""

    def __init__(self, wl, sw: Switches, device: str = "cuda", logits_rows: int = 2048):
        cfg = wl.cfg
        if wl.order is None or cfg.schedule == "semi_ar":
            raise ValueError("the switches are modelled for a pre-generated unmasking order")
        if cfg.layers != 1:
            raise ValueError("the switches are modelled for one attention layer")
        counts = [int(c) for c in wl.counts]
        P, Lg = cfg.prompt_len, cfg.gen_len
        md = max(counts) if sw.truncate else max(max(counts), min(logits_rows, Lg))
        n_reg = cfg.n_registers if sw.truncate else 0
        rows = P + Lg + max(counts) + n_reg
        super().__init__(wl, device=device, fused=False, n_registers=n_reg, max_decode=md,
                         out_rows=rows, n_out=2)
        self.sw = sw
        self.counts = counts
        B = cfg.batch
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        S = P + Lg
        self.S = S
        # [prompt | generated positions in unmasking order]; tokens start as the mask
        rt = np.full((B, S), cfg.vocab, dtype=np.int32)
        rt[:, :P] = wl.prompt_ids
        rp = np.concatenate([wl.prompt_pos, wl.order], axis=1).astype(np.int32)
        self.rows_tok0 = torch.from_numpy(rt).to(dev)
        self.rows_tok = self.rows_tok0.clone()
        self.rows_pos = torch.from_numpy(np.ascontiguousarray(rp)).to(dev)
        # [D | prompt] rows of the "cache res, recompute the prompt" setting
        self.da_stride = max(counts) + P
        self.da_tok = torch.zeros(B, self.da_stride, **i32)
        self.da_pos = torch.zeros(B, self.da_stride, **i32)
        self.conf_x = torch.zeros(B * md, dtype=torch.float32, device=dev)
        self.token_x = torch.zeros(B * md, **i32)
        self.sel_tok = torch.zeros(B * max(counts), **i32)
        self.sel_pos = torch.zeros(B * max(counts), **i32)
        self.last = {}

    # -- helpers ------------------------------------------------------------------
    def _ptr(self, t: torch.Tensor, off_elems: int = 0) -> int:
        return t.data_ptr() + t.element_size() * off_elems

    def _head(self, out: torch.Tensor, n_q: int, r0: int, r1: int):
        """The vocabulary head on rows [r0, r1) of out (n_q rows per sequence),
        in chunks of at most max_decode rows; decisions discarded."""
        hd = self.cfg.hidden
        for c in range(r0, r1, self.max_decode):
            n = min(self.max_decode, r1 - c)
            L.mdm_subset_logits_confidence(self.ctx, self._ptr(out, c * hd), n_q * hd, n, self.conf_x,
                                           self.token_x, None)

    # -- one generation -----------------------------------------------------------
    def prefill(self):
        L.mdm_sparse_step_reset(self.ctx)
        self.rows_tok.copy_(self.rows_tok0)
        self.seq_tokens.copy_(self.seq0)
        if self.sw.cache_prompt:
            P = self.cfg.prompt_len
            L.mdm_kv_append(self.ctx, self.rows_tok, self.rows_pos, self.S, P)

    def step(self, k: int, logits: Optional[torch.Tensor] = None):
        cfg, sw, ctx = self.cfg, self.sw, self.ctx
        P, S, hd = cfg.prompt_len, self.S, cfg.hidden
        c0 = sum(self.counts[:k])
        n_c = self.counts[k]
        n_dprev = self.counts[k - 1] if k else 0
        B = cfg.batch
        out0, out1 = self.outs
        c_ptr = self._ptr(self.order, c0)
        L_ = cfg.gen_len
        if sw.bidirectional:
            L.mdm_sparse_step_reset(ctx)
            L.mdm_kv_append(ctx, self.rows_tok, self.rows_pos, S, S)
            L.mdm_step_attention(ctx, self.rows_tok, self.rows_pos, S, S, None, 0, 0, out0)
            n_q, h_out, h_row = S, out0, P + c0
            self.last = dict(out=out0, n_q=S, c_row=P + c0)
        else:
            # 1. the clean rows of this step
            if sw.cache_prompt and sw.cache_res:
                n_new, d_tok, d_pos, d_stride = n_dprev, self._ptr(self.rows_tok, P + c0 - n_dprev), \
                    self._ptr(self.rows_pos, P + c0 - n_dprev), S
            elif sw.cache_prompt:
                L.mdm_cache_rewind(ctx, P)
                n_new, d_tok, d_pos, d_stride = c0, self._ptr(self.rows_tok, P), self._ptr(self.rows_pos, P), S
            elif sw.cache_res:
                if k:
                    L.mdm_cache_rewind(ctx, L.mdm_cache_len(ctx) - P)     # last step's prompt copy
                if n_dprev:
                    self.da_tok[:, :n_dprev].copy_(self.rows_tok[:, P + c0 - n_dprev:P + c0])
                    self.da_pos[:, :n_dprev].copy_(self.rows_pos[:, P + c0 - n_dprev:P + c0])
                self.da_tok[:, n_dprev:n_dprev + P].copy_(self.rows_tok[:, :P])
                self.da_pos[:, n_dprev:n_dprev + P].copy_(self.rows_pos[:, :P])
                n_new, d_tok, d_pos, d_stride = n_dprev + P, self.da_tok, self.da_pos, self.da_stride
            else:
                L.mdm_sparse_step_reset(ctx)
                n_new, d_tok, d_pos, d_stride = P + c0, self.rows_tok, self.rows_pos, S
            if n_new:
                L.mdm_kv_append(ctx, d_tok, d_pos, d_stride, n_new)
            # 2. attention
            if sw.truncate:
                L.mdm_step_attention(ctx, d_tok, d_pos, d_stride, n_new, c_ptr, L_, n_c, out0)
                n_q, h_out, h_row = n_new + n_c + self.n_registers, out0, n_new
                self.last = dict(out=out0, n_q=n_q, c_row=n_new)
            else:
                if n_new:
                    L.mdm_step_attention(ctx, d_tok, d_pos, d_stride, n_new, None, 0, 0, out0)
                n_m = L_ - c0
                m_tok, m_pos = self._ptr(self.rows_tok, P + c0), self._ptr(self.rows_pos, P + c0)
                L.mdm_kv_append(ctx, m_tok, m_pos, S, n_m)
                L.mdm_step_attention(ctx, m_tok, m_pos, S, n_m, None, 0, 0, out1)
                L.mdm_cache_rewind(ctx, L.mdm_cache_len(ctx) - n_m)
                n_q, h_out, h_row = n_m, out1, 0
                self.last = dict(out=out1, n_q=n_m, c_row=0, clean_out=out0, n_clean=n_new)
        # 3. the vocabulary head and the decisions of the rows decoded now
        L.mdm_subset_logits_confidence(ctx, self._ptr(h_out, h_row * hd), n_q * hd, n_c, self.conf, self.token,
                                       logits)
        if not sw.truncate:
            # every other generated row through the network and not being cached
            self._head(h_out, n_q, h_row + n_c, h_row + (L_ - c0))
            if not sw.bidirectional and not sw.cache_res:
                e0 = 0 if sw.cache_prompt else P
                self._head(out0, self.last["n_clean"], e0, e0 + c0)
            if sw.bidirectional:
                self._head(out0, S, P, P + c0)
        L.mdm_unmask_select(ctx, c_ptr, L_, self.conf, self.token, n_c, n_c, L.MDM_SELECT_ORDER,
                            self.sel_tok, self.sel_pos, None, self.seq_tokens)
        self.rows_tok[:, P + c0:P + c0 + n_c].copy_(self.sel_tok[:B * n_c].view(B, n_c))

    def generate(self, n_steps: Optional[int] = None):
        self.prefill()
        for k in range(len(self.counts) if n_steps is None else n_steps):
            self.step(k)

    def generate_recorded(self, n_steps: Optional[int] = None, keep_o=(), keep_logits=(), trace: bool = False):
        """Eager generation copying each step's decisions (and, for steps in
        keep_o, the attention output of the rows the step's logits read and of
        the clean rows) back to the host."""
        cfg = self.cfg
        B = cfg.batch
        hd = cfg.hidden
        self.prefill()
        recs = []
        n_steps = len(self.counts) if n_steps is None else n_steps
        for k in range(n_steps):
            n_c = self.counts[k]
            lg = None
            if k in keep_logits:
                lg = torch.empty(B * n_c * cfg.vocab, dtype=torch.float32, device=self.device)
            self.step(k, lg)
            torch.cuda.synchronize(self.device)
            c0 = sum(self.counts[:k])
            rec = dict(k=k, conf=self.conf[:B * n_c].view(B, n_c).cpu().numpy().copy(),
                       token=self.token[:B * n_c].view(B, n_c).cpu().numpy().copy(),
                       sel_pos=self.order[:, c0:c0 + n_c].cpu().numpy().copy(),
                       cache_len=L.mdm_cache_len(self.ctx))
            if k in keep_o:
                last = self.last
                n_q = last["n_q"]
                rec["o"] = last["out"][:B * n_q * hd].view(B, n_q, hd).cpu().numpy().copy()
                rec["c_row"] = last["c_row"]
                if "clean_out" in last:
                    nc_ = last["n_clean"]
                    rec["o_clean"] = last["clean_out"][:B * nc_ * hd].view(B, nc_, hd).cpu().numpy().copy()
            if lg is not None:
                rec["logits"] = lg.view(B, n_c, cfg.vocab).cpu().numpy()
            recs.append(rec)
        L.mdm_device_status(self.ctx)
        return recs, self.seq_tokens.cpu().numpy().copy()
