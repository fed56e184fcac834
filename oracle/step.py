"""The incremental sparse sampling loop (test infrastructure).

Page 3, section 3.2 and page 1 (overall framework): the prompt is prefetched
into the KV cache; at every step k the network sees the cached tokens, the
tokens decoded at step k-1 (which enter the cache now), the masked positions
decoded at step k and the registers, and produces logits only for the decoded
positions; the tokens decoded at step k join the cache at step k+1.  Page 1,
key design 1: only the prompt, the decoded tokens and this step's subset are
fed, the rest of the masked positions are truncated.  Page 1, key design 2:
R register tokens with consecutive position ids after the sequence end, the
same R tokens at every step.

Readings (where the pages are silent):

* layer 1's q/k/v rows are table lookups by token id; an optional second
  layer projects the first layer's output (q, k, v = h1 W, no W_o, MLP or
  norm; RoPE at the row's position; q, k and v rounded to the storage type,
  since the cache holds what later steps read); h = the concatenated head
  outputs of the last layer;
* the mask token is one shared table row (id V); register r is row V+1+r;
* registers are re-fed at every step and never cached;
* the prompt is in the cache before step 1 and nothing enters at step 1;
  the last step's tokens are not appended;
* the cache keeps tokens in the order they enter it (append order);
* text infilling: the clean tokens may sit anywhere in the sequence (their
  positions are given), the masked positions are the rest; semi-AR block j
  holds the j-th `block` masked positions in position order, and blocks may
  be decoded in any order (page 3, section 3.2: the network sees only the
  clean tokens and the positions it decodes, so neither changes the step).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import rope
from .attention import attend
from .logits import decide, subset_logits, top_two
from .masks import CACHED, DECODE, NEW, inference_mask, step_mask
from .numerics import round_bf16, round_storage, table_values
from .select import select_all, select_by_confidence


def split_layer2(w_rows: np.ndarray, hq: int, hk: int):
    """Layer-2 projection matrices from the stored weight rows.

    The rows of W_2 [(H + 2 H_kv) d][hidden] are the query heads, then the key
    heads, then the value heads; output feature j of a row is the dot product
    of the layer-1 output h1 with row j.  Returned as (Wq, Wk, Wv) laid out
    [hidden][features], so that q = h1 @ Wq.
    """
    return w_rows[:hq].T, w_rows[hq:hq + hk].T, w_rows[hq + hk:hq + 2 * hk].T


@dataclass
class Model:
    n_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    n_registers: int
    seq_len: int
    tq: np.ndarray            # table rows by token id (bf16 bits, fp32 or fp64)
    tk: np.ndarray
    tv: np.ndarray
    w: np.ndarray             # vocab head [V][hidden] (float64 values)
    precision: str            # storage rounding of RoPE'd q/k: bf16 | fp32 | none
    theta: float = 10000.0
    layer2: Optional[tuple] = None   # (Wq2, Wk2, Wv2) float64 for the 2-layer mode
    cos: np.ndarray = field(init=False, repr=False)
    sin: np.ndarray = field(init=False, repr=False)

    def __post_init__(self):
        self.cos, self.sin = rope.table(self.seq_len + self.n_registers, self.head_dim, self.theta)

    @classmethod
    def from_workload(cls, wl, precision: Optional[str] = None, layer2=None):
        cfg = wl.cfg
        if layer2 is None and getattr(wl, "layer_w", None):
            if len(wl.layer_w) != 1:
                raise ValueError("the oracle models at most two layers")
            layer2 = split_layer2(table_values(wl.layer_w[0]), cfg.n_heads * cfg.head_dim,
                                  cfg.n_kv_heads * cfg.head_dim)
        return cls(n_heads=cfg.n_heads, n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                   vocab=cfg.vocab, n_registers=cfg.n_registers, seq_len=cfg.seq_len,
                   tq=wl.tq, tk=wl.tk, tv=wl.tv, w=table_values(wl.w_vocab),
                   precision=precision or cfg.precision, theta=cfg.rope_theta, layer2=layer2)

    @property
    def hidden(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def mask_id(self) -> int:
        return self.vocab

    def register_ids(self) -> np.ndarray:
        return np.arange(self.vocab + 1, self.vocab + 1 + self.n_registers, dtype=np.int64)

    def register_pos(self) -> np.ndarray:
        return np.arange(self.seq_len, self.seq_len + self.n_registers, dtype=np.int64)

    def _rot(self, x, pos):
        return round_storage(rope.rotate(x, pos, self.cos, self.sin), self.precision)

    def qkv_layer1(self, ids, pos):
        """q, k (RoPE'd at pos, rounded to storage) and v rows for token ids."""
        n = len(ids)
        d, h, hk = self.head_dim, self.n_heads, self.n_kv_heads
        q = table_values(self.tq[ids]).reshape(n, h, d)
        k = table_values(self.tk[ids]).reshape(n, hk, d)
        v = table_values(self.tv[ids]).reshape(n, hk, d)
        return self._rot(q, pos), self._rot(k, pos), v

    def qkv_layer2(self, h1, pos):
        wq, wk, wv = self.layer2
        n = h1.shape[0]
        d, h, hk = self.head_dim, self.n_heads, self.n_kv_heads
        q = (h1 @ wq).reshape(n, h, d)
        k = (h1 @ wk).reshape(n, hk, d)
        v = (h1 @ wv).reshape(n, hk, d)
        # the cache holds what later steps read: v in the storage type too
        return self._rot(q, pos), self._rot(k, pos), round_storage(v, self.precision)


@dataclass
class StepOut:
    o: np.ndarray            # [n_q, H*d] output of the last layer, rows [D | C | R]
    h: np.ndarray            # [n_C, H*d] rows of the decoded subset
    o_layers: list           # per-layer outputs [n_q, H*d]


class SequenceOracle:
    """One sequence: its dense form X, its KV cache (append order) per layer."""

    def __init__(self, model: Model, prompt_ids: np.ndarray, prompt_pos=None):
        self.m = model
        self.layers = 1 if model.layer2 is None else 2
        cap = model.seq_len + model.n_registers
        shape = (cap, model.n_kv_heads, model.head_dim)
        self.k = [np.zeros(shape) for _ in range(self.layers)]
        self.v = [np.zeros(shape) for _ in range(self.layers)]
        self.n = 0
        self.cache_tok: list = []
        self.cache_pos: list = []
        self.x = np.full(model.seq_len, model.mask_id, dtype=np.int64)
        p = len(prompt_ids)
        self.prompt_pos = (np.arange(p, dtype=np.int64) if prompt_pos is None
                           else np.asarray(prompt_pos, dtype=np.int64))
        self.x[self.prompt_pos] = prompt_ids
        self.prompt_ids = np.asarray(prompt_ids, dtype=np.int64)

    # -- the cache -----------------------------------------------------------
    def _commit(self, layer, k, v):
        n = k.shape[0]
        self.k[layer][self.n:self.n + n] = k
        self.v[layer][self.n:self.n + n] = v

    def prefill(self):
        """Prefetch the prompt (the clean tokens) into the cache."""
        self.forward(self.prompt_ids, self.prompt_pos, np.empty(0, np.int64), prefill=True)

    # -- one forward over the query set [D | C | R] -----------------------------
    def forward(self, d_tok, d_pos, c_pos, prefill: bool = False) -> StepOut:
        """Commit D (the rows decoded last step) to the cache, then attend with
        query rows [D | C | R] under the step-causal mask."""
        m = self.m
        d_tok = np.asarray(d_tok, dtype=np.int64)
        d_pos = np.asarray(d_pos, dtype=np.int64)
        c_pos = np.asarray(c_pos, dtype=np.int64)
        n_d, n_c = d_tok.size, c_pos.size
        n_r = 0 if prefill else m.n_registers
        ids = np.concatenate([d_tok, np.full(n_c, m.mask_id, np.int64),
                              m.register_ids()[:n_r]])
        pos = np.concatenate([d_pos, c_pos, m.register_pos()[:n_r]])
        n_cache = self.n
        vis = step_mask(n_cache, n_d, n_c, n_r)
        need_out = not (prefill and self.layers == 1)
        outs = []
        h_prev = None
        for layer in range(self.layers):
            if layer == 0:
                q, k, v = m.qkv_layer1(ids, pos)
            else:
                q, k, v = m.qkv_layer2(h_prev, pos)
            if need_out:
                keys_k = np.concatenate([self.k[layer][:n_cache], k])
                keys_v = np.concatenate([self.v[layer][:n_cache], v])
                o = attend(q, keys_k, keys_v, vis).reshape(len(ids), m.hidden)
                outs.append(o)
                h_prev = o
            self._commit(layer, k[:n_d], v[:n_d])
        self.n += n_d
        self.cache_tok.extend(d_tok.tolist())
        self.cache_pos.extend(d_pos.tolist())
        if not need_out:
            return StepOut(o=np.empty((0, m.hidden)), h=np.empty((0, m.hidden)), o_layers=[])
        o = outs[-1]
        return StepOut(o=o, h=o[n_d:n_d + n_c], o_layers=outs)

    def forward_untruncated(self, d_tok, d_pos, c_pos, m_pos) -> StepOut:
        """The step with truncation switched off (page 1, ablation Table 6:
        "truncate res" off).  Every still-masked position m_pos (a superset of
        c_pos) is present as the mask token and there are no registers, which
        stand in only for truncated tokens (page 3, section 7.2: with every
        masked position present the parameterization is the standard MDM's).
        The step-causal rule still holds: D rows see the cache and D; the
        decoded rows C see everything present.  Returns rows [D | C] (the
        masked rows outside C enter only as keys; their own outputs never reach
        a decision).  One layer: a second would need every masked row's
        first-layer output."""
        if self.layers != 1:
            raise NotImplementedError("the untruncated step is modelled for one layer")
        m = self.m
        d_tok = np.asarray(d_tok, dtype=np.int64)
        d_pos = np.asarray(d_pos, dtype=np.int64)
        c_pos = np.asarray(c_pos, dtype=np.int64)
        m_pos = np.asarray(m_pos, dtype=np.int64)
        if not np.isin(c_pos, m_pos).all():
            raise ValueError("decoded positions must be masked")
        n_d, n_c, n_m = d_tok.size, c_pos.size, m_pos.size
        q_ids = np.concatenate([d_tok, np.full(n_c, m.mask_id, np.int64)])
        q_pos = np.concatenate([d_pos, c_pos])
        q, _, _ = m.qkv_layer1(q_ids, q_pos)
        _, k_dm, v_dm = m.qkv_layer1(np.concatenate([d_tok, np.full(n_m, m.mask_id, np.int64)]),
                                     np.concatenate([d_pos, m_pos]))
        n_cache = self.n
        vis = inference_mask([NEW] * n_d + [DECODE] * n_c,
                             [CACHED] * n_cache + [NEW] * n_d + [DECODE] * n_m)
        keys_k = np.concatenate([self.k[0][:n_cache], k_dm])
        keys_v = np.concatenate([self.v[0][:n_cache], v_dm])
        o = attend(q, keys_k, keys_v, vis).reshape(n_d + n_c, m.hidden)
        self._commit(0, k_dm[:n_d], v_dm[:n_d])
        self.n += n_d
        self.cache_tok.extend(d_tok.tolist())
        self.cache_pos.extend(d_pos.tolist())
        return StepOut(o=o, h=o[n_d:], o_layers=[o])

    def masked_positions(self) -> np.ndarray:
        """Positions still holding the mask token, ascending."""
        return np.flatnonzero(self.x == self.m.mask_id).astype(np.int64)

    def write_tokens(self, pos, tok):
        self.x[np.asarray(pos, dtype=np.int64)] = tok


@dataclass
class StepRecord:
    k: int
    d_pos: list               # per sequence: positions entering the cache
    c_pos: list               # per sequence: positions decoded this step
    token: list               # per sequence: decided tokens [n_C]
    conf32: list
    conf64: list
    margin: list
    top2_idx: list            # per sequence: [n_C, 2] the two best vocabulary indices (float64 logits)
    top2_val: list            # per sequence: [n_C, 2] their logits
    selected: list            # per sequence: indices into c_pos that are unmasked
    conf_gap: list            # per sequence: conf32 gap at the top-n cut (semi-AR), else nan
    o: Optional[list] = None          # per sequence [n_q, hidden] (kept steps only)
    z: Optional[np.ndarray] = None    # stacked [sum n_C, V] exact logits (kept steps only)
    z_mirror: Optional[np.ndarray] = None   # bf16(h) W^T (kept steps, bf16 runs only)


@dataclass
class RunResult:
    batches: list
    tokens: np.ndarray        # [nb, seq_len] final sequences
    unmask: list              # per step: per sequence positions unmasked (selection order)
    records: list             # [StepRecord]


def step_candidates(wl, k, b, remaining):
    """Positions to decode at step k for sequence b (from the workload's plan)."""
    cfg = wl.cfg
    if cfg.schedule == "semi_ar":
        st = wl.semi_ar[k]
        if st.sub == 0:
            start = st.block * cfg.block
            return wl.gen_pos[b, start:start + cfg.block].astype(np.int64)
        return remaining[b]
    c0 = int(np.sum(wl.counts[:k]))
    return wl.order[b, c0:c0 + int(wl.counts[k])].astype(np.int64)


def run_workload(wl, batches=None, n_steps: Optional[int] = None, keep_steps=(),
                 precision: Optional[str] = None, model: Optional[Model] = None,
                 truncate: bool = True) -> RunResult:
    """Run the sparse sampler on sequences `batches` of workload `wl`.
    truncate=False runs every step with all masked positions present and no
    registers (SequenceOracle.forward_untruncated)."""
    cfg = wl.cfg
    batches = list(range(cfg.batch)) if batches is None else list(batches)
    model = model or Model.from_workload(wl, precision=precision)
    n_steps = cfg.n_steps if n_steps is None else n_steps
    seqs = [SequenceOracle(model, wl.prompt_ids[b], wl.prompt_pos[b]) for b in batches]
    for s in seqs:
        s.prefill()
    d_state = [(np.empty(0, np.int64), np.empty(0, np.int64)) for _ in batches]
    remaining = {b: None for b in batches}
    unmask, records = [], []
    keep = set(keep_steps)
    for k in range(n_steps):
        c_list, outs = [], []
        for i, b in enumerate(batches):
            c_pos = step_candidates(wl, k, b, remaining)
            c_list.append(c_pos)
            if truncate:
                outs.append(seqs[i].forward(d_state[i][0], d_state[i][1], c_pos))
            else:
                outs.append(seqs[i].forward_untruncated(d_state[i][0], d_state[i][1], c_pos,
                                                        seqs[i].masked_positions()))
        h = np.concatenate([o.h for o in outs])
        z = subset_logits(h, model.w)
        token, conf32, conf64, margin = decide(z)
        t2_idx, t2_val = top_two(z)
        rec = StepRecord(k=k, d_pos=[d[1] for d in d_state], c_pos=c_list, token=[], conf32=[],
                         conf64=[], margin=[], top2_idx=[], top2_val=[], selected=[], conf_gap=[])
        off = 0
        step_unmask = []
        for i, b in enumerate(batches):
            n_c = c_list[i].size
            tk, c32 = token[off:off + n_c], conf32[off:off + n_c]
            if cfg.schedule == "semi_ar":
                sel, rem = select_by_confidence(c_list[i], c32, wl.semi_ar[k].n_select)
                remaining[b] = c_list[i][rem]
                gap = (np.min(c32[sel]) - np.max(c32[rem])) if rem.size else np.inf
            else:
                sel, rem = select_all(c_list[i])
                gap = np.nan
            rec.token.append(tk)
            rec.conf32.append(c32)
            rec.conf64.append(conf64[off:off + n_c])
            rec.margin.append(margin[off:off + n_c])
            rec.top2_idx.append(t2_idx[off:off + n_c])
            rec.top2_val.append(t2_val[off:off + n_c])
            rec.selected.append(sel)
            rec.conf_gap.append(gap)
            u_pos, u_tok = c_list[i][sel], tk[sel]
            seqs[i].write_tokens(u_pos, u_tok)
            d_state[i] = (u_tok, u_pos)
            step_unmask.append(u_pos)
            off += n_c
        if k in keep:
            rec.o = [o.o for o in outs]
            rec.z = z
            if model.precision == "bf16":
                rec.z_mirror = subset_logits(round_bf16(h), model.w)
        unmask.append(step_unmask)
        records.append(rec)
    tokens = np.stack([s.x for s in seqs])
    return RunResult(batches=batches, tokens=tokens, unmask=unmask, records=records)
