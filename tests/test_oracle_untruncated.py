"""Pins of the oracle's untruncated step (truncation switched off, page 1,
ablation Table 6), each against something other than that function itself:

* the training-form dense forward (page 1, key design 3): the decode history
  as one clean block and every still-masked position as one masked block
  without registers; the decoded rows' outputs must agree;
* page 3, section 7.2: when every masked position is decoded at once (C = B)
  the sparse parameterization is the standard MDM's, so with no registers the
  truncated and the untruncated step coincide;
* brute force: the step rebuilt with Python loops, key kind by key kind;
* a property: the masked keys' order does not matter (attention is a sum
  over keys);
* the whole untruncated run decodes every position once and differs from the
  truncated run (the truncated masked tokens and the registers change the
  decoded rows' context).
"""

import dataclasses

import numpy as np
import pytest

from oracle import attention, dense, masks
from oracle.logits import decide
from oracle.step import Model, SequenceOracle, run_workload
from small_workloads import tiny_bf16, tiny_semi_ar, workload


def _history(res, k, i):
    groups = []
    for r in res.records[:k]:
        sel = r.selected[i]
        groups.append((r.token[i][sel], r.c_pos[i][sel]))
    return groups


@pytest.mark.parametrize("cfgfn", [tiny_bf16, tiny_semi_ar])
def test_untruncated_matches_training_form_forward(cfgfn):
    cfg = cfgfn()
    wl = workload(cfg)
    model = Model.from_workload(wl, precision="none")
    res = run_workload(wl, keep_steps=range(cfg.n_steps), model=model, truncate=False)
    bare = dataclasses.replace(model, n_registers=0)
    for k in range(cfg.n_steps):
        rec = res.records[k]
        for i, b in enumerate(res.batches):
            hist = _history(res, k, i)
            decoded = set(int(p) for _, ps in hist for p in ps)
            masked = np.array([p for p in range(cfg.prompt_len, cfg.seq_len) if p not in decoded])
            clean = [(np.concatenate([t for t, _ in hist]), np.concatenate([p for _, p in hist]))] if hist else []
            ids, pos, blk, m, spans = dense.build_rows(bare, wl.prompt_ids[b], clean, [masked])
            out = dense.dense_forward(bare, ids, pos, blk, m)[0]
            mrows, _ = spans[0]
            row_of = {int(p): int(r) for p, r in zip(pos[mrows], mrows)}
            want = out[[row_of[int(p)] for p in rec.c_pos[i]]]
            n_d = rec.d_pos[i].size
            assert np.allclose(rec.o[i][n_d:], want, rtol=1e-11, atol=1e-12)


def test_c_equals_b_reduces_to_the_untruncated_step():
    cfg = tiny_bf16(n_registers=0, n_steps=1, per_step=16)
    wl = workload(cfg)
    model = Model.from_workload(wl, precision="none")
    assert model.n_registers == 0
    for b in range(cfg.batch):
        s_t = SequenceOracle(model, wl.prompt_ids[b])
        s_u = SequenceOracle(model, wl.prompt_ids[b])
        s_t.prefill()
        s_u.prefill()
        c_pos = wl.order[b].astype(np.int64)              # every masked position at once
        o_t = s_t.forward([], [], c_pos)
        o_u = s_u.forward_untruncated([], [], c_pos, s_u.masked_positions())
        assert np.allclose(o_t.h, o_u.h, rtol=1e-12, atol=1e-13)


def _bruteforce_untruncated(model, cache_tok, cache_pos, d_tok, d_pos, c_pos, m_pos):
    """Rows [D | C] with Python loops; keys: cache, D and every masked position."""
    q_ids = list(d_tok) + [model.mask_id] * len(c_pos)
    q_pos = list(d_pos) + list(c_pos)
    q_kind = ["new"] * len(d_tok) + ["decode"] * len(c_pos)
    k_ids = list(cache_tok) + list(d_tok) + [model.mask_id] * len(m_pos)
    k_pos = list(cache_pos) + list(d_pos) + list(m_pos)
    k_kind = ["cached"] * len(cache_tok) + ["new"] * len(d_tok) + ["decode"] * len(m_pos)
    q, _, _ = model.qkv_layer1(np.array(q_ids), np.array(q_pos))
    _, k, v = model.qkv_layer1(np.array(k_ids), np.array(k_pos))
    vis = np.array([[masks.kind_visible(a, c) for c in k_kind] for a in q_kind])
    return attention.attend_bruteforce(q, k, v, vis).reshape(len(q_ids), -1)


def test_untruncated_step_matches_bruteforce():
    # three steps of four: at step 1 four masked positions are present beyond C
    cfg = tiny_bf16(n_heads=2, n_kv_heads=1, head_dim=8, vocab=20, prompt_len=4, gen_len=12,
                    n_registers=2, n_steps=3, per_step=4)
    wl = workload(cfg)
    model = Model.from_workload(wl)
    res = run_workload(wl, batches=[0], keep_steps=[0, 1], model=model, truncate=False, n_steps=2)
    o0 = wl.order[0]
    r0, r1 = res.records
    m_pos = np.sort(o0[4:])
    o = _bruteforce_untruncated(model, wl.prompt_ids[0], np.arange(cfg.prompt_len), r0.token[0], o0[:4],
                                o0[4:8], m_pos)
    assert np.allclose(o, r1.o[0], rtol=1e-12, atol=1e-13)
    w = model.w
    h = o[4:]
    z = np.array([[sum(h[i, t] * w[vv, t] for t in range(w.shape[1])) for vv in range(w.shape[0])]
                  for i in range(h.shape[0])])
    assert np.allclose(z, r1.z, rtol=1e-12, atol=1e-12)
    assert np.array_equal(decide(z)[0], r1.token[0])


def test_masked_key_order_does_not_matter():
    cfg = tiny_bf16()
    wl = workload(cfg)
    model = Model.from_workload(wl, precision="none")
    rng = np.random.default_rng(5)
    s1, s2 = SequenceOracle(model, wl.prompt_ids[0]), SequenceOracle(model, wl.prompt_ids[0])
    s1.prefill()
    s2.prefill()
    c_pos = wl.order[0][:4].astype(np.int64)
    m = s1.masked_positions()
    a = s1.forward_untruncated([], [], c_pos, m)
    b = s2.forward_untruncated([], [], c_pos, rng.permutation(m))
    assert np.allclose(a.h, b.h, rtol=1e-12, atol=1e-13)


def test_untruncated_run_decodes_every_position_once_and_differs():
    cfg = tiny_bf16()
    wl = workload(cfg)
    model = Model.from_workload(wl)
    r_u = run_workload(wl, model=model, truncate=False)
    r_t = run_workload(wl, model=model)
    for i, b in enumerate(r_u.batches):
        got = np.concatenate([u[i] for u in r_u.unmask])
        assert np.array_equal(np.sort(got), np.arange(cfg.prompt_len, cfg.seq_len))
        assert not np.any(r_u.tokens[i] == model.mask_id)
    # the first step already differs: the decoded rows see other keys
    h_u = np.concatenate([r.z for r in run_workload(wl, model=model, truncate=False, keep_steps=[0],
                                                    n_steps=1).records])
    h_t = np.concatenate([r.z for r in run_workload(wl, model=model, keep_steps=[0], n_steps=1).records])
    assert not np.allclose(h_u, h_t)


def test_untruncated_refuses_two_layers():
    from small_workloads import tiny_two_layer
    cfg = tiny_two_layer()
    wl = workload(cfg)
    with pytest.raises(NotImplementedError):
        run_workload(wl, n_steps=1, truncate=False)
