"""Invariants the pages fix, checked on the oracle's incremental loop.

(a) Cached incremental steps equal a from-scratch forward under the
    training-form block mask (page 1, key design 3; paperlayer.ai summary,
    sections 3.3 and 7.3), for one layer and, with a second layer built on the
    first layer's outputs, for the cached representations too (page 1, worked
    example: cached representations are not polluted by masks or registers).
    Two masked blocks in one forward reproduce two alternative next steps
    (the 0->1->2->3->4 / 0->1->2->3->5 paths of key design 3).
(b) The sparse representation of the running state (cached tokens, their
    positions, the length) recovers the dense partially masked sequence at
    every step (page 1, key design 1).
(d) Brute force: one full step recomputed element by element with Python
    loops equals the vectorised step.
"""

import copy
import math

import numpy as np
import pytest

from oracle import attention, dense, masks, rope, sparse_repr
from oracle.logits import decide
from oracle.numerics import round_storage, table_values
from oracle.step import Model, SequenceOracle, run_workload
from small_workloads import tiny_bf16, tiny_infill, tiny_semi_ar, tiny_two_layer, workload


def _layer2(cfg, seed=7):
    rng = np.random.default_rng(seed)
    hd, kvd = cfg.hidden, cfg.n_kv_heads * cfg.head_dim
    s = 1.0 / math.sqrt(hd)
    return (rng.standard_normal((hd, hd)) * s * 8, rng.standard_normal((hd, kvd)) * s * 8,
            rng.standard_normal((hd, kvd)) * s * 8)


def _history(res, k, i):
    """Decode history (tokens, positions) of steps 0..k-1 for sequence i."""
    groups = []
    for r in res.records[:k]:
        sel = r.selected[i]
        groups.append((r.token[i][sel], r.c_pos[i][sel]))
    return groups


@pytest.mark.parametrize("layers,precision,cfgfn", [
    (1, "bf16", tiny_bf16), (2, "none", tiny_bf16), (1, "bf16", tiny_semi_ar), (2, "none", tiny_semi_ar),
    (1, "bf16", tiny_infill), (2, "none", tiny_infill), (2, "bf16", tiny_two_layer)])
def test_incremental_equals_dense_block_mask(layers, precision, cfgfn):
    cfg = cfgfn()
    wl = workload(cfg)
    # a two-layer workload brings its own layer-2 weights (bf16 storage)
    layer2 = _layer2(cfg) if layers == 2 and cfg.layers == 1 else None
    model = Model.from_workload(wl, precision=precision, layer2=layer2)
    res = run_workload(wl, keep_steps=range(cfg.n_steps), model=model)
    for k in range(cfg.n_steps):
        rec = res.records[k]
        for i, b in enumerate(res.batches):
            hist = _history(res, k, i)
            ids, pos, blk, m, spans = dense.build_rows(model, wl.prompt_ids[b], hist, [rec.c_pos[i]],
                                                       prompt_pos=wl.prompt_pos[b])
            outs = dense.dense_forward(model, ids, pos, blk, m)
            last = outs[-1]
            n_d = rec.d_pos[i].size
            dec_rows, reg_rows = spans[0]
            new_rows = np.nonzero(blk == m)[0] if m > 0 else np.empty(0, int)
            inc = rec.o[i]
            assert new_rows.size == n_d
            assert np.allclose(inc[:n_d], last[new_rows], rtol=1e-11, atol=1e-12)
            assert np.allclose(inc[n_d:n_d + dec_rows.size], last[dec_rows], rtol=1e-11, atol=1e-12)
            assert np.allclose(inc[n_d + dec_rows.size:], last[reg_rows], rtol=1e-11, atol=1e-12)


def test_two_masked_blocks_simulate_two_paths():
    cfg = tiny_bf16()
    wl = workload(cfg)
    for layer2 in (None, _layer2(cfg)):
        model = Model.from_workload(wl, precision="none", layer2=layer2)
        seq = SequenceOracle(model, wl.prompt_ids[0])
        seq.prefill()
        o = wl.order[0]
        hist = []
        d = (np.empty(0, int), np.empty(0, int))
        for j in range(2):                              # two committed steps -> clean blocks
            c = o[4 * j:4 * j + 4]
            seq.forward(d[0], d[1], c)
            tok = np.arange(4) + 10 * j
            seq.write_tokens(c, tok)
            hist.append((tok, c))
            d = (tok, c)
        # the next step's D is the last clean block; two alternative decode sets
        alt_a, alt_b = o[8:11], o[11:16]
        out_a = copy.deepcopy(seq).forward(d[0], d[1], alt_a)
        out_b = copy.deepcopy(seq).forward(d[0], d[1], alt_b)
        ids, pos, blk, m, spans = dense.build_rows(model, wl.prompt_ids[0], hist, [alt_a, alt_b])
        last = dense.dense_forward(model, ids, pos, blk, m)[-1]
        for out, (dec, reg) in zip((out_a, out_b), spans):
            n_d = d[0].size
            assert np.allclose(out.o[n_d:n_d + dec.size], last[dec], rtol=1e-11, atol=1e-12)
            assert np.allclose(out.o[n_d + dec.size:], last[reg], rtol=1e-11, atol=1e-12)
            assert np.allclose(out.o[:n_d], last[blk == m], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("cfgfn", [tiny_bf16, tiny_semi_ar, tiny_infill])
def test_sparse_state_round_trips_every_step(cfgfn):
    cfg = cfgfn()
    wl = workload(cfg)
    model = Model.from_workload(wl)
    seqs = [SequenceOracle(model, wl.prompt_ids[b], wl.prompt_pos[b]) for b in range(cfg.batch)]
    res = run_workload(wl)
    # replay the decisions and check the cache <-> dense sequence correspondence
    for i, s in enumerate(seqs):
        s.prefill()
        d = (np.empty(0, int), np.empty(0, int))
        for r in res.records:
            s.forward(d[0], d[1], r.c_pos[i])
            sel = r.selected[i]
            s.write_tokens(r.c_pos[i][sel], r.token[i][sel])
            d = (r.token[i][sel], r.c_pos[i][sel])
            # the cache plus the tokens about to enter it = the clean part of x
            tok = np.concatenate([s.cache_tok, d[0]])
            pos = np.concatenate([s.cache_pos, d[1]])
            assert np.array_equal(sparse_repr.from_sparse(tok, pos, cfg.seq_len, model.mask_id), s.x)
            t2, p2, n = sparse_repr.to_sparse(s.x, model.mask_id)
            assert n == cfg.seq_len and set(p2.tolist()) == set(pos.tolist())
        assert np.array_equal(s.x, res.tokens[i])
        assert not np.any(s.x == model.mask_id)          # fully unmasked at the end


def _bruteforce_step(model, cache_tok, cache_pos, d_tok, d_pos, c_pos):
    """One step from scratch with Python loops: every key's kind decides
    visibility pair by pair, scores and softmax element by element."""
    m = model
    n_r = m.n_registers
    q_ids = list(d_tok) + [m.mask_id] * len(c_pos) + list(m.register_ids())
    q_pos = list(d_pos) + list(c_pos) + list(m.register_pos())
    q_kind = ["new"] * len(d_tok) + ["decode"] * len(c_pos) + ["register"] * n_r
    k_ids = list(cache_tok) + q_ids
    k_pos = list(cache_pos) + q_pos
    k_kind = ["cached"] * len(cache_tok) + q_kind
    q, _, _ = m.qkv_layer1(np.array(q_ids), np.array(q_pos))
    _, k, v = m.qkv_layer1(np.array(k_ids), np.array(k_pos))
    vis = np.array([[masks.kind_visible(a, b) for b in k_kind] for a in q_kind])
    o = attention.attend_bruteforce(q, k, v, vis).reshape(len(q_ids), -1)
    h = o[len(d_tok):len(d_tok) + len(c_pos)]
    w = m.w
    z = np.array([[sum(h[i, t] * w[vv, t] for t in range(w.shape[1])) for vv in range(w.shape[0])]
                  for i in range(h.shape[0])])
    return o, z


def test_bruteforce_step_matches():
    cfg = tiny_bf16(n_heads=2, n_kv_heads=1, head_dim=8, vocab=20, prompt_len=4, gen_len=8,
                    n_registers=2, n_steps=2, per_step=4)
    wl = workload(cfg)
    model = Model.from_workload(wl)
    res = run_workload(wl, batches=[0], keep_steps=[0, 1], model=model)
    o0 = wl.order[0]
    r1 = res.records[1]
    d_tok = res.records[0].token[0]
    o, z = _bruteforce_step(model, wl.prompt_ids[0], np.arange(cfg.prompt_len), d_tok, o0[:4], o0[4:8])
    assert np.allclose(o, r1.o[0], rtol=1e-12, atol=1e-13)
    assert np.allclose(z, r1.z, rtol=1e-12, atol=1e-12)
    tok = decide(z)[0]
    assert np.array_equal(tok, r1.token[0])


def test_bruteforce_infill_step_matches():
    """Infilling: the clean tokens sit between the masked spans.  The second
    step of the first decoded block, rebuilt from scratch with the prompt at
    its scattered positions, matches the incremental loop."""
    cfg = tiny_infill(n_heads=2, n_kv_heads=1, head_dim=8, vocab=20, n_registers=2)
    wl = workload(cfg)
    assert not np.array_equal(wl.prompt_pos[0], np.arange(cfg.prompt_len))
    model = Model.from_workload(wl)
    res = run_workload(wl, batches=[0], n_steps=2, keep_steps=[0, 1], model=model)
    r0, r1 = res.records
    sel = r0.selected[0]
    o, z = _bruteforce_step(model, wl.prompt_ids[0], wl.prompt_pos[0], r0.token[0][sel], r0.c_pos[0][sel],
                            r1.c_pos[0])
    assert np.allclose(o, r1.o[0], rtol=1e-12, atol=1e-13)
    assert np.allclose(z, r1.z, rtol=1e-12, atol=1e-12)


def test_infill_generation_keeps_prompt_and_follows_block_order():
    """Page 3, section 3.2: the clean tokens are never re-decoded; every masked
    position is unmasked exactly once, block by block in the drawn order, each
    block within its own sub-steps."""
    cfg = tiny_infill()
    wl = workload(cfg)
    res = run_workload(wl)
    n_blocks = cfg.gen_len // cfg.block
    seen_blocks = [st.block for st in wl.semi_ar if st.sub == 0]
    assert sorted(seen_blocks) == list(range(n_blocks)) and seen_blocks != list(range(n_blocks))
    for i, b in enumerate(res.batches):
        assert np.array_equal(res.tokens[i][wl.prompt_pos[b]], wl.prompt_ids[b])
        got = np.concatenate([u[i] for u in res.unmask])
        assert np.array_equal(np.sort(got), wl.gen_pos[b])
        for k, st in enumerate(wl.semi_ar):
            blk = wl.gen_pos[b][st.block * cfg.block:(st.block + 1) * cfg.block]
            assert set(res.unmask[k][i].tolist()) <= set(blk.tolist())


def test_two_layer_workload_reaches_the_second_layer():
    """The workload's layer-2 weights are used, and they matter: the last
    layer's output differs from the first layer's, and the k/v of layer 2 are
    stored in bf16 (rounding them again changes nothing)."""
    cfg = tiny_two_layer()
    wl = workload(cfg)
    model = Model.from_workload(wl)
    assert model.layer2 is not None
    seq = SequenceOracle(model, wl.prompt_ids[0], wl.prompt_pos[0])
    seq.prefill()
    out = seq.forward(np.empty(0, np.int64), np.empty(0, np.int64), wl.order[0, :4])
    assert len(out.o_layers) == 2 and not np.allclose(out.o_layers[0], out.o_layers[1])
    from oracle.numerics import round_bf16
    assert np.array_equal(round_bf16(seq.v[1][:seq.n]), seq.v[1][:seq.n])
    assert np.array_equal(round_bf16(seq.k[1][:seq.n]), seq.k[1][:seq.n])
