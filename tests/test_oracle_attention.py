"""Pins for the oracle's attention, logits and selection.

* brute force: element-by-element attention vs the vectorised one;
* closed form (paperlayer.ai summary, section 7.2): when every masked position
  is decoded in one step and there are no registers, the sparse step equals the
  standard dense MDM step; for one layer the decoded rows equal textbook full
  bidirectional attention over the materialised sequence, computed here by
  PyTorch's scaled_dot_product_attention;
* forbidden keys (invariant c): perturbing keys the mask forbids leaves the
  rows that may not see them bit-identical;
* cache order: softmax is permutation invariant, so the append order of the
  cache does not matter;
* confidence = max softmax probability (scipy), argmax ties -> lowest index.
"""

import copy

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention, logits, masks, select
from oracle.numerics import table_values
from oracle.step import Model, SequenceOracle
from small_workloads import tiny_bf16, workload


def test_attend_matches_bruteforce():
    rng = np.random.default_rng(0)
    for n_h, n_kv in [(2, 2), (4, 2), (4, 1)]:
        q = rng.standard_normal((5, n_h, 6))
        k = rng.standard_normal((9, n_kv, 6))
        v = rng.standard_normal((9, n_kv, 6))
        vis = rng.random((5, 9)) < 0.6
        vis[:, 0] = True
        a = attention.attend(q, k, v, vis)
        b = attention.attend_bruteforce(q, k, v, vis)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def _sdpa(q, k, v):
    """Full bidirectional attention, q/k/v [n, H, d] float64, via torch."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("precision", ["none", "bf16"])
def test_all_masked_decoded_at_once_equals_full_attention(precision):
    cfg = tiny_bf16(n_registers=0)
    wl = workload(cfg)
    model = Model.from_workload(wl, precision=precision)
    seq = SequenceOracle(model, wl.prompt_ids[0])
    seq.prefill()
    # decode some positions first so the cache holds prompt + decoded tokens
    rng = np.random.default_rng(5)
    gen = np.arange(cfg.prompt_len, cfg.seq_len)
    first = rng.choice(gen, 5, replace=False)
    toks = rng.integers(0, cfg.vocab, 5)
    seq.forward(np.empty(0, int), np.empty(0, int), first)        # step that decoded `first`
    seq.write_tokens(first, toks)
    rest = np.setdiff1d(gen, first)                                 # C = every masked position
    out = seq.forward(toks, first, rest)
    # the materialised sequence: prompt + decoded tokens + [MASK] everywhere else
    x = seq.x.copy()
    x[rest] = model.mask_id
    q, k, v = model.qkv_layer1(x, np.arange(cfg.seq_len))
    g = cfg.n_heads // cfg.n_kv_heads
    k = np.repeat(k, g, axis=1)
    v = np.repeat(v, g, axis=1)
    full = _sdpa(q, k, v).reshape(cfg.seq_len, -1)
    assert np.allclose(out.h, full[rest], rtol=1e-12, atol=1e-13)


def test_empty_cache_new_rows_are_plain_self_attention():
    cfg = tiny_bf16(n_registers=0)
    wl = workload(cfg)
    model = Model.from_workload(wl, precision="none")
    seq = SequenceOracle(model, np.empty(0, np.int64))
    ids = np.array([3, 9, 1, 7])
    pos = np.array([2, 11, 4, 8])
    out = seq.forward(ids, pos, np.empty(0, int))
    q, k, v = model.qkv_layer1(ids, pos)
    g = cfg.n_heads // cfg.n_kv_heads
    full = _sdpa(q, np.repeat(k, g, 1), np.repeat(v, g, 1)).reshape(4, -1)
    assert np.allclose(out.o[:4], full, rtol=1e-12, atol=1e-13)


def _state_after_two_steps(model, wl):
    seq = SequenceOracle(model, wl.prompt_ids[0])
    seq.prefill()
    o = wl.order[0]
    seq.forward(np.empty(0, int), np.empty(0, int), o[:4])
    seq.write_tokens(o[:4], np.arange(4))
    seq.forward(np.arange(4), o[:4], o[4:8])
    seq.write_tokens(o[4:8], np.arange(4, 8))
    return seq, o


def test_forbidden_keys_do_not_change_new_rows():
    cfg = tiny_bf16()
    wl = workload(cfg)
    model = Model.from_workload(wl)
    seq, o = _state_after_two_steps(model, wl)
    d_tok, d_pos, c_pos = np.arange(4, 8), o[4:8], o[8:12]
    base = copy.deepcopy(seq).forward(d_tok, d_pos, c_pos)
    # perturb the K/V rows of everything a new row may not see: the mask row and registers
    bad = copy.deepcopy(model)
    bad.tk = table_values(model.tk).copy()
    bad.tv = table_values(model.tv).copy()
    forbidden = [model.mask_id] + list(model.register_ids())
    rng = np.random.default_rng(3)
    bad.tk[forbidden] = rng.standard_normal(bad.tk[forbidden].shape) * 50
    bad.tv[forbidden] = rng.standard_normal(bad.tv[forbidden].shape) * 50
    seq2 = copy.deepcopy(seq)
    seq2.m = bad
    pert = seq2.forward(d_tok, d_pos, c_pos)
    n_d = d_tok.size
    assert np.array_equal(base.o[:n_d], pert.o[:n_d])             # bit-identical
    assert not np.allclose(base.o[n_d:], pert.o[n_d:])            # the others do see them


def test_cache_order_does_not_matter():
    cfg = tiny_bf16()
    wl = workload(cfg)
    model = Model.from_workload(wl)
    seq, o = _state_after_two_steps(model, wl)
    base = copy.deepcopy(seq).forward(np.arange(4, 8), o[4:8], o[8:12])
    perm = np.random.default_rng(0).permutation(seq.n)
    shuf = copy.deepcopy(seq)
    shuf.k[0][:seq.n] = seq.k[0][perm]
    shuf.v[0][:seq.n] = seq.v[0][perm]
    out = shuf.forward(np.arange(4, 8), o[4:8], o[8:12])
    assert np.allclose(base.o, out.o, rtol=1e-12, atol=1e-14)


def test_confidence_is_max_softmax_probability():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((50, 300)) * 4
    tok, c32, c64, margin = logits.decide(z)
    p = scipy.special.softmax(z, axis=1)
    assert np.allclose(c64, p.max(axis=1), rtol=1e-13)
    assert np.array_equal(tok, p.argmax(axis=1))
    assert np.all(c32 == c64.astype(np.float32))
    srt = np.sort(z, axis=1)
    assert np.allclose(margin, srt[:, -1] - srt[:, -2], rtol=0, atol=0)


def test_argmax_ties_go_to_lowest_index_in_fp32():
    z = np.array([[0.5, 2.0, 1.0, 2.0],
                  [1.0, 1.0 + 2.0 ** -30, 0.0, 1.0]])        # second row: an fp32 tie
    tok = logits.decide(z)[0]
    assert tok.tolist() == [1, 0]


def test_select_by_confidence_ties_and_order():
    pos = np.array([40, 12, 33, 7, 25])
    conf = np.array([0.5, 0.9, 0.5, 0.1, 0.5], dtype=np.float32)
    sel, rem = select.select_by_confidence(pos, conf, 3)
    # 0.9 at pos 12, then the 0.5 tie broken towards lower positions: 25, 33
    assert pos[sel].tolist() == [12, 25, 33]
    assert pos[rem].tolist() == [7, 40]
    sel, rem = select.select_by_confidence(pos, conf, 0)
    assert sel.size == 0 and pos[rem].tolist() == [7, 12, 25, 33, 40]


def test_kind_rule_rejects_querying_cached_rows():
    with pytest.raises(ValueError):
        masks.kind_visible("cached", "new")
