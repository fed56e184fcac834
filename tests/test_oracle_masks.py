"""Pins for the step-causal mask and the sparse representation against the
pages' worked examples (tests/golden/*.txt, each with its citation)."""

import os

import numpy as np

from oracle import masks, sparse_repr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.split()
    return out


def test_sparse_example_round_trip():
    g = _read("kd1_sparse_example.txt")
    words = g["tokens"]
    vocab = {w: i for i, w in enumerate(sorted(set(words) - {"[m]"}))}
    mask_id = len(vocab)
    seq = np.array([vocab.get(w, mask_id) for w in words])
    tok, pos, length = sparse_repr.to_sparse(seq, mask_id)
    clean = [w.split("@") for w in g["clean"]]
    assert length == int(g["length"][0])
    assert [p + 1 for p in pos] == [int(p) for _, p in clean]            # 1-indexed on the page
    assert [tok_i for tok_i in tok] == [vocab[w] for w, _ in clean]
    assert [p + 1 for p in sparse_repr.masked_positions(pos, length)] == [int(x) for x in g["masked"]]
    assert np.array_equal(sparse_repr.from_sparse(tok, pos, length, mask_id), seq)
    regs = sparse_repr.register_positions(length, 64)
    assert regs[0] + 1 == int(g["first_register_position"][0])
    assert regs[-1] + 1 == int(g["registers_64_last_position"][0])


def test_sparse_round_trip_random():
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(1, 60))
        seq = rng.integers(0, 9, n)
        seq[rng.random(n) < rng.random()] = 9
        tok, pos, length = sparse_repr.to_sparse(seq, 9)
        assert np.array_equal(sparse_repr.from_sparse(tok, pos, length, 9), seq)
        perm = rng.permutation(tok.size)                  # order of the clean list is free
        assert np.array_equal(sparse_repr.from_sparse(tok[perm], pos[perm], length, 9), seq)


def test_fig3_visibility_table():
    g = _read("fig3_visibility.txt")
    kinds = ["cached", "new", "decode", "register"]
    for qk in ["new", "decode", "register"]:
        want = [int(x) for x in g["row " + qk]]
        got = [int(masks.kind_visible(qk, kk)) for kk in kinds]
        assert got == want, qk
    # the example as a whole step: keys in append order cache|new|decode|registers
    n_cache, n_new, n_dec, n_reg = len(g["cached"]), len(g["new"]), len(g["decode"]), 4
    vis = masks.step_mask(n_cache, n_new, n_dec, n_reg)
    assert vis.shape == (n_new + n_dec + n_reg, n_cache + n_new + n_dec + n_reg)
    assert vis[:n_new, :n_cache + n_new].all() and not vis[:n_new, n_cache + n_new:].any()
    assert vis[n_new:].all()
    # every position of the sequence is cached, new, decoded or truncated exactly once
    allpos = sorted(int(x) for k in ["cached", "new", "decode", "truncated"] for x in g[k])
    assert allpos == list(range(1, int(g["length"][0]) + 1))


def test_step_mask_is_a_per_row_prefix():
    # In append order [cache | new | decode | registers] every row sees a prefix
    # of the keys: new rows the first cache+new keys, the others all keys.
    for n_cache, n_new, n_dec, n_reg in [(0, 3, 2, 1), (5, 0, 4, 2), (7, 3, 0, 3), (2, 2, 2, 0)]:
        vis = masks.step_mask(n_cache, n_new, n_dec, n_reg)
        n_k = vis.shape[1]
        lens = np.array([n_cache + n_new] * n_new + [n_k] * (n_dec + n_reg))
        assert np.array_equal(vis, np.arange(n_k)[None, :] < lens[:, None])


def test_block_mask_rules():
    # prompt block 0, clean blocks 1..3, masked blocks 4 and 5
    blocks = np.array([0, 0, 1, 2, 2, 3, 4, 4, 5, 5])
    vis = masks.block_mask(blocks, blocks, 3)
    for i, bi in enumerate(blocks):
        for j, bj in enumerate(blocks):
            if bi <= 3:
                assert vis[i, j] == (bj <= bi)
            else:
                assert vis[i, j] == (bj == bi or bj <= 3)
    assert not vis[6, 8] and not vis[8, 6]           # masked blocks never see each other


def test_block_mask_single_masked_block_equals_inference_rule():
    # cache = prompt + blocks 1..M-1, new = block M, masked block M+1 = decode + registers
    rng = np.random.default_rng(1)
    for _ in range(20):
        sizes = rng.integers(1, 4, size=int(rng.integers(1, 5)))     # prompt, clean 1..M
        m = sizes.size - 1
        n_dec, n_reg = int(rng.integers(1, 4)), int(rng.integers(0, 3))
        blocks = np.concatenate([np.full(s, j) for j, s in enumerate(sizes)] +
                                [np.full(n_dec + n_reg, m + 1)])
        n_cache = int(sizes[:-1].sum()) if m >= 1 else 0
        n_new = int(sizes[-1]) if m >= 1 else 0
        if m == 0:
            continue
        vis_block = masks.block_mask(blocks, blocks, m)[n_cache:]
        assert np.array_equal(vis_block, masks.step_mask(n_cache, n_new, n_dec, n_reg))
