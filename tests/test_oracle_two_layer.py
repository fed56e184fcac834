"""Brute-force pin of the oracle's second attention layer.

The oracle's two-layer mode (its reading of more than one layer: layer 2
projects every row's layer-1 output with W_2, whose rows are the query heads,
then the key heads, then the value heads; q and k are RoPE'd at the row's
position; q, k and v are rounded to the storage type; each layer keeps its own
cache) is recomputed here from scratch for one sampling step, with plain
Python loops and without any of the oracle's layer code (no
``Model.qkv_layer1/qkv_layer2``, ``split_layer2``, ``attend`` or masks):

* the rows are the sequence's decode groups - the prompt (group 0), then the
  tokens unmasked at each earlier step (groups 1..k), the last of which are
  the rows entering the cache now - followed by this step's masked rows and
  the registers;
* visibility follows the training-form block rule (page 1, key design 3;
  page 3, section 3.3): a committed row of group g sees every committed row of
  group <= g, in every layer (so a cached row's layer-2 key and value come
  from the layer-1 output it had when it entered the cache, page 1, worked
  example = Figure 3: the cache is not polluted by later rows); masked rows
  and registers see every row;
* every dot product, softmax and weighted sum is an explicit loop.

The incremental oracle must reproduce the last layer's outputs of this step's
query rows [new | decode | registers] and the decode rows' logits.  Mutants in
``test_oracle_mutants.py`` (layer-2 queries left unrotated, key and value
blocks of W_2 swapped, the query block transposed, values left unrounded) each
break this pin.
"""

import math

import numpy as np

from oracle import rope
from oracle.numerics import round_bf16, table_values
from oracle.step import Model, run_workload
from small_workloads import tiny_two_layer, workload


def _rotate_row(x, p, cos_t, sin_t):
    """RoPE of one head row x (list of d floats) at position p: interleaved
    pairs (2i, 2i+1) turned by the angle of pair i, products and sums in
    double precision."""
    out = list(x)
    for i in range(len(x) // 2):
        c, s = float(cos_t[p, i]), float(sin_t[p, i])
        out[2 * i] = x[2 * i] * c - x[2 * i + 1] * s
        out[2 * i + 1] = x[2 * i] * s + x[2 * i + 1] * c
    return out


def _round(vals):
    return [float(v) for v in round_bf16(np.array(vals, dtype=np.float64))]


def _attention(q, k, v, sees, n_heads, n_kv, d):
    """o[r][h*d + t] over the rows r' with sees(r, r'); q[r][h] and k/v[r][g]
    are lists of d floats; query head h reads key/value head h // (H / H_kv)."""
    grp = n_heads // n_kv
    n = len(q)
    out = []
    for r in range(n):
        row = []
        keys = [j for j in range(n) if sees(r, j)]
        for h in range(n_heads):
            g = h // grp
            scores = []
            for j in keys:
                acc = 0.0
                for t in range(d):
                    acc += q[r][h][t] * k[j][g][t]
                scores.append(acc / math.sqrt(d))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for t in range(d):
                acc = 0.0
                for wj, j in zip(w, keys):
                    acc += wj * v[j][g][t]
                row.append(acc / tot)
        out.append(row)
    return out


def bruteforce_two_layer_step(wl, b, groups, c_pos):
    """Last-layer outputs of rows [new | decode | registers] and the decode
    rows' logits for one step of sequence b.

    groups: [(token ids, positions)] - group 0 is the prompt, the last group
            holds the rows entering the cache at this step (may be the prompt).
    c_pos:  positions decoded at this step (the mask token's rows)."""
    cfg = wl.cfg
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    V, R, L = cfg.vocab, cfg.n_registers, cfg.seq_len
    hq, hk = H * d, Hk * d
    cos_t, sin_t = rope.table(L + R, d, cfg.rope_theta)
    tq, tk, tv = table_values(wl.tq), table_values(wl.tk), table_values(wl.tv)
    w2 = table_values(wl.layer_w[0])
    wv = table_values(wl.w_vocab)

    ids, pos, grp = [], [], []
    for g, (tok, ps) in enumerate(groups):
        ids += [int(t) for t in tok]
        pos += [int(p) for p in ps]
        grp += [g] * len(tok)
    n_cached = len(ids)
    masked = len(groups)                       # a label above every committed group
    ids += [V] * len(c_pos) + [V + 1 + j for j in range(R)]
    pos += [int(p) for p in c_pos] + [L + j for j in range(R)]
    grp += [masked] * (len(c_pos) + R)
    n = len(ids)

    def sees(r, j):
        if grp[r] == masked:
            return True
        return grp[j] <= grp[r]

    def heads(vec, n_h):
        return [vec[h * d:(h + 1) * d] for h in range(n_h)]

    # layer 1: table rows by id; q and k rotated at the row's position and rounded
    q1 = [[_round(_rotate_row(list(tq[ids[r]][h * d:(h + 1) * d]), pos[r], cos_t, sin_t)) for h in range(H)]
          for r in range(n)]
    k1 = [[_round(_rotate_row(list(tk[ids[r]][g * d:(g + 1) * d]), pos[r], cos_t, sin_t)) for g in range(Hk)]
          for r in range(n)]
    v1 = [heads(list(tv[ids[r]]), Hk) for r in range(n)]
    o1 = _attention(q1, k1, v1, sees, H, Hk, d)

    # layer 2: feature j of a row = <o1 row, W_2 row j>; rows of W_2 are the
    # query heads, the key heads, then the value heads
    q2, k2, v2 = [], [], []
    for r in range(n):
        y = []
        for j in range(hq + 2 * hk):
            acc = 0.0
            wrow = w2[j]
            for c in range(hq):
                acc += o1[r][c] * wrow[c]
            y.append(acc)
        q2.append([_round(_rotate_row(y[h * d:(h + 1) * d], pos[r], cos_t, sin_t)) for h in range(H)])
        k2.append([_round(_rotate_row(y[hq + g * d:hq + (g + 1) * d], pos[r], cos_t, sin_t)) for g in range(Hk)])
        v2.append([_round(y[hq + hk + g * d:hq + hk + (g + 1) * d]) for g in range(Hk)])
    o2 = _attention(q2, k2, v2, sees, H, Hk, d)

    n_new = len(groups[-1][0])
    rows = list(range(n_cached - n_new, n_cached)) + list(range(n_cached, n))
    out = np.array([o2[r] for r in rows])
    dec = list(range(n_cached, n_cached + len(c_pos)))
    z = np.array([[sum(o2[r][c] * wv[t][c] for c in range(hq)) for t in range(V)] for r in dec])
    return out, z


def _groups_before(wl, res, k, i, b):
    groups = [(wl.prompt_ids[b], wl.prompt_pos[b])]
    for r in res.records[:k]:
        sel = r.selected[i]
        groups.append((r.token[i][sel], r.c_pos[i][sel]))
    return groups


def test_two_layer_step_matches_bruteforce():
    cfg = tiny_two_layer(batch=1, n_heads=2, n_kv_heads=1, head_dim=8, vocab=24, prompt_len=5, gen_len=12,
                         n_registers=2, n_steps=3, per_step=4)
    wl = workload(cfg)
    model = Model.from_workload(wl)
    assert model.layer2 is not None and model.precision == "bf16"
    res = run_workload(wl, keep_steps=range(cfg.n_steps), model=model)
    for k in range(cfg.n_steps):
        rec = res.records[k]
        groups = _groups_before(wl, res, k, 0, 0)
        if k == 0:
            groups = groups[:1] + [(np.empty(0, np.int64), np.empty(0, np.int64))]
        o, z = bruteforce_two_layer_step(wl, 0, groups, rec.c_pos[0])
        assert o.shape == rec.o[0].shape
        assert np.allclose(o, rec.o[0], rtol=1e-11, atol=1e-13), f"step {k}: last-layer outputs differ"
        assert np.allclose(z, rec.z, rtol=1e-11, atol=1e-12), f"step {k}: logits differ"
