"""Write the oracle's expected results for the five workloads.

    python tests/golden/make_expected.py [--untruncated] [config ...]

Calls only ``oracle`` (and the shared input generator ``mdm_inputs``); the
HIP path plays no part.  For each workload it stores, in
``tests/golden/expected_<name>.npz``:

  tokens    [B][seq_len] final sequences
  sel_pos   [B][L] positions in the order they were unmasked
  dec_tok   [B][sum n_C] decided token of every decoded row, step by step
  conf      [B][sum n_C] fp32 confidence of every decoded row
  margin    [B][sum n_C] top-1 minus top-2 logit (float64)
  conf_gap  [steps][B] fp32 confidence gap at the top-n cut (semi-AR only)
  o_steps   steps whose attention output rows were sampled
  o_rows    [len(o_steps)][B][6] sampled query-row indices of every sequence
  o_vals    [len(o_steps)][B][6][hidden] attention output (float32)
  top2_idx  [B][sum n_C][2] the two best vocabulary indices of every decision
  top2_val  [B][sum n_C][2] their exact (float64) logits
  h_rows    [len(o_steps)][B][3] decoded-row indices (within the step's C rows
            of every sequence) whose h is stored
  h_vals    [len(o_steps)][B][3][hidden] those rows' h (float64): the tests
            form the exact logits h W^T and the bf16 screen's h_bf16 W^T from
            them

With --untruncated the loop runs with truncation switched off (every masked
position present, no registers; oracle.step.SequenceOracle.forward_untruncated)
and writes ``expected_untruncated_<name>.npz`` with the same fields (query rows
[D | C], no register rows).
"""

from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from mdm_inputs import CONFIGS, get_config, make_workload  # noqa: E402
from oracle.step import run_workload  # noqa: E402


def sample_rows(n_d, n_c, n_r):
    rows = [0, n_d - 1, n_d, n_d + n_c - 1, n_d + n_c, n_d + n_c + n_r - 1]
    return sorted({r for r in rows if 0 <= r < n_d + n_c + n_r})


def o_steps_of(cfg):
    n = cfg.n_steps
    return sorted({1, n // 2, n - 1})


def expected(cfg, truncate=True):
    wl = make_workload(cfg)
    steps = o_steps_of(cfg)
    t = time.time()
    res = run_workload(wl, keep_steps=steps, truncate=truncate)
    dt = time.time() - t
    B = cfg.batch
    sel_pos = [np.concatenate([r.c_pos[b][r.selected[b]] for r in res.records]) for b in range(B)]
    dec_tok = [np.concatenate([r.token[b] for r in res.records]) for b in range(B)]
    conf = [np.concatenate([r.conf32[b] for r in res.records]) for b in range(B)]
    margin = [np.concatenate([r.margin[b] for r in res.records]) for b in range(B)]
    gaps = np.array([[r.conf_gap[b] for b in range(B)] for r in res.records], dtype=np.float64)
    t2i = [np.concatenate([r.top2_idx[b] for r in res.records]) for b in range(B)]
    t2v = [np.concatenate([r.top2_val[b] for r in res.records]) for b in range(B)]
    o_rows, o_vals, h_rows, h_vals = [], [], [], []
    for k in steps:
        r = res.records[k]
        orow, oval, hrow, hval = [], [], [], []
        for b in range(B):
            n_d, n_c = r.d_pos[b].size, r.c_pos[b].size
            rows = sample_rows(n_d, n_c, cfg.n_registers if truncate else 0)
            rows = (rows + [rows[-1]] * 6)[:6]
            orow.append(rows)
            oval.append(r.o[b][rows].astype(np.float32))
            hr = [0, n_c // 2, n_c - 1]
            hrow.append(hr)
            hval.append(r.o[b][[n_d + i for i in hr]])
        o_rows.append(orow)
        o_vals.append(np.stack(oval))
        h_rows.append(hrow)
        h_vals.append(np.stack(hval))
    out = dict(tokens=res.tokens.astype(np.int32), sel_pos=np.stack(sel_pos).astype(np.int32),
               dec_tok=np.stack(dec_tok).astype(np.int32), conf=np.stack(conf).astype(np.float32),
               margin=np.stack(margin), conf_gap=gaps, o_steps=np.array(steps, dtype=np.int32),
               o_rows=np.array(o_rows, dtype=np.int32), o_vals=np.stack(o_vals),
               top2_idx=np.stack(t2i).astype(np.int32), top2_val=np.stack(t2v),
               h_rows=np.array(h_rows, dtype=np.int32), h_vals=np.stack(h_vals))
    return out, dt


def main(args):
    truncate = "--untruncated" not in args
    names = [a for a in args if a != "--untruncated"]
    cfgs = [get_config(n) for n in names] if names else list(CONFIGS)
    for cfg in cfgs:
        out, dt = expected(cfg, truncate)
        stem = "expected_" if truncate else "expected_untruncated_"
        path = os.path.join(HERE, f"{stem}{cfg.name}.npz")
        np.savez_compressed(path, **out)
        print(f"{cfg.name}: oracle {dt:.1f}s, min margin {out['margin'].min():.3g}, "
              f"min conf gap {np.nanmin(out['conf_gap']) if np.isfinite(out['conf_gap']).any() else float('nan'):.3g}"
              f" -> {os.path.relpath(path, ROOT)}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
