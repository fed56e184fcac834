"""The speed-up switches (page 1, ablation Table 6) on the GPU against the oracle.

Every setting of cache prompt / cache res / truncate res, and the plain
bidirectional dense MDM, generates whole sequences through the C ABI
(masked_discrete_diffusion_amd.ablation).  With truncation on, the decisions
must be the sparse loop's (oracle run_workload); with it off, those of the
untruncated loop (run_workload(truncate=False)): every decoded token and the
final sequences bit for bit, confidences within the precision's bar.  On the
small workloads the attention outputs are checked too: the decoded rows
against the oracle's rows, and sampled rows of every other kind a setting
computes (recomputed prompt rows, decoded rows, masked rows that are not
decoded this step, every row of the bidirectional step) against the oracle's
attention over the keys that row sees (clean rows: the prompt and the decoded
tokens; every other row: everything present).  At full size (the 1024- and
4096-token text-to-image workloads) every setting's decisions are compared
with the stored oracle results (tests/golden).
"""

import os

import numpy as np
import pytest

from mdm_inputs import get_config, make_workload
from oracle.attention import attend
from oracle.step import Model, run_workload
from small_workloads import gpu_small_d128, gpu_small_fp32, workload

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}
TIGHT = {"bf16": 2e-4, "fp32": 1e-5}


def _switches():
    from masked_discrete_diffusion_amd.ablation import ALL_SWITCHES
    return ALL_SWITCHES


SW_IDS = ["none", "cache_prompt", "cache_res", "truncate", "cache_prompt+cache_res", "cache_prompt+truncate",
          "all", "dense_bidirectional"]


def _oracle_rows(model, q_tok, q_pos, k_tok, k_pos):
    q, _, _ = model.qkv_layer1(np.asarray(q_tok), np.asarray(q_pos))
    _, k, v = model.qkv_layer1(np.asarray(k_tok), np.asarray(k_pos))
    return attend(q, k, v, np.ones((len(q_tok), len(k_tok)), dtype=bool)).reshape(len(q_tok), -1)


def _pick(n):
    return sorted({0, n // 2, n - 1}) if n else []


@pytest.mark.parametrize("sw_i", range(8), ids=SW_IDS)
@pytest.mark.parametrize("cfgfn", [gpu_small_d128, gpu_small_fp32], ids=["bf16", "fp32"])
def test_switches_match_oracle(cfgfn, sw_i):
    from masked_discrete_diffusion_amd.ablation import AblationRunner
    sw = _switches()[sw_i]
    cfg = cfgfn()
    print(f"switches {sw.name} on {cfg.name}", flush=True)
    wl = workload(cfg)
    model = Model.from_workload(wl)
    keep = sorted({1, cfg.n_steps // 2, cfg.n_steps - 1})
    ref = run_workload(wl, keep_steps=keep, model=model, truncate=sw.truncate)
    run = AblationRunner(wl, sw, device="cuda")
    recs, seq = run.generate_recorded(keep_o=keep)
    run.close()
    rtol, atol = TOL[cfg.precision]
    P, B = cfg.prompt_len, cfg.batch
    for k, rec in enumerate(recs):
        r = ref.records[k]
        want_tok = np.stack(r.token)
        assert np.array_equal(rec["token"], want_tok), f"step {k}: decoded tokens differ"
        want_conf = np.stack(r.conf32).astype(np.float64)
        assert np.all(np.abs(rec["conf"] - want_conf) <= atol + rtol * np.abs(want_conf)), f"step {k}: conf"
    assert np.array_equal(seq, ref.tokens), "final sequences differ"

    counts = [int(c) for c in wl.counts]
    for k in keep:
        rec, r = recs[k], ref.records[k]
        c0, n_c = sum(counts[:k]), counts[k]
        n_dprev = counts[k - 1] if k else 0
        for b in range(B):
            order = wl.order[b].astype(np.int64)
            a_tok, a_pos = wl.prompt_ids[b].astype(np.int64), wl.prompt_pos[b].astype(np.int64)
            e_pos = order[:c0]
            e_tok = ref.tokens[b][e_pos].astype(np.int64)
            m_pos = order[c0:]
            m_tok = np.full(m_pos.size, cfg.vocab, np.int64)
            every_tok = np.concatenate([a_tok, e_tok, m_tok])
            every_pos = np.concatenate([a_pos, e_pos, m_pos])
            clean_tok, clean_pos = np.concatenate([a_tok, e_tok]), np.concatenate([a_pos, e_pos])
            o = rec["o"][b]
            # the decoded rows: the oracle's own rows
            n_d = r.d_pos[b].size
            want = r.o[b][n_d:n_d + n_c]
            got = o[rec["c_row"]:rec["c_row"] + n_c]
            err = np.abs(got - want)
            assert np.all(err <= atol + rtol * np.abs(want)), f"step {k} seq {b}: decoded rows"
            assert err.max() <= TIGHT[cfg.precision] * np.abs(want).max(), f"step {k} seq {b}: decoded rows (tight)"
            checks = []
            if sw.bidirectional:
                rows = _pick(P) + [P + i for i in _pick(c0)] + [P + c0 + n_c + i for i in _pick(cfg.gen_len - c0 - n_c)]
                q_tok, q_pos = every_tok[rows], every_pos[rows]
                checks.append((o[rows], q_tok, q_pos, every_tok, every_pos, "every row"))
            else:
                if sw.cache_prompt and sw.cache_res:
                    c_tok, c_pos = e_tok[c0 - n_dprev:], e_pos[c0 - n_dprev:]
                elif sw.cache_prompt:
                    c_tok, c_pos = e_tok, e_pos
                elif sw.cache_res:
                    c_tok = np.concatenate([e_tok[c0 - n_dprev:], a_tok])
                    c_pos = np.concatenate([e_pos[c0 - n_dprev:], a_pos])
                else:
                    c_tok, c_pos = clean_tok, clean_pos
                oc = o if sw.truncate else rec["o_clean"][b]
                rows = _pick(c_tok.size)
                if rows:
                    assert oc.shape[0] >= c_tok.size
                    checks.append((oc[rows], c_tok[rows], c_pos[rows], clean_tok, clean_pos, "clean rows"))
                if not sw.truncate:
                    rows = [n_c + i for i in _pick(m_pos.size - n_c)]
                    if rows:
                        checks.append((o[rows], m_tok[rows], m_pos[rows], every_tok, every_pos, "masked rows"))
            for got, q_tok, q_pos, k_tok, k_pos, what in checks:
                want = _oracle_rows(model, q_tok, q_pos, k_tok, k_pos)
                err = np.abs(got - want)
                assert np.all(err <= atol + rtol * np.abs(want)), f"step {k} seq {b}: {what}"
                assert err.max() <= TIGHT[cfg.precision] * np.abs(want).max(), f"step {k} seq {b}: {what} (tight)"


@pytest.mark.parametrize("name", ["c2_t2i_1k", "c3_t2i_4k"])
def test_switches_full_size_decisions(name):
    from masked_discrete_diffusion_amd.ablation import AblationRunner
    cfg = get_config(name)
    wl = make_workload(cfg)
    rtol, atol = TOL[cfg.precision]
    exp = {t: np.load(os.path.join(GOLDEN, f"expected_{'' if t else 'untruncated_'}{name}.npz"))
           for t in (True, False)}
    for sw in _switches():
        print(f"full-size switches {sw.name} on {name}", flush=True)
        run = AblationRunner(wl, sw, device="cuda")
        recs, seq = run.generate_recorded()
        run.close()
        e = exp[sw.truncate]
        dec_tok = np.concatenate([r["token"] for r in recs], axis=1)
        sel_pos = np.concatenate([r["sel_pos"] for r in recs], axis=1)
        conf = np.concatenate([r["conf"] for r in recs], axis=1)
        assert np.array_equal(sel_pos, e["sel_pos"]), f"{sw.name}: unmask order"
        assert np.array_equal(dec_tok, e["dec_tok"]), f"{sw.name}: decoded tokens differ"
        assert np.array_equal(seq, e["tokens"]), f"{sw.name}: final sequences differ"
        err = np.abs(conf.astype(np.float64) - e["conf"].astype(np.float64))
        assert np.all(err <= atol + rtol * np.abs(e["conf"])), f"{sw.name}: confidence error {err.max():.3g}"
        print(f"  {sw.name}: {dec_tok.size} decisions identical, max conf err {err.max():.3g}", flush=True)


def test_cache_rewind_bookkeeping_and_errors():
    """mdm_cache_rewind: shortens the host cache length, refuses lengths
    outside [0, length] and contexts with upper layers, and drops the queries
    the last append kept (the fused order step then refuses a non-zero
    n_new_cached)."""
    from masked_discrete_diffusion_amd import _lib as L
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    from small_workloads import gpu_two_layer
    cfg = gpu_small_d128()
    run = SparseStepRunner(workload(cfg), device="cuda", fused=False)
    try:
        run.prefill()
        P = cfg.prompt_len
        assert L.mdm_cache_len(run.ctx) == P
        for bad in (P + 1, -1):
            with pytest.raises(L.MdmError) as e:
                L.mdm_cache_rewind(run.ctx, bad)
            assert e.value.status == L.MDM_E_ARG
        L.mdm_cache_rewind(run.ctx, P)                      # no-op
        assert L.mdm_cache_len(run.ctx) == P
        n = 4
        L.mdm_kv_append(run.ctx, run.prompt_tok, run.prompt_pos, P, n)   # queries kept for these n rows
        L.mdm_cache_rewind(run.ctx, P + n - 1)
        assert L.mdm_cache_len(run.ctx) == P + n - 1
        with pytest.raises(L.MdmError) as e:
            L.mdm_order_step(run.ctx, n - 1, run.order, cfg.gen_len, 1, 0, run.outs[0], run.conf, run.token,
                             None, None)
        assert e.value.status == L.MDM_E_ARG
        L.mdm_device_status(run.ctx)
    finally:
        run.close()
    cfg2 = gpu_two_layer()
    run2 = SparseStepRunner(workload(cfg2), device="cuda")
    try:
        with pytest.raises(L.MdmError) as e:
            L.mdm_cache_rewind(run2.ctx, 0)
        assert e.value.status == L.MDM_E_UNSUPPORTED
    finally:
        run2.close()
