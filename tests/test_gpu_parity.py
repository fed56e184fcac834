"""Parity of the HIP path with the CPU oracle, through the C ABI.

Bars (written here, applied element by element):
* decoded tokens, unmasked positions and their order: bit-exact;
* bf16 path: attention outputs, confidences and screened logits within
  2e-2 relative + 1e-2 absolute; fp32 path: 1e-5 relative + 1e-5 absolute;
* a tighter diagnostic on attention outputs (max |err| / max |ref|) that a
  mask bug would break even where the loose bar would not (2e-4; 4e-3 with
  two layers, where a layer-2 key or value computed in fp32 may round to the
  bf16 neighbour of the oracle's float64 value: one bf16 ulp, 2^-8);
* keys written to the cache: bit-exact (the RoPE rule rounds once from an
  exact double);
* two layers: the logits of a row may further move by ||W_v||_1 times the
  output bound 2^-8 max|O| (an output that moved by one bf16 ulp of a layer-2
  value moves logit v by at most the l1 norm of vocab row v times that).
"""

import numpy as np
import pytest

from mdm_inputs import make_workload
from oracle.numerics import round_bf16, table_values
from oracle.step import Model, SequenceOracle, run_workload
from small_workloads import (gpu_small_bf16, gpu_small_d128, gpu_small_fp32, gpu_small_semi_ar, gpu_text_infill,
                             gpu_two_layer, gpu_two_layer_semi_ar, gpu_two_layer_wide, gpu_wide_fixed,
                             gpu_wide_semi_ar, gpu_wide_semi_ar_192)
from mdm_inputs import get_config

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-5, 1e-5)}
TIGHT = {"bf16": 2e-4, "fp32": 1e-5}
TIGHT_UPPER = 2.0 ** -8


def _say(msg):
    print(msg, flush=True)


def assert_close(got, ref, rtol, atol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside tolerance, "
                           f"max abs err {np.nanmax(err):.3g}")
    return float(np.nanmax(err)) if err.size else 0.0


def bf16_flip_room(h, eps):
    """Per element of h (float64): one bf16 ulp where h lies within eps of a
    bf16 rounding boundary (a value computed with error up to eps may round to
    the other neighbour), else 0."""
    b = round_bf16(h)
    mag = np.where(b != 0, np.abs(b), np.finfo(np.float32).tiny)
    ulp = np.exp2(np.floor(np.log2(mag)) - 7)
    near = (ulp / 2 - np.abs(h - b)) <= eps
    return np.where(near, ulp, 0.0)


def _runner(cfg, **kw):
    import torch
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    wl = make_workload(cfg)
    return wl, SparseStepRunner(wl, device="cuda", **kw)


SMALL = [gpu_small_bf16, gpu_small_d128, gpu_small_semi_ar, gpu_small_fp32,
         lambda: get_config("c1_tiny")]


@pytest.mark.parametrize("cfgfn", SMALL, ids=["bf16_d64", "bf16_d128", "semi_ar", "fp32_d128", "c1_tiny"])
def test_append_keys_bit_exact(cfgfn):
    cfg = cfgfn()
    _say(f"append parity: {cfg.name}")
    wl, run = _runner(cfg)
    run.prefill()
    import torch
    torch.cuda.synchronize()
    P, d, S = cfg.prompt_len, cfg.head_dim, run.slots
    kc = run.k_cache.cpu().numpy().reshape(cfg.batch, cfg.n_kv_heads, S, d)
    # V^T in 64-slot tiles: [B][Hkv][S/64][d][64] -> [B][Hkv][d][S]
    vc = run.v_cache.cpu().numpy().reshape(cfg.batch, cfg.n_kv_heads, S // 64, d, 64)
    vc = vc.transpose(0, 1, 3, 2, 4).reshape(cfg.batch, cfg.n_kv_heads, d, S)
    model = Model.from_workload(wl)
    for b in range(cfg.batch):
        seq = SequenceOracle(model, wl.prompt_ids[b])
        seq.prefill()
        k_ref = seq.k[0][:P]                                  # [P, Hkv, d] float64 storage values
        v_ref = seq.v[0][:P]
        k_gpu = table_values(kc[b].view(np.uint16) if cfg.precision == "bf16" else kc[b])[:, :P]
        v_gpu = table_values(vc[b].view(np.uint16) if cfg.precision == "bf16" else vc[b])[:, :, :P]
        assert np.array_equal(k_gpu.transpose(1, 0, 2), k_ref), f"keys differ (b={b})"
        assert np.array_equal(v_gpu.transpose(2, 0, 1), v_ref), f"values differ (b={b})"
        pos = run.cache_pos.cpu().numpy().reshape(cfg.batch, S)[b, :P]
        tok = run.cache_tok.cpu().numpy().reshape(cfg.batch, S)[b, :P]
        assert np.array_equal(pos, np.arange(P)) and np.array_equal(tok, wl.prompt_ids[b])
    run.close()


@pytest.mark.parametrize("cfgfn", SMALL, ids=["bf16_d64", "bf16_d128", "semi_ar", "fp32_d128", "c1_tiny"])
def test_generation_matches_oracle(cfgfn):
    cfg = cfgfn()
    _say(f"generation parity: {cfg.name}")
    wl, run = _runner(cfg)
    _check_generation(cfg, wl, run)


def test_five_chunk_blocks_match_oracle():
    """Steps with 10 query chunks per head run in blocks of five, the fifth
    chunk split over wavefronts 4-7 by tile parity and key half and merged;
    every row's output is compared with the oracle."""
    from small_workloads import gpu_five_chunks
    cfg = gpu_five_chunks()
    _say(f"generation parity: {cfg.name}")
    wl, run = _runner(cfg)
    _check_generation(cfg, wl, run)


def _tie_note(cfg, wl, g, r, b, rtol, atol):
    """Diagnostic only: where the two sides decided differently, how far the
    oracle's own decision was from a tie (top-1/top-2 logit margin, or the
    confidence gap across the selection cut)."""
    bad = np.nonzero(g["token"][b] != r.token[b])[0]
    if bad.size:
        return f"oracle margins at the differing rows: {np.array2string(r.margin[b][bad], precision=3)}"
    return f"oracle confidence gap at the cut: {r.conf_gap[b]:.3g}"


def _check_generation(cfg, wl, run):
    """Free-running generation compared with the oracle step by step: every
    decided token and the unmask order must be identical at every step (a
    difference fails the test, with the oracle's margin at the differing rows
    in the message), outputs and logits within the bars."""
    steps = list(range(cfg.n_steps))
    recs, seq = run.generate_recorded(keep_o=steps, keep_logits=steps, trace=True)
    counts = run.decision_counts
    run.close()
    res = run_workload(wl, keep_steps=steps)
    rtol, atol = TOL[cfg.precision]
    accurate = bool(run.mc.accurate_conf)
    worst = {"o": 0.0, "conf": 0.0, "logits": 0.0}
    compared = 0
    for k, (g, r) in enumerate(zip(recs, res.records)):
        for b in range(cfg.batch):
            sel = r.selected[b]
            same_tok = np.array_equal(g["token"][b], r.token[b])
            same_sel = np.array_equal(g["sel_pos"][b], r.c_pos[b][sel])
            assert same_tok, f"step {k} b {b}: decoded tokens differ ({_tie_note(cfg, wl, g, r, b, rtol, atol)})"
            assert same_sel, f"step {k} b {b}: unmask order differs ({_tie_note(cfg, wl, g, r, b, rtol, atol)})"
            assert np.array_equal(g["sel_tok"][b], r.token[b][sel])
            tr = g["trace"][b].view(np.int32)
            assert np.array_equal(tr[:, 1], g["token"][b]), f"step {k} b {b}: trace token"
            assert np.all(tr[:, 7] & 8), f"step {k} b {b}: a decision without the kernel's proof"
            worst["conf"] = max(worst["conf"], assert_close(g["conf"][b], r.conf64[b], rtol, atol, f"conf step {k}"))
            o_ref = r.o[b]
            worst["o"] = max(worst["o"], assert_close(g["o"][b], o_ref, rtol, atol, f"O step {k} b {b}"))
            rel = np.max(np.abs(g["o"][b] - o_ref)) / np.max(np.abs(o_ref))
            tight = TIGHT[cfg.precision] if cfg.layers == 1 else TIGHT_UPPER
            assert rel <= tight, f"O step {k} b {b}: max err / max ref = {rel:.3g}"
        compared += 1
        zref = r.z if (cfg.precision == "fp32" or accurate) else r.z_mirror
        z_atol = atol
        if zref is r.z_mirror:
            # the screen rounds h to bf16: where the oracle's h lies within the
            # O bound of a rounding boundary the two sides may hold neighbouring
            # bf16 values, which moves logit v by |W_vi| times one ulp
            h = np.concatenate([r.o[b][len(r.d_pos[b]):len(r.d_pos[b]) + len(r.c_pos[b])] for b in range(cfg.batch)])
            eps = TIGHT[cfg.precision] * max(np.max(np.abs(r.o[b])) for b in range(cfg.batch))
            z_atol = atol + bf16_flip_room(h, eps) @ np.abs(table_values(wl.w_vocab)).T
        if cfg.layers > 1:
            w_l1 = np.abs(table_values(wl.w_vocab)).sum(axis=1)               # [V]
            o_max = max(np.max(np.abs(r.o[b])) for b in range(cfg.batch))
            z_atol = atol + w_l1[None, :] * TIGHT_UPPER * o_max
        worst["logits"] = max(worst["logits"], assert_close(
            g["logits"].reshape(-1, cfg.vocab), zref, rtol, z_atol, f"logits step {k}"))
    assert compared == cfg.n_steps
    assert np.array_equal(seq, res.tokens), "final sequences differ"
    _say(f"  {compared} steps compared, worst abs errors: {worst}; decision counters "
         f"(re-scored beyond the candidates, whole tiles, fp32 ties): {counts}")
    return counts


def test_screen_regimes_match_oracle():
    """An 8192-column vocabulary with 36 to 351 decoded rows per step, so the
    steps take every row tiling and hidden split of the bf16 screen; every
    step's screened logits are compared element by element with bf16(h) W^T
    and the decisions with the oracle's."""
    from small_workloads import gpu_screen_regimes
    cfg = gpu_screen_regimes()
    _say(f"screen regimes: {cfg.name}")
    wl, run = _runner(cfg)
    _check_generation(cfg, wl, run)


def _tied_head(wl, kind):
    """Rewrite the workload's bf16 vocabulary head so that exact ties defeat
    the screen's candidates: 'whole_tiles' repeats 12 distinct rows over the
    whole vocabulary (every 128-column tile holds ten or more copies of each,
    so a tile's third entry ties its first); 'single_entries' copies one row,
    scaled by 4 (exact in bf16), to column 5 of every tile (16 tied columns,
    one per tile).  Tied columns have bit-identical exact logits on both
    sides, so the argmax must take the lowest of their indices."""
    w = wl.w_vocab
    V = w.shape[0]
    if kind == "whole_tiles":
        w[:] = w[np.arange(V) % 12]
    else:
        f = (w[7].astype(np.uint32) << 16).view(np.float32) * np.float32(4.0)
        w[5::128] = (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", ["whole_tiles", "single_entries"])
def test_decision_rescans_on_tied_columns(kind):
    """Both re-scoring paths of the decision kernel (the single entries beyond
    the candidates, shared over the wavefronts, and whole tiles), forced by
    tied vocabulary columns: the generation must match the oracle's, every
    decision carrying the kernel's proof, and the kernel's counters must show
    the path taken."""
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    from small_workloads import gpu_decide_dup
    cfg = gpu_decide_dup()
    _say(f"decision re-scoring on tied columns: {kind}")
    wl = make_workload(cfg)
    _tied_head(wl, kind)
    run = SparseStepRunner(wl, device="cuda")
    counts = _check_generation(cfg, wl, run)
    if kind == "whole_tiles":
        assert counts[1] > 0, f"no whole-tile re-scoring: {counts}"
    else:
        assert counts[0] > 0, f"no re-scoring beyond the candidates: {counts}"


@pytest.mark.parametrize("cfgfn", [gpu_wide_semi_ar, gpu_wide_semi_ar_192, gpu_wide_fixed],
                         ids=["wide_semi_ar", "wide_semi_ar_192", "wide_fixed"])
def test_wide_vocab_tiles_match_oracle(cfgfn):
    """Vocabularies of 115k-120k take the 512-column screen tiles (with and
    without the hi/lo split of h, 64- and 128-row tiles, three 64-row tiles
    for the 144- and 192-row hi/lo steps) streamed from the tiled copy of the
    head; the generation must match the oracle like the small workloads."""
    cfg = cfgfn()
    _say(f"wide vocab parity: {cfg.name}")
    wl, run = _runner(cfg)
    _check_generation(cfg, wl, run)


@pytest.mark.parametrize("kw", [dict(), dict(precision="fp32")], ids=["bf16", "fp32"])
def test_text_infill_random_block_order_matches_oracle(kw):
    """Text variants: the clean tokens sit between four masked spans (their
    keys enter the cache at scattered positions) and the semi-AR blocks are
    decoded in a seeded random order.  Only the positions handed to the calls
    change; decisions, unmask order and outputs must match the oracle."""
    cfg = gpu_text_infill(**kw)
    _say(f"text infill parity: {cfg.name} {cfg.precision}")
    wl, run = _runner(cfg)
    _check_generation(cfg, wl, run)


@pytest.mark.parametrize("cfgfn", [gpu_two_layer, gpu_two_layer_semi_ar, gpu_two_layer_wide],
                         ids=["fixed", "semi_ar_gqa", "wide_projection"])
def test_two_layer_generation_matches_oracle(cfgfn):
    """Layer 2 projects layer 1's outputs of every query row (RoPE'd q, k and
    v rounded to bf16), keeps its own cache of the decoded rows and attends
    under the same step-causal mask; the decisions, unmask order and the last
    layer's outputs must match the oracle's two-layer model."""
    cfg = cfgfn()
    _say(f"two-layer parity: {cfg.name}")
    # screened with h split into hi + lo: the last layer's h carries layer-2
    # rounding, so the screened logits are compared with the exact ones
    wl, run = _runner(cfg, accurate_conf=True)
    _check_generation(cfg, wl, run)


def test_score_jump_falls_back_to_rescaled_path():
    """Scores that rise far above a row's first-tile maximum.  Full key tiles
    run at a reference fixed by the first full tile; when a row's sum of
    exp2(score - reference) reaches 2^50 (or overflows), the block recomputes
    on the lazily rescaled path.  The key-table row of one token is scaled by
    64 (exact in bf16) and the token is placed in the second cache tile only,
    so that (checked here on the CPU) some register row's score against it
    passes its first-tile maximum by far more than 50 in log2 units at step 0;
    the generation must still match the oracle exactly."""
    from mdm_inputs.generate import bf16_bits_from_f32, bf16_bits_to_f32
    from oracle import rope
    cfg = gpu_small_d128(index=114, name="gpu_small_score_jump", prompt_len=150)
    _say(f"score jump: {cfg.name}")
    wl = make_workload(cfg)
    hot = 5
    wl.tk[hot] = bf16_bits_from_f32(bf16_bits_to_f32(wl.tk[hot]) * np.float32(64.0))
    p = wl.prompt_ids
    p[:, :64][p[:, :64] == hot] = hot + 1
    p[:, 64:128:9] = hot
    # precondition on the CPU: register rows of step 0 against the prompt keys
    d, hk = cfg.head_dim, cfg.n_kv_heads
    cos_t, sin_t = rope.table(cfg.seq_len + cfg.n_registers, d)
    g = cfg.n_heads // hk
    jump = 0.0
    for b in range(cfg.batch):
        keys = table_values(wl.tk[p[b]]).reshape(cfg.prompt_len, hk, d)
        keys = rope.rotate(keys, np.arange(cfg.prompt_len), cos_t, sin_t)
        rid = cfg.vocab + 1 + np.arange(cfg.n_registers)
        q = table_values(wl.tq[rid]).reshape(cfg.n_registers, cfg.n_heads, d)
        q = rope.rotate(q, cfg.seq_len + np.arange(cfg.n_registers), cos_t, sin_t)
        for h in range(cfg.n_heads):
            s = q[:, h] @ keys[:, h // g].T * (1.4426950408889634 / np.sqrt(d))
            jump = max(jump, float(np.max(s[:, 64:128].max(axis=1) - s[:, :64].max(axis=1))))
    assert jump > 128.0, jump
    from masked_discrete_diffusion_amd.sampler import SparseStepRunner
    _check_generation(cfg, wl, SparseStepRunner(wl, device="cuda"))


def test_forbidden_keys_nan_poison():
    """Invariant (c) on the GPU: NaN in every key/value a new row may not see
    (this step's masked and register rows, and every slot past the visible
    prefix) leaves the new rows' outputs finite and bit-identical.  The C and R
    keys/values come from tables built at init, so the poisoned tables are
    loaded by a second context on the same buffers, whose cache is rebuilt
    from the recorded sparse representation (token id and position per slot)."""
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    cfg = gpu_small_d128()
    _say("nan poison: gpu_small_d128")
    wl, run = _runner(cfg, fused=False)
    run.prefill()
    for k in range(3):
        run.step(k)
    st = run.plan[3]
    L.mdm_kv_append(run.ctx, run.d_tok[st.d_buf], run.d_pos[st.d_buf], st.n_d, st.n_d)
    c_ptr, c_stride = run._c_src(st)
    n_q = st.n_d + st.n_c + cfg.n_registers

    def attend(ctx):
        L.mdm_step_attention(ctx, run.d_tok[st.d_buf], run.d_pos[st.d_buf], st.n_d, st.n_d,
                             c_ptr, c_stride, st.n_c, run.out)
        torch.cuda.synchronize()
        return run.out[:cfg.batch * n_q * cfg.hidden].view(cfg.batch, n_q, cfg.hidden).clone()

    ref = attend(run.ctx)
    s_len = L.mdm_cache_len(run.ctx)                 # slots past the committed rows
    k_before = run.k_cache.clone()
    v_before = run.v_cache.clone()
    nan = torch.tensor(0x7FC0, dtype=torch.int32).to(torch.int16).item()
    forbidden = [cfg.vocab] + list(range(cfg.vocab + 1, cfg.vocab + 1 + cfg.n_registers))
    run.tk.view(cfg.table_rows, -1)[forbidden] = nan
    run.tv.view(cfg.table_rows, -1)[forbidden] = nan
    ctx2 = L.mdm_sparse_step_init(run.mc, run.bufs, run.stream.cuda_stream)
    try:
        tok = run.cache_tok.clone()
        pos = run.cache_pos.clone()
        L.mdm_kv_append(ctx2, tok, pos, run.slots, s_len)
        torch.cuda.synchronize()
        kc = run.k_cache.view(cfg.batch, cfg.n_kv_heads, run.slots, cfg.head_dim)
        # V^T in 64-slot tiles: view as [B][Hkv][S/64][d][64]; slot s = 64*tile + w
        vc = run.v_cache.view(cfg.batch, cfg.n_kv_heads, run.slots // 64, cfg.head_dim, 64)
        kb = k_before.view(kc.shape)
        vb = v_before.view(vc.shape)
        vis = torch.arange(run.slots, device=vc.device).view(run.slots // 64, 1, 64) < s_len
        assert torch.equal(kc[:, :, :s_len], kb[:, :, :s_len]) and torch.equal(vc[..., vis.expand_as(vc[0, 0])],
                                                                                 vb[..., vis.expand_as(vb[0, 0])])
        kc[:, :, s_len:] = nan
        vc.masked_fill_(~vis, nan)
        got = attend(ctx2)
    finally:
        L.mdm_sparse_step_destroy(ctx2)
    n_d = st.n_d
    assert torch.isfinite(got[:, :n_d]).all()
    assert torch.equal(got[:, :n_d], ref[:, :n_d])
    assert torch.isnan(got[:, n_d:]).any()          # the others do see the poisoned rows
    run.close()


def test_rerun_is_bitwise_deterministic():
    cfg = gpu_small_semi_ar()
    _say("determinism: gpu_small_semi_ar")
    wl, run = _runner(cfg)
    steps = list(range(len(run.plan)))
    a, sa = run.generate_recorded(keep_o=steps)
    b, sb = run.generate_recorded(keep_o=steps)
    run.close()
    assert np.array_equal(sa, sb)
    for x, y in zip(a, b):
        assert np.array_equal(x["o"], y["o"]), f"attention output differs at step {x['k']}"
        assert np.array_equal(x["conf"], y["conf"]) and np.array_equal(x["token"], y["token"])


@pytest.mark.parametrize("name,steps", [("gpu_small_semi_ar", (4, 8)), ("c3_t2i_4k", (27, 40))])
def test_repeated_kernels_are_bitwise_identical(name, steps):
    """Each kernel of a step, launched repeatedly on the same inputs, returns the
    same bits (no read of unwritten or in-flight memory, no order dependence)."""
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    cfg = gpu_small_semi_ar() if name == "gpu_small_semi_ar" else get_config(name)
    _say(f"repeated kernels: {name} steps {steps}")
    wl, run = _runner(cfg, fused=False)
    run.seq_tokens.copy_(run.seq0)
    run.prefill()
    for k in range(max(steps) + 1):
        st = run.plan[k]
        if k not in steps:
            run.step(k)
            continue
        if st.n_d:
            L.mdm_kv_append(run.ctx, run.d_tok[st.d_buf], run.d_pos[st.d_buf], st.n_d, st.n_d)
        c_ptr, c_stride = run._c_src(st)
        n_q = st.n_d + st.n_c + cfg.n_registers
        h_ptr = run.out.data_ptr() + 4 * st.n_d * cfg.hidden
        outs, confs = [], []
        for rep in range(4):
            run.out.fill_(float("nan"))
            L.mdm_step_attention(run.ctx, run.d_tok[st.d_buf], run.d_pos[st.d_buf], st.n_d, st.n_d,
                                 c_ptr, c_stride, st.n_c, run.out)
            torch.cuda.synchronize()
            outs.append(run.out[:cfg.batch * n_q * cfg.hidden].cpu().numpy().copy())
        for rep in range(3):
            L.mdm_subset_logits_confidence(run.ctx, h_ptr, n_q * cfg.hidden, st.n_c, run.conf, run.token)
            torch.cuda.synchronize()
            confs.append((run.conf[:cfg.batch * st.n_c].cpu().numpy().copy(),
                          run.token[:cfg.batch * st.n_c].cpu().numpy().copy()))
        for r in range(1, len(outs)):
            assert np.array_equal(outs[0], outs[r]), \
                f"step {k}: attention repeat {r} differs in {int((outs[0] != outs[r]).sum())} elements"
        for r in range(1, len(confs)):
            assert np.array_equal(confs[0][0], confs[r][0]) and np.array_equal(confs[0][1], confs[r][1])
        rem = run.rem[st.rem_out] if st.rem_out >= 0 else None
        L.mdm_unmask_select(run.ctx, c_ptr, c_stride, run.conf, run.token, st.n_c, st.n_sel, st.mode,
                            run.d_tok[st.out_buf], run.d_pos[st.out_buf], rem, run.seq_tokens)
    torch.cuda.synchronize()
    run.close()


def test_graph_replays_match_eager():
    import torch
    cfg = gpu_small_d128()
    _say("graph replay: gpu_small_d128")
    wl, run = _runner(cfg)
    _, eager = run.generate_recorded()
    graph = run.capture_graph()
    for rep in range(3):
        run.seq_tokens.copy_(run.seq0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(run.seq_tokens.cpu().numpy(), eager), f"replay {rep}"
        _, again = run.generate_recorded(n_steps=2)          # eager work between replays
    run.close()


def test_device_range_check_and_capacity():
    import torch
    from masked_discrete_diffusion_amd import _lib as L
    cfg = gpu_small_bf16()
    _say("range checks: gpu_small_bf16")
    wl, run = _runner(cfg)
    run.prefill()
    bad_tok = torch.full((cfg.batch, 2), cfg.table_rows + 5, dtype=torch.int32, device="cuda")
    pos = torch.full((cfg.batch, 2), cfg.prompt_len, dtype=torch.int32, device="cuda")
    L.mdm_kv_append(run.ctx, bad_tok, pos, 2, 2)
    with pytest.raises(L.MdmError) as e:
        L.mdm_device_status(run.ctx)
    assert e.value.status == L.MDM_E_DEVICE
    L.mdm_device_status(run.ctx)                       # the flag was cleared
    # a sequence row at a register position (seq_len) is out of range too
    ok_tok = torch.zeros((cfg.batch, 1), dtype=torch.int32, device="cuda")
    reg_pos = torch.full((cfg.batch, 1), cfg.seq_len, dtype=torch.int32, device="cuda")
    L.mdm_kv_append(run.ctx, ok_tok, reg_pos, 1, 1)
    with pytest.raises(L.MdmError) as e:
        L.mdm_device_status(run.ctx)
    assert e.value.status == L.MDM_E_DEVICE
    with pytest.raises(L.MdmError) as e:
        L.mdm_kv_append(run.ctx, pos, pos, 2, cfg.seq_len)
    assert e.value.status in (L.MDM_E_CAPACITY, L.MDM_E_ARG)
    n_left = cfg.seq_len - L.mdm_cache_len(run.ctx)
    with pytest.raises(L.MdmError) as e:
        big = torch.zeros(cfg.batch * (n_left + 1), dtype=torch.int32, device="cuda")
        L.mdm_kv_append(run.ctx, big, big, n_left + 1, n_left + 1)
    assert e.value.status == L.MDM_E_CAPACITY
    run.close()
