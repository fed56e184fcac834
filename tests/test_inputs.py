"""Properties of the seeded workload definition (schedules, orders, shapes)."""

import math

import numpy as np
import pytest

from mdm_inputs import CONFIGS, cosine_counts, get_config, make_workload, stratified_order_2d
from mdm_inputs.generate import infill_positions, semi_ar_plan


@pytest.mark.parametrize("L", [1024, 4096])
def test_cosine_schedule(L):
    n = cosine_counts(L, 64)
    assert n.sum() == L and n.min() >= 1 and n.size == 64
    # follows the derivative of L*(1-cos(pi/2 t)): few tokens first, many last
    cont = [L * (math.cos(math.pi / 2 * (k - 1) / 64) - math.cos(math.pi / 2 * k / 64)) for k in range(1, 65)]
    assert np.max(np.abs(n - np.array(cont))) <= 1.0
    assert n[0] < 5 and n[-1] > L / 45


def test_c3_schedule_values():
    n = cosine_counts(4096, 64)
    assert n[:6].tolist() == [2, 3, 7, 8, 11, 14] and n.max() == 101


@pytest.mark.parametrize("grid", [8, 32, 64])
def test_stratified_order(grid):
    rng = np.random.default_rng(0)
    o = stratified_order_2d(grid, rng)
    assert np.array_equal(np.sort(o), np.arange(grid * grid))
    n_cells = (grid // 4) ** 2
    cell = (o // grid // 4) * (grid // 4) + (o % grid) // 4
    for j in range(16):
        run = cell[j * n_cells:(j + 1) * n_cells]
        assert np.array_equal(np.sort(run), np.arange(n_cells))   # one per cell per round


def test_semi_ar_plan():
    plan = semi_ar_plan(get_config("c5_text_semi_ar"))
    assert len(plan) == 128
    assert [s.n_cand for s in plan[:8]] == [32, 24, 16, 8] * 2
    assert all(s.n_select == 8 for s in plan)


def test_workloads_are_deterministic_and_shaped():
    cfg = get_config("c1_tiny")
    a, b = make_workload(cfg), make_workload(cfg)
    assert np.array_equal(a.tq, b.tq) and np.array_equal(a.order, b.order)
    assert a.tq.shape == (cfg.table_rows, cfg.hidden) and a.tq.dtype == np.float32
    assert np.array_equal(np.sort(a.order[0]), np.arange(cfg.prompt_len, cfg.seq_len))
    c = make_workload(cfg, tables=False)
    assert np.array_equal(c.prompt_ids, a.prompt_ids) and np.array_equal(c.order, a.order)
    # variance 1/sqrt(hidden) embeddings and projections give O(1) q/k/v rows
    assert 0.7 < a.tq.std() < 1.3


def test_c3_order_and_prompt_without_tables():
    cfg = get_config("c3_t2i_4k")
    wl = make_workload(cfg, tables=False)
    assert wl.order.shape == (4, 4096) and wl.prompt_ids.shape == (4, 256)
    for b in range(4):
        assert np.array_equal(np.sort(wl.order[b]), np.arange(256, 256 + 4096))
    assert wl.prompt_ids.min() >= 0 and wl.prompt_ids.max() < cfg.vocab


def test_config_table():
    assert [c.name for c in CONFIGS] == ["c1_tiny", "c2_t2i_1k", "c3_t2i_4k", "c4_edit", "c5_text_semi_ar"]
    c5 = get_config(4)
    assert c5.group == 4 and c5.hidden == 4096 and c5.table_rows == 128000 + 1 + 64


@pytest.mark.parametrize("seq_len,gen_len,spans", [(21, 16, 3), (40, 16, 1), (12, 6, 6), (200, 150, 17)])
def test_infill_positions_partition(seq_len, gen_len, spans):
    rng = np.random.default_rng(seq_len * 7 + spans)
    clean, masked = infill_positions(seq_len, gen_len, spans, rng)
    assert masked.size == gen_len and clean.size == seq_len - gen_len
    assert np.array_equal(np.sort(np.concatenate([clean, masked])), np.arange(seq_len))
    m = np.zeros(seq_len, bool)
    m[masked] = True
    starts = np.nonzero(m & ~np.concatenate([[False], m[:-1]]))[0]
    assert starts.size == spans and starts.min() >= 1       # every span follows a clean token


def test_text_variant_workload():
    from small_workloads import tiny_infill
    cfg = tiny_infill()
    wl = make_workload(cfg, tables=False)
    assert wl.prompt_pos.shape == (cfg.batch, cfg.prompt_len) and wl.gen_pos.shape == (cfg.batch, cfg.gen_len)
    for b in range(cfg.batch):
        assert np.array_equal(np.sort(np.concatenate([wl.prompt_pos[b], wl.gen_pos[b]])), np.arange(cfg.seq_len))
    blocks = [st.block for st in wl.semi_ar if st.sub == 0]
    assert sorted(blocks) == list(range(cfg.gen_len // cfg.block))
    # the extra seed stream leaves the tables, prompt and plan sizes of the plain config unchanged
    plain = make_workload(cfg.replace(infill_spans=0, block_order="ltr"), tables=False)
    assert np.array_equal(plain.prompt_ids, wl.prompt_ids)
    assert np.array_equal(plain.prompt_pos[0], np.arange(cfg.prompt_len))
