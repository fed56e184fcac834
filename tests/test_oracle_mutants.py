"""Each pin must catch a plausible mistake.  A mistake is planted in the oracle
(monkeypatched, CPU only) and the pin that guards it is expected to fail."""

import numpy as np
import pytest

import oracle.attention as attention_mod
import oracle.dense as dense_mod
import oracle.masks as masks_mod
import oracle.rope as rope_mod
import oracle.sparse_repr as sparse_mod
import oracle.step as step_mod
import test_oracle_attention as T_att
import test_oracle_invariants as T_inv
import test_oracle_masks as T_mask
import test_oracle_rope as T_rope


def test_mutant_new_rows_see_decode_tokens(monkeypatch):
    bad = dict(masks_mod._SEES)
    bad[masks_mod.NEW] = {masks_mod.CACHED, masks_mod.NEW, masks_mod.DECODE}
    monkeypatch.setattr(masks_mod, "_SEES", bad)
    with pytest.raises(AssertionError):
        T_mask.test_fig3_visibility_table()
    with pytest.raises(AssertionError):
        T_att.test_forbidden_keys_do_not_change_new_rows()


def test_mutant_registers_invisible_to_decode_rows(monkeypatch):
    bad = dict(masks_mod._SEES)
    bad[masks_mod.DECODE] = {masks_mod.CACHED, masks_mod.NEW, masks_mod.DECODE}
    monkeypatch.setattr(masks_mod, "_SEES", bad)
    with pytest.raises(AssertionError):
        T_mask.test_fig3_visibility_table()


def test_mutant_masked_blocks_see_each_other(monkeypatch):
    def block_mask(q_blocks, k_blocks, m):
        qb = np.asarray(q_blocks)[:, None]
        kb = np.asarray(k_blocks)[None, :]
        return np.where(qb <= m, kb <= qb, (kb > m) | (kb <= m))
    monkeypatch.setattr(masks_mod, "block_mask", block_mask)
    monkeypatch.setattr(dense_mod, "block_mask", block_mask)
    with pytest.raises(AssertionError):
        T_mask.test_block_mask_rules()
    with pytest.raises(AssertionError):
        T_inv.test_two_masked_blocks_simulate_two_paths()


def test_mutant_rope_half_split_pairs(monkeypatch):
    def rotate(x, pos, c_t, s_t):
        x = np.asarray(x, dtype=np.float64)
        c = c_t[np.asarray(pos)].astype(np.float64)
        s = s_t[np.asarray(pos)].astype(np.float64)
        while c.ndim < x.ndim:
            c, s = c[..., None, :], s[..., None, :]
        h = x.shape[-1] // 2
        out = np.empty_like(x)
        out[..., :h] = x[..., :h] * c - x[..., h:] * s
        out[..., h:] = x[..., :h] * s + x[..., h:] * c
        return out
    monkeypatch.setattr(rope_mod, "rotate", rotate)
    with pytest.raises(AssertionError):
        T_rope.test_pairs_are_interleaved_and_rotate_counterclockwise()


def test_mutant_rope_clockwise(monkeypatch):
    orig = rope_mod.rotate
    monkeypatch.setattr(rope_mod, "rotate", lambda x, pos, c, s: orig(x, pos, c, -s))
    with pytest.raises(AssertionError):
        T_rope.test_pairs_are_interleaved_and_rotate_counterclockwise()


def test_mutant_attention_without_scale(monkeypatch):
    orig = attention_mod.attend

    def attend(q, k, v, vis):
        return orig(q * np.sqrt(q.shape[-1]), k, v, vis)
    monkeypatch.setattr(attention_mod, "attend", attend)
    monkeypatch.setattr(step_mod, "attend", attend)
    with pytest.raises(AssertionError):
        T_att.test_all_masked_decoded_at_once_equals_full_attention("none")


def test_mutant_gqa_wrong_grouping(monkeypatch):
    orig = attention_mod.attend

    def attend(q, k, v, vis):      # query head h -> kv head h % H_kv instead of h // G
        n_q, n_h, d = q.shape
        n_kv = k.shape[1]
        g = n_h // n_kv
        perm = np.array([(h % n_kv) * g + h // n_kv for h in range(n_h)])
        inv = np.argsort(perm)
        return orig(q[:, inv], k, v, vis)[:, perm]
    monkeypatch.setattr(step_mod, "attend", attend)
    with pytest.raises(AssertionError):
        T_att.test_all_masked_decoded_at_once_equals_full_attention("none")


def test_mutant_register_positions_off_by_one(monkeypatch):
    monkeypatch.setattr(sparse_mod, "register_positions",
                        lambda n, r: np.arange(n + 1, n + 1 + r))
    with pytest.raises(AssertionError):
        T_mask.test_sparse_example_round_trip()


def test_mutant_new_rows_not_committed_before_attention(monkeypatch):
    orig = step_mod.step_mask
    # keys of the rows entering the cache are dropped from the new rows' view
    monkeypatch.setattr(step_mod, "step_mask",
                        lambda nc, nn, nd, nr: orig(nc, nn, nd, nr) & ~np.pad(
                            np.eye(nn + nd + nr, dtype=bool)[:, :nn], ((0, 0), (nc, nd + nr)))
                        if nn else orig(nc, nn, nd, nr))
    with pytest.raises(AssertionError):
        T_inv.test_incremental_equals_dense_block_mask(1, "bf16", T_inv.tiny_bf16)


# ---- second layer: each planted mistake must break the brute-force pin ------
import test_oracle_two_layer as T_two
from oracle.numerics import round_storage


def _qkv_layer2_variant(rotate_q=True, round_v=True):
    def qkv_layer2(self, h1, pos):
        wq, wk, wv = self.layer2
        n = h1.shape[0]
        d, h, hk = self.head_dim, self.n_heads, self.n_kv_heads
        q = (h1 @ wq).reshape(n, h, d)
        k = (h1 @ wk).reshape(n, hk, d)
        v = (h1 @ wv).reshape(n, hk, d)
        q = self._rot(q, pos) if rotate_q else round_storage(q, self.precision)
        v = round_storage(v, self.precision) if round_v else v
        return q, self._rot(k, pos), v
    return qkv_layer2


def test_mutant_layer2_queries_unrotated(monkeypatch):
    monkeypatch.setattr(step_mod.Model, "qkv_layer2", _qkv_layer2_variant(rotate_q=False))
    with pytest.raises(AssertionError):
        T_two.test_two_layer_step_matches_bruteforce()


def test_mutant_layer2_values_unrounded(monkeypatch):
    monkeypatch.setattr(step_mod.Model, "qkv_layer2", _qkv_layer2_variant(round_v=False))
    with pytest.raises(AssertionError):
        T_two.test_two_layer_step_matches_bruteforce()


def test_mutant_layer2_key_value_blocks_swapped(monkeypatch):
    orig = step_mod.split_layer2

    def split(w, hq, hk):
        q, k, v = orig(w, hq, hk)
        return q, v, k
    monkeypatch.setattr(step_mod, "split_layer2", split)
    with pytest.raises(AssertionError):
        T_two.test_two_layer_step_matches_bruteforce()


def test_mutant_layer2_query_block_transposed(monkeypatch):
    orig = step_mod.split_layer2

    def split(w, hq, hk):
        q, k, v = orig(w, hq, hk)
        return q.T, k, v                      # square block: the shapes still fit
    monkeypatch.setattr(step_mod, "split_layer2", split)
    with pytest.raises(AssertionError):
        T_two.test_two_layer_step_matches_bruteforce()


# ---- untruncated step: each planted mistake must break one of its pins -----
import test_oracle_untruncated as T_unt


def test_mutant_untruncated_keeps_only_the_decoded_masks(monkeypatch):
    orig = step_mod.SequenceOracle.forward_untruncated
    monkeypatch.setattr(step_mod.SequenceOracle, "forward_untruncated",
                        lambda self, dt, dp, c, m: orig(self, dt, dp, c, c))
    with pytest.raises(AssertionError):
        T_unt.test_untruncated_matches_training_form_forward(T_unt.tiny_bf16)
    with pytest.raises(AssertionError):
        T_unt.test_untruncated_step_matches_bruteforce()


def test_mutant_untruncated_new_rows_see_masks(monkeypatch):
    orig = step_mod.inference_mask

    def inference_mask(qk, kk):
        return orig([masks_mod.DECODE if q == masks_mod.NEW else q for q in qk], kk)
    monkeypatch.setattr(step_mod, "inference_mask", inference_mask)
    with pytest.raises(AssertionError):
        T_unt.test_untruncated_step_matches_bruteforce()


def test_mutant_untruncated_masked_rows_at_wrong_positions(monkeypatch):
    orig = step_mod.SequenceOracle.masked_positions
    monkeypatch.setattr(step_mod.SequenceOracle, "masked_positions",
                        lambda self: np.unique(np.concatenate([orig(self), orig(self) - 1])))
    with pytest.raises(AssertionError):
        T_unt.test_untruncated_matches_training_form_forward(T_unt.tiny_bf16)
