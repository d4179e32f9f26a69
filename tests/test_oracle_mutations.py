"""Plant plausible mistakes in the oracle and check that its pins catch them.

Each mutant patches the oracle on the CPU for the duration of one test and
runs a pin from test_oracle_pins; the pin must fail.  This shows that the
pins can see a dropped term, a wrong sign or index, or a transposed operand.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as oa
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, FloatingPointError):
        return True
    return False


def test_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "scaled_scores",
                        lambda q_rows, k, scale: np.asarray(q_rows) @ np.asarray(k).T)
    assert _fails(pins.test_single_visible_key_closed_form)
    assert _fails(pins.test_brute_force_every_mask_combination_tiny)


def test_transposed_operand_is_caught(monkeypatch):
    # S^T = k q^T in place of S = q k^T (shapes agree for square problems)
    monkeypatch.setattr(oa, "scaled_scores",
                        lambda q_rows, k, scale: float(scale) * (np.asarray(k) @ np.asarray(q_rows).T)
                        if np.asarray(q_rows).shape == np.asarray(k).shape
                        else float(scale) * np.asarray(q_rows) @ np.asarray(k).T)
    assert _fails(pins.test_brute_force_every_mask_combination_tiny)


def test_causal_off_by_one_is_caught(monkeypatch):
    real = oa.visible_mask

    def strict(rows, n_keys, causal, length=None, keys=None, offset=0):
        vis = real(rows, n_keys, causal, length, keys, offset)
        if causal:
            rows_a = np.asarray(rows).reshape(-1)
            keys_a = np.arange(n_keys) if keys is None else np.asarray(keys).reshape(-1)
            vis &= keys_a[None, :] < rows_a[:, None] + offset
        return vis

    monkeypatch.setattr(oa, "visible_mask", strict)
    assert _fails(pins.test_single_visible_key_closed_form)
    assert _fails(pins.test_brute_force_every_mask_combination_tiny)


def test_length_off_by_one_is_caught(monkeypatch):
    real = oa.visible_mask

    def loose(rows, n_keys, causal, length=None, keys=None, offset=0):
        return real(rows, n_keys, causal, None if length is None else int(length) + 1, keys,
                    offset)

    monkeypatch.setattr(oa, "visible_mask", loose)
    assert _fails(pins.test_brute_force_every_mask_combination_tiny)
    assert _fails(pins.test_empty_rows_return_zeros_and_neg_inf_lse)


def test_wrong_backward_scale_is_caught(monkeypatch):
    real = oa.attention_backward

    def no_scale_in_dq(q, k, v, o, do, lse, scale, causal=False, lengths=None, row_block=512):
        dq, dk, dv = real(q, k, v, o, do, lse, scale, causal, lengths, row_block)
        return dq / scale, dk, dv

    monkeypatch.setattr(oracle, "attention_backward", no_scale_in_dq)
    assert _fails(pins.test_backward_matches_finite_differences, True, None)


def test_swapped_backward_outputs_are_caught(monkeypatch):
    real = oa.attention_backward

    def swapped(*a, **kw):
        dq, dk, dv = real(*a, **kw)
        return dq, dv, dk

    monkeypatch.setattr(oracle, "attention_backward", swapped)
    assert _fails(pins.test_backward_matches_finite_differences, False, None)
    assert _fails(pins.test_backward_invariants)


def test_merge_without_max_subtraction_is_caught(monkeypatch):
    def unsafe(o_parts, lse_parts):
        o = np.asarray(o_parts, np.float64)
        with np.errstate(over="ignore", invalid="ignore"):
            w = np.exp(np.asarray(lse_parts, np.float64))
            return (w[..., None] * o).sum(-2) / w.sum(-1, keepdims=True), np.log(w.sum(-1))

    monkeypatch.setattr(oracle, "merge_states", unsafe)
    assert _fails(pins.test_merge_is_finite_at_large_lse)


def test_merge_ignoring_weights_is_caught(monkeypatch):
    real = oa.merge_states

    def plain_mean(o_parts, lse_parts):
        _, lse = real(o_parts, lse_parts)
        return np.asarray(o_parts, np.float64).mean(axis=-2), lse

    monkeypatch.setattr(oracle, "merge_states", plain_mean)
    assert _fails(pins.test_merge_reproduces_toy_two_tiles)


def test_decode_key_range_off_by_one_is_caught(monkeypatch):
    real = oa.attention_decode

    def one_more(q, k, v, scale, lengths=None, chunk=None):
        longer = None if lengths is None else np.minimum(np.asarray(lengths) + 1, k.shape[2])
        return real(q, k, v, scale, longer, chunk)

    monkeypatch.setattr(oracle, "attention_decode", one_more)
    assert _fails(pins.test_decode_matches_torch_sdpa_with_lengths, 7)
    assert _fails(pins.test_decode_closed_forms)


def test_top_left_rectangular_alignment_is_caught(monkeypatch):
    """Dropping the Nk - Nq offset (top-left alignment) breaks the rectangular
    pins while every square pin still holds."""
    real = oa.visible_mask

    def top_left(rows, n_keys, causal, length=None, keys=None, offset=0):
        return real(rows, n_keys, causal, length, keys, 0)

    monkeypatch.setattr(oa, "visible_mask", top_left)
    assert _fails(pins.test_fewer_queries_are_the_last_rows_of_the_square_problem)
    assert _fails(pins.test_one_causal_query_sees_the_whole_cache)
    assert _fails(pins.test_more_queries_than_keys_leave_the_first_rows_empty)


def test_packed_keys_taken_from_query_offsets_is_caught(monkeypatch):
    """Slicing each sequence's keys with the query offsets (a plausible
    mix-up of the two offset arrays) breaks the packed pins."""
    real = oa.attention_packed

    def mixed(q, k, v, cu_q, cu_k, scale, causal=False):
        return real(q, k, v, cu_q, cu_q, scale, causal)

    monkeypatch.setattr(oracle, "attention_packed", mixed)
    assert _fails(pins.test_packed_queries_are_the_last_rows_of_each_sequence)
