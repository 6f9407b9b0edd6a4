"""Pins for the oracle's decode attention (grouped-query, one query row per
head over the cached K/V rows).

Page: turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs --
Qwen3AsrMetalEngine::step (encode_attention_decode over [0, position]).
"""
import numpy as np
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_row_returns_its_value():
    # one cached row: softmax is 1, the output is that row's V
    q = _rand((4, 16), 0)
    k = _rand((3, 2, 16), 1)
    v = _rand((3, 2, 16), 2)
    out = oracle.attention_decode(q, k, v, 1, 0.25)
    assert np.array_equal(out, v[0, [0, 0, 1, 1], :])


def test_equal_keys_average_the_values():
    # identical keys give equal weights: the mean of V over the rows
    q = _rand((2, 8), 3)
    k = np.broadcast_to(_rand((1, 1, 8), 4), (5, 1, 8)).copy()
    v = _rand((5, 1, 8), 5)
    out = oracle.attention_decode(q, k, v, 5, 1.0)
    assert np.allclose(out, np.broadcast_to(v[:, 0, :].mean(axis=0), (2, 8)), rtol=0, atol=1e-15)


def test_kv_start_window_and_dominant_row():
    # rows before kv_start are ignored; a row with a far larger score wins
    q = np.zeros((1, 4))
    q[0, 0] = 1.0
    k = np.zeros((6, 1, 4))
    k[4, 0, 0] = 1000.0
    k[1, 0, 0] = 2000.0  # outside the window
    v = _rand((6, 1, 4), 6)
    out = oracle.attention_decode(q, k, v, 6, 1.0, kv_start=2)
    assert np.allclose(out[0], v[4, 0], rtol=0, atol=1e-300)


def test_matches_torch_sdpa_with_repeated_kv_heads():
    # torch's attention (an independent implementation) in f64, K/V heads
    # repeated over their query groups
    heads, kv_heads, d, length = 8, 2, 32, 37
    q = _rand((heads, d), 7)
    k = _rand((50, kv_heads, d), 8)
    v = _rand((50, kv_heads, d), 9)
    scale = 1.0 / np.sqrt(d)
    out = oracle.attention_decode(q, k, v, length, scale)
    kt = torch.from_numpy(k[:length]).permute(1, 0, 2).repeat_interleave(heads // kv_heads, 0)
    vt = torch.from_numpy(v[:length]).permute(1, 0, 2).repeat_interleave(heads // kv_heads, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], kt, vt, scale=scale)[:, 0, :].numpy()
    assert np.max(np.abs(out - ref)) <= 1e-13


def test_shift_invariance_of_scores():
    # adding the same vector c to every key adds q.c to every score: unchanged
    heads, kv_heads, d, length = 4, 4, 16, 9
    q = _rand((heads, d), 10)
    k = _rand((length, kv_heads, d), 11)
    v = _rand((length, kv_heads, d), 12)
    a = oracle.attention_decode(q, k, v, length, 0.5)
    b = oracle.attention_decode(q, k + _rand((1, kv_heads, d), 13), v, length, 0.5)
    assert np.max(np.abs(a - b)) <= 1e-12
