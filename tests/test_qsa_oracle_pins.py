"""Pins of the QSA indexer oracle (compressed keys, block scores, top-k selection) against facts
fixed by the pages and by mathematics: brute-force loops on tiny inputs, closed-form rotations,
the relative-position property of rotary embeddings, the block-start position of a compressed key
and the token budget the pages state (Qwen3.8-Flash-Next analysis notes, §04 indexer data flow).
"""
import math

import numpy as np
import pytest

import oracle as O


def test_budget_constants():
    """512 blocks of 4 keys make the 2048-token budget (§04: K_B = K / r)."""
    assert O.QSA_BLOCK == 4 and O.QSA_TOPK == 512
    assert O.QSA_TOPK * O.QSA_BLOCK == 2048


def test_rope_closed_form():
    """A unit vector on dim 0 (frequency 1) at position p turns into (cos p, sin p) on dims 0 and
    32; dim 31 turns at frequency 1e4^(-31/32); dims 64.. do not move; position 0 is the identity."""
    x = np.zeros(128)
    x[0] = 1.0
    y = O.partial_rope(x, 3.0)
    assert y[0] == pytest.approx(math.cos(3.0), abs=1e-15)
    assert y[32] == pytest.approx(math.sin(3.0), abs=1e-15)
    assert np.count_nonzero(np.delete(y, [0, 32])) == 0
    x = np.zeros(128)
    x[31] = 1.0
    f = 10000.0 ** (-31 / 32)
    y = O.partial_rope(x, 1000.0)
    assert y[31] == pytest.approx(math.cos(1000.0 * f), abs=1e-12)
    assert y[63] == pytest.approx(math.sin(1000.0 * f), abs=1e-12)
    rng = np.random.default_rng(3)
    z = rng.standard_normal(128)
    assert np.array_equal(O.partial_rope(z, 0.0), z)
    assert np.array_equal(O.partial_rope(z, 12345.0)[64:], z[64:])


def test_rope_scores_depend_on_offset_only():
    """rope(q, p) . rope(k, p') depends on p - p' only, and each pair keeps its length."""
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    base = O.partial_rope(q, 900.0) @ O.partial_rope(k, 100.0)
    for s in (1.0, 37.0, 65536.0):
        assert O.partial_rope(q, 900.0 + s) @ O.partial_rope(k, 100.0 + s) == pytest.approx(base, rel=1e-9)
    y = O.partial_rope(q, 777.0)
    assert np.allclose(y[:32] ** 2 + y[32:64] ** 2, q[:32] ** 2 + q[32:64] ** 2, rtol=1e-12)


def test_compress_brute_force():
    """Loop version: mean of 4 keys, divide by the root mean square, times the gain, then rotate to
    position 4b; the incomplete tail block (43 = 4*10 + 3) gives no compressed key."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((43, 128))
    w = rng.uniform(0.5, 1.5, 128)
    kb = O.qsa_compress(k, w)
    assert kb.shape == (10, 128)
    assert O.qsa_compress(k[:0], w).shape == (0, 128) and O.qsa_compress(k[:3], w).shape == (0, 128)
    for b in range(10):
        m = [sum(k[4 * b + j, d] for j in range(4)) / 4 for d in range(128)]
        r = math.sqrt(sum(x * x for x in m) / 128 + 1e-6)
        y = np.array([m[d] / r * w[d] for d in range(128)])
        for d in range(32):
            a = 4 * b * 10000.0 ** (-d / 32)
            y[d], y[d + 32] = (y[d] * math.cos(a) - y[d + 32] * math.sin(a),
                               y[d] * math.sin(a) + y[d + 32] * math.cos(a))
        assert np.allclose(kb[b], y, rtol=1e-12, atol=1e-12)


def test_compressed_key_sits_at_block_start():
    """A sequence that repeats one key: every block has the same content summary, so compressed
    key b is compressed key 0 (position 0, not rotated) turned to position 4b -- not 4b + 3 or b --
    and pooling before rotating keeps its full length (rotating first would shrink the mean)."""
    rng = np.random.default_rng(6)
    key = rng.standard_normal(128)
    kb = O.qsa_compress(np.tile(key, (64, 1)), np.ones(128))
    assert np.allclose(kb[0], key / math.sqrt(np.mean(key * key) + 1e-6), rtol=1e-12)
    for b in (1, 5, 15):
        assert np.allclose(kb[b], O.partial_rope(kb[0], 4.0 * b), rtol=1e-11, atol=1e-12)
        assert not np.allclose(kb[b], O.partial_rope(kb[0], 4.0 * b + 3), atol=1e-3)
    assert np.allclose(np.sum(kb * kb, axis=1), 128 / (1 + 1e-6 / np.mean(key * key)), rtol=1e-12)


def test_scores_brute_force_and_causality():
    """I[i, b] = sum_h max(0, <rope(q_ih, i), kbar_b>) for blocks with 4b + 3 <= i, by loops; a query
    at position 3 sees block 0 and one at position 2 sees none."""
    rng = np.random.default_rng(7)
    T = 23
    k = rng.standard_normal((T, 128))
    q = rng.standard_normal((T, 4, 128))
    kb = O.qsa_compress(k, np.ones(128))
    sc = O.qsa_scores(q, kb, np.arange(T))
    for i in range(T):
        for b in range(kb.shape[0]):
            if 4 * b + 3 > i:
                assert sc[i, b] == -np.inf
                continue
            s = 0.0
            for h in range(4):
                s += max(0.0, float(O.partial_rope(q[i, h], float(i)) @ kb[b]))
            assert sc[i, b] == pytest.approx(s, rel=1e-12, abs=1e-12)
    assert np.isfinite(sc[3, 0]) and not np.isfinite(sc[2]).any()


def test_scores_sum_relu_per_head():
    """ReLU acts per head before the sum: heads v and -v give |<v, kbar>|, not max(0, 0)."""
    rng = np.random.default_rng(8)
    kb = rng.standard_normal((3, 128))
    v = rng.standard_normal(128)
    q = np.stack([v, -v, np.zeros(128), np.zeros(128)])[None]
    sc = O.qsa_scores(q, kb, np.array([11]))
    assert np.allclose(sc[0], np.abs(O.partial_rope(v, 11.0) @ kb.T), rtol=1e-12)


def test_select_against_lexsort():
    """Top-k by (score descending, block ascending) from numpy's lexsort, with planted ties; every
    complete block when there are at most k; the tail starts at the incomplete block."""
    rng = np.random.default_rng(9)
    M, N, k = 40, 60, 16
    sc = np.round(rng.uniform(0, 4, (M, N)), 1)  # coarse values: many exact ties
    pos = rng.integers(0, 4 * N, M)
    valid = (4 * np.arange(N)[None, :] + 3) <= pos[:, None]
    sc = np.where(valid, sc, -np.inf)
    sel, tail = O.qsa_select(sc, pos, topk=k)
    for i in range(M):
        nb = int(valid[i].sum())
        order = np.lexsort((np.arange(nb), -sc[i, :nb]))
        assert np.array_equal(sel[i], np.sort(order[:k]))
        assert len(sel[i]) == min(k, nb)
        assert tail[i] == 4 * ((pos[i] + 1) // 4) and tail[i] <= pos[i] + 1 < tail[i] + 4 + 1


def test_rope_width():
    """Other rotated widths: 128 pairs dim d with d + 64 at frequency 1e4^(-d/64) (dim 0 with 64 at
    frequency 1, dim 63 with 127); 16 pairs d with d + 8 and leaves dims 16.. alone; 0 is the identity."""
    x = np.zeros(128)
    x[0] = 1.0
    y = O.partial_rope(x, 2.0, rope_dims=128)
    assert y[0] == pytest.approx(math.cos(2.0), abs=1e-15) and y[64] == pytest.approx(math.sin(2.0), abs=1e-15)
    x = np.zeros(128)
    x[63] = 1.0
    y = O.partial_rope(x, 500.0, rope_dims=128)
    f = 10000.0 ** (-63 / 64)
    assert y[63] == pytest.approx(math.cos(500.0 * f), abs=1e-12) and y[127] == pytest.approx(math.sin(500.0 * f), abs=1e-12)
    z = np.random.default_rng(10).standard_normal(128)
    y = O.partial_rope(z, 77.0, rope_dims=16)
    assert np.array_equal(y[16:], z[16:])
    assert np.allclose(y[:8] ** 2 + y[8:16] ** 2, z[:8] ** 2 + z[8:16] ** 2, rtol=1e-12)
    assert np.array_equal(O.partial_rope(z, 77.0, rope_dims=0), z)
