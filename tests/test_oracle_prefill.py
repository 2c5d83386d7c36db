"""Pins of the prefill / ground-truth oracle (oracle/prefill_gt.py) against
things other than itself: torch's attention and pooling routines, a
tile-by-tile statement of the fused extraction of [CP Knowl 4], closed forms
and the invariants [CP Knowl 3] states.  CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle as O


def _rand(rng, *shape):
    return rng.normal(size=shape)


@pytest.mark.parametrize("L,d,scale", [(1, 8, 0.3), (37, 16, 0.25), (200, 32, 1 / math.sqrt(32))])
def test_prefill_attention_matches_torch_sdpa(L, d, scale):
    rng = np.random.default_rng(L + d)
    q, k, v = _rand(rng, L, d), _rand(rng, L, d), _rand(rng, L, d)
    o, lse, prob = O.prefill_attention(q, k, v, np.arange(L), scale)
    qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=scale)[0, 0].numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)
    s = torch.from_numpy(q @ k.T * scale)
    s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), -math.inf)
    assert np.allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(prob, torch.softmax(s, dim=1).numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("L,b", [(64, 64), (200, 64), (130, 16), (5, 8)])
def test_pooled_map_matches_torch_max_pool(L, b):
    rng = np.random.default_rng(L * b)
    prob = rng.uniform(size=(7, L))
    ref = torch.nn.functional.max_pool1d(torch.from_numpy(prob)[None], kernel_size=b, stride=b,
                                         ceil_mode=True)[0].numpy()
    assert np.array_equal(O.pooled_attention_map(prob, b), ref)


def _knowl4_tiles(q, k, scale, b, row_tile):
    """The fused extraction written tile by tile: query tiles of row_tile
    rows, key tiles of b keys; each tile's row maximum r_ij is stored, the
    running max and normaliser are updated online, and at the end every
    stored r_ij becomes exp(r_ij - m_i) / l_i."""
    n, L = q.shape[0], k.shape[0]
    nb = -(-L // b)
    gt = np.zeros((n, nb))
    for i0 in range(0, n, row_tile):
        rows = np.arange(i0, min(i0 + row_tile, n))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        r = np.full((len(rows), nb), -np.inf)
        for j in range(nb):
            t = np.arange(j * b, min((j + 1) * b, L))
            s = q[rows] @ k[t].T * scale
            s = np.where(t[None, :] <= rows[:, None], s, -np.inf)
            r[:, j] = s.max(axis=1)
            m_new = np.maximum(m, r[:, j])
            live = np.isfinite(m_new)
            alpha = np.where(live, np.exp(np.where(live, m - m_new, 0.0)), 1.0)
            p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
            l = l * alpha + p.sum(axis=1)
            m = m_new
        gt[rows] = np.exp(r - m[:, None]) / l[:, None]
    return gt


@pytest.mark.parametrize("L,b,row_tile", [(128, 64, 32), (300, 64, 64), (257, 128, 16),
                                          (70, 16, 7)])
def test_ground_truth_equals_fused_tile_form(L, b, row_tile):
    rng = np.random.default_rng(L + b)
    g, d = 3, 16
    q, k, v = _rand(rng, g, L, d) * 1.7, _rand(rng, L, d), _rand(rng, L, d)
    scale = 1 / math.sqrt(d)
    _, _, per_head, gt = O.prefill_group(q, k, v, np.arange(L), scale, b)
    for h in range(g):
        tiles = _knowl4_tiles(q[h], k, scale, b, row_tile)
        assert np.allclose(per_head[h], tiles, rtol=1e-12, atol=1e-300)
    ref = np.max([_knowl4_tiles(q[h], k, scale, b, row_tile) for h in range(g)], axis=0)
    assert np.allclose(gt, ref / ref.sum(axis=1, keepdims=True), rtol=1e-12, atol=1e-300)


def test_ground_truth_closed_forms_and_invariants():
    rng = np.random.default_rng(3)
    L, d, b, g = 150, 8, 32, 2
    pos = np.arange(L)
    nb = -(-L // b)
    # identical keys: uniform attention over the visible keys
    k = np.tile(_rand(rng, 1, d), (L, 1))
    q = _rand(rng, g, L, d)
    _, lse, per_head, gt = O.prefill_group(q, k, _rand(rng, L, d), pos, 0.5, b)
    for p in [0, 1, 31, 32, 100, 149]:
        nvis = p // b + 1
        want_h = np.where(np.arange(nb) < nvis, 1.0 / (p + 1), 0.0)
        assert np.allclose(per_head[:, p], want_h[None], rtol=1e-13, atol=0)
        assert np.allclose(gt[p], np.where(np.arange(nb) < nvis, 1.0 / nvis, 0.0), rtol=1e-13)
        assert np.allclose(lse[:, p], q[:, p] @ k[0] * 0.5 + math.log(p + 1), rtol=1e-13)
    # every row sums to 1; blocks wholly after the query are exactly 0
    q, k, v = _rand(rng, g, L, d), _rand(rng, L, d), _rand(rng, L, d)
    _, _, per_head, gt = O.prefill_group(q, k, v, pos, 0.7, b)
    assert np.allclose(gt.sum(axis=1), 1.0, rtol=1e-13)
    for p in range(L):
        assert np.all(gt[p, p // b + 1:] == 0) and np.all(per_head[:, p, p // b + 1:] == 0)
        assert np.all(gt[p, :p // b + 1] > 0)
    # the values do not enter the ground truth
    _, _, _, gt_v = O.prefill_group(q, k, 5 * v + 1, pos, 0.7, b)
    assert np.array_equal(gt, gt_v)


def test_ground_truth_group_max_and_dominant_key():
    rng = np.random.default_rng(4)
    L, d, b = 96, 8, 16
    pos = np.arange(L)
    k, v = _rand(rng, L, d), _rand(rng, L, d)
    # head 0 attends uniformly (q = 0); head 1 is dominated by key 40 for every
    # query that sees it
    u = k[40] / np.linalg.norm(k[40])
    k[40] = 60 * u
    q = np.zeros((2, L, d))
    q[1] = u[None, :]
    _, _, per_head, gt = O.prefill_group(q, k, v, pos, 1.0, b)
    for p in range(40, L):
        assert per_head[1, p, 40 // b] > 1 - 1e-12
        nvis = p // b + 1
        uniform = np.where(np.arange(L // b) < nvis, 1.0 / (p + 1), 0.0)
        assert np.allclose(per_head[0, p], uniform, rtol=1e-13)
        want = np.maximum(per_head[0, p], per_head[1, p])  # the group's max, head by head
        assert np.allclose(gt[p], want / want.sum(), rtol=1e-13)
        assert gt[p, 40 // b] > 0.5
    # a single head: the ground truth is its pooled map, normalised
    _, _, ph1, gt1 = O.prefill_group(q[1:], k, v, pos, 1.0, b)
    assert np.allclose(gt1, ph1[0] / ph1[0].sum(axis=1, keepdims=True), rtol=1e-14)


def test_sampled_rows_equal_full_prefill():
    """Rows computed alone at their positions (as the full-size parity tests
    sample them) equal the rows of the whole prefill."""
    rng = np.random.default_rng(5)
    L, d, b, g = 140, 16, 64, 2
    q, k, v = _rand(rng, g, L, d), _rand(rng, L, d), _rand(rng, L, d)
    o, lse, ph, gt = O.prefill_group(q, k, v, np.arange(L), 0.25, b)
    rows = np.array([0, 63, 64, 65, 139])
    o2, lse2, ph2, gt2 = O.prefill_group(q[:, rows], k, v, rows, 0.25, b)
    assert np.allclose(o2, o[:, rows], rtol=1e-14, atol=1e-15)
    assert np.allclose(lse2, lse[:, rows], rtol=1e-14)
    assert np.allclose(gt2, gt[rows], rtol=1e-14, atol=0)
    assert np.allclose(ph2, ph[:, rows], rtol=1e-14, atol=0)
