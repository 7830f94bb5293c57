"""Pins of the oracle's merge forms (CPU only).

Random token sets are cut into random pieces; each piece's partial state is
computed on its own and the pieces are merged with every printed form.  The
result must equal one full softmax over the unsplit set (a library
logsumexp and a direct matrix product), in any merge order, with empty
pieces carrying no weight.
"""
import numpy as np
import pytest
import torch

import oracle


def _full(qrows, K, V, scale):
    s = torch.from_numpy(scale * (qrows @ K.T))
    lse = torch.logsumexp(s, dim=1).numpy()
    p = torch.softmax(s, dim=1).numpy()
    return p @ V, lse


def _pieces(rng, n, k):
    cuts = np.sort(rng.choice(np.arange(0, n + 1), size=k - 1, replace=True))
    bounds = [0] + list(cuts) + [n]
    return [(bounds[i], bounds[i + 1]) for i in range(k)]


@pytest.mark.parametrize("seed", range(8))
def test_split_merge_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    n, d, R = int(rng.integers(5, 400)), int(rng.choice([8, 64, 128])), int(rng.integers(1, 6))
    qrows = rng.standard_normal((R, d)) * (3.0 if seed % 2 else 1.0)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    scale = 1 / np.sqrt(d)
    Oref, Lref = _full(qrows, K, V, scale)
    parts = [oracle.partial_attend(qrows, K[a:b], V[a:b], scale) for a, b in _pieces(rng, n, int(rng.integers(1, 9)))]
    # CoDec POR chain (binary merges), in a random order: associativity and commutativity.
    order = rng.permutation(len(parts))
    Oc, mc, sc = oracle.por_chain([(parts[i][0], parts[i][1], parts[i][2]) for i in order])
    assert np.abs(Oc - Oref).max() <= 1e-12
    assert np.abs(mc + np.log(sc) - Lref).max() <= 1e-12
    # FlashDecoding G-way reduction.
    Of = oracle.flashdecoding_merge([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
    assert np.abs(Of - Oref).max() <= 1e-12
    # LSE form.
    Ol, Ll = oracle.lse_merge([p[0] for p in parts], [p[3] for p in parts])
    assert np.abs(Ol - Oref).max() <= 1e-12 and np.abs(Ll - Lref).max() <= 1e-12
    # CoDec's streaming (M, D, U) accumulators take unnormalised contributions u = s * O.
    Os, Ls = oracle.streaming_merge([(p[1], p[2], p[0] * p[2][:, None]) for p in parts if np.isfinite(p[1]).all()])
    assert np.abs(Os - Oref).max() <= 1e-12 and np.abs(Ls - Lref).max() <= 1e-12


def test_empty_partial_has_no_weight():
    rng = np.random.default_rng(3)
    qrows = rng.standard_normal((2, 16))
    K, V = rng.standard_normal((10, 16)), rng.standard_normal((10, 16))
    full = oracle.partial_attend(qrows, K, V, 0.25)
    empty = oracle.partial_attend(qrows, K[:0], V[:0], 0.25)
    O, m, s = oracle.por_pair(empty[0], empty[1], empty[2], full[0], full[1], full[2])
    assert np.abs(O - full[0]).max() == 0
    O2, L2 = oracle.lse_merge([full[0], empty[0]], [full[3], empty[3]])
    assert np.abs(O2 - full[0]).max() == 0 and np.abs(L2 - full[3]).max() == 0


def test_merge_is_not_a_plain_average():
    """A dropped weight (plain mean of partials) must be caught: the two differ."""
    rng = np.random.default_rng(4)
    qrows = rng.standard_normal((1, 8)) * 4
    K, V = rng.standard_normal((30, 8)), rng.standard_normal((30, 8))
    a = oracle.partial_attend(qrows, K[:5], V[:5], 1.0)
    b = oracle.partial_attend(qrows, K[5:], V[5:], 1.0)
    O, _ = oracle.lse_merge([a[0], b[0]], [a[3], b[3]])
    assert np.abs(O - 0.5 * (a[0] + b[0])).max() > 1e-3
