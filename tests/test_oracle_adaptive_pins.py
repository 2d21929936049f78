"""Pins of the adaptive-layout oracle.

* The block similarity equals torch's cosine_similarity of block means built
  by explicit slicing (a different code path).
* Closed forms: a key block that is a positive multiple of the query block
  has similarity 1, a negative multiple -1, an orthogonal one 0.
* Brute force: Python loops over tokens, blocks and dimensions on a tiny
  case give the same layout.
* Invariants: positive rescaling of q or k leaves the layout unchanged;
  tau = -1 makes every (causal) pair live; tau > 1 leaves only the diagonal.
"""

import math

import numpy as np
import pytest
import torch

from oracle import bsa_oracle as O


def test_similarity_is_cosine_of_block_means():
    rng = np.random.default_rng(0)
    H, Hkv, bs, Mb, Nb, d = 4, 2, 8, 5, 6, 16
    q = rng.standard_normal((H, Mb * bs, d))
    k = rng.standard_normal((Hkv, Nb * bs, d))
    _, sim = O.adaptive_layout(q, k, bs, 0.0)
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    for h in range(H):
        for m in range(Mb):
            qm = tq[h, m * bs:(m + 1) * bs].mean(0)
            for n in range(Nb):
                kn = tk[h // 2, n * bs:(n + 1) * bs].mean(0)
                ref = torch.nn.functional.cosine_similarity(qm, kn, dim=0).item()
                assert abs(sim[h, m, n] - ref) <= 1e-12


def test_closed_forms():
    bs, d = 4, 8
    rng = np.random.default_rng(1)
    base = rng.standard_normal((bs, d))
    ortho = rng.standard_normal((bs, d))
    # make the mean of `ortho` orthogonal to the mean of `base`
    mb, mo = base.mean(0), ortho.mean(0)
    ortho -= (mo @ mb) / (mb @ mb) * mb
    q = base[None]                                    # one block
    k = np.concatenate([2.5 * base, -0.5 * base, ortho])[None]
    _, sim = O.adaptive_layout(q, k, bs, 0.5, keep_diagonal=False)
    assert abs(sim[0, 0, 0] - 1.0) <= 1e-12
    assert abs(sim[0, 0, 1] + 1.0) <= 1e-12
    assert abs(sim[0, 0, 2]) <= 1e-12
    lay, _ = O.adaptive_layout(q, k, bs, 0.5, keep_diagonal=False)
    assert lay.tolist() == [[[1, 0, 0]]]
    # a zero block has similarity 0 with everything
    z = np.zeros((1, bs, d))
    _, sim0 = O.adaptive_layout(z, k, bs, 0.5, keep_diagonal=False)
    assert np.all(sim0 == 0.0)


@pytest.mark.parametrize("causal,keep", [(False, False), (True, True), (False, True)])
def test_brute_force(causal, keep):
    rng = np.random.default_rng(2)
    H, bs, Mb, Nb, d = 2, 3, 4, 5, 4
    q = rng.standard_normal((H, Mb * bs, d)).tolist()
    k = rng.standard_normal((H, Nb * bs, d)).tolist()
    tau = 0.2
    lay, _ = O.adaptive_layout(np.array(q), np.array(k), bs, tau, causal=causal,
                               keep_diagonal=keep)
    for h in range(H):
        for m in range(Mb):
            qm = [sum(q[h][m * bs + t][c] for t in range(bs)) / bs for c in range(d)]
            for n in range(Nb):
                kn = [sum(k[h][n * bs + t][c] for t in range(bs)) / bs for c in range(d)]
                dot = sum(a * b for a, b in zip(qm, kn))
                den = math.sqrt(sum(a * a for a in qm)) * math.sqrt(sum(b * b for b in kn))
                live = dot / den >= tau
                if causal and n > m:
                    live = False
                if keep and n == m:
                    live = True
                assert lay[h, m, n] == int(live), (h, m, n)


def test_invariants():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 32, 8))
    k = rng.standard_normal((3, 40, 8))
    lay, _ = O.adaptive_layout(q, k, 8, 0.1, causal=True)
    lay2, _ = O.adaptive_layout(3.0 * q, 0.25 * k, 8, 0.1, causal=True)
    assert np.array_equal(lay, lay2)
    full, _ = O.adaptive_layout(q, k, 8, -1.0, causal=True, keep_diagonal=False)
    m = np.arange(4)[:, None]
    n = np.arange(5)[None, :]
    assert np.array_equal(full, np.broadcast_to((n <= m).astype(np.int32), full.shape))
    diag, _ = O.adaptive_layout(q, k, 8, 1.5)
    assert np.array_equal(diag, np.broadcast_to((n == m).astype(np.int32), diag.shape))
