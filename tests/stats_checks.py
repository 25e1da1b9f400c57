"""Statistical checks of a verification round on the 32-token toy workload.

Given the outputs of many independent rounds that share one set of logits, they
check what the rayaq.ca page "Speculative decoding" derives (sections "Why the
output is exactly the target's" and "Tokens per round and speedup"):

  * the token emitted at every reached position is distributed as that
    position's target p (chi-square);
  * the number of accepted drafts K has P(K = k) = prod_{j<k} alpha_j (1 - alpha_k)
    for k < gamma and prod_j alpha_j for k = gamma, alpha_j = sum min(p_j, q_j);
  * E[K + 1] = sum_{k=0..gamma} prod_{j<k} alpha_j, which is (1 - alpha^(gamma+1)) /
    (1 - alpha) when every position has the same alpha.

p_j and q_j come from scipy's softmax of the logits, not from the code under test.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special

from pins import _chi2_ok


def position_probs(w):
    T = float(w.temperature[0])
    tgt = w.meta["base_target"].astype(np.float64)
    drf = w.meta["base_draft"].astype(np.float64)
    p = scipy.special.softmax(tgt / T, axis=1)
    q = scipy.special.softmax(drf / T, axis=1)
    alpha = np.minimum(p[:-1], q).sum(axis=1)
    return p, q, alpha


def check_draft_tokens(w):
    """The generator's draft tokens are draws from q (Gumbel-max)."""
    _, q, _ = position_probs(w)
    g = int(w.gamma[0])
    x = w.draft_tokens.reshape(-1, g)
    for j in range(g):
        _chi2_ok(np.bincount(x[:, j], minlength=w.vocab), q[j], f"draft tokens ~ q_{j}")


def check_emitted_distribution(w, n_accepted, emitted):
    p, _, _ = position_probs(w)
    g = int(w.gamma[0])
    em = np.asarray(emitted).reshape(-1, g + 1)
    K = np.asarray(n_accepted)
    for j in range(g + 1):
        reached = K >= j
        toks = em[reached, j]
        assert np.all(toks >= 0) and np.all(toks < w.vocab)
        if reached.sum() >= 50:
            _chi2_ok(np.bincount(toks, minlength=w.vocab), p[j], f"emitted at position {j} ~ p_{j}")
        assert np.all(em[~reached, j] == -1)


def check_accept_counts(w, n_accepted):
    _, _, alpha = position_probs(w)
    g = int(w.gamma[0])
    K = np.asarray(n_accepted)
    pk = [np.prod(alpha[:k]) * (1 - alpha[k]) for k in range(g)] + [np.prod(alpha)]
    _chi2_ok(np.bincount(K, minlength=g + 1), pk, "P(K = k)")
    tokens = K + 1
    expect = sum(np.prod(alpha[:k]) for k in range(g + 1))
    se = tokens.std() / math.sqrt(len(tokens))
    assert abs(tokens.mean() - expect) < 4 * se, (tokens.mean(), expect, se)
    if np.allclose(alpha, alpha[0], rtol=0, atol=1e-12):
        a = alpha[0]
        closed = (1 - a ** (g + 1)) / (1 - a)
        assert abs(closed - expect) < 1e-12
        assert abs(tokens.mean() - closed) < 4 * se, (tokens.mean(), closed, se)
    return tokens.mean(), expect, se
