"""Pins of the fp64 CPU oracle to things other than itself.

Every function here checks the oracle against something the pages or the
mathematics fix: values the pages print for their worked examples (under
tests/golden, each with its citation), closed forms, identities of the method,
special cases that reduce to a library routine (scipy's softmax, numpy's
argmax / searchsorted), brute force on tiny inputs, and Monte Carlo against exact
page fractions.  Each raises AssertionError on a mismatch.

The same functions are run against planted mistakes in the oracle (see
test_oracle_mutants.py), which must each fail at least one of them.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np
import scipy.special
import scipy.stats

import oracle
from pagevals import LOGP, LOGQ, MARKOV, P, P_MAT, Q, Q_MAT, ROUNDS, TOK, load

U24 = 2.0 ** -24
F32_BELOW_ONE = float(np.float32(1.0 - U24))


def _close(a, b, tol, what):
    assert abs(float(a) - float(b)) <= tol, f"{what}: {a!r} vs {b!r} (tol {tol})"


def _chi2_ok(observed, probs, what, pmin=1e-3):
    observed = np.asarray(observed, np.float64)
    probs = np.asarray(probs, np.float64)
    n = observed.sum()
    exp = probs * n
    keep = exp >= 5
    obs_k, exp_k = list(observed[keep]), list(exp[keep])
    if (~keep).any():  # merge thin bins
        obs_k.append(observed[~keep].sum())
        exp_k.append(exp[~keep].sum())
    obs_k, exp_k = np.array(obs_k), np.array(exp_k)
    if len(obs_k) < 2:
        return
    assert np.all(obs_k[exp_k == 0] == 0), f"{what}: mass where none is expected"
    m = exp_k > 0
    pval = scipy.stats.chisquare(obs_k[m], exp_k[m] * obs_k[m].sum() / exp_k[m].sum()).pvalue
    assert pval > pmin, f"{what}: chi-square p = {pval:.2e}, observed {observed}, expected {exp}"


def snapped(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape).astype(np.float64) * U24).astype(np.float32)


# --------------------------------------------------------------------------- #
# Markov three-token example: drafter simulation and packed rounds
# --------------------------------------------------------------------------- #
def markov_drafts(rng, ctx, gamma):
    """Draft tokens from the Markov drafter q, one round per entry of ctx."""
    cq = np.cumsum(Q_MAT, axis=1)
    out = np.empty((len(ctx), gamma), np.int32)
    prev = np.asarray(ctx)
    for j in range(gamma):
        u = rng.random(len(ctx))
        x = np.minimum((u[:, None] >= cq[prev]).sum(axis=1), 2)
        out[:, j] = x
        prev = x
    return out


def markov_verify(ctx, drafts, uniforms, **kw):
    """Run the oracle on rounds from contexts ctx with the given drafts and uniforms."""
    N, g = drafts.shape
    seq = np.concatenate([np.asarray(ctx)[:, None], drafts], axis=1)  # context of each position
    target = LOGP[seq].reshape(-1, 3)
    draft = LOGQ[seq[:, :g]].reshape(-1, 3)
    return oracle.verify(target, draft, "f64", 3, np.full(N, g, np.int32), drafts.reshape(-1),
                         np.asarray(uniforms, np.float32).reshape(-1), np.ones(N, np.float32), **kw)


def markov_round(rng, ctx, gamma):
    drafts = markov_drafts(rng, ctx, gamma)
    u = snapped(rng, (len(ctx), gamma + 1))
    r = markov_verify(ctx, drafts, u)
    em = r["emitted"].reshape(len(ctx), gamma + 1)
    return r["n_accepted"], em


def markov_emit(rng, start, n_tokens, N, gamma=3):
    """Chain rounds from `start` until n_tokens are out; returns [N, n_tokens]."""
    seq = np.full((N, n_tokens), -1, np.int64)
    cnt = np.zeros(N, np.int64)
    ctx = np.full(N, start, np.int64)
    while True:
        idx = np.nonzero(cnt < n_tokens)[0]
        if len(idx) == 0:
            return seq
        K, em = markov_round(rng, ctx[idx], gamma)
        for k in range(gamma + 1):
            take = (k <= K) & (cnt[idx] < n_tokens)
            rows = idx[take]
            seq[rows, cnt[rows]] = em[take, k]
            cnt[rows] += 1
        ctx[idx] = em[np.arange(len(idx)), K]


# --------------------------------------------------------------------------- #
# softmax and argmax
# --------------------------------------------------------------------------- #
def pin_softmax_constant():
    """Constant logits give 1/V exactly (up to rounding)."""
    for V in (1, 7, 32000):
        p = oracle.softmax(np.full(V, 3.25), 0.7)
        assert np.all(p == 1.0 / V), "constant logits"


def pin_softmax_two_level():
    """n1 logits at a, n2 at b: p(a) = 1 / (n1 + n2 exp((b-a)/T))."""
    for (n1, n2, a, b, T) in [(1, 3, 2.0, -1.0, 1.0), (5, 11, 0.5, 1.75, 0.8), (2, 1000, 9.0, 0.0, 1.3)]:
        z = np.array([a] * n1 + [b] * n2)
        p = oracle.softmax(z, T)
        pa = 1.0 / (n1 + n2 * math.exp((b - a) / T))
        pb = 1.0 / (n2 + n1 * math.exp((a - b) / T))
        tol = 4e-16 * (n1 + n2)  # sequential fp64 sum of n1 + n2 terms
        _close(p[0] / pa, 1.0, tol, "two-level p(a)")
        _close(p[-1] / pb, 1.0, tol, "two-level p(b)")


def pin_softmax_vs_scipy():
    """Temperature softmax equals scipy.special.softmax(z / T) for all input dtypes."""
    rng = np.random.default_rng(11)
    import workloads
    for dtype in ("f64", "f32", "bf16"):
        for T in (0.5, 0.8, 1.0, 1.5):
            z = rng.standard_normal(4099) * 3.0
            if dtype == "bf16":
                zin = workloads.to_bf16_bits(z.astype(np.float32))
                zf = workloads.bf16_bits_to_f32(zin).astype(np.float64)
            elif dtype == "f32":
                zin = z.astype(np.float32)
                zf = zin.astype(np.float64)
            else:
                zin, zf = z, z
            p = oracle.softmax(zin, T, dtype)
            ref = scipy.special.softmax(zf / T)
            assert np.max(np.abs(p - ref) / ref) < 1e-12, f"softmax vs scipy ({dtype}, T={T})"


def pin_softmax_one_hot_and_masked():
    """A dominant logit gives ~1; -inf logits get probability 0; all -inf is rejected."""
    z = np.zeros(100)
    z[17] = 1000.0
    p = oracle.softmax(z, 1.0)
    _close(p[17], 1.0, 1e-300, "dominant logit")
    z = np.array([0.0, -np.inf, 0.0, -np.inf])
    p = oracle.softmax(z, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0 and abs(p[0] - 0.5) < 1e-16, "masked logits"
    for bad in ([-np.inf] * 3, [0.0, np.nan], [np.inf, 0.0]):
        try:
            oracle.softmax(np.array(bad), 1.0)
        except ValueError:
            continue
        raise AssertionError(f"softmax accepted {bad}")


def pin_argmax_first_index():
    """Greedy argmax is numpy's argmax (first index of the maximum) on raw logits."""
    rng = np.random.default_rng(5)
    import workloads
    for _ in range(50):
        z = rng.integers(-3, 4, size=257).astype(np.float32)  # many ties
        assert oracle.argmax(z, "f32") == int(np.argmax(z)), "argmax ties (f32)"
        zb = workloads.to_bf16_bits(z)
        assert oracle.argmax(zb, "bf16") == int(np.argmax(z)), "argmax ties (bf16)"


# --------------------------------------------------------------------------- #
# the three-token Markov example (rayaq.ca "Speculative decoding", "Worked example")
# --------------------------------------------------------------------------- #
def pin_markov_alpha_and_residual():
    """alpha and the residual for previous tokens a, b, c match the page's table."""
    for c in "abc":
        r = oracle.position(LOGP[TOK[c]], LOGQ[TOK[c]], 1.0)
        for v in range(3):
            _close(r["p"][v], float(P[c][v]), 1e-15, f"p(.|{c})")
            _close(r["q"][v], float(Q[c][v]), 1e-15, f"q(.|{c})")
            _close(r["residual"][v], float(Fraction(MARKOV["residual"][c][v])), 1e-12,
                   f"residual(.|{c})")
        _close(r["alpha"], float(Fraction(MARKOV["alpha"][c])), 1e-15, f"alpha({c})")
        _close(r["resid_mass"], 1.0 - float(Fraction(MARKOV["alpha"][c])), 1e-15, f"W({c})")


def pin_markov_reject_round():
    """Drafts c, c, a after 'a' with u = 0.085, 0.835: keep c (ratio 1), reject c
    (ratio 5/7), residual gives a; the round emits 'c a' and accepts one draft."""
    spec = ROUNDS["reject_round"]
    drafts = np.array([[TOK[t] for t in spec["drafts"]]], np.int32)
    for u_draw in (0.0, 0.3, 0.7, F32_BELOW_ONE):
        for u3 in (0.0, 0.5, F32_BELOW_ONE):  # the third draft is never checked
            u = np.array([[spec["positions"][0]["u"], spec["positions"][1]["u"], u3, u_draw]])
            r = markov_verify([TOK["a"]], drafts, u)
            assert r["n_accepted"][0] == spec["n_accepted"], r
            em = [t for t in r["emitted"] if t >= 0]
            assert em == [TOK[t] for t in spec["emitted"]], em
            assert r["flag_pos"][0] == -1
            _close(r["p_x"][0], float(Fraction(spec["positions"][0]["p"])), 1e-15, "p(c|a)")
            _close(r["q_x"][0], float(Fraction(spec["positions"][0]["q"])), 1e-15, "q(c|a)")
            _close(r["p_x"][1], float(Fraction(spec["positions"][1]["p"])), 1e-15, "p(c|c)")
            _close(r["q_x"][1], float(Fraction(spec["positions"][1]["q"])), 1e-15, "q(c|c)")
            _close(r["p_x"][1] / r["q_x"][1], 5 / 7, 1e-15, "ratio 5/7")
            _close(r["resid_mass"][0], 1 - 4 / 5, 1e-15, "W after c")


def pin_markov_all_accept_round():
    """Drafts b, c, c after 'a' (ratios 3/4, 1, 5/7) all kept; the bonus from
    p(.|c) = (3/10, 1/5, 1/2) gives c for u in [1/2, 1): 'b c c c'."""
    spec = ROUNDS["all_accept_round"]
    drafts = np.array([[TOK[t] for t in spec["drafts"]]], np.int32)
    ratios = [Fraction(3, 10) / Fraction(2, 5), Fraction(1), Fraction(1, 2) / Fraction(7, 10)]
    below = [float(np.nextafter(np.float32(float(x)), np.float32(0))) for x in ratios]
    u = np.array([[below[0], F32_BELOW_ONE, below[2], 0.75]])
    r = markov_verify([TOK["a"]], drafts, u)
    assert r["n_accepted"][0] == 3, r
    assert list(r["emitted"]) == [TOK[t] for t in spec["emitted"]], r["emitted"]
    for j in range(3):
        _close(r["p_x"][j] / r["q_x"][j], float(ratios[j]), 1e-15, f"ratio {j}")
    for u_draw, tok in ((0.0, "a"), (0.2999, "a"), (0.3001, "b"), (0.4999, "b"), (0.5001, "c"),
                        (F32_BELOW_ONE, "c")):
        u[0, 3] = u_draw
        r = markov_verify([TOK["a"]], drafts, u)
        assert r["emitted"][3] == TOK[tok], (u_draw, r["emitted"])
    # a uniform just above a ratio below 1 rejects there
    for j in (0, 2):
        uu = u.copy()
        uu[0, j] = float(np.nextafter(np.float32(float(ratios[j])), np.float32(1)))
        r = markov_verify([TOK["a"]], drafts, uu)
        assert r["n_accepted"][0] == j, (j, r["n_accepted"])


def pin_markov_distinct_sequences():
    """Every draft and every accept-or-reject outcome from 'a' with gamma = 3 gives
    94 distinct emitted sequences."""
    seqs = set()
    grid = (np.arange(256) + 0.5) / 256
    for drafts in itertools.product(range(3), repeat=3):
        for pattern in itertools.product((0.0, F32_BELOW_ONE), repeat=3):
            n = len(grid)
            u = np.empty((n, 4), np.float32)
            u[:, :3] = pattern
            u[:, 3] = grid
            r = markov_verify(np.zeros(n, np.int64), np.tile(np.array(drafts, np.int32), (n, 1)), u)
            em = r["emitted"].reshape(n, 4)
            for row in em:
                seqs.add(tuple(int(t) for t in row if t >= 0))
    assert len(seqs) == ROUNDS["distinct_sequences_from_a_gamma3"], len(seqs)


def pin_markov_accept_counts():
    """P(K = 0..3) from 'a' is 1/10, 13/100, 61/500, 81/125, so E[tokens] = 1659/500
    (not the 3.439 of the i.i.d. formula)."""
    rng = np.random.default_rng(2024)
    N = 400_000
    K, _ = markov_round(rng, np.zeros(N, np.int64), 3)
    probs = [float(Fraction(ROUNDS["accepted_count_from_a_gamma3"][str(k)])) for k in range(4)]
    _chi2_ok(np.bincount(K, minlength=4), probs, "P(K) from a")
    mean = (K + 1).mean()
    se = (K + 1).std() / math.sqrt(N)
    exact = float(Fraction(ROUNDS["expected_tokens_from_a_gamma3"]))
    assert abs(mean - exact) < 4 * se, (mean, exact, se)
    assert abs(mean - ROUNDS["iid_formula_alpha_9_10_gamma3"]) > 50 * se


def pin_markov_joint_two_tokens():
    """Chaining rounds from 'a' until two tokens are out reproduces the target's joint."""
    rng = np.random.default_rng(7)
    N = 300_000
    seq = markov_emit(rng, TOK["a"], 2, N)
    counts = np.zeros(9)
    np.add.at(counts, seq[:, 0] * 3 + seq[:, 1], 1)
    table = ROUNDS["joint_two_tokens_from_a"]
    probs = [float(Fraction(table[a + b])) for a in "abc" for b in "abc"]
    _chi2_ok(counts, probs, "two-token joint from a")


def pin_markov_joint_three_tokens():
    """From every start, three emitted tokens follow the target chain p exactly."""
    rng = np.random.default_rng(8)
    N = 150_000
    for s in range(3):
        seq = markov_emit(rng, s, 3, N)
        counts = np.zeros(27)
        np.add.at(counts, seq[:, 0] * 9 + seq[:, 1] * 3 + seq[:, 2], 1)
        probs = [P_MAT[s, a] * P_MAT[a, b] * P_MAT[b, c]
                 for a in range(3) for b in range(3) for c in range(3)]
        _chi2_ok(counts, probs, f"three-token joint from {s}")


# --------------------------------------------------------------------------- #
# the four-token hand example (cgnarendiran.github.io, "The correction that makes it exact")
# --------------------------------------------------------------------------- #
def _four_token():
    ex = load("four_token_example.json")
    return ex, np.log(np.array(ex["target_p"])), np.log(np.array(ex["draft_q"]))


def pin_four_token_alpha_residual():
    ex, lp, lq = _four_token()
    r = oracle.position(lp, lq, 1.0)
    _close(r["alpha"], ex["alpha"], 1e-15, "alpha")
    _close(1 - r["alpha"], ex["reject_probability"], 1e-15, "reject probability")
    for v in range(4):
        _close(r["residual"][v], float(Fraction(ex["residual"][v])), 1e-14, f"residual {v}")
        _close(r["residual"][v], ex["residual_printed"][v], 5e-4, f"printed residual {v}")
    # exactness: min(p, q) + (1 - alpha) r = p
    emit = np.minimum(r["p"], r["q"]) + (1 - r["alpha"]) * r["residual"]
    assert np.max(np.abs(emit - np.array(ex["target_p"]))) < 1e-15


def pin_four_token_decision_and_emit():
    """The proposed token is kept with probability 1/2, and what is emitted is p."""
    ex, lp, lq = _four_token()
    x = ex["tokens"].index(ex["proposed"])

    def run(u):
        u = np.asarray(u, np.float32).reshape(-1, 2)
        n = u.shape[0]
        target = np.tile(np.stack([lp, lp]), (n, 1))
        draft = np.tile(lq[None], (n, 1))
        return oracle.verify(target, draft, "f64", 4, np.ones(n, np.int32), np.full(n, x, np.int32),
                             u, np.ones(n, np.float32))

    r = run([0.4999, 0.0])
    assert r["n_accepted"][0] == 1 and r["emitted"][0] == x
    _close(r["p_x"][0] / r["q_x"][0], ex["accept_probability"], 1e-15, "keep probability")
    r = run([0.5001, 0.0])
    assert r["n_accepted"][0] == 0
    # on rejection the residual CDF is (0, 2/3, 5/6, 1): a, my, your
    for ud, tok in ((0.1, 1), (0.666, 1), (0.667, 2), (0.83, 2), (0.834, 3), (0.99, 3)):
        r = run([0.9, ud])
        assert r["emitted"][0] == tok, (ud, r["emitted"])
    # Monte Carlo: the token emitted at the position is distributed as p
    rng = np.random.default_rng(99)
    N = 200_000
    xq = rng.choice(4, size=N, p=np.array(ex["draft_q"]))
    u = snapped(rng, (N, 2))
    target = np.tile(np.stack([lp, lp]), (N, 1))
    draft = np.tile(lq[None], (N, 1))
    r = oracle.verify(target, draft, "f64", 4, np.ones(N, np.int32), xq.astype(np.int32), u,
                      np.ones(N, np.float32))
    em0 = r["emitted"].reshape(N, 2)[:, 0]
    _chi2_ok(np.bincount(em0, minlength=4), ex["target_p"], "four-token emit distribution")
    acc = (r["n_accepted"] == 1) & (xq == x)
    _close(acc.sum() / (xq == x).sum(), 0.5, 4 * math.sqrt(0.25 / (xq == x).sum()), "keep rate")


# --------------------------------------------------------------------------- #
# quiz values (rayaq.ca "Speculative decoding", self-check questions)
# --------------------------------------------------------------------------- #
def pin_quiz_keep_probability():
    qz = load("quiz.json")["keep_probability"]
    lp = np.log([qz["p"], 1 - qz["p"]])
    lq = np.log([qz["q"], 1 - qz["q"]])
    target = np.stack([lp, lp])
    for u, acc in ((0.2499, 1), (0.2501, 0)):
        r = oracle.verify(target, lq[None], "f64", 2, [1], [0], [u, 0.5], [1.0])
        _close(r["p_x"][0] / r["q_x"][0], qz["expected"], 1e-15, "keep probability")
        assert r["n_accepted"][0] == acc


def pin_quiz_expected_tokens():
    """alpha = 0.8 at every position, gamma = 4: E[tokens] = (1 - 0.8^5)/0.2 = 3.3616."""
    qz = load("quiz.json")["expected_tokens_iid"]
    p = np.array([0.6, 0.4])
    q = np.array([0.8, 0.2])  # sum min(p, q) = 0.8
    assert abs(np.minimum(p, q).sum() - qz["alpha"]) < 1e-15
    g = qz["gamma"]
    rng = np.random.default_rng(31)
    N = 400_000
    x = rng.choice(2, size=(N, g), p=q).astype(np.int32)
    u = snapped(rng, (N, g + 1))
    target = np.tile(np.log(p), (N * (g + 1), 1))
    draft = np.tile(np.log(q), (N * g, 1))
    r = oracle.verify(target, draft, "f64", 2, np.full(N, g, np.int32), x.reshape(-1), u,
                      np.ones(N, np.float32))
    tokens = r["n_accepted"] + 1
    se = tokens.std() / math.sqrt(N)
    closed = (1 - qz["alpha"] ** (g + 1)) / (1 - qz["alpha"])
    assert abs(closed - qz["expected"]) < 5e-3
    assert abs(tokens.mean() - closed) < 4 * se, (tokens.mean(), closed, se)


# --------------------------------------------------------------------------- #
# identities of the method on random inputs
# --------------------------------------------------------------------------- #
def pin_identities_random():
    """min(p,q) + max(0,p-q) = p; sum max(0,p-q) = 1 - alpha; alpha = 1 - TV(p, q);
    min(p,q) + (1-alpha) r = p."""
    import workloads
    rng = np.random.default_rng(3)
    for dtype in ("f32", "bf16"):
        for T in (0.6, 1.0, 1.4):
            zt = rng.standard_normal(2000).astype(np.float32) * 3
            zd = (zt + rng.standard_normal(2000) * 1.0).astype(np.float32)
            if dtype == "bf16":
                zt, zd = workloads.to_bf16_bits(zt), workloads.to_bf16_bits(zd)
            r = oracle.position(zt, zd, T, dtype)
            p, q, a = r["p"], r["q"], r["alpha"]
            lhs = np.minimum(p, q) + np.maximum(0.0, p - q)
            assert np.all(np.abs(lhs - p) <= np.spacing(p)), "min + max(0, p-q) = p"
            _close(r["resid_mass"], 1 - a, 1e-12, "W = 1 - alpha")
            _close(a, 1 - 0.5 * np.abs(p - q).sum(), 1e-12, "alpha = 1 - TV")
            emit = np.minimum(p, q) + (1 - a) * r["residual"]
            assert np.max(np.abs(emit - p)) < 1e-12, "P(emit) = p"
            assert abs(p.sum() - 1) < 1e-12 and abs(q.sum() - 1) < 1e-12


def pin_px_qx_vs_scipy():
    """p(x_j) and q(x_j) reported by a batched, ragged, tempered round equal
    scipy's softmax(z / T) at the draft token."""
    import workloads
    w = workloads.small(seed=12, batch=9, vocab=301, dtype="f32", gamma=[0, 1, 2, 3, 4, 5, 6, 7, 3],
                        temperature=[0.55, 0.8, 1.0, 1.3, 0.7, 2.0, 0.9, 1.1, 0.6])
    r = oracle.verify_workload(w)
    t_off, d_off = w.offsets()
    for i in range(w.batch):
        T = float(w.temperature[i])
        for j in range(int(w.gamma[i])):
            x = int(w.draft_tokens[d_off[i] + j])
            pz = scipy.special.softmax(w.target[t_off[i] + j].astype(np.float64) / T)[x]
            qz = scipy.special.softmax(w.draft[d_off[i] + j].astype(np.float64) / T)[x]
            _close(r["p_x"][d_off[i] + j] / pz, 1.0, 1e-12, "p_x vs scipy")
            _close(r["q_x"][d_off[i] + j] / qz, 1.0, 1e-12, "q_x vs scipy")


def pin_rows_independent():
    """Each row of a ragged batch gives what it gives alone (packed offsets)."""
    import workloads
    w = workloads.small(seed=13, batch=7, vocab=97, dtype="bf16", gamma=[3, 0, 5, 1, 0, 7, 2],
                        temperature=[0.7, 1.0, 1.2, 0.9, 1.0, 0.5, 1.5])
    full = oracle.verify_workload(w)
    t_off, d_off = w.offsets()
    for i in range(w.batch):
        g = int(w.gamma[i])
        r = oracle.verify(w.target[t_off[i]:t_off[i + 1]], w.draft[d_off[i]:d_off[i + 1]], "bf16",
                          w.vocab, [g], w.draft_tokens[d_off[i]:d_off[i + 1]],
                          w.uniforms[t_off[i]:t_off[i + 1]], w.temperature[i:i + 1])
        assert r["n_accepted"][0] == full["n_accepted"][i]
        assert np.array_equal(r["emitted"], full["emitted"][t_off[i]:t_off[i + 1]])


# --------------------------------------------------------------------------- #
# the draw
# --------------------------------------------------------------------------- #
def pin_inverse_cdf_vs_searchsorted():
    """The draw is numpy's searchsorted(cumsum(w), u*W, side='right'); a uniform at
    the middle of a token's CDF interval selects that token; u = 0 skips leading
    zero weights."""
    rng = np.random.default_rng(17)
    for _ in range(200):
        V = int(rng.integers(1, 300))
        w = rng.random(V) * (rng.random(V) < 0.6)
        if w.sum() == 0:
            w[rng.integers(V)] = 1.0
        C = np.cumsum(w)
        for u in list(rng.random(5)) + [0.0]:
            tok, W, _ = oracle.inverse_cdf(w, u)
            assert tok == int(np.searchsorted(C, u * C[-1], side="right")), (u, tok)
            assert w[tok] > 0
        v = int(np.nonzero(w)[0][rng.integers(np.count_nonzero(w))])
        mid = ((C[v] - w[v]) + C[v]) / 2 / C[-1]
        assert oracle.inverse_cdf(w, mid)[0] == v


def pin_gamma_zero_is_bonus():
    """A row with no drafts emits one draw from p_0 with its single uniform."""
    rng = np.random.default_rng(4)
    z = rng.standard_normal((50, 64))
    u = snapped(rng, 50)
    r = oracle.verify(z, np.zeros((0, 64)), "f64", 64, np.zeros(50, np.int32),
                      np.zeros(0, np.int32), u, np.full(50, 0.9, np.float32))
    for i in range(50):
        p = scipy.special.softmax(z[i] / np.float32(0.9).astype(np.float64))
        assert r["n_accepted"][i] == 0
        assert r["emitted"][i] == int(np.searchsorted(np.cumsum(p), float(u[i]) * p.sum(), side="right"))


# --------------------------------------------------------------------------- #
# special cases that reduce to something simpler
# --------------------------------------------------------------------------- #
def pin_q_equals_p_accepts_all():
    rng = np.random.default_rng(6)
    N, g, V = 500, 5, 40
    z = rng.standard_normal((N * (g + 1), V))
    d = z.reshape(N, g + 1, V)[:, :g].reshape(-1, V)
    x = rng.integers(0, V, N * g).astype(np.int32)
    r = oracle.verify(z, d, "f64", V, np.full(N, g, np.int32), x, snapped(rng, N * (g + 1)),
                      np.ones(N, np.float32))
    assert np.all(r["n_accepted"] == g)


def pin_one_hot_draft():
    """A one-hot q (a greedy drafter) keeps x with probability p(x) and otherwise
    draws from p with x removed."""
    rng = np.random.default_rng(8)
    V, x = 12, 5
    zt = rng.standard_normal(V)
    zd = np.full(V, -np.inf)
    zd[x] = 0.0
    r = oracle.position(zt, zd, 1.0)
    p = scipy.special.softmax(zt)
    _close(r["alpha"], p[x], 1e-15, "alpha = p(x)")
    expect = p.copy()
    expect[x] = 0.0
    expect /= 1 - p[x]
    assert np.max(np.abs(r["residual"] - expect)) < 1e-14


def pin_greedy_brute_force():
    """Greedy mode keeps drafts while they equal numpy's argmax of the target logits,
    then emits that argmax."""
    import workloads
    rng = np.random.default_rng(21)
    for dtype in ("f32", "bf16"):
        B, V = 60, 16
        gam = rng.integers(0, 6, B).astype(np.int32)
        nT, nD = int((gam + 1).sum()), int(gam.sum())
        zt = rng.integers(-2, 3, (nT, V)).astype(np.float32)  # ties everywhere
        t_off = np.concatenate([[0], np.cumsum(gam + 1)])
        am = np.argmax(zt, axis=1)
        x = np.empty(nD, np.int32)
        k = 0
        for i in range(B):
            for j in range(gam[i]):
                x[k] = am[t_off[i] + j] if rng.random() < 0.7 else rng.integers(V)
                k += 1
        zin = workloads.to_bf16_bits(zt) if dtype == "bf16" else zt
        r = oracle.verify(zin, np.zeros((nD, V), zin.dtype), dtype, V, gam, x, np.zeros(nT, np.float32),
                          np.ones(B, np.float32), mode="greedy")
        d = 0
        for i in range(B):
            K = gam[i]
            for j in range(gam[i]):
                if x[d + j] != am[t_off[i] + j]:
                    K = j
                    break
            assert r["n_accepted"][i] == K
            exp = list(x[d:d + K]) + [am[t_off[i] + K]] + [-1] * (gam[i] - K)
            assert list(r["emitted"][t_off[i]:t_off[i + 1]]) == exp
            d += gam[i]


def pin_low_temperature_is_greedy():
    """At a temperature far below the logit gaps, sampling gives the greedy result
    whatever the uniforms; T <= 0 rows are greedy rows."""
    rng = np.random.default_rng(23)
    B, g, V = 40, 4, 50
    base = rng.permutation(V).astype(np.float64) * 0.5  # distinct logits, gaps >= 0.5
    zt = np.stack([rng.permutation(base) for _ in range(B * (g + 1))])
    zd = np.stack([rng.permutation(base) for _ in range(B * g)])
    am = np.argmax(zt, axis=1).reshape(B, g + 1)
    x = np.where(rng.random((B, g)) < 0.6, am[:, :g], rng.integers(0, V, (B, g))).astype(np.int32)
    gam = np.full(B, g, np.int32)
    greedy = oracle.verify(zt, zd, "f64", V, gam, x.reshape(-1), np.zeros(B * (g + 1), np.float32),
                           np.ones(B, np.float32), mode="greedy")
    for trial in range(3):
        u = snapped(rng, B * (g + 1))
        cold = oracle.verify(zt, zd, "f64", V, gam, x.reshape(-1), u, np.full(B, 1e-3, np.float32))
        assert np.array_equal(cold["n_accepted"], greedy["n_accepted"])
        assert np.array_equal(cold["emitted"], greedy["emitted"])
        for t in (0.0, -1.0):
            zero = oracle.verify(zt, zd, "f64", V, gam, x.reshape(-1), u, np.full(B, t, np.float32))
            assert np.array_equal(zero["emitted"], greedy["emitted"])


# --------------------------------------------------------------------------- #
# decisions at a threshold
# --------------------------------------------------------------------------- #
def pin_strict_threshold_and_flags():
    """The test is strict (u = ratio rejects); decisions within 1e-5 of their
    threshold are flagged, decisions further away are not."""
    # p = (1/2, 1/2) and q = (1, 0): the ratio at x = 0 is exactly 1/2
    zt2, zd2 = np.array([0.0, 0.0]), np.array([0.0, -np.inf])
    target = np.stack([zt2, zt2])

    def run(u):
        return oracle.verify(target, zd2[None], "f64", 2, [1], [0], [u, 0.25], [1.0])

    r = run(0.5)
    assert r["n_accepted"][0] == 0 and r["flag_pos"][0] == 0, "u = ratio must reject, flagged"
    r = run(0.5 - U24)
    assert r["n_accepted"][0] == 1 and r["flag_pos"][0] == 0
    r = run(0.5 + 2e-5)
    assert r["n_accepted"][0] == 0 and r["flag_pos"][0] == -1
    r = run(0.5 - 2e-5)
    assert r["n_accepted"][0] == 1 and r["flag_pos"][0] == -1
    # draw near a CDF edge: residual after rejection is (0, 1) -> no edge at u=0.25;
    # the bonus p = (1/2, 1/2) has an edge at u = 1/2
    r = oracle.verify(target, zd2[None], "f64", 2, [1], [0], [0.1, 0.5], [1.0])
    assert r["n_accepted"][0] == 1 and r["emitted"][1] == 1 and r["flag_pos"][0] == 1
    r = oracle.verify(target, zd2[None], "f64", 2, [1], [0], [0.1, 0.5 - 4e-6], [1.0])
    assert r["emitted"][1] == 0 and r["flag_pos"][0] == 1
    r = oracle.verify(target, zd2[None], "f64", 2, [1], [0], [0.1, 0.5 - 4e-5], [1.0])
    assert r["emitted"][1] == 0 and r["flag_pos"][0] == -1


def pin_every_near_decision_flagged():
    """Each decision within 1e-5 of its threshold is flagged, not only the first, and
    only decisions are: the page's all-accept round (ratios 3/4, 1, 5/7, bonus from
    p(.|c) = (3/10, 1/5, 1/2)) with uniforms just below 3/4 and 5/7, far from 1, and
    a draw 3e-6 above the CDF edge 1/2 between b and c; then the page's rejection
    round with a uniform just above 5/7 and one near the unread third ratio."""
    spec = ROUNDS["all_accept_round"]
    drafts = np.array([[TOK[t] for t in spec["drafts"]]], np.int32)
    below = lambda x: float(np.nextafter(np.float32(x), np.float32(0)))
    u = np.array([[below(3 / 4), 0.5, below(5 / 7), float(np.float32(0.5 + 3e-6))]])
    r = markov_verify([TOK["a"]], drafts, u)
    assert r["n_accepted"][0] == 3 and r["emitted"][3] == TOK["c"], r
    assert list(r["flags"]) == [oracle.FLAG_NEAR, 0, oracle.FLAG_NEAR, oracle.FLAG_NEAR], r["flags"]
    assert r["flag_pos"][0] == 0
    # the tokens a draw within 1e-5 of the edge could return: b and c
    assert (r["draw_lo"][0], r["draw_hi"][0]) == (TOK["b"], TOK["c"])
    u[0, 3] = 0.75
    r = markov_verify([TOK["a"]], drafts, u)
    assert r["flags"][3] == 0 and r["draw_lo"][0] == r["draw_hi"][0] == TOK["c"]
    rej = ROUNDS["reject_round"]
    drafts = np.array([[TOK[t] for t in rej["drafts"]]], np.int32)
    above = float(np.nextafter(np.float32(5 / 7), np.float32(1)))
    r = markov_verify([TOK["a"]], drafts, np.array([[0.085, above, F32_BELOW_ONE, 0.4]]))
    assert r["n_accepted"][0] == 1 and r["emitted"][1] == TOK["a"], r
    # the residual after c is (1, 0, 0): one token, no interior edge
    assert list(r["flags"]) == [0, oracle.FLAG_NEAR, 0, 0], r["flags"]
    assert r["draw_lo"][0] == r["draw_hi"][0] == TOK["a"]


def pin_draw_range_by_perturbation():
    """[lo, hi] of a draw are the first and last tokens that the plain inverse CDF
    returns for thresholds within eps * W of t = u W: the draw is repeated over a
    grid of uniforms in [u - eps, u + eps], with windows of one to several tokens."""
    rng = np.random.default_rng(29)
    for trial in range(300):
        V = int(rng.integers(2, 60))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if np.count_nonzero(w) < 2:
            w[:2] = [0.3, 0.7]
        C = np.cumsum(w) / w.sum()
        eps = float(rng.choice([1e-5, 1e-3, 0.05]))
        # uniforms near an interior edge, and anywhere
        edges = C[:-1][(C[:-1] > 0) & (C[:-1] < 1)]
        u = float(rng.choice(edges) + rng.uniform(-0.9, 0.9) * eps) if trial % 3 and edges.size else float(rng.random())
        u = min(max(u, 0.0), 1.0 - 1e-12)
        tok, W, near, lo, hi = oracle.inverse_cdf_range(w, u, eps)
        assert tok == oracle.inverse_cdf(w, u, eps)[0]
        grid = np.clip(np.linspace(u - eps, u + eps, 4001), 0.0, 1.0 - 1e-12)
        seen = sorted({oracle.inverse_cdf(w, g)[0] for g in grid})
        if not near:
            assert lo == hi == tok
            continue
        assert seen[0] == lo and seen[-1] == hi, (trial, u, eps, seen, lo, hi)
        assert w[lo] > 0 and w[hi] > 0 and lo <= tok <= hi


# --------------------------------------------------------------------------- #
# status rules
# --------------------------------------------------------------------------- #
def pin_status_rules():
    rng = np.random.default_rng(41)
    V, g = 16, 3
    zt = rng.standard_normal((4 * (g + 1), V))
    zd = rng.standard_normal((4 * g, V))
    x = rng.integers(0, V, 4 * g).astype(np.int32)
    u = snapped(rng, 4 * (g + 1))
    gam = np.full(4, g, np.int32)
    T = np.ones(4, np.float32)

    def run(zt=zt, zd=zd, x=x, gam=gam, T=T, n=None, mode="sample"):
        return oracle.verify(zt, zd, "f64", V, gam, x, u, T, mode=mode, n_target_rows=n)

    base = run()
    assert np.all(base["row_status"] & oracle.INVALID_MASK == 0)
    # draft token out of range invalidates only its row
    xb = x.copy()
    xb[g + 1] = V
    r = run(x=xb)
    assert r["row_status"][1] & oracle.BAD_TOKEN and r["n_accepted"][1] == -1
    assert np.all(r["emitted"][g + 1:2 * (g + 1)] == -1)
    assert np.array_equal(r["emitted"][:g + 1], base["emitted"][:g + 1])
    # NaN / +inf / all -inf invalidate their row; a single -inf does not
    for bad, invalid in ((np.nan, True), (np.inf, True), (-np.inf, False)):
        zb = zd.copy()
        zb[2 * g + 1, 3] = bad
        r = run(zd=zb)
        assert bool(r["row_status"][2] & oracle.NONFINITE) == invalid, bad
        assert (r["n_accepted"][2] == -1) == invalid
    zb = zt.copy()
    zb[3 * (g + 1) + 2] = -np.inf
    r = run(zt=zb)
    assert r["row_status"][3] & oracle.NONFINITE
    # greedy rows never read draft logits
    zb = zd.copy()
    zb[0, 0] = np.nan
    r = run(zd=zb, mode="greedy")
    assert r["row_status"][0] == 0 and r["n_accepted"][0] >= 0
    # bad gamma: negative, or a row count that does not match
    r = run(gam=np.array([g, -1, g, g], np.int32))
    assert np.all(r["row_status"] == oracle.BAD_GAMMA) and np.all(r["n_accepted"] == -1)
    r = run(n=4 * (g + 1) - 1)
    assert np.all(r["row_status"] == oracle.BAD_GAMMA)
    # temperature: non-finite or subnormal is invalid, <= 0 is greedy
    Tb = np.array([np.nan, np.inf, 1e-39, 1.0], np.float32)
    r = run(T=Tb)
    assert np.all(r["row_status"][:3] & oracle.BAD_TEMP) and r["row_status"][3] == 0
    # q(x) = 0 with p(x) > 0: ratio 1, flagged; q(x) = p(x) = 0 with p = q elsewhere:
    # rejection with zero residual mass falls back to p
    zt3 = np.array([[0.0, 0.0, -np.inf]] * 2)
    zd3 = np.array([[0.0, 0.0, -np.inf]])
    r = oracle.verify(zt3, zd3, "f64", 3, [1], [2], [0.3, 0.7], [1.0])
    assert r["n_accepted"][0] == 0 and r["row_status"][0] == oracle.Q_ZERO | oracle.ZERO_RESID
    assert r["emitted"][0] == 1  # 0.7 of (1/2, 1/2, 0)
    zt4 = np.array([[0.0, 0.0, 0.0]] * 2)
    zd4 = np.array([[0.0, 0.0, -np.inf]])
    r = oracle.verify(zt4, zd4, "f64", 3, [1], [2], [F32_BELOW_ONE, 0.7], [1.0])
    assert r["n_accepted"][0] == 1 and r["row_status"][0] == oracle.Q_ZERO



# --------------------------------------------------------------------------- #
# the drafter's draw (x ~ q)
# --------------------------------------------------------------------------- #
def pin_sample_closed_form():
    """Hand-computed draws: logits (0, ln 3, 0, 0) give (1, 3, 1, 1)/6 at T = 1 and
    (1, 9, 1, 1)/12 at T = 1/2; bf16 logits (0, 1, 0, 0) give (1, e, 1, 1)/(3 + e)."""
    z = np.array([0.0, math.log(3.0), 0.0, 0.0])
    cases = [(1.0, [0.1, 0.2, 0.6, 0.7, 0.95], [0, 1, 1, 2, 3]),
             (0.5, [0.05, 0.5, 0.85, 0.99], [0, 1, 2, 3])]
    for T, us, want in cases:
        r = oracle.sample(np.tile(z, (len(us), 1)), "f64", 4, [T] * len(us), us)
        assert list(r["tokens"]) == want, (T, r["tokens"])
        assert not r["status"].any()
    zb = np.tile(np.array([0x0000, 0x3F80, 0x0000, 0x0000], np.uint16), (5, 1))
    # edges 1/(3+e) = 0.1749, (1+e)/(3+e) = 0.6501, (2+e)/(3+e) = 0.8251
    r = oracle.sample(zb, "bf16", 4, [1.0] * 5, [0.17, 0.18, 0.65, 0.66, 0.83])
    assert list(r["tokens"]) == [0, 1, 1, 2, 3], r["tokens"]


def pin_sample_stratified_counts():
    """Uniforms on a regular grid (k + 1/2)/N hit every token v within one count of
    N p_v, with p = scipy's softmax of z/T."""
    rng = np.random.default_rng(23)
    V, N = 10, 20000
    z = rng.standard_normal(V) * 2.0
    T = 0.7
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    r = oracle.sample(np.tile(z, (N, 1)), "f64", V, np.full(N, T, np.float32), u)
    p = scipy.special.softmax(z / np.float64(np.float32(T)))
    counts = np.bincount(r["tokens"], minlength=V)
    assert np.all(np.abs(counts - N * p) <= 1.0 + 1e-9), (counts, N * p)


def pin_sample_greedy_and_status():
    """T <= 0 takes the first argmax; a bad temperature or a vector without a softmax
    gives token -1 with its status bit; -inf logits are never drawn."""
    z = np.array([[1.0, 3.0, 3.0, 2.0]] * 6)
    z[4, 2] = np.nan
    z[5, :] = -np.inf
    T = np.array([0.0, -1.0, np.nan, 1e-39, 1.0, 1.0], np.float32)
    r = oracle.sample(z, "f64", 4, T, np.full(6, 0.5, np.float32))
    assert list(r["tokens"][:2]) == [1, 1]
    assert r["status"][2] & oracle.BAD_TEMP and r["status"][3] & oracle.BAD_TEMP
    assert r["status"][4] & oracle.NONFINITE and r["status"][5] & oracle.NONFINITE
    assert np.all(r["tokens"][2:] == -1)
    zm = np.array([[-np.inf, 0.0, -np.inf, 0.0]] * 4)
    r = oracle.sample(zm, "f64", 4, np.ones(4, np.float32), [0.0, 0.49, 0.51, F32_BELOW_ONE])
    assert list(r["tokens"]) == [1, 1, 3, 3] and not r["status"].any()



# --------------------------------------------------------------------------- #
# greedy verification of a candidate tree
# --------------------------------------------------------------------------- #
def _tree_brute(z, counts, tokens, parents):
    """Every node's root path by walking parents; a node is kept when every edge on
    it has the child's token equal to numpy's first argmax at the parent; the deepest
    kept node wins, the lowest index on ties."""
    out_n, out_path, out_emit = [], [], []
    o = 0
    for c in counts:
        pred = [int(np.argmax(z[o + k])) for k in range(c)]
        best, best_len = 0, 1
        for k in range(c):
            chain = [k]
            while parents[o + chain[-1]] >= 0:
                chain.append(int(parents[o + chain[-1]]))
            chain.reverse()
            ok = all(tokens[o + chain[d]] == pred[chain[d - 1]] for d in range(1, len(chain)))
            if ok and len(chain) > best_len:
                best, best_len = k, len(chain)
        chain = [best]
        while parents[o + chain[-1]] >= 0:
            chain.append(int(parents[o + chain[-1]]))
        chain.reverse()
        out_n.append(len(chain) - 1)
        out_path.append(chain + [-1] * (c - len(chain)))
        out_emit.append([int(tokens[o + j]) for j in chain[1:]] + [pred[best]] + [-1] * (c - len(chain)))
        o += c
    return np.array(out_n), np.concatenate(out_path), np.concatenate(out_emit)


def _random_trees(rng, B, nmax, V):
    counts = rng.integers(1, nmax + 1, B).astype(np.int32)
    parents, tokens = [], []
    for c in counts:
        parents += [-1] + [int(rng.integers(0, k)) for k in range(1, c)]
    n = int(counts.sum())
    # small integer logits: ties everywhere, so the lowest-index rule is exercised
    z = rng.integers(-2, 3, (n, V)).astype(np.float64)
    o = 0
    for c in counts:
        for k in range(c):
            par = parents[o + k]
            if par < 0 or rng.random() < 0.3:
                tokens.append(int(rng.integers(0, V)))
            else:
                tokens.append(int(np.argmax(z[o + par])))   # a child that will be kept
        o += c
    return z, counts, np.array(tokens, np.int32), np.array(parents, np.int32)


def pin_tree_brute_force():
    rng = np.random.default_rng(31)
    for _ in range(30):
        z, counts, tokens, parents = _random_trees(rng, 6, 12, 5)
        r = oracle.tree_greedy(z, "f64", 5, counts, tokens, parents)
        n, path, emit = _tree_brute(z, counts, tokens, parents)
        assert not r["status"].any()
        assert np.array_equal(r["n_accepted"], n), (r["n_accepted"], n)
        assert np.array_equal(r["path"], path)
        assert np.array_equal(r["emitted"], emit)


def pin_tree_chain_is_linear_greedy():
    """A chain (node k's parent is k - 1) is a row of drafts: the result is the linear
    greedy verification of tokens 1 .. n-1 against the nodes' logits."""
    rng = np.random.default_rng(32)
    B, V = 40, 30
    counts = rng.integers(1, 9, B).astype(np.int32)
    n = int(counts.sum())
    z = rng.standard_normal((n, V))
    parents, tokens = [], []
    o = 0
    for c in counts:
        am = np.argmax(z[o:o + c], axis=1)
        for k in range(c):
            parents.append(k - 1)
            tokens.append(int(am[k - 1]) if k > 0 and rng.random() < 0.75 else int(rng.integers(0, V)))
        o += c
    tokens = np.array(tokens, np.int32)
    r = oracle.tree_greedy(z, "f64", V, counts, tokens, parents)
    drafts = np.concatenate([tokens[o + 1:o + c] for o, c in zip(np.cumsum(counts) - counts, counts)])
    lin = oracle.verify(z, np.zeros((n - B, V)), "f64", V, counts - 1, drafts.astype(np.int32),
                        np.zeros(n, np.float32), np.ones(B, np.float32), mode="greedy")
    assert np.array_equal(r["n_accepted"], lin["n_accepted"])
    assert np.array_equal(r["emitted"], lin["emitted"])
    for i, (o, c) in enumerate(zip(np.cumsum(counts) - counts, counts)):
        K = lin["n_accepted"][i]
        assert list(r["path"][o:o + c]) == list(range(K + 1)) + [-1] * (c - K - 1)


def pin_tree_hand_example():
    """Root 0 with children 1 (token 3) and 2 (token 1); node 3 (token 0) under 1,
    nodes 4 (token 2) and 5 (token 4) under 2, node 6 (token 0) under 4.  The argmax
    is 1 at the root, 2 at node 2, 0 at node 4 and 3 at node 6, so the kept path is
    0 -> 2 -> 4 -> 6 and the next token is 3."""
    parents = np.array([-1, 0, 0, 1, 2, 2, 4], np.int32)
    tokens = np.array([9, 3, 1, 0, 2, 4, 0], np.int32)
    am = [1, 4, 2, 0, 0, 1, 3]
    z = np.zeros((7, 10))
    for k, a in enumerate(am):
        z[k, a] = 5.0
    r = oracle.tree_greedy(z, "f64", 10, [7], tokens, parents)
    assert r["n_accepted"][0] == 3
    assert list(r["path"]) == [0, 2, 4, 6, -1, -1, -1]
    assert list(r["emitted"]) == [1, 2, 0, 3, -1, -1, -1]
    # two kept paths of equal length: the one ending at the lower node index wins
    tokens2 = np.array([9, 1, 1, 4, 4, 2, 0], np.int32)
    am2 = [1, 4, 4, 7, 8, 1, 3]
    z2 = np.zeros((7, 10))
    for k, a in enumerate(am2):
        z2[k, a] = 5.0
    r = oracle.tree_greedy(z2, "f64", 10, [7], tokens2, parents)
    assert r["n_accepted"][0] == 2 and list(r["path"][:3]) == [0, 1, 3]
    assert list(r["emitted"][:3]) == [1, 4, 7]


def pin_tree_status():
    z = np.zeros((5, 4))
    z[:, 1] = 1.0
    ok = oracle.tree_greedy(z, "f64", 4, [2, 3], [0, 1, 0, 1, 1], [-1, 0, -1, 0, 1])
    assert list(ok["n_accepted"]) == [1, 2] and not ok["status"].any()
    r = oracle.tree_greedy(z, "f64", 4, [2, 3], [0, 1, 0, 1, 1], [-1, 0, -1, 0, 2])   # parent not earlier
    assert r["status"][1] & oracle.BAD_TREE and r["n_accepted"][1] == -1 and r["status"][0] == 0
    r = oracle.tree_greedy(z, "f64", 4, [2, 3], [0, 1, 0, 1, 1], [0, 0, -1, 0, 1])    # root with a parent
    assert r["status"][0] & oracle.BAD_TREE
    r = oracle.tree_greedy(z, "f64", 4, [2, 3], [0, 7, 0, 1, 1], [-1, 0, -1, 0, 1])   # token out of range
    assert r["status"][0] & oracle.BAD_TOKEN and np.all(r["emitted"][:2] == -1)
    zn = z.copy()
    zn[3, 2] = np.nan
    r = oracle.tree_greedy(zn, "f64", 4, [2, 3], [0, 1, 0, 1, 1], [-1, 0, -1, 0, 1])
    assert r["status"][1] & oracle.NONFINITE and r["status"][0] == 0
    r = oracle.tree_greedy(z, "f64", 4, [2, 2], [0, 1, 0, 1, 1], [-1, 0, -1, 0, 1])   # counts != nodes
    assert np.all(r["status"] == oracle.BAD_GAMMA) and np.all(r["emitted"] == -1)



# --------------------------------------------------------------------------- #
# early exit and the cache entries to keep
# --------------------------------------------------------------------------- #
def pin_early_exit_page_round():
    """The page's round with a rejection, read left to right: the same decisions and
    page values, nothing computed after the rejection, and the page's cache counts:
    5 entries before the round, 9 after the verification pass wrote the last token and
    the three drafts, 7 kept once one draft is accepted (rayaq.ca "Speculative
    decoding", section "A round with a rejection")."""
    spec = ROUNDS["reject_round"]
    drafts = np.array([[TOK[t] for t in spec["drafts"]]], np.int32)
    u = np.array([[spec["positions"][0]["u"], spec["positions"][1]["u"], 0.5, 0.3]])
    before = spec["cache_entries_before"]
    # the fixture is the page's: the verification pass adds the last token and gamma drafts
    assert before + 1 + spec["gamma"] == spec["cache_entries_after_verify"]
    r = markov_verify([TOK["a"]], drafts, u, early_exit=True, cache_len=[before])
    assert r["n_accepted"][0] == spec["n_accepted"] == 1
    assert [t for t in r["emitted"] if t >= 0] == [TOK[t] for t in spec["emitted"]]
    _close(r["p_x"][1] / r["q_x"][1], 5 / 7, 1e-15, "ratio 5/7")
    assert np.isnan(r["p_x"][2]) and np.isnan(r["q_x"][2])
    assert r["crop_len"][0] == spec["cache_entries_kept"], r["crop_len"]
    full = markov_verify([TOK["a"]], drafts, u, cache_len=[before])
    assert not np.isnan(full["p_x"][2])
    assert full["crop_len"][0] == spec["cache_entries_kept"]


def pin_early_exit_matches_full_round():
    """On finite logits the early-exit round keeps the same drafts, draws the same
    token with the same mass, and agrees on p(x_j), q(x_j) up to the rejection."""
    rng = np.random.default_rng(41)
    B, V = 60, 50
    gam = rng.integers(0, 7, B).astype(np.int32)
    nT = int(gam.sum() + B)
    zt = rng.standard_normal((nT, V)) * 2
    zd = np.concatenate([zt[o:o + g] for o, g in zip(np.cumsum(gam + 1) - gam - 1, gam)]) + \
        rng.standard_normal((int(gam.sum()), V)) * 0.7
    x = rng.integers(0, V, int(gam.sum())).astype(np.int32)
    u = snapped(rng, nT)
    T = (0.5 + rng.random(B)).astype(np.float32)
    n = rng.integers(0, 1000, B).astype(np.int32)
    a = oracle.verify(zt, zd, "f64", V, gam, x, u, T, cache_len=n)
    b = oracle.verify(zt, zd, "f64", V, gam, x, u, T, early_exit=True, cache_len=n)
    for k in ("n_accepted", "emitted", "row_status", "flag_pos", "resid_mass", "crop_len"):
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(b["crop_len"], n + a["n_accepted"] + 1)
    d0 = np.cumsum(gam) - gam
    for i in range(B):
        K = a["n_accepted"][i]
        for j in range(gam[i]):
            if j <= K:
                assert b["p_x"][d0[i] + j] == a["p_x"][d0[i] + j]
            else:
                assert np.isnan(b["p_x"][d0[i] + j]) and np.isnan(b["q_x"][d0[i] + j])


def pin_early_exit_reads_only_up_to_the_rejection():
    """A NaN logit after the first rejection leaves the early-exit row valid (the full
    round flags it); one at or before the rejection invalidates both; greedy rows
    likewise; a bad token anywhere invalidates both."""
    V, g = 6, 4
    zt = np.zeros((g + 1, V))
    zt[:, 2] = 3.0
    zd = np.zeros((g, V))
    zd[:, 2] = 3.0
    zd[1, 2] = -3.0               # position 1: q(2) small, p(2) large: kept
    x = np.array([2, 2, 4, 2], np.int32)   # position 2: token 4 with p < q: rejected at u = 0.99
    u = np.array([0.5, 0.5, 0.99, 0.5, 0.5], np.float32)
    run = lambda zt_, zd_, xx=x, **kw: oracle.verify(zt_, zd_, "f64", V, [g], xx, u, [1.0], **kw)
    zd4 = zd.copy()
    zd4[2, 4] = 4.0
    assert run(zt, zd4)["n_accepted"][0] == 2
    for early, ok in ((True, True), (False, False)):
        zt_nan = zt.copy()
        zt_nan[3, 0] = np.nan
        r = run(zt_nan, zd4, early_exit=early)
        assert (r["row_status"][0] == 0) == ok and (r["n_accepted"][0] == 2) == ok
        zd_nan = zd4.copy()
        zd_nan[3, 1] = np.nan
        assert (run(zt, zd_nan, early_exit=early)["row_status"][0] == 0) == ok
        zt_nan2 = zt.copy()
        zt_nan2[2, 0] = np.nan
        assert run(zt_nan2, zd4, early_exit=early)["row_status"][0] & oracle.NONFINITE
        bad = x.copy()
        bad[3] = V
        assert run(zt, zd4, bad, early_exit=early)["row_status"][0] & oracle.BAD_TOKEN
    # greedy: the argmax is 2 everywhere, so the draft 4 at position 2 is the mismatch
    zt_nan = zt.copy()
    zt_nan[4, 0] = np.nan
    r = run(zt_nan, zd4, mode="greedy", early_exit=True)
    assert r["row_status"][0] == 0 and r["n_accepted"][0] == 2 and r["emitted"][2] == 2
    assert run(zt_nan, zd4, mode="greedy")["row_status"][0] & oracle.NONFINITE



# --------------------------------------------------------------------------- #
# top-k and top-p filtering of p and q
# --------------------------------------------------------------------------- #
def pin_filter_closed_forms():
    """Hand-counted thresholds: probabilities (0.5, 0.3, 0.15, 0.05) keep 1, 2, 3, 4
    tokens at top-p 0.49, 0.79, 0.81, 0.96; top-k counts ties; top-k = 3 before top-p
    renormalizes (0.4, 0.3, 0.2, 0.1) to (4, 3, 2)/9, so top-p 0.75 keeps 2 tokens
    instead of 3."""
    z = np.log([0.5, 0.3, 0.15, 0.05])
    for tp, kept in ((0.49, 1), (0.79, 2), (0.81, 3), (0.96, 4)):
        th, near = oracle.filter_threshold(z, 1.0, top_p=tp)
        assert np.sum(z >= th) == kept and not near, (tp, th)
    zt = np.array([3.0, 1.0, 1.0, 1.0, 0.0])
    assert oracle.filter_threshold(zt, 1.0, top_k=2)[0] == 1.0          # keeps 4 (ties)
    assert oracle.filter_threshold(zt, 1.0, top_k=1)[0] == 3.0
    assert oracle.filter_threshold(zt, 1.0, top_k=5)[0] == -np.inf      # k >= V: no filter
    z4 = np.log([0.4, 0.3, 0.2, 0.1])
    assert np.sum(z4 >= oracle.filter_threshold(z4, 1.0, top_p=0.75)[0]) == 3
    assert np.sum(z4 >= oracle.filter_threshold(z4, 1.0, top_k=3, top_p=0.75)[0]) == 2
    # temperature sharpens before top-p: T = 1/2 squares the odds, (25, 9, 2.25, 0.25)/36.5
    assert np.sum(z >= oracle.filter_threshold(z, 0.5, top_p=0.9)[0]) == 2
    # bf16 logits (2, 1, 1, 0): e^(z) = (7.389, 2.718, 2.718, 1) over 13.825
    zb = np.array([[0x4000, 0x3F80, 0x3F80, 0x0000]], np.uint16)
    th, _ = oracle.filter_threshold(zb, 1.0, top_p=0.6, dtype="bf16")
    assert th == 1.0                                                   # 0.534 < 0.6 <= 0.928


def pin_filter_vs_sorting():
    """Thresholds against numpy: the top_k-th largest value, then the first group of
    equal logits (in decreasing order) where scipy's softmax over the kept tokens
    reaches top_p."""
    rng = np.random.default_rng(43)
    for _ in range(300):
        V = int(rng.integers(2, 60))
        z = rng.integers(-6, 7, V).astype(np.float64) * 0.5   # many ties
        T = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.integers(0, V + 2))
        tp = float(rng.choice([1.0, rng.random()]))
        th, near = oracle.filter_threshold(z, T, top_k=k, top_p=tp)
        desc = np.sort(z)[::-1]
        want = desc[k - 1] if 0 < k < V else -np.inf
        if 0 < tp < 1:
            kept = z[z >= want]
            p = scipy.special.softmax(kept / T)
            vals = np.unique(kept)[::-1]
            cum = np.cumsum([p[kept == v].sum() for v in vals])
            i = int(np.argmax(cum >= tp)) if (cum >= tp).any() else len(vals) - 1
            if abs(cum[i] - tp) < 1e-9 or (i > 0 and abs(tp - cum[i - 1]) < 1e-9):
                continue
            want = vals[i]
        assert th == want, (z, T, k, tp, th, want)


def pin_top1_sampling_is_greedy():
    """top_k = 1 on both models makes p and q one-hot at their argmaxes: with drafts
    equal to the drafter's argmax, the sampling round is the greedy round whatever the
    uniforms."""
    rng = np.random.default_rng(44)
    B, V = 50, 40
    gam = rng.integers(0, 6, B).astype(np.int32)
    nT, nD = int(gam.sum() + B), int(gam.sum())
    zt = rng.standard_normal((nT, V))
    d_off = np.cumsum(gam) - gam
    t_off = np.cumsum(gam + 1) - gam - 1
    zd = np.concatenate([zt[o:o + g] for o, g in zip(t_off, gam)]) + rng.standard_normal((nD, V)) * 0.8
    x = np.argmax(zd, axis=1).astype(np.int32)
    u = snapped(rng, nT)
    T = np.full(B, 0.9, np.float32)
    a = oracle.verify(zt, zd, "f64", V, gam, x, u, T, top_k=np.ones(B, np.int32))
    g = oracle.verify(zt, zd, "f64", V, gam, x, u, T, mode="greedy")
    assert np.array_equal(a["n_accepted"], g["n_accepted"])
    assert np.array_equal(a["emitted"], g["emitted"])
    # and no filter (top_k >= V, top_p >= 1) is the plain round
    b = oracle.verify(zt, zd, "f64", V, gam, x, u, T, top_k=np.full(B, V, np.int32),
                      top_p=np.ones(B, np.float32))
    c = oracle.verify(zt, zd, "f64", V, gam, x, u, T)
    for k in ("n_accepted", "emitted", "p_x", "q_x", "resid_mass"):
        assert np.array_equal(b[k], c[k], equal_nan=True), k


def pin_filtered_output_distribution():
    """With p and q both filtered (top-k 5, top-p 0.8) and drafts drawn from the
    filtered q, the token emitted at the first position is distributed as the filtered
    p (chi-square over 40,000 rounds)."""
    rng = np.random.default_rng(45)
    V, g, N = 10, 2, 40000
    zt1 = rng.standard_normal(V) * 1.5
    zd1 = zt1 + rng.standard_normal(V)
    zt = np.tile(zt1, (g + 1, 1))
    zd = np.tile(zd1, (g, 1))
    def filtered(z):
        th, _ = oracle.filter_threshold(z, 1.0, top_k=5, top_p=0.8)
        p = np.where(z >= th, np.exp(z - z.max()), 0.0)
        return p / p.sum()
    pf, qf = filtered(zt1), filtered(zd1)
    x = rng.choice(V, size=(N, g), p=qf).astype(np.int32)
    u = snapped(rng, N * (g + 1))
    r = oracle.verify(np.tile(zt, (N, 1)), np.tile(zd, (N, 1)), "f64", V, np.full(N, g, np.int32),
                      x.reshape(-1), u, np.ones(N, np.float32), top_k=np.full(N, 5, np.int32),
                      top_p=np.full(N, 0.8, np.float32))
    first = r["emitted"].reshape(N, g + 1)[:, 0]
    _chi2_ok(np.bincount(first, minlength=V), pf, "filtered emission")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
