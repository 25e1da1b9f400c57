"""Seeded synthetic workloads for the speculative-sampling verification step.

This module only *produces inputs*: logits, draft tokens, uniforms, temperatures
and per-row draft lengths.  It holds none of the verification arithmetic (no
temperature softmax, no acceptance ratio, no residual, no inverse-CDF draw), so
both the HIP path and the CPU oracle may consume what it makes.

Layout (the packed layout of the library's C ABI):
  * row i has gamma_i drafts; target rows t_off[i] .. t_off[i]+gamma_i hold the
    target logits of the gamma_i+1 verified positions, draft rows
    d_off[i] .. d_off[i]+gamma_i-1 hold the drafter logits of the gamma_i drafts;
  * t_off / d_off are exclusive prefix sums of gamma_i+1 / gamma_i;
  * logits are row-major [rows, V]; bf16 logits are stored as their uint16 bit
    patterns (round-to-nearest-even from float32), fp32 logits as float32;
  * uniforms[t_off[i] + j] (j < gamma_i) drives the accept test of draft j, and
    uniforms[t_off[i] + gamma_i] drives the single residual-or-bonus draw;
    every uniform is k * 2^-24 for an integer k in [0, 2^24), so it is exact in
    float32 and in float64.

Draft tokens are what a drafter would have produced: in sampling mode a sample
of softmax(draft/T) drawn with the Gumbel-max construction (argmax of logits/T
plus Gumbel noise), in greedy mode the argmax of the draft logits (the greedy
drafter).  Both are input generation, done before and apart from verification.

Every random number comes from numpy's Philox bit generator, keyed per
(seed, workload, row) through a SeedSequence, so a workload is reproducible and
its rows can be generated in parallel.

The five workloads follow the configurations the verification step is measured
on: a 32-token toy for the statistical checks, and bf16/fp32 batches at
V = 32000, 128256, 152064 and 256000.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

U24 = float(2.0 ** -24)


# --------------------------------------------------------------------------- #
# container
# --------------------------------------------------------------------------- #
@dataclass
class Workload:
    name: str
    dtype: str                 # "bf16" | "f32"
    vocab: int
    gamma: np.ndarray          # int32 [B]
    target: np.ndarray         # uint16 bits (bf16) or float32, [n_target_rows, V]
    draft: np.ndarray          # same dtype, [n_draft_rows, V]
    draft_tokens: np.ndarray   # int32 [n_draft_rows]
    uniforms: np.ndarray       # float32 [n_target_rows]
    temperature: np.ndarray    # float32 [B]
    mode: str = "sample"       # "sample" | "greedy"
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.gamma.shape[0])

    @property
    def n_target_rows(self) -> int:
        return int(self.target.shape[0])

    @property
    def n_draft_rows(self) -> int:
        return int(self.draft.shape[0])

    @property
    def dense_gamma(self):
        """The common draft length if every row has the same one, else None."""
        if self.batch and np.all(self.gamma == self.gamma[0]):
            return int(self.gamma[0])
        return None

    def offsets(self):
        """(t_off, d_off) as int64 arrays of length B+1 (layout bookkeeping)."""
        t = np.zeros(self.batch + 1, np.int64)
        d = np.zeros(self.batch + 1, np.int64)
        np.cumsum(self.gamma.astype(np.int64) + 1, out=t[1:])
        np.cumsum(self.gamma.astype(np.int64), out=d[1:])
        return t, d

    def logit_bytes(self) -> int:
        return int(self.target.nbytes + self.draft.nbytes)

    def with_mode(self, mode: str) -> "Workload":
        w = Workload(**{**self.__dict__})
        w.mode = mode
        return w


# --------------------------------------------------------------------------- #
# helpers (input generation only)
# --------------------------------------------------------------------------- #
def _rng(seed: int, stream: int, row: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=(int(stream), int(row)))
    return np.random.Generator(np.random.Philox(ss))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def logits_as_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(arr) if dtype == "bf16" else np.asarray(arr, np.float32)


def snapped_uniforms(rng: np.random.Generator, n: int) -> np.ndarray:
    k = rng.integers(0, 1 << 24, size=n, dtype=np.int64)
    return (k.astype(np.float64) * U24).astype(np.float32)


def gumbel_max_token(rng: np.random.Generator, logits_f32: np.ndarray, temperature: float,
                     top_k: int = 0) -> int:
    """One draw from softmax(logits / T) by the Gumbel-max construction; with top_k > 0,
    from the top_k largest logits only (Gumbel-max over that index set: a draw from the
    distribution restricted to them, chosen by rank alone).  T <= 0 is a greedy drafter:
    the first argmax of the raw logits (the Gumbel noise is still drawn, so the stream
    stays aligned)."""
    z = logits_f32.astype(np.float64)
    idx = None
    if 0 < top_k < z.shape[0]:
        idx = np.sort(np.argpartition(-z, top_k - 1)[:top_k])
        z = z[idx]
    g = -np.log(rng.standard_exponential(z.shape[0]))
    if not (float(temperature) > 0.0):
        pick = int(np.argmax(z))
    else:
        pick = int(np.argmax(z / float(temperature) + g))
    return int(idx[pick]) if idx is not None else pick


def _store(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x_f32) if dtype == "bf16" else x_f32.astype(np.float32)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------- #
# generic builder
# --------------------------------------------------------------------------- #
def build(name: str, dtype: str, vocab: int, gamma, temperature, seed: int,
          target_fn, draft_fn, mode: str = "sample", draft_tokens_fn=None,
          meta=None, draft_top_k: int = 0) -> Workload:
    """Assemble a packed workload row by row.

    target_fn(rng, row, n_pos) -> float32 [n_pos, V]   (pre-rounding target logits)
    draft_fn(rng, row, tgt)    -> float32 [gamma, V]    (pre-rounding draft logits)
    draft_tokens_fn(rng, row, draft_stored_f32, T) -> int32 [gamma] (optional)
    draft_top_k > 0: sampled drafts come from the draft_top_k largest draft logits of
    their position (a drafter that samples from its own top-k set)
    """
    gamma = np.asarray(gamma, np.int32)
    B = gamma.shape[0]
    temperature = np.asarray(temperature, np.float32)
    if temperature.ndim == 0:
        temperature = np.full(B, float(temperature), np.float32)
    t_off = np.concatenate([[0], np.cumsum(gamma.astype(np.int64) + 1)])
    d_off = np.concatenate([[0], np.cumsum(gamma.astype(np.int64))])
    store_dt = np.uint16 if dtype == "bf16" else np.float32
    target = np.empty((int(t_off[-1]), vocab), store_dt)
    draft = np.empty((int(d_off[-1]), vocab), store_dt)
    tokens = np.empty(int(d_off[-1]), np.int32)
    uniforms = np.empty(int(t_off[-1]), np.float32)

    def one_row(i: int):
        g = int(gamma[i])
        rng = _rng(seed, 1, i)
        tgt = target_fn(rng, i, g + 1)
        target[t_off[i]:t_off[i + 1]] = _store(tgt, dtype)
        if g > 0:
            drf = draft_fn(rng, i, tgt[:g])
            draft[d_off[i]:d_off[i + 1]] = _store(drf, dtype)
            stored = logits_as_f32(draft[d_off[i]:d_off[i + 1]], dtype)
            if draft_tokens_fn is not None:
                tok = draft_tokens_fn(rng, i, stored, float(temperature[i]))
            elif mode == "greedy":
                tok = np.argmax(stored, axis=1)
            else:
                tok = [gumbel_max_token(rng, stored[j], float(temperature[i]), draft_top_k) for j in range(g)]
            tokens[d_off[i]:d_off[i + 1]] = np.asarray(tok, np.int32)
        uniforms[t_off[i]:t_off[i + 1]] = snapped_uniforms(_rng(seed, 2, i), g + 1)

    if B * vocab >= (1 << 20):
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one_row, range(B)))
    else:
        for i in range(B):
            one_row(i)
    return Workload(name=name, dtype=dtype, vocab=vocab, gamma=gamma, target=target,
                    draft=draft, draft_tokens=tokens, uniforms=uniforms,
                    temperature=temperature, mode=mode, meta=dict(meta or {}, seed=seed))


# --------------------------------------------------------------------------- #
# logit shapes
# --------------------------------------------------------------------------- #
def _normal_target(vocab: int, sigma: float):
    def fn(rng, row, n_pos):
        return rng.standard_normal((n_pos, vocab), dtype=np.float32) * np.float32(sigma)
    return fn


def _boosted_target(vocab: int, sigma: float, n_boost: int, boost: float):
    """N(0, sigma) logits with n_boost distinct random entries per position raised by +boost."""
    def fn(rng, row, n_pos):
        x = rng.standard_normal((n_pos, vocab), dtype=np.float32) * np.float32(sigma)
        for j in range(n_pos):
            idx = rng.choice(vocab, size=n_boost, replace=False)
            x[j, idx] += np.float32(boost)
        return x
    return fn


def _zipf_target(vocab: int, sigma: float, s: float):
    """N(0, sigma) logits plus -s*ln(rank) under a fresh random token permutation per
    position, i.e. probabilities tilted by a Zipf(s) factor rank^-s."""
    log_rank = (-s * np.log(np.arange(1, vocab + 1, dtype=np.float64))).astype(np.float32)

    def fn(rng, row, n_pos):
        x = rng.standard_normal((n_pos, vocab), dtype=np.float32) * np.float32(sigma)
        for j in range(n_pos):
            x[j] += log_rank[rng.permutation(vocab)]
        return x
    return fn


def _noisy_draft(scale: float, sigma):
    """draft = scale * target + N(0, sigma_row)."""
    def fn(rng, row, tgt):
        sg = sigma(row) if callable(sigma) else sigma
        return (np.float32(scale) * tgt
                + rng.standard_normal(tgt.shape, dtype=np.float32) * np.float32(sg))
    return fn


# --------------------------------------------------------------------------- #
# the five configurations
# --------------------------------------------------------------------------- #
def toy(seed: int = 1, rounds: int = 10_000, gamma: int = 4, vocab: int = 32,
        shared_position: bool = False) -> Workload:
    """B=1, gamma=4, V=32 fp32 toy: target ~ N(0,2), draft = target + N(0,0.5), T=1.

    The single row's logits are fixed and replicated over `rounds` independent
    rounds (one packed row per round); every round draws its own draft tokens
    from q and its own uniforms.  With shared_position=True every position uses
    the same (p, q) pair, so the acceptance rate is the same at every position.
    """
    base = _rng(seed, 0, 0)
    if shared_position:
        t1 = base.standard_normal(vocab) * 2.0
        tgt = np.tile(t1, (gamma + 1, 1))
        d1 = t1 + base.standard_normal(vocab) * 0.5
        drf = np.tile(d1, (gamma, 1))
    else:
        tgt = base.standard_normal((gamma + 1, vocab)) * 2.0
        drf = tgt[:gamma] + base.standard_normal((gamma, vocab)) * 0.5
    tgt = tgt.astype(np.float32)
    drf = drf.astype(np.float32)
    B = rounds
    target = np.tile(tgt, (B, 1))
    draft = np.tile(drf, (B, 1))
    # Gumbel-max draws of every round's drafts from softmax(draft), fp64
    rng = _rng(seed, 3, 0)
    g = -np.log(rng.standard_exponential((B, gamma, vocab)))
    tokens = np.argmax(drf.astype(np.float64)[None] + g, axis=2).astype(np.int32).reshape(-1)
    uniforms = snapped_uniforms(_rng(seed, 2, 0), B * (gamma + 1))
    return Workload(name="toy" + ("_shared" if shared_position else ""), dtype="f32",
                    vocab=vocab, gamma=np.full(B, gamma, np.int32), target=target,
                    draft=draft, draft_tokens=tokens, uniforms=uniforms,
                    temperature=np.ones(B, np.float32), mode="sample",
                    meta=dict(seed=seed, rounds=rounds, base_target=tgt, base_draft=drf))


def c2(seed: int = 2) -> Workload:
    """B=8, gamma=4, V=32000 bf16; target N(0,3) with 5 logits +8 per position;
    draft = target + N(0,1); T=1."""
    V = 32000
    return build("c2_b8_g4_v32000_bf16", "bf16", V, np.full(8, 4), 1.0, seed,
                 _boosted_target(V, 3.0, 5, 8.0), _noisy_draft(1.0, 1.0))


def c3(seed: int = 3, mode: str = "sample", batch: int = 64, draft_scale: float = 0.8,
       draft_sigma: float = 1.5, draft_top_k: int = 0) -> Workload:
    """B=64, gamma=5, V=128256 bf16; target N(0,3) + Zipf(1.1) log-boost on a random
    permutation; draft = 0.8*target + N(0,1.5); T=0.8; sampling or greedy.  draft_scale
    and draft_sigma change the draft (1.0 and 0.2: a draft close to its target, whose
    rows mostly keep every draft); draft_top_k > 0 samples the drafts from the draft's
    top-k set."""
    V = 128256
    tag = "" if (draft_scale, draft_sigma, draft_top_k) == (0.8, 1.5, 0) else \
        f"_d{draft_scale:g}x_n{draft_sigma:g}" + (f"_dk{draft_top_k}" if draft_top_k else "")
    return build(f"c3_b{batch}_g5_v128256_bf16_{mode}{tag}", "bf16", V, np.full(batch, 5), 0.8, seed,
                 _zipf_target(V, 3.0, 1.1), _noisy_draft(draft_scale, draft_sigma), mode=mode,
                 draft_top_k=draft_top_k)


def c4(seed: int = 4, batch: int = 256, draft_top_k: int = 0) -> Workload:
    """B=256, gamma=8, V=152064 bf16 as c2; per-row T ~ U[0.5,1.5]; per-row draft
    noise sigma ~ U[0.2,3.0].  draft_top_k > 0 samples the drafts from the draft's
    top-k set."""
    V = 152064
    prm = _rng(seed, 9, 0)
    temps = prm.uniform(0.5, 1.5, batch).astype(np.float32)
    sig = prm.uniform(0.2, 3.0, batch)
    return build(f"c4_b{batch}_g8_v152064_bf16" + (f"_dk{draft_top_k}" if draft_top_k else ""), "bf16", V,
                 np.full(batch, 8), temps, seed,
                 _boosted_target(V, 3.0, 5, 8.0), _noisy_draft(1.0, lambda r: float(sig[r])),
                 meta=dict(draft_sigma=sig), draft_top_k=draft_top_k)


def c5(seed: int = 5, batch: int = 512) -> Workload:
    """Ragged B=512, gamma_i ~ U{0..7}, V=256000 fp32; target N(0,4); draft = target + N(0,1); T=1."""
    V = 256000
    prm = _rng(seed, 9, 0)
    gam = prm.integers(0, 8, batch).astype(np.int32)
    return build(f"c5_b{batch}_ragged_v256000_f32", "f32", V, gam, 1.0, seed,
                 _normal_target(V, 4.0), _noisy_draft(1.0, 1.0))


def small(seed: int, batch: int, vocab: int, dtype: str, gamma, temperature=1.0,
          sigma: float = 3.0, noise: float = 1.0, mode: str = "sample", n_boost: int = 0) -> Workload:
    """Small generic workload for parity tests (ragged gamma allowed)."""
    gamma = np.asarray(gamma, np.int32)
    if gamma.ndim == 0:
        gamma = np.full(batch, int(gamma), np.int32)
    tf = _boosted_target(vocab, sigma, n_boost, 8.0) if n_boost else _normal_target(vocab, sigma)
    return build(f"small_b{batch}_v{vocab}_{dtype}_{mode}", dtype, vocab, gamma, temperature, seed,
                 tf, _noisy_draft(1.0, noise), mode=mode)


@dataclass
class SampleInputs:
    """Inputs of the drafter's draw: n logit vectors, one temperature and one uniform
    each."""
    name: str
    dtype: str
    vocab: int
    logits: np.ndarray         # uint16 bits (bf16) or float32, [n, V]
    temperature: np.ndarray    # float32 [n]
    uniforms: np.ndarray       # float32 [n], k * 2^-24

    @property
    def n(self) -> int:
        return int(self.logits.shape[0])


def sample_inputs(w: Workload, seed: int, side: str = "draft", limit: int | None = None) -> SampleInputs:
    """The vectors of one side of a workload (its draft rows, or its target rows), each
    with its row's temperature and a fresh uniform from its own Philox stream."""
    t_off, d_off = w.offsets()
    if side == "draft":
        logits = w.draft
        temp = np.repeat(w.temperature, w.gamma)
    else:
        logits = w.target
        temp = np.repeat(w.temperature, w.gamma + 1)
    if limit is not None:
        logits, temp = logits[:limit], temp[:limit]
    u = snapped_uniforms(_rng(seed, 7, 0), logits.shape[0])
    return SampleInputs(f"{w.name}_{side}", w.dtype, w.vocab, np.ascontiguousarray(logits),
                        np.ascontiguousarray(temp, np.float32), u)


@dataclass
class TreeInputs:
    """Candidate trees for greedy tree verification, packed tree after tree: node k of
    tree i is row off_i + k of `logits`; parents are tree-local, -1 for the root,
    listed before their children."""
    name: str
    dtype: str
    vocab: int
    counts: np.ndarray         # int32 [B]
    tokens: np.ndarray         # int32 [n_nodes]
    parents: np.ndarray        # int32 [n_nodes]
    logits: np.ndarray         # uint16 bits (bf16) or float32, [n_nodes, V]

    @property
    def n_nodes(self) -> int:
        return int(self.tokens.shape[0])


def medusa_shape(top_k: int, heads: int):
    """Parents and depths of a Medusa candidate tree: the root, then per level every
    node of the previous level gets top_k children, level by level."""
    parents, depths, level = [-1], [0], [0]
    for d in range(1, heads + 1):
        nxt = []
        for par in level:
            for _ in range(top_k):
                nxt.append(len(parents))
                parents.append(par)
                depths.append(d)
        level = nxt
    return np.array(parents, np.int32), np.array(depths, np.int32)


def trees(seed: int, batch: int, vocab: int, dtype: str, top_k=2, heads=5, accept: float = 0.7,
          sigma: float = 3.0, random_shape: bool = False) -> TreeInputs:
    """Medusa-shaped trees (or, with random_shape, random trees in parents-first
    order) over normal logits.  Every level has top_k candidate tokens shared by all
    its nodes, as when each level's tokens come from one head.  With probability
    `accept` a node's logits are shaped so that their argmax is one of the next
    level's candidates (so that child is kept), else a random token."""
    counts, toks, pars, rows = [], [], [], []
    tk = np.atleast_1d(np.asarray(top_k))
    hd = np.atleast_1d(np.asarray(heads))
    for i in range(batch):
        rng = _rng(seed, 11, i)
        k_i, h_i = int(tk[i % tk.size]), int(hd[i % hd.size])
        if random_shape:
            n = int(rng.integers(1, max(2, k_i ** h_i) + 1))
            par = np.array([-1] + [int(rng.integers(0, j)) for j in range(1, n)], np.int32)
            dep = np.zeros(n, np.int32)
            for j in range(1, n):
                dep[j] = dep[par[j]] + 1
        else:
            par, dep = medusa_shape(k_i, h_i)
        n = par.shape[0]
        dmax = int(dep.max())
        cand = [rng.choice(vocab, size=min(k_i, vocab), replace=False) for _ in range(dmax + 2)]
        tok = np.empty(n, np.int32)
        tok[0] = rng.integers(0, vocab)
        slot = np.zeros(n, np.int64)
        for j in range(1, n):
            c = cand[dep[j]]
            # children of one parent take the level's candidates in order
            sib = int(np.sum(par[:j] == par[j]))
            slot[j] = sib % c.shape[0]
            tok[j] = c[slot[j]]
        z = rng.standard_normal((n, vocab)).astype(np.float32) * np.float32(sigma)
        for j in range(n):
            if rng.random() < accept:
                t = int(rng.choice(cand[dep[j] + 1]))
                z[j, t] = z[j].max() + np.float32(1.0)
        counts.append(n)
        toks.append(tok)
        pars.append(par)
        rows.append(_store(z, dtype))
    name = f"trees_b{batch}_{'random' if random_shape else f'k{top_k}_h{heads}'}_v{vocab}_{dtype}"
    return TreeInputs(name, dtype, vocab, np.array(counts, np.int32), np.concatenate(toks),
                      np.concatenate(pars), np.ascontiguousarray(np.concatenate(rows)))


CONFIGS = {
    "toy": toy,
    "c2": c2,
    "c3": c3,
    "c4": c4,
    "c5": c5,
}
