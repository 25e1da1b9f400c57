"""Seeded random shapes against the CPU oracle, through the C ABI: vocabularies at and
around the streaming pass's piece and half boundaries (4096 and 2048 logits) and at
odd sizes (rows that are not 16-byte aligned), ragged gammas, per-row temperatures
that include greedy rows (T <= 0) and unusable ones (NaN, inf, subnormal), and draft
noise from near-equal to unrelated distributions; the full round, the filtered round,
both early-exit plans, the drafter's draw and greedy tree verification (random tree
shapes and depths)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
import test_gpu_early_exit as ee
import test_gpu_filtered as filt
from test_gpu_parity import _parity

pytestmark = pytest.mark.gpu

BOUNDARY_V = [2047, 2048, 2049, 4095, 4096, 4097, 4104, 6143, 8191, 8192, 8193, 12289, 16384, 24584]


@pytest.fixture(scope="module")
def H():
    import gpu_harness
    return gpu_harness


def random_case(seed: int, max_vocab: int = 40000, max_batch: int = 12) -> dict:
    """Arguments of workloads.small for one random shape."""
    rng = np.random.default_rng(seed)
    dtype = str(rng.choice(["bf16", "f32"]))
    vocab = int(rng.choice(BOUNDARY_V)) if rng.random() < 0.5 else int(rng.integers(1, max_vocab + 1))
    batch = int(rng.integers(1, max_batch + 1))
    gmax = int(rng.choice([0, 1, 3, 6, 9]))
    gamma = rng.integers(0, gmax + 1, batch)
    temperature = rng.choice([0.5, 0.8, 1.0, 1.3, 2.0], batch).astype(np.float64)
    kind = rng.random(batch)
    temperature[kind < 0.15] = 0.0      # greedy rows inside a sampling call (T <= 0)
    temperature[kind < 0.05] = -1.0
    bad = kind > 0.96                   # unusable temperature (NaN, inf, subnormal): invalid row
    temperature[bad] = rng.choice([np.nan, np.inf, 1e-40], int(bad.sum()))
    return dict(seed=seed, batch=batch, vocab=vocab, dtype=dtype, gamma=gamma.tolist(),
                temperature=temperature.tolist(), sigma=float(rng.choice([1.0, 3.0, 6.0])),
                noise=float(rng.choice([0.02, 0.3, 1.0, 3.0])))


@pytest.mark.parametrize("case", range(60))
def test_random_rounds(H, case):
    _parity(H, workloads.small(**random_case(1000 + case)))


@pytest.mark.parametrize("case", range(12))
def test_random_greedy_rounds(H, case):
    kw = random_case(2000 + case)
    kw["temperature"] = 1.0
    _parity(H, workloads.small(**kw, mode="greedy"), mode="greedy")


@pytest.mark.parametrize("case", range(30))
def test_random_filtered_rounds(H, case):
    w = workloads.small(**random_case(3000 + case))
    k, p = filt.filters(w, seed=3100 + case)
    filt.parity(H, w, k, p)


@pytest.mark.parametrize("case", range(20))
def test_random_early_exit_rounds(H, case):
    ee.parity(H, workloads.small(**random_case(4000 + case)), seed=4100 + case)


@pytest.mark.parametrize("case", range(16))
def test_random_drafter_draws(case):
    import test_gpu_sample as samp
    w = workloads.small(**random_case(5000 + case))
    side = "target" if case % 3 == 0 else "draft"
    if side == "draft" and w.draft.shape[0] == 0:
        side = "target"
    samp.parity(workloads.sample_inputs(w, seed=5100 + case, side=side))


@pytest.mark.parametrize("case", range(16))
def test_random_trees(case):
    import test_gpu_tree as tree
    rng = np.random.default_rng(6000 + case)
    vocab = int(rng.choice(BOUNDARY_V)) if rng.random() < 0.5 else int(rng.integers(2, 40001))
    top_k = int(rng.integers(1, 4))
    tree.parity(workloads.trees(seed=6100 + case, batch=int(rng.integers(1, 9)), vocab=vocab,
                                dtype=str(rng.choice(["bf16", "f32"])), top_k=top_k,
                                heads=int(rng.integers(0, 7 if top_k < 3 else 6)),
                                accept=float(rng.choice([0.3, 0.7, 0.95])),
                                random_shape=bool(rng.random() < 0.4)))
