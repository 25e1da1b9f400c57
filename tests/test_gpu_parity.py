"""HIP path against the CPU oracle, through the C ABI, on seeded synthetic inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def H():
    import gpu_harness
    return gpu_harness


def _parity(H, w, mode=None, dense=False, strict_eps=1e-7, assert_strict=False):
    """Parity with the oracle (see gpu_harness.compare).  Also counts the rows whose
    decisions all lie further than strict_eps from their thresholds but differ; with
    assert_strict that count must be 0."""
    _say(f"[case] {w.name} mode={mode or w.mode} dense={dense} B={w.batch} V={w.vocab}")
    gpu = H.run_gpu(w, mode=mode, dense=dense)
    ref = oracle.verify_workload(w, mode=mode)
    rep = H.compare(w, gpu, ref, mode=mode)
    if (mode or w.mode) == "sample":
        strict = oracle.verify_workload(w, mode=mode, flag_eps=strict_eps)
        rep["strict_checked_mismatched"] = H.check_strict(w, gpu, strict)
        if assert_strict:
            assert rep["strict_checked_mismatched"][1] == 0, rep
    _say(f"[ok] {rep}")
    return gpu, ref, rep


# --------------------------------------------------------------------------- #
# toy workload: bit parity plus the statistics of 10,000 rounds
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("shared", [False, True], ids=["per_position", "shared_position"])
def test_toy_parity_and_statistics(H, shared):
    import stats_checks
    w = workloads.toy(seed=1 if not shared else 2, shared_position=shared)
    gpu, ref, rep = _parity(H, w)
    stats_checks.check_emitted_distribution(w, gpu["n_accepted"], gpu["emitted"])
    stats_checks.check_accept_counts(w, gpu["n_accepted"])


# --------------------------------------------------------------------------- #
# small shapes: ragged, unaligned, multi-segment, degenerate vocabularies
# --------------------------------------------------------------------------- #
SMALL = [
    dict(seed=21, batch=9, vocab=4096, dtype="bf16", gamma=[3, 0, 5, 2, 4, 1, 7, 0, 2],
         temperature=[0.8, 1.0, 1.2, 0.7, 1.0, 0.0, 1.5, -1.0, 0.6]),
    dict(seed=22, batch=7, vocab=997, dtype="bf16", gamma=[1, 2, 0, 6, 3, 3, 1]),
    dict(seed=23, batch=5, vocab=20000, dtype="bf16", gamma=[4, 4, 4, 4, 4], n_boost=5),
    dict(seed=24, batch=6, vocab=1024, dtype="f32", gamma=[2, 0, 3, 5, 1, 4],
         temperature=[0.9, 1.1, 0.5, 2.0, 1.0, 0.75]),
    dict(seed=25, batch=6, vocab=1001, dtype="f32", gamma=[3, 1, 0, 2, 6, 2]),
    dict(seed=26, batch=4, vocab=1004, dtype="f32", gamma=[2, 2, 2, 2]),
    dict(seed=27, batch=4, vocab=1, dtype="f32", gamma=[0, 1, 3, 2]),
    dict(seed=28, batch=8, vocab=8, dtype="bf16", gamma=[1, 2, 3, 4, 5, 6, 7, 0]),
    dict(seed=29, batch=5, vocab=513, dtype="bf16", gamma=[3, 3, 0, 1, 2]),
    dict(seed=30, batch=3, vocab=40, dtype="f32", gamma=[100, 70, 0], noise=0.05),
    dict(seed=31, batch=33, vocab=65536, dtype="bf16", gamma=[2] * 33, noise=0.3),
    dict(seed=32, batch=4, vocab=300000, dtype="f32", gamma=[1, 3, 0, 2], sigma=4.0),
    # drafts very close to the target: the residual is a small difference of near-equal
    # probabilities, which the fp32 weights must resolve to the 1e-6 relative bound
    dict(seed=33, batch=5, vocab=2003, dtype="f32", gamma=[3, 2, 4, 1, 6], noise=0.01),
    dict(seed=34, batch=3, vocab=60001, dtype="f32", gamma=[2, 5, 3], noise=0.02, temperature=0.7),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_sample(H, case):
    kw = dict(SMALL[case])
    _parity(H, workloads.small(**kw))


@pytest.mark.parametrize("case", [0, 1, 3, 4, 7, 9])
def test_small_greedy(H, case):
    kw = dict(SMALL[case])
    w = workloads.small(**{**kw, "mode": "greedy"})
    _parity(H, w, mode="greedy")


def test_greedy_ties(H):
    """Integer-valued bf16 logits tie everywhere: the lowest index must win."""
    rng = np.random.default_rng(3)
    B, g, V = 16, 4, 3000
    gam = np.full(B, g, np.int32)
    tgt = rng.integers(-3, 4, (B * (g + 1), V)).astype(np.float32)
    am = np.argmax(tgt, axis=1).reshape(B, g + 1)
    tok = np.where(rng.random((B, g)) < 0.8, am[:, :g], 0).astype(np.int32).reshape(-1)
    w = workloads.Workload("ties", "bf16", V, gam, workloads.to_bf16_bits(tgt),
                           workloads.to_bf16_bits(np.zeros((B * g, V), np.float32)), tok,
                           np.zeros(B * (g + 1), np.float32), np.ones(B, np.float32), mode="greedy")
    _parity(H, w, mode="greedy")


def _offset_copy(t, elems):
    """The same values in a buffer whose first element sits `elems` elements past an
    allocation's start (a base address that is not 16-byte aligned)."""
    import torch
    flat = torch.empty(t.numel() + elems, dtype=t.dtype, device=t.device)
    view = flat[elems:].view(t.shape)
    view.copy_(t)
    return view


@pytest.mark.parametrize("vocab,dtype,gamma,offset", [
    (128257, "bf16", [2, 0, 3, 1, 4], 0),
    (50257, "bf16", [3, 3, 2, 0], 0),
    (32001, "f32", [2, 1, 0], 0),
    (8192, "bf16", [2, 3], 3),
    (4096, "f32", [1, 2], 1),
])
def test_unaligned_rows(H, vocab, dtype, gamma, offset):
    """Rows that start at every 2- or 4-byte offset within 16 bytes (vocabularies
    that are not a multiple of 16 bytes, or a base address past an aligned one): the
    streaming pass loads aligned blocks and moves the bytes into place."""
    w = workloads.small(seed=60 + len(gamma), batch=len(gamma), vocab=vocab, dtype=dtype, gamma=gamma)
    d = H.to_device(w)
    if offset:
        d["target"] = _offset_copy(d["target"], offset)
        d["draft"] = _offset_copy(d["draft"], offset)
    for mode in ("sample", "greedy"):
        g = H.run_gpu(w, mode=mode, tensors=d)
        ref = oracle.verify_workload(w, mode=mode)
        H.compare(w, g, ref, mode=mode)


def test_dense_equals_ragged(H):
    w = workloads.small(seed=41, batch=12, vocab=8192, dtype="bf16", gamma=3)
    a = H.run_gpu(w, dense=True)
    b = H.run_gpu(w, dense=False)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_deterministic(H):
    w = workloads.small(seed=42, batch=16, vocab=50000, dtype="bf16", gamma=4, n_boost=5)
    d = H.to_device(w)
    a = H.run_gpu(w, tensors=d)
    b = H.run_gpu(w, tensors=d)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


# --------------------------------------------------------------------------- #
# status rules and special inputs
# --------------------------------------------------------------------------- #
def _edit(w, **kw):
    return workloads.Workload(**{**w.__dict__, **kw})


def test_status_rules(H):
    base = workloads.small(seed=51, batch=10, vocab=2048, dtype="f32", gamma=3)
    tgt = base.target.copy()
    drf = base.draft.copy()
    tok = base.draft_tokens.copy()
    T = base.temperature.copy()
    drf[1 * 3 + 1, 7] = np.nan                 # row 1: NaN in a draft position
    tgt[2 * 4 + 3, 100] = np.inf               # row 2: +inf at the bonus position
    tgt[3 * 4 + 0, :] = -np.inf                # row 3: a position with all -inf
    tgt[4 * 4 + 2, :1000] = -np.inf            # row 4: masked tokens, still valid
    drf[4 * 3 + 1, 1000:] = -np.inf
    tok[5 * 3 + 2] = 2048                      # row 5: token out of range
    tok[6 * 3 + 0] = -1                        # row 6: negative token
    T[7] = np.nan                              # row 7: NaN temperature
    T[8] = 1e-39                               # row 8: subnormal temperature
    T[9] = 0.0                                 # row 9: greedy row
    w = _edit(base, target=tgt, draft=drf, draft_tokens=tok, temperature=T)
    gpu, ref, rep = _parity(H, w)
    st = gpu["row_status"]
    assert st[1] & oracle.NONFINITE and st[2] & oracle.NONFINITE and st[3] & oracle.NONFINITE
    assert not st[4] & oracle.INVALID_MASK
    assert st[5] & oracle.BAD_TOKEN and st[6] & oracle.BAD_TOKEN
    assert st[7] & oracle.BAD_TEMP and st[8] & oracle.BAD_TEMP
    assert st[9] == 0 and gpu["n_accepted"][9] >= 0
    # greedy mode never reads draft logits: the NaN draft row is valid there
    gg, rg, _ = _parity(H, w, mode="greedy")
    assert not gg["row_status"][1] & oracle.INVALID_MASK


@pytest.mark.parametrize("V,dtype", [(16, "f32"), (16, "bf16"), (5000, "f32"), (5000, "bf16")])
def test_q_zero_and_zero_residual(H, V, dtype):
    """q(x) = 0 with p(x) > 0 keeps the draft (ratio 1); q(x) = p(x) = 0 with p = q
    elsewhere rejects with zero residual mass and draws from p (over several tiles at
    V = 5000: the residual's terms cancel to exactly 0 in every tile)."""
    z = np.zeros((2, V), np.float32)
    tgt1 = z.copy()
    drf1 = z[:1].copy()
    drf1[0, 5] = -np.inf
    tgt2 = z.copy()
    tgt2[:, 9] = -np.inf
    drf2 = z[:1].copy()
    drf2[0, 9] = -np.inf
    store = (lambda a: workloads.to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    w = workloads.Workload("qzero", dtype, V, np.array([1, 1], np.int32), store(np.concatenate([tgt1, tgt2])),
                           store(np.concatenate([drf1, drf2])), np.array([5, 9], np.int32),
                           np.array([0.999, 0.3, 0.2, 0.55], np.float32), np.ones(2, np.float32))
    gpu, ref, rep = _parity(H, w)
    assert gpu["row_status"][0] == oracle.Q_ZERO and gpu["n_accepted"][0] == 1
    assert gpu["row_status"][1] == oracle.Q_ZERO | oracle.ZERO_RESID and gpu["n_accepted"][1] == 0


@pytest.mark.parametrize("vocab,dtype", [(40, "f32"), (2003, "f32"), (60001, "f32"), (4096, "bf16")])
def test_near_equal_rejections(H, vocab, dtype):
    """Drafts within about 1 % of the target and test uniforms just below 1: rows reject
    where p(x) is a hair below q(x), so the residual max(0, p - q) is a small
    difference of near-equal probabilities, its mass a few percent at most."""
    w = workloads.small(seed=70 + vocab % 7, batch=12, vocab=vocab, dtype=dtype, gamma=3, noise=0.01)
    u = w.uniforms.copy()
    off = np.concatenate([[0], np.cumsum(w.gamma.astype(np.int64) + 1)])
    for i in range(w.batch):
        u[off[i]:off[i] + w.gamma[i]] = np.float32(0.999999)
    w2 = _edit(w, uniforms=u)
    gpu, ref, rep = _parity(H, w2)
    assert (ref["n_accepted"] < w2.gamma).sum() >= w.batch // 2
    W = ref["resid_mass"][ref["n_accepted"] < w2.gamma]
    assert np.nanmax(W) < 0.1


def test_extreme_scales_f32(H):
    """fp32 logits at extreme scales: temperatures from 1e-3 to 1e30 (a near-uniform
    distribution), rows shifted by +1e7 (their exponents m c lie far beyond 2^20, so
    the draw subtracts m first and the streaming pass works against large
    references), a draft shifted by -1e6 against its target (the same softmax from
    very different maxima), rows with -inf entries away from the drafted tokens, and a
    row shifted by 1e6 at T = 1e-4, whose m c ~ 1.4e10 is far beyond where a reference
    taken with the scale's fp32 part alone would overflow the sums."""
    g = 3
    w = workloads.small(seed=91, batch=9, vocab=5000, dtype="f32", gamma=g)
    T = np.array([1e-3, 0.05, 1.0, 1e3, 1e30, 1.0, 0.5, 2.0, 1e-4], np.float32)
    tgt, drf = w.target.copy(), w.draft.copy()
    tr = lambda i: slice(i * (g + 1), (i + 1) * (g + 1))
    dr = lambda i: slice(i * g, (i + 1) * g)
    tgt[tr(5)] += np.float32(1e7)
    drf[dr(5)] += np.float32(1e7)
    rng = np.random.default_rng(92)
    drafted = set(w.draft_tokens[dr(6)].tolist())
    holes = np.array([v for v in rng.choice(w.vocab, 150, replace=False) if v not in drafted][:100])
    tgt[tr(6), holes[:50, None].T] = -np.inf
    drf[dr(6), holes[50:, None].T] = -np.inf
    drf[dr(7)] -= np.float32(1e6)
    tgt[tr(8)] += np.float32(1e6)   # m c ~ 1.4e10 at T = 1e-4
    drf[dr(8)] += np.float32(1e6)
    w2 = _edit(w, target=tgt, draft=drf, temperature=T)
    _parity(H, w2)
    _parity(H, w2, mode="greedy")


def test_bad_gamma(H):
    w = workloads.small(seed=52, batch=6, vocab=512, dtype="bf16", gamma=[2, 1, 3, 0, 2, 1])
    d = H.to_device(w)
    import torch
    import speculative_sampling_verify_02_amd as sv
    for bad in ([2, 1, 3, 0, 2, 2], [2, 1, -1, 0, 2, 5]):
        g = torch.tensor(bad, dtype=torch.int32, device=d["target"].device)
        n, e, dg = sv.spec_verify(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"],
                                  g, diag=True)
        torch.cuda.synchronize()
        assert (n.cpu().numpy() == -1).all() and (e.cpu().numpy() == -1).all()
        assert (dg["row_status"].cpu().numpy() == oracle.BAD_GAMMA).all()


# --------------------------------------------------------------------------- #
# the five configurations at full size
# --------------------------------------------------------------------------- #
def test_c2_full(H):
    _parity(H, workloads.c2())


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_c3_full(H, mode):
    _parity(H, workloads.c3(mode=mode), mode=mode, dense=True, assert_strict=True)


def test_c4_full(H):
    _parity(H, workloads.c4(), dense=True, assert_strict=True)


def test_c5_full(H):
    _parity(H, workloads.c5(), assert_strict=True)


@pytest.mark.parametrize("seed", [13, 23])
def test_c3_more_seeds(H, seed):
    _parity(H, workloads.c3(seed=seed), dense=True, assert_strict=True)


@pytest.mark.parametrize("vocab,dtype,batch", [(152063, "bf16", 80), (65537, "f32", 164)])
def test_long_pass_staged_records(H, vocab, dtype, batch):
    """A pass long enough (over 46875 pieces) for the bf16 streaming kernel to keep its
    records in LDS and write them out at the end, with rows that are not 16-byte
    aligned (the kernel that realigns its loads) and greedy rows (T = 0, argmax
    records) among the sampling rows; and an fp32 pass of that length (bound by its
    arithmetic, it stores its records piece by piece)."""
    w = workloads.small(seed=97, batch=batch, vocab=vocab, dtype=dtype, gamma=8, n_boost=5 if dtype == "bf16" else 0,
                        temperature=[0.0 if i % 7 == 3 else 0.9 for i in range(batch)])
    assert (2 * w.target.shape[0] - w.batch) * ((w.vocab + 4095) // 4096) * 8192 / 6.4e12 >= 60e-6
    _parity(H, w, dense=True)


def test_c4_second_seed(H):
    _parity(H, workloads.c4(seed=14), dense=True, assert_strict=True)


def test_c3_near_target_draft_reaches_bonus(H):
    """The V = 128256 batch with a draft close to its target (draft = target + N(0, 0.2)):
    most rows keep every draft, so the bonus draw from the streaming pass's piece sums
    runs on most rows at full size (rayaq.ca "Speculative decoding", section "One
    round", step 5)."""
    w = workloads.c3(seed=33, draft_scale=1.0, draft_sigma=0.2)
    gpu, ref, rep = _parity(H, w, dense=True, assert_strict=True)
    bonus = int((ref["n_accepted"] == w.gamma).sum())
    _say(f"[ok] bonus rows {bonus} of {w.batch}")
    assert bonus >= 0.3 * w.batch


def test_many_rows(H):
    """3000 ragged rows (gamma 0..7): the packed offsets are scanned over several
    1024-row chunks, and every per-row kernel runs thousands of workgroups."""
    gam = np.random.default_rng(95).integers(0, 8, 3000).astype(np.int32)
    _parity(H, workloads.small(seed=95, batch=3000, vocab=2048, dtype="bf16", gamma=gam))
    wg = workloads.small(seed=96, batch=3000, vocab=2048, dtype="bf16", gamma=gam, mode="greedy")
    _parity(H, wg, mode="greedy")


def test_profile_events(H):
    """Events handed to spec_verify_set_profile_events are attached to the streaming
    kernel's dispatch: after a call they bound a short, positive interval."""
    import torch
    import bench
    import speculative_sampling_verify_02_amd as sv
    ev = bench.HipEvents()
    a, b = ev.create(), ev.create()
    w = workloads.small(seed=97, batch=6, vocab=8192, dtype="bf16", gamma=3)
    d = H.to_device(w)
    dev = d["target"].device
    try:
        sv.set_profile_events(a, b)
        sv.spec_verify(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"], int(w.gamma[0]))
        torch.cuda.synchronize()
        t_verify = ev.elapsed_ms(a, b)
        n = d["target"].shape[0]
        sv.spec_sample(d["target"], torch.rand(n, device=dev), torch.ones(n, device=dev))
        torch.cuda.synchronize()
        t_sample = ev.elapsed_ms(a, b)
    finally:
        sv.set_profile_events(None, None)
        ev.destroy(a)
        ev.destroy(b)
    _say(f"[ok] streaming kernel {t_verify * 1e3:.1f} us (verify), {t_sample * 1e3:.1f} us (sample)")
    assert 0.0 < t_verify < 50.0 and 0.0 < t_sample < 50.0


def test_binding_rejects_mismatched_draft_logits(H):
    """A drafter whose vocabulary or row count does not match the target's is refused
    by the binding before anything is launched (the kernels would read past the
    draft tensor or stride the wrong rows)."""
    import torch
    import speculative_sampling_verify_02_amd as sv
    w = workloads.small(seed=98, batch=4, vocab=1000, dtype="bf16", gamma=2)
    d = H.to_device(w)
    padded = torch.zeros((w.n_draft_rows, 1024), dtype=torch.bfloat16, device=d["draft"].device)
    short = d["draft"][:-1]
    for bad, msg in ((padded, "logits per row"), (short, "draft rows expected")):
        with pytest.raises(ValueError, match=msg):
            sv.spec_verify(d["target"], bad, d["tokens"], d["uniforms"], d["temperature"], d["gamma"])
        with pytest.raises(ValueError, match=msg):
            sv.spec_verify_filtered(d["target"], bad, d["tokens"], d["uniforms"], d["temperature"], d["gamma"],
                                    top_k=torch.full((4,), 5, dtype=torch.int32, device=bad.device))
        with pytest.raises(ValueError, match=msg):
            sv.spec_verify_early_exit(d["target"], bad, d["tokens"], d["uniforms"], d["temperature"],
                                      d["gamma"], gamma_max=2)
    with pytest.raises(ValueError, match="required in sampling mode"):
        sv.spec_verify(d["target"], None, d["tokens"], d["uniforms"], d["temperature"], d["gamma"])
    torch.cuda.synchronize()


def invalid_from_start(dtype="f32", seed=55):
    """Rows invalid from the start that also hold non-finite logits further on: an
    unusable temperature (NaN, subnormal) with a NaN, +inf or all -inf position, and a
    bad token with a NaN at the last position.  The round reads every position, so the
    oracle reports the non-finite logits too."""
    w = workloads.small(seed=seed, batch=8, vocab=3000, dtype=dtype, gamma=3)
    tgt, drf, tok, T = w.target.copy(), w.draft.copy(), w.draft_tokens.copy(), w.temperature.copy()
    nan = np.float32(np.nan) if dtype == "f32" else 0x7FC0
    pinf = np.float32(np.inf) if dtype == "f32" else 0x7F80
    ninf = np.float32(-np.inf) if dtype == "f32" else 0xFF80
    T[0] = np.nan
    drf[0 * 3 + 2, 11] = nan                   # row 0: bad T, NaN in the last draft position
    T[1] = 1e-39
    tgt[1 * 4 + 3, 5] = pinf                   # row 1: subnormal T, +inf at the bonus position
    T[2] = np.inf
    tgt[2 * 4 + 1, :] = ninf                   # row 2: infinite T, a position with all -inf
    tok[3 * 3 + 0] = 3000
    tgt[3 * 4 + 3, 7] = nan                    # row 3: bad token, NaN at the bonus position
    tok[4 * 3 + 1] = -5                        # row 4: bad token only
    T[5] = np.nan                              # row 5: bad T only
    return workloads.Workload(**{**w.__dict__, "target": tgt, "draft": drf, "draft_tokens": tok, "temperature": T})


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_invalid_rows_still_report_nonfinite(H, dtype):
    w = invalid_from_start(dtype)
    gpu, ref, rep = _parity(H, w)
    st = gpu["row_status"]
    assert st[0] == oracle.BAD_TEMP | oracle.NONFINITE and st[1] == oracle.BAD_TEMP | oracle.NONFINITE
    assert st[2] == oracle.BAD_TEMP | oracle.NONFINITE and st[3] == oracle.BAD_TOKEN | oracle.NONFINITE
    assert st[4] == oracle.BAD_TOKEN and st[5] == oracle.BAD_TEMP
    gg, rg, _ = _parity(H, w, mode="greedy")
    assert gg["row_status"][3] == oracle.BAD_TOKEN | oracle.NONFINITE
