"""Verification on top-k / top-p filtered distributions (spec_verify_filtered)
against the CPU oracle, through the C ABI."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def H():
    import gpu_harness
    return gpu_harness


def filters(w, seed, kinds=("k", "p", "kp", "none", "k1")):
    """Per-row top-k / top-p settings cycling through the given kinds."""
    rng = np.random.default_rng(seed)
    B, V = w.batch, w.vocab
    k = np.zeros(B, np.int32)
    p = np.ones(B, np.float32)
    for i in range(B):
        kind = kinds[i % len(kinds)]
        if "k" in kind:
            k[i] = 1 if kind == "k1" else int(rng.integers(1, max(2, min(V, 200))))
        if "p" in kind:
            p[i] = float(rng.choice([0.5, 0.8, 0.9, 0.95, 0.99]))
    return k, p


def run_filtered(H, w, k, p, dense=False):
    import speculative_sampling_verify_02_amd as sv
    d = H.to_device(w)
    gamma = w.dense_gamma if dense else d["gamma"]
    n, e, dg = sv.spec_verify_filtered(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"],
                                       gamma, top_k=torch.from_numpy(k).cuda(), top_p=torch.from_numpy(p).cuda(),
                                       diag=True)
    torch.cuda.synchronize()
    out = dict(n_accepted=n.cpu().numpy(), emitted=e.cpu().numpy())
    for key, v in dg.items():
        out[key] = v.cpu().numpy()
    return out


def parity(H, w, k, p, dense=False):
    _say(f"[case] filtered {w.name} B={w.batch} V={w.vocab} top_k={k[:4]} top_p={p[:4]}")
    g = run_filtered(H, w, k, p, dense=dense)
    ref = oracle.verify_workload(w, top_k=k, top_p=p)
    rep = H.compare(w, g, ref, oracle_kw=dict(top_k=k, top_p=p))
    _say(f"[ok] {rep}")
    return g, ref


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small(H, case):
    w = workloads.small(**SMALL[case])
    k, p = filters(w, seed=200 + case)
    parity(H, w, k, p)


def test_ties_and_tiny_vocabularies(H):
    """Integer-valued logits (ties at every threshold) and V = 8."""
    rng = np.random.default_rng(5)
    w = workloads.small(seed=81, batch=10, vocab=3000, dtype="bf16", gamma=3)
    tgt = workloads.to_bf16_bits(rng.integers(-4, 5, w.target.shape).astype(np.float32))
    dft = workloads.to_bf16_bits(rng.integers(-4, 5, w.draft.shape).astype(np.float32))
    w2 = workloads.Workload(**{**w.__dict__, "target": tgt, "draft": dft})
    k, p = filters(w2, seed=6)
    parity(H, w2, k, p)
    w3 = workloads.small(seed=82, batch=8, vocab=8, dtype="bf16", gamma=[1, 2, 3, 4, 5, 6, 7, 0])
    parity(H, w3, *filters(w3, seed=7))


def test_top1_is_greedy(H):
    """top_k = 1 on both models with drafts at the drafter's argmax: the greedy round."""
    w = workloads.small(seed=83, batch=16, vocab=4096, dtype="f32", gamma=4, mode="greedy")
    k = np.ones(w.batch, np.int32)
    p = np.ones(w.batch, np.float32)
    g = run_filtered(H, w.with_mode("sample"), k, p)
    ref = oracle.verify_workload(w, mode="greedy")
    assert np.array_equal(g["n_accepted"], ref["n_accepted"])
    assert np.array_equal(g["emitted"], ref["emitted"])


def _filtered_path_exercised(w, ref, min_bonus=0):
    """The drafts come from the drafter's top-k set, so the filtered ratio and residual
    path runs on most positions: few rows see q(x) = 0, most reject with a residual of
    positive mass, and (where asked) rows reach the filtered bonus draw."""
    st, K = ref["row_status"], ref["n_accepted"]
    q_zero = float(((st & oracle.Q_ZERO) != 0).mean())
    rejects = int(((K >= 0) & (K < w.gamma) & (ref["resid_mass"] > 0)).sum())
    bonus = int((K == w.gamma).sum())
    _say(f"[ok] q(x)=0 on {q_zero:.3f} of rows, {rejects} residual draws, {bonus} bonus draws")
    assert q_zero < 0.10
    assert rejects >= min(w.batch // 2, 20) or bonus >= 0.3 * w.batch
    assert bonus >= min_bonus


def test_c3_full(H):
    """The V = 128256 bf16 batch with top-k 50 and top-p 0.9 on every row, drafts drawn
    from the drafter's 20 largest logits (inside its kept set on nearly every
    position, as a drafter that samples from filtered q would draw them)."""
    w = workloads.c3(draft_top_k=20)
    g, ref = parity(H, w, np.full(w.batch, 50, np.int32), np.full(w.batch, 0.9, np.float32), dense=True)
    _filtered_path_exercised(w, ref)


def test_c3_full_near_target_bonus(H):
    """The same filter on the V = 128256 batch with a draft close to its target: most
    rows keep every draft and draw the bonus from the filtered p at full size."""
    w = workloads.c3(seed=33, draft_scale=1.0, draft_sigma=0.2, draft_top_k=20)
    g, ref = parity(H, w, np.full(w.batch, 50, np.int32), np.full(w.batch, 0.9, np.float32), dense=True)
    _filtered_path_exercised(w, ref, min_bonus=int(0.3 * w.batch))


def test_c4_full(H):
    """The V = 152064 bf16 batch (B = 256, gamma = 8) with top-k 50 and top-p 0.9: 4352
    vectors, more than the select workgroups that fit at once; drafts from the
    drafter's 20 largest logits."""
    w = workloads.c4(draft_top_k=20)
    g, ref = parity(H, w, np.full(w.batch, 50, np.int32), np.full(w.batch, 0.9, np.float32), dense=True)
    _filtered_path_exercised(w, ref, min_bonus=1)


def test_c3_full_top_p_only(H):
    w = workloads.c3()
    parity(H, w, np.zeros(w.batch, np.int32), np.full(w.batch, 0.95, np.float32), dense=True)


def test_large_k_and_crowded_tops(H):
    """top-k above 1024 and more than 4096 logits tied at the top, beyond what the
    kernel gathers in LDS: the thresholds come from searches over the whole vector."""
    rng = np.random.default_rng(8)
    w = workloads.small(seed=84, batch=6, vocab=20000, dtype="bf16", gamma=2)
    tgt = workloads.to_bf16_bits(rng.integers(0, 2, w.target.shape).astype(np.float32))
    dft = workloads.to_bf16_bits(rng.integers(0, 2, w.draft.shape).astype(np.float32))
    w2 = workloads.Workload(**{**w.__dict__, "target": tgt, "draft": dft})
    k = np.array([50, 2000, 5, 3000, 100, 1], np.int32)
    p = np.array([1.0, 0.9, 0.5, 1.0, 0.99, 1.0], np.float32)
    parity(H, w2, k, p)
    w3 = workloads.small(seed=85, batch=6, vocab=20000, dtype="f32", gamma=2)
    parity(H, w3, k, p)
    # about 2000 logits tied at the top: more candidates than one wave selects from,
    # few enough for the searches in LDS
    for dt, seed in (("bf16", 86), ("f32", 87)):
        w4 = workloads.small(seed=seed, batch=6, vocab=20000, dtype=dt, gamma=2)
        conv = workloads.to_bf16_bits if dt == "bf16" else (lambda a: a)
        t4 = conv(rng.integers(0, 10, w4.target.shape).astype(np.float32))
        d4 = conv(rng.integers(0, 10, w4.draft.shape).astype(np.float32))
        w4 = workloads.Workload(**{**w4.__dict__, "target": t4, "draft": d4})
        parity(H, w4, np.array([300, 1000, 7, 1024, 50, 2], np.int32),
               np.array([0.9, 1.0, 0.5, 0.99, 1.0, 0.7], np.float32))


def test_fp32_key_buckets(H):
    """fp32 logits whose largest values share one 16-bit key bucket: the top of each
    vector is a cluster -4 - j 2^-20 (j <= 40, negative, so the bucket's least float
    is its most negative one), spread over different 64-logit units, everything else
    below -5, and top-k cuts inside the cluster.  The threshold search's bound from
    the units' 16-bit keys must be the least float of the bucket for all of the
    cluster to be among the candidates."""
    rng = np.random.default_rng(95)
    w = workloads.small(seed=95, batch=6, vocab=8192, dtype="f32", gamma=2)

    def clustered(shape):
        x = (-10.0 + 0.5 * rng.standard_normal(shape)).astype(np.float32)
        x = np.minimum(x, np.float32(-5.0))
        for r in range(shape[0]):
            units = rng.choice(shape[1] // 64, size=41, replace=False)
            pos = units * 64 + rng.integers(0, 64, size=41)
            x[r, pos] = (np.float32(-4.0) - np.arange(41, dtype=np.float32) * np.float32(2.0 ** -20))
        return x

    w2 = workloads.Workload(**{**w.__dict__, "target": clustered(w.target.shape), "draft": clustered(w.draft.shape)})
    k = np.array([10, 5, 30, 40, 1, 10], np.int32)
    p = np.array([1.0, 0.9, 1.0, 0.5, 1.0, 0.99], np.float32)
    parity(H, w2, k, p)


def test_vocab_sizes_around_the_unit_budgets(H):
    """Vocabularies at the edges of the threshold kernel's unit budgets (8, 16, 24, 32
    and 64 unit maxima of 64 logits per thread of a 128-thread workgroup: up to 65536,
    131072, 196608, 262144 and 524288 logits) and just beyond the last (the threshold
    kernel that reads the whole vector), bf16 and fp32, with top-k, top-p, both and
    neither."""
    cases = ((65536, "bf16"), (65544, "bf16"), (131080, "f32"), (196608, "bf16"),
             (196616, "bf16"), (262152, "f32"), (524288, "bf16"), (524296, "bf16"))
    for i, (V, dt) in enumerate(cases):
        w = workloads.small(seed=90 + i, batch=4, vocab=V, dtype=dt, gamma=[2, 0, 3, 1],
                            temperature=[1.0, 0.7, 1.3, 0.0])
        parity(H, w, *filters(w, seed=300 + i, kinds=("kp", "p", "k", "none")))


def test_status_rules_bf16(H):
    """NaN, +inf, all -inf, bad tokens and temperatures, and a greedy row in a
    filtered bf16 call."""
    base = workloads.small(seed=53, batch=10, vocab=2048, dtype="bf16", gamma=3)
    tgt = base.target.copy()
    drf = base.draft.copy()
    tok = base.draft_tokens.copy()
    T = base.temperature.copy()
    nan, pinf, ninf = 0x7FC0, 0x7F80, 0xFF80
    drf[1 * 3 + 1, 7] = nan                    # row 1: NaN in a draft position
    tgt[2 * 4 + 3, 100] = pinf                 # row 2: +inf at the bonus position
    tgt[3 * 4 + 0, :] = ninf                   # row 3: a position with all -inf
    tgt[4 * 4 + 2, :1000] = ninf               # row 4: masked tokens, still valid
    drf[4 * 3 + 1, 1000:] = ninf
    tok[5 * 3 + 2] = 2048                      # row 5: token out of range
    T[7] = np.nan                              # row 7: NaN temperature
    T[8] = 1e-39                               # row 8: subnormal temperature
    T[9] = 0.0                                 # row 9: greedy row
    w = workloads.Workload(**{**base.__dict__, "target": tgt, "draft": drf, "draft_tokens": tok,
                              "temperature": T})
    for kinds in (("kp",), ("k",), ("p",), ("none",)):
        g, ref = parity(H, w, *filters(w, seed=9, kinds=kinds))
        st = g["row_status"]
        assert st[1] & oracle.NONFINITE and st[2] & oracle.NONFINITE and st[3] & oracle.NONFINITE
        assert st[5] & oracle.BAD_TOKEN and st[7] & oracle.BAD_TEMP and st[8] & oracle.BAD_TEMP
        assert st[9] == 0 and g["n_accepted"][9] >= 0


def test_bad_gamma(H):
    import speculative_sampling_verify_02_amd as sv
    w = workloads.small(seed=54, batch=6, vocab=512, dtype="bf16", gamma=[2, 1, 3, 0, 2, 1])
    d = H.to_device(w)
    k, p = filters(w, seed=10)
    for bad in ([2, 1, 3, 0, 2, 2], [2, 1, -1, 0, 2, 5]):
        g = torch.tensor(bad, dtype=torch.int32, device=d["target"].device)
        n, e, dg = sv.spec_verify_filtered(d["target"], d["draft"], d["tokens"], d["uniforms"],
                                           d["temperature"], g, top_k=torch.from_numpy(k).cuda(),
                                           top_p=torch.from_numpy(p).cuda(), diag=True)
        torch.cuda.synchronize()
        assert (n.cpu().numpy() == -1).all() and (e.cpu().numpy() == -1).all()
        assert (dg["row_status"].cpu().numpy() == oracle.BAD_GAMMA).all()


def test_many_vectors_mixed_rows(H):
    """Many vectors with rows of every kind interleaved: top-k, top-p, both, neither,
    top-k 1, greedy (T = 0), a bad temperature and a NaN logit."""
    w = workloads.small(seed=91, batch=100, vocab=32000, dtype="bf16", gamma=4)
    T = w.temperature.copy()
    T[7::10] = 0.0
    T[13] = np.nan
    tgt = w.target.copy()
    tgt[5 * 5 + 2, 99] = 0x7FC0                # row 5: NaN logit
    w2 = workloads.Workload(**{**w.__dict__, "temperature": T, "target": tgt})
    g, ref = parity(H, w2, *filters(w2, seed=12))
    assert g["row_status"][5] & oracle.NONFINITE and g["row_status"][13] & oracle.BAD_TEMP


@pytest.mark.parametrize("vocab", [152064, 152063])
def test_long_pass_staged_keys(H, vocab):
    """A bf16 pass long enough (82688 pieces) for the streaming kernel to keep the unit
    keys of its pieces in LDS and write them out at the end, on rows of every kind
    (top-k, top-p, both, neither, top-k 1), with 16-byte aligned rows and with rows
    that are not (the kernel that realigns its loads)."""
    w = workloads.small(seed=96, batch=128, vocab=vocab, dtype="bf16", gamma=8, n_boost=5)
    assert (2 * w.target.shape[0] - w.batch) * ((vocab + 4095) // 4096) >= 78125
    parity(H, w, *filters(w, seed=15), dense=True)


@pytest.mark.parametrize("vocab,dtype", [(8192, "bf16"), (6001, "f32"), (4101, "bf16")])
def test_more_vectors_than_resident_selects(H, vocab, dtype):
    """More vectors (5100) than the select workgroups that fit on the device at once
    (16 a CU), so the last ones start in a second round, on rows of every kind: top-k
    from 1 to 300 (above 128 the per-wave bound does not apply and the select runs over
    every unit key), top-p, both, neither, greedy (T = 0) and a bad temperature;
    aligned and unaligned rows, bf16 and fp32."""
    w = workloads.small(seed=94, batch=300, vocab=vocab, dtype=dtype, gamma=8)
    T = w.temperature.copy()
    T[11::17] = 0.0
    T[5] = np.inf
    w2 = workloads.Workload(**{**w.__dict__, "temperature": T})
    assert 2 * w2.target.shape[0] - w2.batch > 16 * 256
    k, p = filters(w2, seed=14)
    k[3::20] = 300
    k[8::20] = 65
    parity(H, w2, k, p, dense=True)


@pytest.mark.parametrize("vocab,dtype", [(50257, "bf16"), (32001, "f32"), (128257, "bf16")])
def test_unaligned_vocabularies(H, vocab, dtype):
    """Rows that do not start 16-byte aligned: the streaming pass and the threshold
    kernel read them with aligned loads shifted into place."""
    w = workloads.small(seed=93, batch=5, vocab=vocab, dtype=dtype, gamma=[2, 3, 0, 1, 2])
    parity(H, w, *filters(w, seed=13))


def test_invalid_rows_still_report_nonfinite(H):
    """Rows with an unusable temperature or a bad token and non-finite logits further on,
    in a filtered call (bf16 rows take the one-pass filter kernel)."""
    from test_gpu_parity import invalid_from_start
    for dtype in ("bf16", "f32"):
        w = invalid_from_start(dtype, seed=56)
        g, ref = parity(H, w, *filters(w, seed=14, kinds=("kp", "k", "p", "none")))
        assert g["row_status"][0] == oracle.BAD_TEMP | oracle.NONFINITE
        assert g["row_status"][3] == oracle.BAD_TOKEN | oracle.NONFINITE
