"""The early-exit round (spec_verify_early_exit) against the CPU oracle's early-exit
round and against the GPU's full round, through the C ABI."""
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


def run_early(H, w, mode=None, dense=False, cache_len=None, tensors=None, gamma_max=None, plan="steps"):
    import speculative_sampling_verify_02_amd as sv
    d = tensors or H.to_device(w)
    gamma = w.dense_gamma if dense else d["gamma"]
    cl = None if cache_len is None else torch.from_numpy(np.ascontiguousarray(cache_len, np.int32)).cuda()
    gm = int(w.gamma.max()) if gamma_max is None else gamma_max
    n, e, crop, dg = sv.spec_verify_early_exit(d["target"], d["draft"], d["tokens"], d["uniforms"],
                                               d["temperature"], gamma, gamma_max=gm,
                                               cache_len=cl, mode=mode or w.mode, diag=True, plan=plan)
    torch.cuda.synchronize()
    out = dict(n_accepted=n.cpu().numpy(), emitted=e.cpu().numpy(), crop_len=crop.cpu().numpy())
    for k, v in dg.items():
        out[k] = v.cpu().numpy()
    return out


def same_outputs(a, b):
    """Every output of two early-exit calls is identical (NaN diagnostics included)."""
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=a[k].dtype.kind == "f"), k


def parity(H, w, mode=None, dense=False, seed=0):
    """The steps plan against the oracle's early-exit round; the one-pass plan gives
    identical outputs."""
    mode = mode or w.mode
    _say(f"[case] early exit {w.name} mode={mode} dense={dense} B={w.batch} V={w.vocab}")
    cache = np.random.default_rng(seed).integers(0, 4096, w.batch).astype(np.int32)
    g = run_early(H, w, mode=mode, dense=dense, cache_len=cache)
    same_outputs(g, run_early(H, w, mode=mode, dense=dense, cache_len=cache, plan="one_pass"))
    ref = oracle.verify_workload(w, mode=mode, early_exit=True, cache_len=cache)
    # compare() also holds crop_len to cache_len + K + 1 of the (possibly re-run) oracle row
    rep = H.compare(w, g, ref, mode=mode, oracle_kw=dict(early_exit=True, cache_len=cache))
    # the full round on the GPU keeps the same drafts and draws the same tokens
    full = H.run_gpu(w, mode=mode, dense=dense)
    ok = full["row_status"] == 0
    assert np.array_equal(full["n_accepted"][ok], g["n_accepted"][ok])
    t_off, _ = w.offsets()
    for i in np.nonzero(ok)[0]:
        a, b = t_off[i], t_off[i + 1]
        assert np.array_equal(full["emitted"][a:b], g["emitted"][a:b]), i
    _say(f"[ok] {rep}")
    return g, ref


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_sample(H, case):
    parity(H, workloads.small(**SMALL[case]), seed=case)


@pytest.mark.parametrize("case", [0, 1, 3, 7, 9])
def test_small_greedy(H, case):
    w = workloads.small(**{**SMALL[case], "mode": "greedy"})
    parity(H, w, mode="greedy", seed=case)


def test_long_rows(H):
    """Rows of up to 250 drafts with drafts close to the target: the chunk of positions
    [127, 255) is longer than a wave, so its positions are decided 64 at a time, and
    rows are decided in both of its parts (K = 250 and 200 at the bonus, 136 by a
    rejection)."""
    w = workloads.small(seed=89, batch=4, vocab=64, dtype="f32", gamma=[250, 200, 5, 140], noise=0.004)
    g, ref = parity(H, w, seed=89)
    assert sorted(g["n_accepted"].tolist()) == [5, 136, 200, 250]


def test_dense(H):
    parity(H, workloads.small(seed=71, batch=24, vocab=8192, dtype="bf16", gamma=4, noise=0.4), dense=True)


def test_nan_after_the_rejection(H):
    """A NaN logit beyond a row's rejection is never read: the row stays valid (the
    full round marks it invalid)."""
    w = workloads.small(seed=72, batch=16, vocab=4096, dtype="f32", gamma=6, noise=2.0)
    ref = oracle.verify_workload(w)
    t_off, d_off = w.offsets()
    tgt, dft = w.target.copy(), w.draft.copy()
    rows = []
    for i in range(w.batch):
        K = ref["n_accepted"][i]
        if 0 <= K < w.gamma[i] - 1:
            tgt[t_off[i] + K + 1, 5] = np.nan
            dft[d_off[i] + K + 1, 7] = np.nan
            rows.append(i)
    assert rows, "no row rejects early enough"
    w2 = workloads.Workload(**{**w.__dict__, "target": tgt, "draft": dft})
    g, _ = parity(H, w2)
    assert np.all(g["row_status"][rows] == 0)


def test_q_zero_then_nan(H):
    """q(x) = 0 with p(x) > 0 at position 0 (kept, ratio 1), then a NaN target logit
    at position 1: the row is invalid and reports only NONFINITE, like the full
    round."""
    V = 64
    rng = np.random.default_rng(11)
    tgt = rng.normal(0.0, 1.0, (2 * 4, V)).astype(np.float32)
    drf = rng.normal(0.0, 1.0, (2 * 3, V)).astype(np.float32)
    tok = np.array([5, 6, 7, 5, 6, 7], np.int32)
    drf[0, 5] = -np.inf          # row 0, position 0: q(x) = 0
    tgt[1, 9] = np.nan           # row 0, position 1: NaN
    drf[3, 5] = -np.inf          # row 1, position 0: q(x) = 0, and the row stays valid
    u = np.full(8, 0.5, np.float32)
    w = workloads.Workload("qzero_nan", "f32", V, np.array([3, 3], np.int32), tgt, drf, tok, u,
                           np.ones(2, np.float32))
    g, ref = parity(H, w)
    assert g["row_status"][0] == oracle.NONFINITE
    assert g["row_status"][1] & oracle.Q_ZERO


def test_c3_full(H):
    parity(H, workloads.c3(), dense=True, seed=3)


def test_c5_full(H):
    parity(H, workloads.c5(), seed=5)


def test_c4_full(H):
    """The shape where the automatic plan takes the steps: four chunks of positions
    over 256 rows of 152064 logits."""
    import speculative_sampling_verify_02_amd as sv
    w = workloads.c4()
    assert sv.early_exit_plan(w.batch, w.n_target_rows, w.vocab, sv.SV_BF16, "sample", int(w.gamma.max())) == "steps"
    g, _ = parity(H, w, dense=True, seed=4)
    assert np.all(g["row_status"] & oracle.INVALID_MASK == 0)
    assert len(set(g["n_accepted"].tolist())) >= 4   # rows decided in several different chunks


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_invalid_rows_read_to_the_end(H, dtype):
    """A row invalid from the start (bad temperature or token) decides nothing, so the
    early-exit round, like the full one, still reads its every position and reports
    non-finite logits there."""
    from test_gpu_parity import invalid_from_start
    w = invalid_from_start(dtype)
    g, ref = parity(H, w, seed=7)
    st = g["row_status"]
    assert st[0] == oracle.BAD_TEMP | oracle.NONFINITE and st[3] == oracle.BAD_TOKEN | oracle.NONFINITE
    assert st[4] == oracle.BAD_TOKEN and st[5] == oracle.BAD_TEMP


def test_rows_beyond_gamma_max(H):
    """A ragged row longer than the caller's gamma_max is invalid (BAD_GAMMA): it emits
    nothing and keeps no cache count, and the other rows decide exactly as in a call
    whose bound covers every row (which the oracle checks)."""
    w = workloads.small(seed=83, batch=6, vocab=3000, dtype="bf16", gamma=[2, 5, 1, 3, 0, 4], noise=0.05)
    full, _ = parity(H, w, seed=83)
    cache = np.random.default_rng(83).integers(0, 4096, w.batch).astype(np.int32)   # parity()'s
    _say("[case] early exit with gamma_max 3 under row gammas up to 5")
    cut = run_early(H, w, cache_len=cache, gamma_max=3)
    same_outputs(cut, run_early(H, w, cache_len=cache, gamma_max=3, plan="one_pass"))
    t_off, _ = w.offsets()
    assert np.any(w.gamma > 3) and np.any(full["n_accepted"][w.gamma <= 3] >= 1)
    for i in range(w.batch):
        a, b = t_off[i], t_off[i + 1]
        if w.gamma[i] > 3:
            assert cut["n_accepted"][i] == -1 and cut["crop_len"][i] == -1, i
            assert cut["row_status"][i] == oracle.BAD_GAMMA and np.all(cut["emitted"][a:b] == -1), i
            assert np.all(np.isnan(cut["p_x"][w.offsets()[1][i]:w.offsets()[1][i + 1]])), i
        else:
            for k in ("n_accepted", "crop_len", "row_status"):
                assert cut[k][i] == full[k][i], (k, i)
            assert np.array_equal(cut["emitted"][a:b], full["emitted"][a:b]), i


def test_auto_plan(H):
    """plan="auto" takes one of the two plans and so gives their outputs.  On 64 rows
    of 131072 bf16 logits with 12 drafts each (inputs drawn on the GPU, drafts sampled
    from q), a hint of 0 makes it take the steps and a hint of 1 the one pass."""
    import speculative_sampling_verify_02_amd as sv
    B, g, V = 64, 12, 131072
    gen = torch.Generator(device="cuda").manual_seed(85)
    tgt = (torch.randn(B, g + 1, V, device="cuda", generator=gen) * 3.0).to(torch.bfloat16)
    drf = (tgt[:, :g].float() + 0.3 * torch.randn(B, g, V, device="cuda", generator=gen)).to(torch.bfloat16)
    tok = torch.multinomial(torch.softmax(drf.float().reshape(B * g, V), -1), 1, generator=gen)
    tok = tok.reshape(B, g).to(torch.int32)
    uni = torch.rand(B, g + 1, device="cuda", generator=gen)
    T = torch.ones(B, device="cuda")
    outs, chosen = [], []
    for plan, hint in (("steps", None), ("one_pass", None), ("auto", 0.0), ("auto", 1.0)):
        if plan == "auto":
            chosen.append(sv.early_exit_plan(B, B * (g + 1), V, sv.SV_BF16, "sample", g, accept_hint=hint))
        _say(f"[case] early exit plan={plan} hint={hint} B={B} gamma={g} V={V}")
        n, e, crop, dg = sv.spec_verify_early_exit(tgt, drf, tok, uni, T, diag=True, plan=plan, accept_hint=hint)
        torch.cuda.synchronize()
        outs.append(dict(n_accepted=n.cpu().numpy(), emitted=e.cpu().numpy(), crop_len=crop.cpu().numpy(),
                         **{k: v.cpu().numpy() for k, v in dg.items()}))
    assert chosen == ["steps", "one_pass"]
    assert np.all(outs[0]["row_status"] & oracle.INVALID_MASK == 0) and 0 < outs[0]["n_accepted"].mean() < g
    for o in outs[1:]:
        same_outputs(outs[0], o)
