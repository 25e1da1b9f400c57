"""The drafter's draw (spec_sample) against the CPU oracle, through the C ABI.

Parity rule: status bits identical on every vector; the token identical wherever
the oracle finds the draw's threshold farther than 1e-5 W from an interior edge of
the drawn token's CDF interval; elsewhere one of the tokens whose CDF interval comes
within 1e-5 W of the threshold (the oracle's [lo, hi]).  Greedy vectors (T <= 0)
match bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _device_logits(si, dev="cuda:0"):
    if si.dtype == "bf16":
        return torch.from_numpy(si.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(si.logits, np.float32)).to(dev)


def run_gpu(si, dev="cuda:0"):
    import speculative_sampling_verify_02_amd as sv
    z = _device_logits(si, dev)
    u = torch.from_numpy(si.uniforms).to(dev)
    T = torch.from_numpy(si.temperature).to(dev)
    tok, st = sv.spec_sample(z, u, T, status=True)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), st.cpu().numpy()


def check(si, tok, st, ref):
    bad = np.nonzero(st != ref["status"])[0]
    assert bad.size == 0, f"status differs at {bad[:10]}: gpu {st[bad[:10]]} oracle {ref['status'][bad[:10]]}"
    free = ref["flags"] == 0
    diff = np.nonzero(free & (tok != ref["tokens"]))[0]
    assert diff.size == 0, f"tokens differ at {diff[:10]}: gpu {tok[diff[:10]]} oracle {ref['tokens'][diff[:10]]}"
    flagged = np.nonzero(~free)[0]
    out = flagged[(tok[flagged] < ref["lo"][flagged]) | (tok[flagged] > ref["hi"][flagged])]
    assert out.size == 0, (f"near draws outside the oracle's admissible tokens at {out[:10]}: gpu {tok[out[:10]]} "
                           f"range {ref['lo'][out[:10]]}..{ref['hi'][out[:10]]}")
    return dict(n=si.n, flagged=int(flagged.size), flagged_differ=int((tok[flagged] != ref["tokens"][flagged]).sum()))


def parity(si):
    _say(f"[case] spec_sample {si.name} n={si.n} V={si.vocab} {si.dtype}")
    tok, st = run_gpu(si)
    ref = oracle.sample(si.logits, si.dtype, si.vocab, si.temperature, si.uniforms)
    rep = check(si, tok, st, ref)
    _say(f"[ok] {rep}")
    return tok, st, ref


SMALL = [
    dict(seed=51, batch=9, vocab=4096, dtype="bf16", gamma=[3, 0, 5, 2, 4, 1, 7, 0, 2],
         temperature=[0.8, 1.0, 1.2, 0.7, 1.0, 0.0, 1.5, -1.0, 0.6]),
    dict(seed=52, batch=7, vocab=997, dtype="bf16", gamma=[1, 2, 0, 6, 3, 3, 1]),
    dict(seed=53, batch=5, vocab=20000, dtype="bf16", gamma=[4, 4, 4, 4, 4], n_boost=5),
    dict(seed=54, batch=6, vocab=1024, dtype="f32", gamma=[2, 0, 3, 5, 1, 4],
         temperature=[0.9, 1.1, 0.5, 2.0, 1.0, 0.0]),
    dict(seed=55, batch=6, vocab=1001, dtype="f32", gamma=[3, 1, 0, 2, 6, 2]),
    dict(seed=56, batch=4, vocab=1, dtype="bf16", gamma=[0, 1, 3, 2]),
    dict(seed=57, batch=8, vocab=8, dtype="bf16", gamma=[1, 2, 3, 4, 5, 6, 7, 0]),
    dict(seed=58, batch=33, vocab=65536, dtype="bf16", gamma=[2] * 33),
    dict(seed=59, batch=4, vocab=300000, dtype="f32", gamma=[1, 3, 0, 2], sigma=4.0),
    dict(seed=60, batch=3, vocab=24577, dtype="bf16", gamma=[40, 10, 0], sigma=0.5),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("side", ["target", "draft"])
def test_small(case, side):
    w = workloads.small(**SMALL[case])
    parity(workloads.sample_inputs(w, seed=100 + case, side=side))


def test_status_and_special_vectors():
    """NaN, +inf and all -inf vectors are invalid; bad temperatures are invalid; -inf
    logits are never drawn; T <= 0 takes the first argmax."""
    w = workloads.small(seed=61, batch=8, vocab=3000, dtype="f32", gamma=[1] * 8)
    si = workloads.sample_inputs(w, seed=61, side="target")
    z = si.logits.copy()
    z[0, 17] = np.nan
    z[1, 2999] = np.inf
    z[2, :] = -np.inf
    z[3, ::2] = -np.inf
    z[4, :] = 1.0            # all tied: argmax 0 at T <= 0, uniform draw otherwise
    z[5, :] = 1.0
    T = si.temperature.copy()
    T[4] = 0.0
    T[6] = np.nan
    T[7] = 1e-39
    T[8] = np.inf
    T[9] = -2.0
    si = workloads.SampleInputs("special", "f32", si.vocab, z, T, si.uniforms)
    tok, st, ref = parity(si)
    assert tok[3] % 2 == 1 and tok[4] == 0 and tok[9] >= 0
    assert np.all(tok[[0, 1, 2, 6, 7, 8]] == -1)


def test_equals_verify_without_drafts():
    """spec_sample gives what spec_verify gives for rows without drafts."""
    import speculative_sampling_verify_02_amd as sv
    w = workloads.small(seed=62, batch=24, vocab=50000, dtype="bf16", gamma=2)
    si = workloads.sample_inputs(w, seed=62, side="target")
    z = _device_logits(si)
    u = torch.from_numpy(si.uniforms).cuda()
    T = torch.from_numpy(si.temperature).cuda()
    a = sv.spec_sample(z, u, T)
    _, b = sv.spec_verify(z, None, None, u, T, 0, mode="sample")
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_c3_draft_full():
    """All 320 draft vectors of the V = 128256 bf16 batch in one call."""
    parity(workloads.sample_inputs(workloads.c3(), seed=3, side="draft"))


def test_c4_draft_long_pass():
    """1300 draft vectors of the V = 152064 bf16 batch: 49400 pieces, a pass long
    enough for the streaming kernel to keep its records in LDS and write them out
    after its last piece."""
    si = workloads.sample_inputs(workloads.c4(), seed=4, side="draft", limit=1300)
    assert si.n * ((si.vocab + 4095) // 4096) * 8192 / 6.4e12 >= 60e-6
    parity(si)


def test_c2_target_full():
    parity(workloads.sample_inputs(workloads.c2(), seed=2, side="target"))


def test_c5_draft_subset():
    """fp32 logits at V = 256000: the first 256 draft vectors."""
    parity(workloads.sample_inputs(workloads.c5(), seed=5, side="draft", limit=256))


def test_bad_temperature_and_nonfinite_vector():
    """A vector with an unusable temperature and a NaN, +inf or all -inf logits reports
    both, as the oracle does."""
    w = workloads.small(seed=63, batch=4, vocab=2000, dtype="f32", gamma=[1] * 4)
    si = workloads.sample_inputs(w, seed=63, side="target")
    z = si.logits.copy()
    T = si.temperature.copy()
    z[0, 3] = np.nan
    T[0] = np.nan
    z[1, 1999] = np.inf
    T[1] = 1e-39
    z[2, :] = -np.inf
    T[2] = np.inf
    T[3] = np.nan
    si = workloads.SampleInputs("bad_t_nonfinite", "f32", si.vocab, z, T, si.uniforms)
    tok, st, ref = parity(si)
    assert list(st[:3]) == [oracle.BAD_TEMP | oracle.NONFINITE] * 3 and st[3] == oracle.BAD_TEMP
