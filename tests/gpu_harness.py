"""Run the HIP path through the C ABI on a workload, and compare it with the oracle.

Parity rule.  A decision is "near" when the oracle finds it within eps = 1e-5 of its
threshold: |u - ratio| < eps for an accept test, |C - t| < eps * W at an interior CDF
edge for the draw.  The GPU computes in fp32 where the oracle computes in fp64, so
only a near decision may go either way; every other one must be taken identically.
Per row:
  * row status bits are identical;
  * decisions are compared left to right: an accept test taken the same way moves on;
    one taken the other way must be near, and then the oracle is run again on that
    row with that test's uniform forced to the GPU's branch (0 keeps the draft, 1
    rejects it), and the comparison goes on against that run, so the rest of the row
    is still held to the oracle;
  * with the same K, the kept drafts are identical and the drawn token is identical,
    or, for a near draw, lies among the tokens the oracle finds within eps * W of the
    threshold ([draw_lo, draw_hi]); the slots after K are -1;
  * p(x_j), q(x_j) and the residual mass agree within `tol` relative (1e-4 for bf16
    logits, 1e-6 for fp32), and are NaN at the same places.
A top-p boundary within 1e-10 of top_p (filtered calls) may move a threshold by one
group of tokens; from such a position on only the prefix before it is compared.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import speculative_sampling_verify_02_amd as sv
import workloads

TOL = {"bf16": 1e-4, "f32": 1e-6}


def to_device(w, dev="cuda:0"):
    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if w.dtype == "bf16":
        target = t(w.target.view(np.int16)).view(torch.bfloat16)
        draft = t(w.draft.view(np.int16)).view(torch.bfloat16)
    else:
        target, draft = t(w.target), t(w.draft)
    return dict(target=target, draft=draft, tokens=t(w.draft_tokens), uniforms=t(w.uniforms),
                temperature=t(w.temperature), gamma=t(w.gamma))


def run_gpu(w, mode=None, dense=False, dev="cuda:0", tensors=None):
    d = tensors or to_device(w, dev)
    gamma = w.dense_gamma if dense else d["gamma"]
    n, e, dg = sv.spec_verify(d["target"], d["draft"], d["tokens"], d["uniforms"],
                              d["temperature"], gamma, mode=mode or w.mode, diag=True)
    torch.cuda.synchronize()
    out = dict(n_accepted=n.cpu().numpy(), emitted=e.cpu().numpy())
    for k, v in dg.items():
        out[k] = v.cpu().numpy()
    return out


def _rel_ok(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb), f"{what}: NaN pattern differs at {np.nonzero(fa != fb)[0][:10]}"
    if not fb.any():
        return 0.0
    err = np.abs(a[fb] - b[fb]) / np.maximum(np.abs(b[fb]), 1e-300)
    worst = float(err.max())
    assert worst <= tol, f"{what}: max relative error {worst:.3e} > {tol:.0e} at {np.argmax(err)}"
    return worst


def row_workload(w, i, uniforms=None):
    """Row i of a packed workload as a workload of its own (optionally with other
    uniforms for that row)."""
    t_off, d_off = w.offsets()
    a, b, c, d = t_off[i], t_off[i + 1], d_off[i], d_off[i + 1]
    return workloads.Workload(name=f"{w.name}_row{i}", dtype=w.dtype, vocab=w.vocab, gamma=w.gamma[i:i + 1],
                              target=w.target[a:b], draft=w.draft[c:d], draft_tokens=w.draft_tokens[c:d],
                              uniforms=(w.uniforms[a:b] if uniforms is None else uniforms),
                              temperature=w.temperature[i:i + 1], mode=w.mode)


class RowRef:
    """The oracle's result for one row: from a batch run, or from a run of that row alone."""

    def __init__(self, ref, i, a, b, c, d, uniforms):
        self.K = int(ref["n_accepted"][i])
        self.emitted = ref["emitted"][a:b]
        self.flags = ref["flags"][a:b]
        self.lo, self.hi = int(ref["draw_lo"][i]), int(ref["draw_hi"][i])
        self.status = int(ref["row_status"][i])
        self.resid = ref["resid_mass"][i:i + 1]
        self.p_x, self.q_x = ref["p_x"][c:d], ref["q_x"][c:d]
        self.crop = int(ref["crop_len"][i])
        self.uniforms = uniforms


def compare(w, gpu, ref, mode=None, tol=None, oracle_kw=None):
    """Assert the parity rule on every row; return a small report.  oracle_kw holds the
    per-row oracle options of the call (top_k, top_p, early_exit, cache_len) for the
    forced re-runs."""
    mode = mode or w.mode
    tol = TOL[w.dtype] if tol is None else tol
    oracle_kw = dict(oracle_kw or {})
    t_off, d_off = w.offsets()
    rep = dict(rows=w.batch, near_decisions=int(np.count_nonzero(ref["flags"] & oracle.FLAG_NEAR)),
               rows_with_near=int((ref["flag_pos"] >= 0).sum()), diverged_at_near_test=0,
               near_draws=0, near_draws_differ=0, filter_boundary_rows=0)
    worst = dict(p_x=0.0, q_x=0.0, resid_mass=0.0)

    def rerun(i, u):
        kw = {}
        for k in ("top_k", "top_p", "cache_len"):
            if oracle_kw.get(k) is not None:
                kw[k] = np.asarray(oracle_kw[k])[i:i + 1]
        r = oracle.verify_workload(row_workload(w, i, u), mode=mode, early_exit=oracle_kw.get("early_exit", False),
                                   **kw)
        g = int(w.gamma[i])
        return RowRef(r, 0, 0, g + 1, 0, g, u)

    for i in range(w.batch):
        a, b, c, d = t_off[i], t_off[i + 1], d_off[i], d_off[i + 1]
        g = b - a - 1
        R = RowRef(ref, i, a, b, c, d, w.uniforms[a:b].copy())
        Kg = int(gpu["n_accepted"][i])
        eg = gpu["emitted"][a:b]
        where = f"row {i} (gamma {g})"
        for depth in range(g + 2):
            ff = np.nonzero(R.flags & oracle.FLAG_FILTER)[0]
            ff = int(ff[0]) if ff.size else g + 1
            forced = False
            for j in range(min(g, ff)):
                ga, ra = Kg > j, R.K > j
                if ga == ra:
                    if not ga:
                        break
                    continue
                assert R.flags[j] & oracle.FLAG_NEAR, (
                    f"{where}: accept test {j} taken differently and not near its threshold: "
                    f"gpu K={Kg} {eg} oracle K={R.K} {R.emitted}")
                u = R.uniforms.copy()
                u[j] = 0.0 if ga else 1.0
                R = rerun(i, u)
                assert (R.K > j) == ga, f"{where}: forcing test {j} did not take the GPU's branch"
                rep["diverged_at_near_test"] += 1
                forced = True
                break
            if not forced:
                break
        if gpu["row_status"][i] != R.status:
            raise AssertionError(f"{where}: row status gpu {gpu['row_status'][i]} oracle {R.status}")
        if ff <= min(Kg, R.K):
            # a top-p boundary at or before the decision: compare the prefix before it
            rep["filter_boundary_rows"] += 1
            assert np.array_equal(eg[:ff], R.emitted[:ff]), f"{where}: prefix before a top-p boundary differs"
            continue
        assert Kg == R.K, f"{where}: gpu K={Kg} {eg} oracle K={R.K} {R.emitted}"
        K = Kg
        if K < 0:
            assert np.all(eg == -1), f"{where}: invalid row with outputs {eg}"
        else:
            assert np.array_equal(eg[:K], R.emitted[:K]), f"{where}: kept drafts differ: {eg} vs {R.emitted}"
            assert np.all(eg[K + 1:] == -1), f"{where}: slots after K are not -1: {eg}"
            if R.flags[g] & oracle.FLAG_NEAR:
                rep["near_draws"] += 1
                rep["near_draws_differ"] += int(eg[K] != R.emitted[K])
                assert R.lo <= eg[K] <= R.hi, (f"{where}: near draw gives {eg[K]}, outside the tokens "
                                               f"[{R.lo}, {R.hi}] within eps of the threshold")
            else:
                assert eg[K] == R.emitted[K], f"{where}: drawn token {eg[K]} vs oracle {R.emitted[K]}"
        if "crop_len" in gpu:
            assert gpu["crop_len"][i] == R.crop, f"{where}: crop_len {gpu['crop_len'][i]} vs {R.crop}"
        if mode == "sample":
            worst["p_x"] = max(worst["p_x"], _rel_ok(gpu["p_x"][c:d], R.p_x, tol, f"{where} p_x"))
            worst["q_x"] = max(worst["q_x"], _rel_ok(gpu["q_x"][c:d], R.q_x, tol, f"{where} q_x"))
            worst["resid_mass"] = max(worst["resid_mass"],
                                      _rel_ok(gpu["resid_mass"][i:i + 1], R.resid, tol, f"{where} resid_mass"))
    if mode == "sample":
        rep.update(worst)
    return rep


def check_strict(w, gpu, ref_strict):
    """Among rows whose decisions are all further than a tighter eps from their
    thresholds, count those that do not match exactly: (checked, mismatched)."""
    t_off, _ = w.offsets()
    ok = ref_strict["flag_pos"] < 0
    bad = 0
    for i in np.nonzero(ok)[0]:
        a, b = t_off[i], t_off[i + 1]
        if gpu["n_accepted"][i] != ref_strict["n_accepted"][i] or \
                not np.array_equal(gpu["emitted"][a:b], ref_strict["emitted"][a:b]):
            bad += 1
    return int(ok.sum()), bad
