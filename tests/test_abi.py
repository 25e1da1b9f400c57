"""The C-ABI library loads and exports every function include/*.h declares; host-side
argument checks return their documented status without touching a GPU."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b([a-z_][a-z0-9_]*)\s*\(", text):
            name = m.group(1)
            if name.startswith("spec_"):
                names.add(name)
    return names


@pytest.fixture(scope="module")
def sv():
    import speculative_sampling_verify_02_amd as sv
    return sv


def test_exports_every_declared_symbol(sv):
    names = _declared()
    assert {"spec_verify", "spec_verify_workspace_bytes", "spec_verify_strerror",
            "spec_verify_set_profile_events", "spec_verify_version"} <= names
    for n in names:
        assert hasattr(sv.lib, n), f"{n} declared in include/ but not exported"
    assert set(sv.EXPORTED) == names


def test_strerror_and_version(sv):
    for code in (sv.SV_OK, sv.SV_EINVAL, sv.SV_EDTYPE, sv.SV_EWORKSPACE, sv.SV_EHIP, sv.SV_ESCRATCH):
        assert sv.strerror(code) and sv.strerror(code) != "unknown status"
    assert sv.strerror(12345) == "unknown status"
    assert "gfx950" in sv.version()


def test_workspace_bytes(sv):
    a = sv.workspace_bytes(64, 64 * 6, 128256, sv.SV_BF16)
    b = sv.workspace_bytes(256, 256 * 9, 152064, sv.SV_BF16)
    assert 0 < a < b < 64 << 20
    assert a % 256 == 0
    assert sv.workspace_bytes(-1, 0, 10, sv.SV_BF16) == 0
    assert sv.workspace_bytes(4, 3, 10, sv.SV_BF16) == 0
    assert sv.workspace_bytes(4, 8, 0, sv.SV_F32) == 0
    assert sv.workspace_bytes(4, 8, 10, 7) == 0


def _call(sv, **kw):
    args = dict(target=1 << 20, draft=1 << 21, dtype=sv.SV_BF16, vocab=32, batch=2, nT=6,
                tokens=1 << 22, uniforms=1 << 23, temperature=1 << 24, gamma=None, gamma_u=2,
                mode=sv.SV_SAMPLE, n_acc=1 << 25, emitted=1 << 26, ws=1 << 27, ws_bytes=1 << 30)
    args.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return sv.lib.spec_verify(vp(args["target"]), vp(args["draft"]), args["dtype"], args["vocab"],
                              args["batch"], args["nT"], vp(args["tokens"]), vp(args["uniforms"]),
                              vp(args["temperature"]), vp(args["gamma"]), args["gamma_u"], args["mode"],
                              vp(args["n_acc"]), vp(args["emitted"]), None, vp(args["ws"]),
                              args["ws_bytes"], None)


def test_host_argument_errors(sv):
    # every case below is rejected before any HIP call (the pointers are never used)
    assert _call(sv, dtype=5) == sv.SV_EDTYPE
    assert _call(sv, mode=3) == sv.SV_EINVAL
    assert _call(sv, vocab=0) == sv.SV_EINVAL
    assert _call(sv, nT=1) == sv.SV_EINVAL                 # fewer target rows than rows
    assert _call(sv, nT=7) == sv.SV_EINVAL                 # dense count mismatch
    assert _call(sv, gamma_u=-1) == sv.SV_EINVAL
    assert _call(sv, target=None) == sv.SV_EINVAL
    assert _call(sv, uniforms=None) == sv.SV_EINVAL
    assert _call(sv, tokens=None) == sv.SV_EINVAL
    assert _call(sv, draft=None) == sv.SV_EINVAL           # sampling needs draft logits
    assert _call(sv, ws=None) == sv.SV_EINVAL
    assert _call(sv, ws_bytes=100) == sv.SV_EWORKSPACE
    assert _call(sv, ws=(1 << 27) + 64) == sv.SV_EWORKSPACE  # misaligned
    assert _call(sv, batch=0, nT=0) == sv.SV_OK              # empty batch: nothing to do
    assert sv.lib.spec_verify_set_profile_events(ctypes.c_void_p(1), None) == sv.SV_EINVAL


def _call_sample(sv, **kw):
    args = dict(logits=1 << 20, dtype=sv.SV_BF16, vocab=32, n=4, temperature=1 << 24,
                uniforms=1 << 23, tokens=1 << 25, status=None, ws=1 << 27, ws_bytes=1 << 30)
    args.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return sv.lib.spec_sample(vp(args["logits"]), args["dtype"], args["vocab"], args["n"],
                              vp(args["temperature"]), vp(args["uniforms"]), vp(args["tokens"]),
                              vp(args["status"]), vp(args["ws"]), args["ws_bytes"], None)


def test_sample_host_argument_errors(sv):
    assert _call_sample(sv, dtype=5) == sv.SV_EDTYPE
    assert _call_sample(sv, vocab=0) == sv.SV_EINVAL
    assert _call_sample(sv, n=-1) == sv.SV_EINVAL
    assert _call_sample(sv, n=1 << 31) == sv.SV_EINVAL
    assert _call_sample(sv, logits=None) == sv.SV_EINVAL
    assert _call_sample(sv, uniforms=None) == sv.SV_EINVAL
    assert _call_sample(sv, temperature=None) == sv.SV_EINVAL
    assert _call_sample(sv, tokens=None) == sv.SV_EINVAL
    assert _call_sample(sv, ws=None) == sv.SV_EINVAL
    assert _call_sample(sv, ws_bytes=100) == sv.SV_EWORKSPACE
    assert _call_sample(sv, ws=(1 << 27) + 64) == sv.SV_EWORKSPACE
    assert _call_sample(sv, n=0) == sv.SV_OK
    a = sv.sample_workspace_bytes(320, 128256, sv.SV_BF16)
    assert 0 < a < 64 << 20 and a % 256 == 0
    assert sv.sample_workspace_bytes(-1, 10, sv.SV_BF16) == 0
    assert sv.sample_workspace_bytes(4, 0, sv.SV_F32) == 0
    assert sv.sample_workspace_bytes(4, 10, 7) == 0


def test_tree_host_argument_errors(sv):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(**kw):
        a = dict(logits=1 << 20, dtype=sv.SV_BF16, vocab=32, B=2, n=6, counts=1 << 21, tokens=1 << 22,
                 parents=1 << 23, n_acc=1 << 24, path=1 << 25, emitted=1 << 26, status=None, ws=1 << 27,
                 ws_bytes=1 << 30)
        a.update(kw)
        return sv.lib.spec_tree_verify_greedy(vp(a["logits"]), a["dtype"], a["vocab"], a["B"], a["n"],
                                              vp(a["counts"]), vp(a["tokens"]), vp(a["parents"]),
                                              vp(a["n_acc"]), vp(a["path"]), vp(a["emitted"]),
                                              vp(a["status"]), vp(a["ws"]), a["ws_bytes"], None)
    assert call(dtype=9) == sv.SV_EDTYPE
    assert call(vocab=0) == sv.SV_EINVAL
    assert call(B=-1) == sv.SV_EINVAL
    assert call(n=-1) == sv.SV_EINVAL
    assert call(B=0, n=3) == sv.SV_EINVAL
    assert call(B=0, n=0) == sv.SV_OK
    for k in ("logits", "counts", "tokens", "parents", "n_acc", "path", "emitted", "ws"):
        assert call(**{k: None}) == sv.SV_EINVAL, k
    assert call(ws_bytes=10) == sv.SV_EWORKSPACE
    assert call(ws=(1 << 27) + 8) == sv.SV_EWORKSPACE
    assert sv.tree_workspace_bytes(4032, 128256, sv.SV_BF16) > 0
    assert sv.tree_workspace_bytes(-1, 10, sv.SV_BF16) == 0


def test_early_exit_host_argument_errors(sv):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(**kw):
        a = dict(target=1 << 20, draft=1 << 21, dtype=sv.SV_BF16, vocab=32, batch=2, nT=6, tokens=1 << 22,
                 uniforms=1 << 23, temperature=1 << 24, gamma=None, gamma_u=2, gamma_max=2, mode=sv.SV_SAMPLE,
                 cache=None, n_acc=1 << 25, emitted=1 << 26, crop=None, plan=sv.SV_EE_AUTO, hint=-1.0,
                 ws=1 << 27, ws_bytes=1 << 30)
        a.update(kw)
        return sv.lib.spec_verify_early_exit(vp(a["target"]), vp(a["draft"]), a["dtype"], a["vocab"], a["batch"],
                                             a["nT"], vp(a["tokens"]), vp(a["uniforms"]), vp(a["temperature"]),
                                             vp(a["gamma"]), a["gamma_u"], a["gamma_max"], a["mode"],
                                             vp(a["cache"]), vp(a["n_acc"]), vp(a["emitted"]), vp(a["crop"]),
                                             None, a["plan"], a["hint"], vp(a["ws"]), a["ws_bytes"], None)
    assert call(dtype=4) == sv.SV_EDTYPE
    assert call(mode=2) == sv.SV_EINVAL
    assert call(nT=7) == sv.SV_EINVAL
    assert call(gamma_u=-1) == sv.SV_EINVAL
    assert call(gamma=1 << 28, gamma_max=-1) == sv.SV_EINVAL   # ragged needs a bound
    assert call(target=None) == sv.SV_EINVAL
    assert call(draft=None) == sv.SV_EINVAL
    assert call(ws_bytes=64) == sv.SV_EWORKSPACE
    assert call(ws=(1 << 27) + 16) == sv.SV_EWORKSPACE
    assert call(plan=3) == sv.SV_EINVAL and call(plan=-1) == sv.SV_EINVAL
    assert call(batch=0, nT=0) == sv.SV_OK
    a = sv.early_exit_workspace_bytes(64, 384, 128256, sv.SV_BF16)
    assert a > sv.workspace_bytes(64, 384, 128256, sv.SV_BF16) and a % 256 == 0


def test_filtered_host_argument_errors(sv):
    vp = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(**kw):
        a = dict(target=1 << 20, draft=1 << 21, dtype=sv.SV_BF16, vocab=32, batch=2, nT=6, tokens=1 << 22,
                 uniforms=1 << 23, temperature=1 << 24, gamma=None, gamma_u=2, top_k=1 << 28, top_p=None,
                 n_acc=1 << 25, emitted=1 << 26, ws=1 << 27, ws_bytes=1 << 30)
        a.update(kw)
        return sv.lib.spec_verify_filtered(vp(a["target"]), vp(a["draft"]), a["dtype"], a["vocab"], a["batch"],
                                           a["nT"], vp(a["tokens"]), vp(a["uniforms"]), vp(a["temperature"]),
                                           vp(a["gamma"]), a["gamma_u"], vp(a["top_k"]), vp(a["top_p"]),
                                           vp(a["n_acc"]), vp(a["emitted"]), None, vp(a["ws"]), a["ws_bytes"], None)
    assert call(top_k=None, top_p=None) == sv.SV_EINVAL
    assert call(dtype=3) == sv.SV_EDTYPE
    assert call(nT=5) == sv.SV_EINVAL
    assert call(draft=None) == sv.SV_EINVAL
    assert call(ws_bytes=sv.workspace_bytes(2, 6, 32, sv.SV_BF16)) == sv.SV_EWORKSPACE   # no room for thresholds
    assert call(batch=0, nT=0) == sv.SV_OK
    assert sv.filtered_workspace_bytes(2, 6, 32, sv.SV_BF16) > sv.workspace_bytes(2, 6, 32, sv.SV_BF16)


def test_bench_refuses_several_gpus():
    """The benchmark runs on one GPU: asking for more exits with status 2 and one JSON
    line that says so, before anything touches a GPU."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU only" in line["error"]


def test_noalloc_host_argument_errors(sv):
    """spec_verify_noalloc refuses, before touching a device, a shape whose workspace
    exceeds its fixed scratch array, and bad dtypes or sizes."""
    L = sv.lib
    p = 1 << 20

    def call(dtype, V, B, nT, gu):
        return L.spec_verify_noalloc(p, p, dtype, V, B, nT, p, p, p, None, gu, sv.SV_SAMPLE, p, p, None, None)

    # 4096 rows of 8 drafts over V = 256000 fp32: beyond 16 MiB of workspace
    assert sv.workspace_bytes(4096, 4096 * 9, 256000, sv.SV_F32) > sv.NOALLOC_SCRATCH_BYTES
    assert call(sv.SV_F32, 256000, 4096, 4096 * 9, 8) == sv.SV_ESCRATCH
    assert call(7, 1000, 2, 6, 2) == sv.SV_EDTYPE
    assert call(sv.SV_BF16, 0, 2, 6, 2) == sv.SV_EINVAL
    assert call(sv.SV_BF16, 1000, 2, 1, 2) == sv.SV_EINVAL


def test_early_exit_plan_choice(sv):
    """The automatic plan of the round with early exit (host only).  Few, short vectors
    per position (64 rows of 128256 bf16 logits, 5 drafts) cannot pay for the steps'
    fixed cost, so one pass is taken; 256 rows of 152064 logits with 8 drafts read a
    third of their logits at the default acceptance rate, so the steps are taken.  A
    draft that is never kept makes the steps read position 0 only; one that is always
    kept makes them read everything, so one pass.  (Even then the small shape keeps one
    pass: its three steps' fixed cost exceeds what they save.)"""
    plan = sv.early_exit_plan
    assert plan(64, 64 * 6, 128256, sv.SV_BF16, "sample", 5) == "one_pass"
    assert plan(64, 64 * 6, 128256, sv.SV_BF16, "greedy", 5) == "one_pass"
    assert plan(256, 256 * 9, 152064, sv.SV_BF16, "sample", 8) == "steps"
    assert plan(256, 256 * 9, 152064, sv.SV_BF16, "sample", 8, accept_hint=0.0) == "steps"
    assert plan(256, 256 * 9, 152064, sv.SV_BF16, "sample", 8, accept_hint=1.0) == "one_pass"
    assert plan(256, 256 * 9, 152064, sv.SV_BF16, "sample", 8, accept_hint=float("nan")) == "steps"
    assert plan(64, 64 * 6, 128256, sv.SV_BF16, "sample", 5, accept_hint=0.0) == "one_pass"
    for bad in (dict(batch=0), dict(gamma_max=-1), dict(dtype=7), dict(mode=5)):
        a = dict(batch=4, nT=8, vocab=100, dtype=sv.SV_F32, mode=sv.SV_SAMPLE, gamma_max=1)
        a.update(bad)
        assert sv.lib.spec_verify_early_exit_plan(a["batch"], a["nT"], a["vocab"], a["dtype"], a["mode"],
                                                  a["gamma_max"], -1.0) < 0, bad
