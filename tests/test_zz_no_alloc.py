"""spec_verify_noalloc (the entry point that allocates nothing: its workspace is the
library's fixed scratch array) against spec_verify, through the C ABI, on two calls
in a row, the second with a smaller input."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _noalloc(sv, d, w, dense):
    """One spec_verify_noalloc call through the C ABI, with diagnostics."""
    dev = d["target"].device
    B, nT = w.batch, w.n_target_rows
    out = dict(n_accepted=torch.full((B,), -7, dtype=torch.int32, device=dev),
               emitted=torch.full((nT,), -7, dtype=torch.int32, device=dev),
               p_x=torch.empty(nT - B, dtype=torch.float64, device=dev),
               q_x=torch.empty(nT - B, dtype=torch.float64, device=dev),
               resid_mass=torch.empty(B, dtype=torch.float64, device=dev),
               row_status=torch.empty(B, dtype=torch.int32, device=dev))
    diag = sv.Diag(out["p_x"].data_ptr(), out["q_x"].data_ptr(), out["resid_mass"].data_ptr(),
                   out["row_status"].data_ptr())
    dt = sv.SV_BF16 if w.dtype == "bf16" else sv.SV_F32
    gptr = None if dense else ctypes.c_void_p(d["gamma"].data_ptr())
    gu = int(w.gamma[0]) if dense else 0
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = sv.lib.spec_verify_noalloc(ctypes.c_void_p(d["target"].data_ptr()), ctypes.c_void_p(d["draft"].data_ptr()),
                                    dt, w.vocab, B, nT, ctypes.c_void_p(d["tokens"].data_ptr()),
                                    ctypes.c_void_p(d["uniforms"].data_ptr()),
                                    ctypes.c_void_p(d["temperature"].data_ptr()), gptr, gu, sv.SV_SAMPLE,
                                    ctypes.c_void_p(out["n_accepted"].data_ptr()),
                                    ctypes.c_void_p(out["emitted"].data_ptr()), ctypes.byref(diag),
                                    ctypes.c_void_p(stream))
    assert rc == sv.SV_OK, sv.strerror(rc)
    return out


def _host(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_noalloc_matches_spec_verify():
    import gpu_harness as H
    import speculative_sampling_verify_02_amd as sv
    big = workloads.small(seed=401, batch=40, vocab=50000, dtype="bf16",
                          gamma=np.random.default_rng(401).integers(0, 8, 40))
    small = workloads.small(seed=402, batch=6, vocab=4096, dtype="bf16", gamma=3)
    cases = [(big, False), (small, True)]
    dev_in = [H.to_device(w) for w, _ in cases]
    # the existing entry point (caller workspace), then the no-alloc one on both inputs
    # in a row, the second smaller, so the second call finds the first call's contents
    ref_gpu = [H.run_gpu(w, dense=dense, tensors=d) for (w, dense), d in zip(cases, dev_in)]
    outs = [_noalloc(sv, d, w, dense) for (w, dense), d in zip(cases, dev_in)]
    torch.cuda.synchronize()
    for (w, dense), a, b in zip(cases, ref_gpu, outs):
        b = _host(b)
        _say(f"[case] noalloc {w.name} dense={dense}")
        for k in ("n_accepted", "emitted", "row_status"):
            assert np.array_equal(a[k], b[k]), k
        for k in ("p_x", "q_x", "resid_mass"):
            assert np.array_equal(a[k], b[k], equal_nan=True), k
        rep = H.compare(w, b, oracle.verify_workload(w))
        _say(f"[ok] {rep}")


def test_noalloc_refuses_oversized_shape():
    import speculative_sampling_verify_02_amd as sv
    w = workloads.small(seed=403, batch=4, vocab=1000, dtype="bf16", gamma=2)
    import gpu_harness as H
    d = H.to_device(w)
    # a shape claimed far beyond the scratch array: refused before anything is enqueued
    n = torch.full((4,), -7, dtype=torch.int32, device=d["target"].device)
    rc = sv.lib.spec_verify_noalloc(ctypes.c_void_p(d["target"].data_ptr()), ctypes.c_void_p(d["draft"].data_ptr()),
                                    sv.SV_F32, 256000, 4096, 4096 * 9, ctypes.c_void_p(d["tokens"].data_ptr()),
                                    ctypes.c_void_p(d["uniforms"].data_ptr()),
                                    ctypes.c_void_p(d["temperature"].data_ptr()), None, 8, sv.SV_SAMPLE,
                                    ctypes.c_void_p(n.data_ptr()), ctypes.c_void_p(n.data_ptr()), None, None)
    torch.cuda.synchronize()
    assert rc == sv.SV_ESCRATCH
    assert (n.cpu().numpy() == -7).all()
