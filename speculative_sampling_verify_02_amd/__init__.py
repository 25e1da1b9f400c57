"""spec_verify: the verification step of speculative sampling on AMD MI355X (gfx950).

This module is a thin ctypes binding of the HIP library libspecverify.so: it
marshals torch tensors into the C ABI declared in include/spec_verify.h (device
pointers, sizes, the current HIP stream) and nothing else.  Every step of the
computation runs in the library's kernels.  Importing this package fails loudly if
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

# sv_status
SV_OK, SV_EINVAL, SV_EDTYPE, SV_EWORKSPACE, SV_EHIP, SV_ESCRATCH = 0, -1, -2, -3, -4, -5
# fixed scratch array of spec_verify_noalloc (bytes)
NOALLOC_SCRATCH_BYTES = 16 << 20
# sv_dtype / sv_mode
SV_BF16, SV_F32 = 0, 1
SV_SAMPLE, SV_GREEDY = 0, 1
SV_EE_AUTO, SV_EE_STEPS, SV_EE_ONE_PASS = 0, 1, 2
# row status bits
ROW_BAD_TOKEN = 1
ROW_Q_ZERO = 2
ROW_NONFINITE = 4
ROW_BAD_GAMMA = 8
ROW_ZERO_RESID = 16
ROW_BAD_TEMP = 32
ROW_BAD_TREE = 64
ROW_INVALID = ROW_BAD_TOKEN | ROW_NONFINITE | ROW_BAD_GAMMA | ROW_BAD_TEMP | ROW_BAD_TREE

EXPORTED = ("spec_verify", "spec_verify_workspace_bytes", "spec_verify_strerror",
            "spec_verify_set_profile_events", "spec_verify_version", "spec_sample",
            "spec_sample_workspace_bytes", "spec_tree_verify_greedy",
            "spec_tree_verify_greedy_workspace_bytes", "spec_verify_early_exit",
            "spec_verify_early_exit_workspace_bytes", "spec_verify_filtered",
            "spec_verify_filtered_workspace_bytes", "spec_verify_noalloc", "spec_verify_early_exit_plan")


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"spec_verify failed ({status}): {message}")
        self.status = status


class Diag(ctypes.Structure):
    _fields_ = [("p_x", ctypes.c_void_p), ("q_x", ctypes.c_void_p),
                ("resid_mass", ctypes.c_void_p), ("row_status", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first (python -c "
            "'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.spec_verify_workspace_bytes.argtypes = [i32, i64, i64, i32]
    L.spec_verify_workspace_bytes.restype = sz
    L.spec_verify.argtypes = [vp, vp, i32, i64, i32, i64, vp, vp, vp, vp, i32, i32, vp, vp,
                              ctypes.POINTER(Diag), vp, sz, vp]
    L.spec_verify.restype = ctypes.c_int
    L.spec_verify_strerror.argtypes = [i32]
    L.spec_verify_strerror.restype = ctypes.c_char_p
    L.spec_verify_set_profile_events.argtypes = [vp, vp]
    L.spec_verify_set_profile_events.restype = ctypes.c_int
    L.spec_verify_version.argtypes = []
    L.spec_verify_version.restype = ctypes.c_char_p
    L.spec_sample_workspace_bytes.argtypes = [i64, i64, i32]
    L.spec_sample_workspace_bytes.restype = sz
    L.spec_sample.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    L.spec_sample.restype = ctypes.c_int
    L.spec_tree_verify_greedy_workspace_bytes.argtypes = [i64, i64, i32]
    L.spec_tree_verify_greedy_workspace_bytes.restype = sz
    L.spec_tree_verify_greedy.argtypes = [vp, i32, i64, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.spec_tree_verify_greedy.restype = ctypes.c_int
    L.spec_verify_early_exit_workspace_bytes.argtypes = [i32, i64, i64, i32]
    L.spec_verify_early_exit_workspace_bytes.restype = sz
    L.spec_verify_early_exit.argtypes = [vp, vp, i32, i64, i32, i64, vp, vp, vp, vp, i32, i32, i32, vp, vp,
                                         vp, vp, ctypes.POINTER(Diag), i32, ctypes.c_float, vp, sz, vp]
    L.spec_verify_early_exit.restype = ctypes.c_int
    L.spec_verify_early_exit_plan.argtypes = [i32, i64, i64, i32, i32, i32, ctypes.c_float]
    L.spec_verify_early_exit_plan.restype = ctypes.c_int
    L.spec_verify_filtered_workspace_bytes.argtypes = [i32, i64, i64, i32]
    L.spec_verify_filtered_workspace_bytes.restype = sz
    L.spec_verify_filtered.argtypes = [vp, vp, i32, i64, i32, i64, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                       ctypes.POINTER(Diag), vp, sz, vp]
    L.spec_verify_filtered.restype = ctypes.c_int
    L.spec_verify_noalloc.argtypes = [vp, vp, i32, i64, i32, i64, vp, vp, vp, vp, i32, i32, vp, vp,
                                      ctypes.POINTER(Diag), vp]
    L.spec_verify_noalloc.restype = ctypes.c_int
    return L


lib = _load()


def strerror(status: int) -> str:
    return lib.spec_verify_strerror(int(status)).decode()


def version() -> str:
    return lib.spec_verify_version().decode()


def workspace_bytes(batch: int, n_target_rows: int, vocab: int, dtype: int) -> int:
    return int(lib.spec_verify_workspace_bytes(batch, n_target_rows, vocab, dtype))


def sample_workspace_bytes(n: int, vocab: int, dtype: int) -> int:
    return int(lib.spec_sample_workspace_bytes(n, vocab, dtype))


def early_exit_workspace_bytes(batch: int, n_target_rows: int, vocab: int, dtype: int) -> int:
    return int(lib.spec_verify_early_exit_workspace_bytes(batch, n_target_rows, vocab, dtype))


def filtered_workspace_bytes(batch: int, n_target_rows: int, vocab: int, dtype: int) -> int:
    return int(lib.spec_verify_filtered_workspace_bytes(batch, n_target_rows, vocab, dtype))


def tree_workspace_bytes(n_nodes: int, vocab: int, dtype: int) -> int:
    return int(lib.spec_tree_verify_greedy_workspace_bytes(n_nodes, vocab, dtype))


def set_profile_events(start_event, stop_event) -> None:
    """Raw hipEvent_t handles (ints) attached to the streaming kernel's dispatch in
    every following call (around the position steps for early exit); (None, None)
    stops."""
    rc = lib.spec_verify_set_profile_events(start_event, stop_event)
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))


_workspaces: dict = {}


def _workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtypes, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def spec_verify(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                gamma_per_row=None, *, mode: str = "sample", diag: bool = False,
                workspace: torch.Tensor | None = None, out=None):
    return _verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, gamma_per_row,
                   mode=mode, diag=diag, workspace=workspace, out=out)


EE_PLANS = {"auto": SV_EE_AUTO, "steps": SV_EE_STEPS, "one_pass": SV_EE_ONE_PASS}


def spec_verify_early_exit(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                           gamma_per_row=None, *, gamma_max: int | None = None, cache_len=None,
                           mode: str = "sample", diag: bool = False, workspace: torch.Tensor | None = None,
                           out=None, plan: str = "auto", accept_hint: float | None = None):
    """spec_verify with early exit (nothing after a row's first rejection counts).
    gamma_max bounds gamma_i of a ragged batch (default: read from gamma_per_row, which
    synchronizes).  cache_len: int32 [B] device tensor of cached prefix lengths (None:
    0).  plan: "steps" (positions read left to right in doubling chunks by the rows
    still undecided), "one_pass" (one pass over every position) or "auto" (the one
    expected faster for the shape, given accept_hint, the expected per-draft acceptance
    rate; None for the library's default).  Every plan gives the same outputs.  Returns
    (n_accepted, emitted, crop_len) and, with diag=True, the diagnostics dict;
    crop_len[i] = cache_len[i] + n_accepted[i] + 1."""
    if plan not in EE_PLANS:
        raise ValueError(f"plan must be one of {sorted(EE_PLANS)}")
    return _verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, gamma_per_row,
                   mode=mode, diag=diag, workspace=workspace, out=out, early_exit=True,
                   gamma_max=gamma_max, cache_len=cache_len, ee_plan=EE_PLANS[plan],
                   accept_hint=-1.0 if accept_hint is None else float(accept_hint))


def early_exit_plan(batch: int, n_target_rows: int, vocab: int, dtype: int, mode: str, gamma_max: int,
                    accept_hint: float | None = None) -> str:
    """The plan spec_verify_early_exit(plan="auto") takes for a shape: "steps" or
    "one_pass" (host only)."""
    rc = int(lib.spec_verify_early_exit_plan(batch, n_target_rows, vocab, dtype,
                                             SV_SAMPLE if mode == "sample" else SV_GREEDY, gamma_max,
                                             -1.0 if accept_hint is None else float(accept_hint)))
    if rc < 0:
        raise SpecVerifyError(rc, strerror(rc))
    return {SV_EE_STEPS: "steps", SV_EE_ONE_PASS: "one_pass"}[rc]


def spec_verify_filtered(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                         gamma_per_row=None, *, top_k=None, top_p=None, diag: bool = False,
                         workspace: torch.Tensor | None = None, out=None):
    """spec_verify (sampling) with each row's top-k / top-p filter applied to both p and
    q.  top_k: int32 [B] device tensor or None; top_p: float32 [B] device tensor or
    None (one of the two is required)."""
    return _verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, gamma_per_row,
                   mode="sample", diag=diag, workspace=workspace, out=out, top_k=top_k, top_p=top_p,
                   filtered=True)


def _verify(target_logits, draft_logits, draft_tokens, uniforms, temperature, gamma_per_row=None, *,
            mode="sample", diag=False, workspace=None, out=None, early_exit=False, gamma_max=None,
            cache_len=None, top_k=None, top_p=None, filtered=False, ee_plan=0, accept_hint=-1.0):
    """Verify a batch of drafted rows on the GPU.

    target_logits  bf16/fp32 [n_target_rows, V] (packed) or [B, gamma+1, V] (dense)
    draft_logits   same dtype, [n_draft_rows, V] or [B, gamma, V]; may be None in greedy mode
    draft_tokens   int32 [n_draft_rows] (or [B, gamma])
    uniforms       float32 [n_target_rows] (or [B, gamma+1]); slot gamma_i of a row drives
                   the draw, the others the accept tests
    temperature    float32 [B] tensor, or a Python float for every row
    gamma_per_row  int32 [B] device tensor (ragged rows), an int (dense), or None (dense,
                   gamma read from a 3-D target tensor)
    mode           "sample" or "greedy"
    Returns (n_accepted int32 [B], emitted int32 [n_target_rows]) and, with diag=True,
    a third dict of p_x, q_x (float64 [n_draft_rows]), resid_mass (float64 [B]) and
    row_status (int32 [B]).  Asynchronous on torch's current stream.
    """
    device = target_logits.device
    if device.type != "cuda":
        raise ValueError("target_logits must be a GPU tensor")
    if target_logits.dtype == torch.bfloat16:
        dtype = SV_BF16
    elif target_logits.dtype == torch.float32:
        dtype = SV_F32
    else:
        raise ValueError(f"unsupported logits dtype {target_logits.dtype}")
    if mode not in ("sample", "greedy"):
        raise ValueError("mode must be 'sample' or 'greedy'")
    V = int(target_logits.shape[-1])
    n_target_rows = target_logits.numel() // V if V else 0

    gamma_t = None
    if isinstance(gamma_per_row, torch.Tensor):
        gamma_t = gamma_per_row
        B = int(gamma_t.numel())
        gamma_uniform = 0
    else:
        if gamma_per_row is None:
            if target_logits.dim() != 3:
                raise ValueError("pass gamma_per_row for a packed 2-D target tensor")
            B, gp1 = int(target_logits.shape[0]), int(target_logits.shape[1])
            gamma_uniform = gp1 - 1
        else:
            gamma_uniform = int(gamma_per_row)
            B = n_target_rows // (gamma_uniform + 1)
    if not isinstance(temperature, torch.Tensor):
        temperature = torch.full((B,), float(temperature), dtype=torch.float32, device=device)

    _check(target_logits, "target_logits", (target_logits.dtype,), device)
    _check(draft_logits, "draft_logits", (target_logits.dtype,), device)
    _check(draft_tokens, "draft_tokens", (torch.int32,), device)
    _check(uniforms, "uniforms", (torch.float32,), device)
    _check(temperature, "temperature", (torch.float32,), device)
    _check(gamma_t, "gamma_per_row", (torch.int32,), device)
    if temperature.numel() != B:
        raise ValueError("temperature must have one entry per row")
    if uniforms.numel() != n_target_rows:
        raise ValueError("uniforms must have one entry per target row")
    if draft_tokens is not None and draft_tokens.numel() != n_target_rows - B:
        raise ValueError("draft_tokens must have one entry per draft row")
    n_draft_rows = n_target_rows - B
    if draft_logits is not None:
        # the kernels read n_draft_rows rows of V logits from this pointer
        if draft_logits.dim() < 1 or int(draft_logits.shape[-1]) != V:
            raise ValueError(f"draft_logits has {int(draft_logits.shape[-1]) if draft_logits.dim() else 0} "
                             f"logits per row, the target {V}")
        if draft_logits.numel() != n_draft_rows * V:
            raise ValueError(f"draft_logits holds {draft_logits.numel() // max(V, 1)} rows, "
                             f"{n_draft_rows} draft rows expected")
    elif mode == "sample" and n_draft_rows > 0:
        raise ValueError("draft_logits is required in sampling mode when rows have drafts")
    if n_draft_rows > 0 and draft_tokens is None:
        raise ValueError("draft_tokens is required when rows have drafts")

    if out is None:
        n_acc = torch.empty(B, dtype=torch.int32, device=device)
        emitted = torch.empty(n_target_rows, dtype=torch.int32, device=device)
    else:
        n_acc, emitted = out
        _check(n_acc, "n_accepted", (torch.int32,), device)
        _check(emitted, "emitted", (torch.int32,), device)
    dg = None
    d = None
    if diag:
        n_draft = n_target_rows - B
        dg = dict(p_x=torch.empty(n_draft, dtype=torch.float64, device=device),
                  q_x=torch.empty(n_draft, dtype=torch.float64, device=device),
                  resid_mass=torch.empty(B, dtype=torch.float64, device=device),
                  row_status=torch.empty(B, dtype=torch.int32, device=device))
        d = Diag(dg["p_x"].data_ptr(), dg["q_x"].data_ptr(), dg["resid_mass"].data_ptr(),
                 dg["row_status"].data_ptr())

    stream = torch.cuda.current_stream(device).cuda_stream
    need = (early_exit_workspace_bytes if early_exit else
            filtered_workspace_bytes if filtered else workspace_bytes)(B, n_target_rows, V, dtype)
    if workspace is None:
        workspace = _workspace(device, stream, need)
    elif workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    md = SV_SAMPLE if mode == "sample" else SV_GREEDY
    dptr = ctypes.byref(d) if d is not None else None

    if filtered:
        _check(top_k, "top_k", (torch.int32,), device)
        _check(top_p, "top_p", (torch.float32,), device)
        for t, name in ((top_k, "top_k"), (top_p, "top_p")):
            if t is not None and t.numel() != B:
                raise ValueError(f"{name} must have one entry per row")
        rc = lib.spec_verify_filtered(_ptr(target_logits), _ptr(draft_logits), dtype, V, B, n_target_rows,
                                      _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), _ptr(gamma_t),
                                      gamma_uniform, _ptr(top_k), _ptr(top_p), _ptr(n_acc), _ptr(emitted), dptr,
                                      _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, strerror(rc))
        return (n_acc, emitted, dg) if diag else (n_acc, emitted)

    if not early_exit:
        rc = lib.spec_verify(_ptr(target_logits), _ptr(draft_logits), dtype, V, B, n_target_rows,
                             _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), _ptr(gamma_t),
                             gamma_uniform, md, _ptr(n_acc), _ptr(emitted), dptr,
                             _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
        if rc != SV_OK:
            raise SpecVerifyError(rc, strerror(rc))
        return (n_acc, emitted, dg) if diag else (n_acc, emitted)

    _check(cache_len, "cache_len", (torch.int32,), device)
    if cache_len is not None and cache_len.numel() != B:
        raise ValueError("cache_len must have one entry per row")
    if gamma_t is not None and gamma_max is None:
        gamma_max = int(gamma_t.max().item()) if B else 0
    crop = torch.empty(B, dtype=torch.int32, device=device)
    rc = lib.spec_verify_early_exit(_ptr(target_logits), _ptr(draft_logits), dtype, V, B, n_target_rows,
                                    _ptr(draft_tokens), _ptr(uniforms), _ptr(temperature), _ptr(gamma_t),
                                    gamma_uniform, int(gamma_max or 0), md, _ptr(cache_len), _ptr(n_acc),
                                    _ptr(emitted), _ptr(crop), dptr, ee_plan, accept_hint, _ptr(workspace),
                                    workspace.numel(), ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))
    return (n_acc, emitted, crop, dg) if diag else (n_acc, emitted, crop)


def spec_sample(logits, uniforms, temperature, *, status: bool = False,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """The drafter's draw on the GPU: one token per logit vector, x ~ softmax(z/T) by
    inverse CDF with that vector's uniform (first argmax where T <= 0).

    logits       bf16/fp32 [n, V] (or any shape [..., V]: every vector is one draw)
    uniforms     float32, one per vector
    temperature  float32 tensor with one entry per vector, or a Python float
    Returns int32 tokens [n] (-1 for an invalid vector) and, with status=True, also
    the int32 status bits per vector.  Asynchronous on torch's current stream.
    """
    device = logits.device
    if device.type != "cuda":
        raise ValueError("logits must be a GPU tensor")
    if logits.dtype == torch.bfloat16:
        dtype = SV_BF16
    elif logits.dtype == torch.float32:
        dtype = SV_F32
    else:
        raise ValueError(f"unsupported logits dtype {logits.dtype}")
    V = int(logits.shape[-1])
    n = logits.numel() // V if V else 0
    if not isinstance(temperature, torch.Tensor):
        temperature = torch.full((n,), float(temperature), dtype=torch.float32, device=device)
    _check(logits, "logits", (logits.dtype,), device)
    _check(uniforms, "uniforms", (torch.float32,), device)
    _check(temperature, "temperature", (torch.float32,), device)
    if uniforms.numel() != n or temperature.numel() != n:
        raise ValueError("one uniform and one temperature per vector")
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=device)
    else:
        _check(out, "out", (torch.int32,), device)
        if out.numel() != n:
            raise ValueError("out must hold one token per vector")
    st = torch.empty(n, dtype=torch.int32, device=device) if status else None
    stream = torch.cuda.current_stream(device).cuda_stream
    need = sample_workspace_bytes(n, V, dtype)
    if workspace is None:
        workspace = _workspace(device, stream, need)
    elif workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    rc = lib.spec_sample(_ptr(logits), dtype, V, n, _ptr(temperature), _ptr(uniforms), _ptr(out),
                         _ptr(st), _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))
    return (out, st) if status else out


def spec_tree_verify_greedy(target_logits, node_counts, tokens, parents, *, status: bool = False,
                            workspace: torch.Tensor | None = None, out=None):
    """Greedy verification of packed candidate trees on the GPU.

    target_logits  bf16/fp32 [n_nodes, V]: node k of tree i at row off_i + k
    node_counts    int32 [B] device tensor (each in [1, 2048])
    tokens         int32 [n_nodes]; parents int32 [n_nodes], tree-local, -1 for roots,
                   parents before children
    Returns (n_accepted [B], path [n_nodes], emitted [n_nodes]) and, with status=True,
    also the int32 status bits per tree.  Asynchronous on torch's current stream.
    """
    device = target_logits.device
    if device.type != "cuda":
        raise ValueError("target_logits must be a GPU tensor")
    if target_logits.dtype == torch.bfloat16:
        dtype = SV_BF16
    elif target_logits.dtype == torch.float32:
        dtype = SV_F32
    else:
        raise ValueError(f"unsupported logits dtype {target_logits.dtype}")
    V = int(target_logits.shape[-1])
    n = target_logits.numel() // V if V else 0
    for t, name in ((target_logits, "target_logits"), (node_counts, "node_counts"), (tokens, "tokens"),
                    (parents, "parents")):
        _check(t, name, (t.dtype,) if name == "target_logits" else (torch.int32,), device)
    if tokens.numel() != n or parents.numel() != n:
        raise ValueError("one token and one parent per node")
    B = int(node_counts.numel())
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=device), torch.empty(n, dtype=torch.int32, device=device),
               torch.empty(n, dtype=torch.int32, device=device))
    else:
        for t in out:
            _check(t, "out", (torch.int32,), device)
    n_acc, path, emitted = out
    st = torch.empty(B, dtype=torch.int32, device=device) if status else None
    stream = torch.cuda.current_stream(device).cuda_stream
    need = tree_workspace_bytes(n, V, dtype)
    if workspace is None:
        workspace = _workspace(device, stream, need)
    elif workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    rc = lib.spec_tree_verify_greedy(_ptr(target_logits), dtype, V, B, n, _ptr(node_counts), _ptr(tokens),
                                     _ptr(parents), _ptr(n_acc), _ptr(path), _ptr(emitted), _ptr(st),
                                     _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))
    return (n_acc, path, emitted, st) if status else (n_acc, path, emitted)


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, uniforms, temperature, gamma_per_row, *,
                        mode: str = "sample", out=None):
    """spec_verify through the entry point that allocates nothing on the device: the
    workspace is the library's fixed scratch array (NOALLOC_SCRATCH_BYTES per GPU).
    gamma_per_row is an int32 [B] device tensor or an int (dense); out, if given, is
    (n_accepted, emitted).  Calls that overlap on one GPU race on the scratch array."""
    device = target_logits.device
    dtype = SV_BF16 if target_logits.dtype == torch.bfloat16 else SV_F32
    if target_logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported logits dtype {target_logits.dtype}")
    V = int(target_logits.shape[-1])
    nT = target_logits.numel() // V
    gamma_t = gamma_per_row if isinstance(gamma_per_row, torch.Tensor) else None
    gu = 0 if gamma_t is not None else int(gamma_per_row)
    B = int(gamma_t.numel()) if gamma_t is not None else nT // (gu + 1)
    for t, name, dts in ((target_logits, "target_logits", (target_logits.dtype,)),
                         (draft_logits, "draft_logits", (target_logits.dtype,)),
                         (draft_tokens, "draft_tokens", (torch.int32,)), (uniforms, "uniforms", (torch.float32,)),
                         (temperature, "temperature", (torch.float32,)), (gamma_t, "gamma_per_row", (torch.int32,))):
        _check(t, name, dts, device)
    if draft_logits is not None and draft_logits.numel() != (nT - B) * V:
        raise ValueError("draft_logits must hold one row of V logits per draft row")
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=device), torch.empty(nT, dtype=torch.int32, device=device))
    n_acc, emitted = out
    md = SV_SAMPLE if mode == "sample" else SV_GREEDY
    stream = torch.cuda.current_stream(device).cuda_stream
    rc = lib.spec_verify_noalloc(_ptr(target_logits), _ptr(draft_logits), dtype, V, B, nT, _ptr(draft_tokens),
                                 _ptr(uniforms), _ptr(temperature), _ptr(gamma_t), gu, md, _ptr(n_acc),
                                 _ptr(emitted), None, ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, strerror(rc))
    return n_acc, emitted


spec_verify.__doc__ = _verify.__doc__
