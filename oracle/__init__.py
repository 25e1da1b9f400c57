"""ctypes binding of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg of
the benchmark import this package; the product package never does.  It shares no
code with the HIP path: the only things both sides consume are the seeded inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

BF16, F32, F64 = 0, 1, 2
SAMPLE, GREEDY = 0, 1

BAD_TOKEN = 1
Q_ZERO = 2
NONFINITE = 4
BAD_GAMMA = 8
ZERO_RESID = 16
BAD_TEMP = 32
BAD_TREE = 64
INVALID_MASK = BAD_TOKEN | NONFINITE | BAD_GAMMA | BAD_TEMP | BAD_TREE
# per-decision flags (verify()["flags"])
FLAG_NEAR = 1     # the decision lies within flag_eps of its threshold
FLAG_FILTER = 2   # a top-p boundary within 1e-10 at this position

_DTYPES = {"bf16": BF16, "f32": F32, "f64": F64}


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, fp64, OpenMP over rows)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fPIC", "-shared",
           SRC_PATH, "-o", LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=_HERE)
    return LIB_PATH


_lib = None


def _load(path: str):
    L = ctypes.CDLL(path)
    vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    L.oracle_softmax.argtypes = [vp, ctypes.c_int, i64, dbl, vp]
    L.oracle_softmax.restype = ctypes.c_int
    L.oracle_argmax.argtypes = [vp, ctypes.c_int, i64]
    L.oracle_argmax.restype = i64
    L.oracle_position.argtypes = [vp, vp, ctypes.c_int, i64, dbl, vp, vp, vp, vp, vp]
    L.oracle_position.restype = ctypes.c_int
    L.oracle_inverse_cdf.argtypes = [vp, i64, dbl, dbl, vp, vp]
    L.oracle_inverse_cdf.restype = i64
    L.oracle_inverse_cdf_range.argtypes = [vp, i64, dbl, dbl, vp, vp, vp, vp]
    L.oracle_inverse_cdf_range.restype = i64
    L.oracle_verify.argtypes = [vp, vp, ctypes.c_int, i64, i32, i64, vp, vp, vp, vp,
                                ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, dbl, ctypes.c_int]
    L.oracle_verify.restype = ctypes.c_int
    L.oracle_verify_ex.argtypes = [vp, vp, ctypes.c_int, i64, i32, i64, vp, vp, vp, vp,
                                   ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, dbl, ctypes.c_int,
                                   ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
    L.oracle_verify_ex.restype = ctypes.c_int
    L.oracle_filter_threshold.argtypes = [vp, ctypes.c_int, i64, dbl, i64, dbl, dbl, vp, vp]
    L.oracle_filter_threshold.restype = ctypes.c_int
    L.oracle_sample.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, vp, vp, dbl, ctypes.c_int, vp, vp]
    L.oracle_sample.restype = ctypes.c_int
    L.oracle_tree_greedy.argtypes = [vp, ctypes.c_int, i64, i32, i64, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_int]
    L.oracle_tree_greedy.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        _lib = _load(LIB_PATH)
    return _lib


class using:
    """Context manager that points this binding at another build of oracle.c (used
    to check that planted mistakes in a copy of the oracle fail its pins)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _load(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(z, dtype):
    if dtype == "bf16":
        return np.ascontiguousarray(z, np.uint16)
    if dtype == "f32":
        return np.ascontiguousarray(z, np.float32)
    return np.ascontiguousarray(z, np.float64)


def softmax(z, T: float, dtype: str = "f64") -> np.ndarray:
    z = _logits(z, dtype)
    p = np.empty(z.shape[-1], np.float64)
    rc = lib().oracle_softmax(_ptr(z), _DTYPES[dtype], z.shape[-1], float(T), _ptr(p))
    if rc != 0:
        raise ValueError(f"oracle_softmax status {rc}")
    return p


def argmax(z, dtype: str = "f64") -> int:
    z = _logits(z, dtype)
    return int(lib().oracle_argmax(_ptr(z), _DTYPES[dtype], z.shape[-1]))


def position(zt, zd, T: float, dtype: str = "f64") -> dict:
    """p, q, alpha = sum min(p,q), residual mass and residual r at one position."""
    zt = _logits(zt, dtype)
    zd = _logits(zd, dtype)
    V = zt.shape[-1]
    p, q, r = (np.empty(V, np.float64) for _ in range(3))
    a = np.zeros(1, np.float64)
    w = np.zeros(1, np.float64)
    rc = lib().oracle_position(_ptr(zt), _ptr(zd), _DTYPES[dtype], V, float(T), _ptr(p), _ptr(q),
                               _ptr(a), _ptr(w), _ptr(r))
    if rc != 0:
        raise ValueError(f"oracle_position status {rc}")
    return dict(p=p, q=q, alpha=float(a[0]), resid_mass=float(w[0]), residual=r)


def inverse_cdf(w, u: float, eps: float = 1e-5):
    """(token, W, near_edge) of the inverse-CDF draw with weights w and uniform u."""
    w = np.ascontiguousarray(w, np.float64)
    W = np.zeros(1, np.float64)
    near = np.zeros(1, np.int32)
    tok = lib().oracle_inverse_cdf(_ptr(w), w.shape[0], float(u), float(eps), _ptr(W), _ptr(near))
    return int(tok), float(W[0]), bool(near[0])


def inverse_cdf_range(w, u: float, eps: float = 1e-5):
    """(token, W, near_edge, lo, hi): the draw, and the first and last tokens with
    weight whose CDF interval comes within eps * W of the threshold u * W (lo = hi =
    token when the draw is not near an edge)."""
    w = np.ascontiguousarray(w, np.float64)
    W = np.zeros(1, np.float64)
    near = np.zeros(1, np.int32)
    lo = np.zeros(1, np.int64)
    hi = np.zeros(1, np.int64)
    tok = lib().oracle_inverse_cdf_range(_ptr(w), w.shape[0], float(u), float(eps), _ptr(W), _ptr(near),
                                         _ptr(lo), _ptr(hi))
    return int(tok), float(W[0]), bool(near[0]), int(lo[0]), int(hi[0])


def verify(target, draft, dtype: str, vocab: int, gamma, draft_tokens, uniforms, temperature,
           mode: str = "sample", n_target_rows=None, threads: int = 0,
           flag_eps: float = 1e-5, early_exit: bool = False, cache_len=None, top_k=None,
           top_p=None) -> dict:
    """One verification round over a packed batch; returns numpy arrays.  flag_pos[i] is
    the first decision of row i within flag_eps of its threshold (accept test j, or
    gamma_i for the draw), -1 if none; flags[t_off[i] + j] has FLAG_NEAR for every
    such decision (test j < gamma_i, or the draw at j = gamma_i) and FLAG_FILTER where
    a top-p boundary lies within 1e-10; [draw_lo[i], draw_hi[i]] are the tokens a near
    draw could return (both equal the drawn token otherwise).  early_exit reads positions left to right and
    stops at the first rejection; crop_len[i] = cache_len[i] + K_i + 1 (-1 if invalid).
    top_k (int32 [B]) and top_p (float32 [B]) filter p and q of each sampling row
    (see filter_threshold)."""
    gamma = np.ascontiguousarray(gamma, np.int32)
    B = gamma.shape[0]
    target = _logits(target, dtype)
    draft = None if draft is None else _logits(draft, dtype)
    tokens = np.ascontiguousarray(draft_tokens, np.int32)
    uniforms = np.ascontiguousarray(uniforms, np.float32)
    temperature = np.ascontiguousarray(temperature, np.float32)
    if n_target_rows is None:
        n_target_rows = target.shape[0] if target.ndim == 2 else target.size // vocab
    n_draft = tokens.shape[0]
    out = dict(
        n_accepted=np.empty(B, np.int32),
        emitted=np.empty(n_target_rows, np.int32),
        p_x=np.empty(n_draft, np.float64),
        q_x=np.empty(n_draft, np.float64),
        resid_mass=np.empty(B, np.float64),
        row_status=np.empty(B, np.int32),
        flag_pos=np.empty(B, np.int32),
        flags=np.empty(n_target_rows, np.int32),
        draw_lo=np.empty(B, np.int32),
        draw_hi=np.empty(B, np.int32),
    )
    out["crop_len"] = np.empty(B, np.int32)
    cl = None if cache_len is None else np.ascontiguousarray(cache_len, np.int32)
    tk = None if top_k is None else np.ascontiguousarray(top_k, np.int32)
    tp = None if top_p is None else np.ascontiguousarray(top_p, np.float32)
    rc = lib().oracle_verify_ex(_ptr(target), _ptr(draft), _DTYPES[dtype], int(vocab), B,
                                int(n_target_rows), _ptr(tokens), _ptr(uniforms), _ptr(temperature),
                                _ptr(gamma), SAMPLE if mode == "sample" else GREEDY,
                                _ptr(out["n_accepted"]), _ptr(out["emitted"]), _ptr(out["p_x"]),
                                _ptr(out["q_x"]), _ptr(out["resid_mass"]), _ptr(out["row_status"]),
                                _ptr(out["flag_pos"]), float(flag_eps), int(threads), int(bool(early_exit)),
                                _ptr(cl), _ptr(out["crop_len"]), _ptr(tk), _ptr(tp), _ptr(out["flags"]),
                                _ptr(out["draw_lo"]), _ptr(out["draw_hi"]))
    if rc != 0:
        raise ValueError(f"oracle_verify status {rc}")
    return out


def filter_threshold(z, T: float, top_k: int = 0, top_p: float = 1.0, dtype: str = "f64",
                     eps: float = 1e-10):
    """(theta, near): tokens with logit >= theta survive top-k then top-p filtering."""
    z = _logits(z, dtype)
    th = np.zeros(1, np.float64)
    near = np.zeros(1, np.int32)
    rc = lib().oracle_filter_threshold(_ptr(z), _DTYPES[dtype], z.shape[-1], float(T), int(top_k),
                                       float(top_p), float(eps), _ptr(th), _ptr(near))
    if rc != 0:
        raise ValueError(f"oracle_filter_threshold status {rc}")
    return float(th[0]), bool(near[0])


def sample(logits, dtype: str, vocab: int, temperature, uniforms, threads: int = 0,
           flag_eps: float = 1e-5) -> dict:
    """The drafter's draw: one token per logit vector (x ~ softmax(z/T) by inverse CDF
    with that vector's uniform; argmax where T <= 0).  Returns tokens, status and
    flags (1 where the draw's threshold is within flag_eps * W of an interior edge),
    and lo / hi, the tokens such a draw could return (both = the token otherwise)."""
    z = _logits(logits, dtype)
    n = z.size // vocab
    temperature = np.ascontiguousarray(temperature, np.float32)
    uniforms = np.ascontiguousarray(uniforms, np.float32)
    if temperature.shape[0] != n or uniforms.shape[0] != n:
        raise ValueError("one temperature and one uniform per vector")
    out = dict(tokens=np.empty(n, np.int32), status=np.empty(n, np.int32),
               flags=np.empty(n, np.int32), lo=np.empty(n, np.int32), hi=np.empty(n, np.int32))
    rc = lib().oracle_sample(_ptr(z), _DTYPES[dtype], int(vocab), int(n), _ptr(temperature),
                             _ptr(uniforms), _ptr(out["tokens"]), _ptr(out["status"]),
                             _ptr(out["flags"]), float(flag_eps), int(threads), _ptr(out["lo"]),
                             _ptr(out["hi"]))
    if rc != 0:
        raise ValueError(f"oracle_sample status {rc}")
    return out


def tree_greedy(logits, dtype: str, vocab: int, counts, tokens, parents, threads: int = 0) -> dict:
    """Greedy verification of a batch of candidate trees (nodes packed tree after tree,
    parents tree-local and listed before their children).  Returns n_accepted [B],
    path, emitted [n_nodes] and status [B]."""
    z = _logits(logits, dtype)
    counts = np.ascontiguousarray(counts, np.int32)
    tokens = np.ascontiguousarray(tokens, np.int32)
    parents = np.ascontiguousarray(parents, np.int32)
    n = tokens.shape[0]
    if parents.shape[0] != n or z.size // vocab != n:
        raise ValueError("one token, one parent and one logit vector per node")
    B = counts.shape[0]
    out = dict(n_accepted=np.empty(B, np.int32), path=np.empty(n, np.int32),
               emitted=np.empty(n, np.int32), status=np.empty(B, np.int32))
    rc = lib().oracle_tree_greedy(_ptr(z), _DTYPES[dtype], int(vocab), B, n, _ptr(counts), _ptr(tokens),
                                  _ptr(parents), _ptr(out["n_accepted"]), _ptr(out["path"]),
                                  _ptr(out["emitted"]), _ptr(out["status"]), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_tree_greedy status {rc}")
    return out


def verify_workload(w, threads: int = 0, mode: str | None = None, flag_eps: float = 1e-5,
                    early_exit: bool = False, cache_len=None, top_k=None, top_p=None) -> dict:
    """verify() on any object with the packed-workload attributes."""
    return verify(w.target, w.draft, w.dtype, w.vocab, w.gamma, w.draft_tokens, w.uniforms,
                  w.temperature, mode=mode or w.mode, threads=threads, flag_eps=flag_eps,
                  early_exit=early_exit, cache_len=cache_len, top_k=top_k, top_p=top_p)
