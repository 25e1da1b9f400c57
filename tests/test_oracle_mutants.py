"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is one plausible slip (a non-strict test, an inverted ratio, a wrong
residual sign, the wrong uniform for the draw, ...), applied textually to a
temporary copy of oracle.c and compiled on the CPU.  The committed oracle is never
modified.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

import oracle
import pins

MUTANTS = {
    "nonstrict_accept": ("if (!(u < ratio)) {", "if (!(u <= ratio)) {"),
    "inverted_ratio": ("ratio = px / qx;", "ratio = qx / px;"),
    "residual_sign": ("w[v] = fmax(0.0, P[v] - Q[v]);", "w[v] = fmax(0.0, Q[v] - P[v]);"),
    "bonus_wrong_position": (
        "softmax_kept(vector_ptr(target, dtype, t0 + K, V), dtype, V, T, THETA_T(K), P);",
        "softmax_kept(vector_ptr(target, dtype, t0 + (K == g && K > 0 ? K - 1 : K), V), dtype, V, T, THETA_T(K), P);"),
    "draw_reuses_test_uniform": ("(double)uniforms[t0 + g], eps, &W, &near, &lo, &hi)",
                                 "(double)uniforms[t0 + K], eps, &W, &near, &lo, &hi)"),
    "q_sum_without_temperature": ("vector_max_sumexp(zd, dtype, V, T, theta_d, &md, &Sd);",
                                  "vector_max_sumexp(zd, dtype, V, 1.0, theta_d, &md, &Sd);"),
    "sumexp_without_temperature": ("S += exp((kept_logit(z, dtype, v, theta) - m) / T);",
                                   "S += exp(kept_logit(z, dtype, v, theta) - m);"),
    "greedy_bonus_off_by_one": (
        "int64_t aK = oracle_argmax(vector_ptr(target, dtype, t0 + K, V), dtype, V);",
        "int64_t aK = oracle_argmax(vector_ptr(target, dtype, t0 + (K > 0 ? K - 1 : 0), V), dtype, V);"),
    "greedy_last_index_on_ties": ("        if (x > bv) {", "        if (x >= bv) {"),
    "cdf_nonstrict": ("        if (C > t) {", "        if (C >= t) {"),
    "draw_unnormalized": ("    double t = u * W;", "    double t = u;"),
    "alpha_with_max": ("a += fmin(pp[v], qq[v]);", "a += fmax(pp[v], qq[v]);"),
    "flag_threshold_too_wide": ("if (fabs(u - ratio) < eps) {", "if (fabs(u - ratio) < 100 * eps) {"),
    "no_zero_residual_fallback": ("                if (W == 0.0) {", "                if (W < 0.0) {"),
    "sample_without_temperature": ("oracle_softmax(z, dtype, V, T, w);", "oracle_softmax(z, dtype, V, 1.0, w);"),
    "sample_first_uniform": ("oracle_inverse_cdf_range(w, V, (double)uniforms[i], eps, NULL, &near, &a, &b);",
                             "oracle_inverse_cdf_range(w, V, (double)uniforms[0], eps, NULL, &near, &a, &b);"),
    "sample_greedy_below_one": ("                if (T <= 0) {", "                if (T < 1) {"),
    "tree_own_prediction": ("(int64_t)tokens[o + k] == pred[par]", "(int64_t)tokens[o + k] == pred[k]"),
    "tree_last_longest": ("                if (len[k] > len[best])", "                if (len[k] >= len[best])"),
    "tree_ignores_parent": ("len[k] = (len[par] > 0 && ", "len[k] = (len[par] >= 0 && "),
    "early_exit_keeps_reading": ("                if (early_exit && decided)\n                    break;",
                                 "                if (early_exit && decided && 0)\n                    break;"),
    "crop_without_last_token": ("    return n + K + 1;", "    return n + K;"),
    "top_k_off_by_one": ("double theta = use_k ? s[top_k - 1] : -INFINITY;",
                         "double theta = use_k ? s[top_k] : -INFINITY;"),
    "top_p_before_top_k": ("for (int64_t i = 0; i < V && s[i] >= theta; ++i)\n            S += exp",
                           "for (int64_t i = 0; i < V; ++i)\n            S += exp"),
    "top_p_overshoots": ("            if (cum >= target) {", "            if (cum > target * 1.05) {"),
    "filter_only_target": ("                        oracle_filter_threshold(vector_ptr(draft, dtype, d0 + j, V), dtype, V, T, row_k,",
                           "                        oracle_filter_threshold(vector_ptr(draft, dtype, d0 + j, V), dtype, V, T, 0 * row_k,"),
    "flags_only_first_near": ("                        if (flags)\n                            flags[t0 + j] |= ORACLE_FLAG_NEAR;",
                              "                        if (flags && flag == j)\n                            flags[t0 + j] |= ORACLE_FLAG_NEAR;"),
    "draw_range_drops_lower": ("if (w[v] > 0 && c >= t - eps * W && before <= t + eps * W) {",
                               "if (w[v] > 0 && c > t && before <= t + eps * W) {"),
    "neg_inf_is_nonfinite": ("if (isnan(x) || x == INFINITY)", "if (isnan(x) || isinf(x))"),
}


# Each mutant is compiled and run against the pins in a worker process of its own (one
# OpenMP thread each), all of them at once, so the suite's wall time stays a few
# minutes; a worker prints the name of the first pin that fails, or nothing.
_WORKER = """
import sys
sys.path[:0] = [sys.argv[2], sys.argv[3]]
import oracle, pins
with oracle.using(sys.argv[1]):
    for pin in pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            print(pin.__name__)
            break
"""


def _run_mutant(name, root):
    old, new = MUTANTS[name]
    src = open(oracle.SRC_PATH).read()
    if src.count(old) != 1:
        return f"!site: mutation site for {name} not unique/found"
    d = root / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(oracle.SRC_PATH), "oracle.h"), d / "oracle.h")
    (d / "oracle.c").write_text(src.replace(old, new))
    so = str(d / "liboracle.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(d / "oracle.c"),
                    "-o", so, "-lm"], check=True)
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _WORKER, so, os.path.dirname(here), here], env=env,
                       capture_output=True, text=True, timeout=1200)
    if r.returncode != 0:
        return f"!worker: {r.stderr[-2000:]}"
    return r.stdout.strip()


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    root = tmp_path_factory.mktemp("oracle_mutants")
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = {name: ex.submit(_run_mutant, name, root) for name in MUTANTS}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_results):
    caught = mutant_results[name]
    assert not caught.startswith("!"), caught
    assert caught, f"mutant {name} passes every pin"
