"""The oracle on the toy workload: 10,000 independent rounds (B=1, gamma=4, V=32,
fp32, target ~ N(0,2), draft = target + N(0,0.5), T=1), checked statistically."""
import pytest

import oracle
import stats_checks
import workloads


@pytest.fixture(scope="module", params=[False, True], ids=["per_position", "shared_position"])
def toy(request):
    w = workloads.toy(seed=1 if not request.param else 2, shared_position=request.param)
    return w, oracle.verify_workload(w)


def test_toy_draft_tokens_follow_q(toy):
    stats_checks.check_draft_tokens(toy[0])


def test_toy_emitted_tokens_follow_p(toy):
    w, r = toy
    stats_checks.check_emitted_distribution(w, r["n_accepted"], r["emitted"])


def test_toy_accept_counts_and_expected_tokens(toy):
    w, r = toy
    stats_checks.check_accept_counts(w, r["n_accepted"])


def test_toy_no_invalid_rows(toy):
    w, r = toy
    assert (r["row_status"] & oracle.INVALID_MASK == 0).all()
