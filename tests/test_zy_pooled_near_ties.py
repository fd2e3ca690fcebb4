"""The session's pooled near-tie rate over every GPU parity test that ran
before this one (collected after them: pytest orders files by name).

Each parity test adds its decisions and counted near-ties (a mismatch at a
decision whose oracle margin is below 1e-5) to tests.parity.POOL; the pooled
fraction must stay below 1e-4."""
import pytest

from tests.parity import MAX_NEAR_TIE_FRACTION, POOL

pytestmark = pytest.mark.gpu


def test_pooled_near_tie_rate():
    if POOL["tests"] == 0:
        pytest.skip("no parity test ran in this session")
    rate = POOL["near_ties"] / max(POOL["decisions"], 1)
    print("pooled over %d parity tests: %d decisions, %d counted near-ties (rate %.2e), %d excluded"
          % (POOL["tests"], POOL["decisions"], POOL["near_ties"], rate, POOL["excluded"]), flush=True)
    for line in POOL["with_ties"]:
        print("  near-ties in: " + line, flush=True)
    assert rate < MAX_NEAR_TIE_FRACTION, "; ".join(POOL["with_ties"])
