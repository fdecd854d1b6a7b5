"""Session-wide mismatch rates of the GPU parity suite (collected last).

Every GPU-vs-oracle comparison adds its flagged-boundary mismatches and entry
counts to tests/parity.py TOTALS; the rule is that mismatches stay under 1e-6
of all compared entries."""

import pytest

import parity

pytestmark = pytest.mark.gpu


def test_session_mismatch_rates():
    t = parity.TOTALS
    if t["code_entries"] == 0:
        pytest.skip("no GPU parity comparisons ran in this session")
    print(t)
    assert t["code_mismatch"] < 1e-6 * t["code_entries"]
    assert t["sign_mismatch"] < 1e-6 * t["sign_entries"]
