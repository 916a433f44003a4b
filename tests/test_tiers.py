"""Q2_0 row-tier selection (host only, nothing is launched).

Page "w4a16_gemv_tiers.rs": select_tier picks the narrowest present tier that
covers m and nothing for m = 0; "Kill switch": the presence of an environment
variable, read once per process, hides the exact-row tiers and leaves the base
tiers; "Why this module exists": a launch on a wider tier than m pays for rows
that are not there, hence the narrowest choice.  Here the base tiers are the
widths 1 and 8 and the exact-row tiers 2, 4 and 6.
"""
import itertools
import json
import os
import subprocess
import sys

import pytest

from weight_quantized_decode_block_amd import wqd

WIDTHS = wqd.Q2_0_TIER_WIDTHS
EXACT = {2, 4, 6}
ALL = (1 << len(WIDTHS)) - 1
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_widths_match_binding():
    text = open(wqd.HEADER).read()
    assert "#define WQD_Q2_0_TIER_WIDTHS {1u, 2u, 4u, 6u, 8u}" in text
    assert f"#define WQD_Q2_0_TIER_COUNT {len(WIDTHS)}" in text


@pytest.mark.parametrize("exact", [True, False])
def test_every_m_from_1_to_8_all_tiers_present(exact):
    got = [WIDTHS[wqd.q2_0_select_tier(m, ALL, exact)] for m in range(1, 9)]
    if exact:
        assert got == [1, 2, 4, 4, 6, 6, 8, 8]
    else:  # only the base tiers 1 and 8 remain
        assert got == [1, 8, 8, 8, 8, 8, 8, 8]


@pytest.mark.parametrize("exact", [True, False])
def test_m0_and_uncovered_m_select_nothing(exact):
    assert wqd.q2_0_select_tier(0, ALL, exact) is None
    assert wqd.q2_0_select_tier(9, ALL, exact) is None
    assert wqd.q2_0_select_tier(1, 0, exact) is None
    # without the 8-row tier nothing covers 7 rows
    assert wqd.q2_0_select_tier(7, ALL & ~(1 << 4), exact) is None


def test_narrowest_present_covering_over_every_mask():
    """For every subset of tiers, every m in 0..9 and both switch states: the
    choice covers m, is present and allowed, and no narrower present allowed
    tier covers m; nothing is chosen exactly when no such tier exists."""
    for mask, m, exact in itertools.product(range(1 << len(WIDTHS)), range(10), (True, False)):
        allowed = [i for i, w in enumerate(WIDTHS)
                   if (mask >> i) & 1 and (exact or w not in EXACT) and w >= m]
        got = wqd.q2_0_select_tier(m, mask, exact)
        if m == 0 or not allowed:
            assert got is None, (mask, m, exact)
            continue
        assert got is not None, (mask, m, exact)
        assert (mask >> got) & 1 and WIDTHS[got] >= m
        assert exact or WIDTHS[got] not in EXACT
        assert WIDTHS[got] == min(WIDTHS[i] for i in allowed)


def test_tier_width_in_this_process():
    enabled = wqd.q2_0_exact_m_tiers_enabled()
    assert enabled == ("WQD_NO_EXACT_M_TIERS" not in os.environ)
    assert wqd.q2_0_tier_width(0) == 0
    assert wqd.q2_0_tier_width(9) == 0
    for m in range(1, 9):
        assert wqd.q2_0_tier_width(m) == WIDTHS[wqd.q2_0_select_tier(m, ALL, enabled)]


_CHILD = r"""
import json, os, sys
sys.path.insert(0, sys.argv[1])
from weight_quantized_decode_block_amd import wqd
first = [wqd.q2_0_exact_m_tiers_enabled(), [wqd.q2_0_tier_width(m) for m in range(10)]]
# the switch is read once: changing the environment later changes nothing
if "WQD_NO_EXACT_M_TIERS" in os.environ:
    del os.environ["WQD_NO_EXACT_M_TIERS"]
else:
    os.environ["WQD_NO_EXACT_M_TIERS"] = "1"
second = [wqd.q2_0_exact_m_tiers_enabled(), [wqd.q2_0_tier_width(m) for m in range(10)]]
print(json.dumps([first, second]))
"""


@pytest.mark.parametrize("value", [None, "1", "0", ""])
def test_kill_switch_presence_checked_and_read_once(value):
    env = {k: v for k, v in os.environ.items() if k != "WQD_NO_EXACT_M_TIERS"}
    if value is not None:
        env["WQD_NO_EXACT_M_TIERS"] = value
    out = subprocess.run([sys.executable, "-c", _CHILD, ROOT], env=env, capture_output=True, text=True,
                         check=True, timeout=120)
    first, second = json.loads(out.stdout.strip().splitlines()[-1])
    assert first == second
    enabled, widths = first
    if value is None:
        assert enabled and widths == [0, 1, 2, 4, 4, 6, 6, 8, 8, 0]
    else:  # any value, "0" and the empty string included, switches the exact tiers off
        assert not enabled and widths == [0, 1, 8, 8, 8, 8, 8, 8, 8, 0]
