"""The driver-facing smoke check (__graft_entry__.smoke) as a GPU test: one
tiny decode, unsplit and split, against the oracle, with the launch counters
it asserts -- so a plan change that breaks its expectations shows here."""
import pytest

import __graft_entry__

pytestmark = pytest.mark.gpu


def test_smoke(gpu):
    __graft_entry__.smoke()
