"""The step kernels' occupancy caps, measured: the LDS each launch reserves
(plus the kernel's static LDS) lets exactly the intended number of its
workgroups share a compute unit.  lema_probe_residency runs workgroups of
the same size with the same LDS and counts how many are resident on one CU
at once; LDS is handed out in whole granules, so a reservation computed
without the granule or the static LDS would fit one workgroup fewer."""
from __future__ import annotations

import pytest

import optimizer_step_lema_amd as L

pytestmark = pytest.mark.gpu

KERNELS = {0: "fp32 step", 1: "fp32 step, 8 resident micro-batches", 2: "int8 step",
           3: "fp32 step, launches under 2^18 tiles"}
INTENDED = {0: 12, 1: 9, 2: 3, 3: 16}


@pytest.mark.parametrize("kernel", sorted(KERNELS))
def test_reservation_gives_intended_count(kernel):
    plan = L.step_occupancy(kernel)
    print(KERNELS[kernel], plan, flush=True)
    lds = plan["static_lds"] + plan["reserved_lds"]
    assert lds % plan["lds_granule"] == 0          # whole granules: nothing rounds up
    got = L.probe_residency(plan["lanes"], lds)
    assert got["cus_seen"] == L.device_info()["compute_units"]
    assert plan["intended_per_cu"] == INTENDED[kernel]
    assert got["max_per_cu"] == got["min_per_cu"] == plan["intended_per_cu"]
    # registers alone would allow at least as many
    assert plan["per_cu_by_registers"] >= plan["intended_per_cu"]


def test_granule_measured():
    """LDS is handed out in granules of lds_granule bytes: one byte beyond a
    whole number of granules costs a whole granule."""
    g = L.step_occupancy(0)["lds_granule"]
    per_cu = L.device_info()["lds_per_cu"] // g      # granules per CU
    for k in (8, 10, 13):
        assert L.probe_residency(64, k * g)["max_per_cu"] == min(32, per_cu // k)
        assert L.probe_residency(64, k * g + 4)["max_per_cu"] == min(32, per_cu // (k + 1))
