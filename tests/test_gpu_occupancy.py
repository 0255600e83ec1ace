"""The planner's resident-slot counts against the device's occupancy calculator.

fg_plan_pass deals a plan's first launch rounds onto CUs assuming a number of
work-groups per CU for the attention kernel the plan launches (it depends on
the head dim, the block size and whether the plan has matrix-core items).
Only speed depends on it; these tests check it against what the HIP occupancy
calculator reports for the compiled kernels, for every supported pair."""
import pytest

from ragged_paged_attention_splitfuse_amd import binding
from ragged_paged_attention_splitfuse_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [(d, b, kind) for d in (64, 128) for b in (16, 32, 64) for kind in ("decodes", "tiles")]


def _spec(d, b, kind):
    if kind == "decodes":   # vector-ALU items only: the decode-only kernel
        return wl.custom_spec("dec", [1] * 40, [3000] * 40, 8, 8, d, b, seed=d + b)
    # a 300-token chunk beside decodes: matrix-core tiles in the launch
    return wl.custom_spec("tile", [1] * 8 + [300], [3000] * 8 + [500], 8, 8, d, b, seed=d + b + 1)


@pytest.mark.parametrize("d,b,kind", CASES, ids=[f"d{d}-b{b}-{k}" for d, b, k in CASES])
def test_planned_slots_match_the_occupancy_calculator(d, b, kind):
    plan = binding.Plan.from_spec(_spec(d, b, kind))
    assert (plan.info["num_mfma_items"] > 0) == (kind == "tiles")
    planned, device = plan.resident_slots()
    print(f"D {d} B {b} {kind}: planned {planned} device {device}", flush=True)
    assert device > 0
    assert planned == device
