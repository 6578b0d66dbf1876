"""Pins for the host dispatch predicates (CPU)."""
from conftest import read_golden
from oracle import demand_capacity_ok, prefill_on_demand


def test_threshold_cases_printed_on_the_page():
    for T, N, want in read_golden("dispatch_threshold.txt"):
        assert prefill_on_demand(int(T), int(N)) == bool(int(want)), (T, N)


def test_capacity_guard():
    # the capacity guard: the layer's distinct experts must fit in the slots
    assert demand_capacity_ok(96, 10, 512, 1100)
    assert not demand_capacity_ok(96, 10, 512, 400)
    assert demand_capacity_ok(4096, 10, 512, 512)
    # the stricter half-cache rule: 200 tokens x top-10 over 512 experts needs 512 slots
    assert demand_capacity_ok(200, 10, 512, 1100, half=True)       # 512 <= 550
    assert not demand_capacity_ok(200, 10, 512, 1000, half=True)   # 512 > 500
    assert demand_capacity_ok(40, 10, 512, 1000, half=True)        # 400 <= 500
