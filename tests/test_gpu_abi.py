"""The C ABI with a device present: the argument checks of the CPU suite, run
where the library drives a device (nothing may be enqueued by a rejected call),
and scr_bank_init against a state written from the host."""
import numpy as np
import pytest
import torch

import test_abi as A

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import slot_cache_routed_amd._lib as L
    torch.cuda.init()
    return L.load()


@pytest.mark.parametrize("call", A.BAD_CALLS)
def test_bad_arguments_rejected_with_a_device_present(lib, call):
    A.test_bad_arguments_are_rejected_before_any_launch(lib, call)
    torch.cuda.synchronize()       # no launch was enqueued, so nothing can fault


def test_bank_and_view_validation_with_a_device_present(lib):
    A.test_bank_and_view_validation(lib)
    A.test_plan_chunk_validation(lib)
    torch.cuda.synchronize()


def test_bank_init_sets_the_state_and_rebuilds_the_map(lib):
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    S, NL, E = 24, 3, 8
    bank = LY.Bank(S, NL, E, L.SCR_W_BF16, 256)
    g = np.random.default_rng(11)
    keys = np.full(S, -1, np.int32)
    stamps = np.zeros(S, np.uint64)
    slots = g.choice(S, 15, replace=False)
    keys[slots] = g.choice(NL * E, 15, replace=False)
    stamps[slots] = g.permutation(np.arange(1, 16, dtype=np.uint64))
    # leftovers of an earlier use that bank_init must clear
    bank.stats.fill_(7)
    bank.decode_freq.fill_(3)
    bank.err.fill_(1)
    bank.key_to_slot.fill_(5)
    L.bank_init(bank.desc, keys, stamps, 20, torch.cuda.current_stream().cuda_stream)
    snap = bank.snapshot()
    assert np.array_equal(snap["slot_key"], keys)
    assert np.array_equal(snap["slot_stamp"], stamps)
    assert snap["clock"] == 20 and snap["err"] == 0
    assert not snap["stats"].any() and not snap["decode_freq"].any()
    want = np.full(NL * E, -1, np.int32)
    want[keys[slots]] = slots
    assert np.array_equal(snap["key_to_slot"], want)
    # a refused state leaves the bank as it was
    for k2, s2, c2 in A.BAD_BANK_STATES:
        kk = np.full(S, -1, np.int32)
        ss = np.zeros(S, np.uint64)
        kk[:4], ss[:4] = k2, s2
        if max(k2) >= 16:
            kk[1] = NL * E            # beyond this bank's L * E
        with pytest.raises(L.ScrError):
            L.bank_init(bank.desc, kk, ss, c2, torch.cuda.current_stream().cuda_stream)
    snap2 = bank.snapshot()
    assert np.array_equal(snap2["slot_key"], keys) and np.array_equal(snap2["key_to_slot"], want)
