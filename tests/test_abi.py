"""The C ABI: the library loads, exports every declared entry point, and
rejects bad arguments before touching the device (CPU only)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

L = pytest.importorskip("slot_cache_routed_amd._lib")


def _declared():
    src = open(os.path.join(ROOT, "include", "scr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(scr_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libscr.so not built")
    return L.load()


def test_every_declared_entry_point_is_exported(lib):
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_version_and_host_helpers(lib):
    assert "gfx950" in L.version()
    assert L.prefill_on_demand(96, 96) and not L.prefill_on_demand(97, 96)
    assert not L.prefill_on_demand(1, 0) and L.prefill_on_demand(2, 2)
    assert L.demand_capacity_ok(96, 10, 512, 1100) and not L.demand_capacity_ok(96, 10, 512, 100)


def test_tile_config_depends_on_the_layer_only(lib):
    a = L.tile_config(600, 2, 8, L.SCR_W_BF16).as_tuple()
    assert a == L.tile_config(600, 2, 8, L.SCR_W_BF16).as_tuple()
    assert L.tile_config(96, 10, 512, L.SCR_W_BF16).m_chunk == 32      # ~2 rows per expert
    assert L.tile_config(4096, 10, 512, L.SCR_W_NVFP4).m_chunk == 112  # ~80 rows per expert


def test_record_layouts(lib):
    b = L.record_layout_of(L.SCR_W_BF16, 2048, 512)
    assert b.record_bytes == 6291456 and b.w2_off == 4194304
    f = L.record_layout_of(L.SCR_W_NVFP4, 2048, 512)
    assert f.w13_scale_off == 1 << 20 and f.w2_off == (1 << 20) + (128 << 10)
    assert f.g13_off == 1769472 and f.record_bytes % 256 == 0 and f.record_bytes >= 1769472 + 8
    p = L.record_layout_of(L.SCR_W_FP8, 2048, 512)
    assert p.w2_off == 2 << 20 and p.g13_off == 3 << 20 and p.record_bytes == (3 << 20) + 256
    m = L.record_layout_of(L.SCR_W_MXFP4, 2048, 512)
    assert m.w13_scale_off == 1 << 20 and m.w2_off == (1 << 20) + (64 << 10)
    assert m.w2_scale_off == m.w2_off + (512 << 10) and m.record_bytes == m.w2_scale_off + (32 << 10)


def _ws_bytes(T, k, E, H, I, B, wd, f32_rows):
    """The forward's workspace as include/scr.h lays it out, each part 256-byte
    aligned: h (A8: x's and h's codes), the per-route rows (fp32, or fp16 with
    one exponent byte per 32 columns), the flags, the two scales, and NVFP4's
    fp16 copy of x with its row exponents."""
    al = lambda v: (v + 255) // 256 * 256
    R = T * k
    rows = (R + min(R, E) * (B - 1) + B - 1) // B * B
    end = al(T * H) + rows * I if wd == L.SCR_W_MXFP4_A8 else rows * I * 2
    o_end = al(end) + R * H * (4 if f32_rows else 2)
    oe_end = al(o_end) + (0 if f32_rows else R * (H // 32))
    total = al(al(al(oe_end) + R * 4) + 8)
    if wd in (L.SCR_W_NVFP4, L.SCR_W_NVFP4_A4):
        total = al(al(total + T * H * 2) + T * 4)
    return total


@pytest.mark.parametrize("T,k,E,H,I,wd,f32_rows", [
    (96, 10, 512, 2048, 512, "SCR_W_BF16", True),     # few rows per expert: fp32 rows for bf16
    (4096, 10, 512, 2048, 512, "SCR_W_BF16", False),  # the long-chunk kernels: fp16 rows
    (4096, 10, 512, 384, 512, "SCR_W_BF16", True),    # a hidden size those kernels do not take
    (96, 10, 512, 2048, 512, "SCR_W_NVFP4", False),
    (4096, 10, 512, 2048, 512, "SCR_W_NVFP4", False),
    (4096, 10, 512, 2048, 512, "SCR_W_MXFP4_A8", False),
    (4096, 10, 512, 2048, 512, "SCR_W_NVFP4_A4", False),
    (0, 2, 8, 256, 128, "SCR_W_FP8", False),
])
def test_moe_workspace_follows_its_documented_layout(lib, T, k, E, H, I, wd, f32_rows):
    code = getattr(L, wd)
    cfg = L.tile_config(T, k, E, code)
    assert L.moe_workspace(T, k, E, H, I, cfg) == _ws_bytes(T, k, E, H, I, cfg.block_m, code, f32_rows)


def test_align_capacity_formula(lib):
    assert L.align_capacity(960, 1100, 16) == 960 + 960 * 15
    assert L.align_capacity(40960, 512, 16) == 40960 + 512 * 15
    assert L.align_capacity(0, 8, 16) == 0
    assert L.align_workspace(40960, 512) > 0


BAD_CALLS = [
    lambda: L.route(0, 4, 8, 0, 0, 0, None),                 # k = 0
    lambda: L.route(0, 4, 8, 9, 0, 0, None),                 # k > E
    lambda: L.route(0, 4, 5000, 2, 0, 0, None),              # E too large
    lambda: L.route(0, 4, 64, 33, 0, 0, None),               # k > 32
    lambda: L.route(None, 4, 8, 2, None, None, None),        # null pointers
    lambda: L.dedup(None, 10, 0, None, None, None, None),    # E = 0
    lambda: L.align_blocks(0, 10, None, 0, 0, 16, 1, 1, 1, 1, 1, 1, 1, 1 << 20, None),   # 0 buckets
    lambda: L.align_blocks(0, 10, None, 0, 8, 24, 1, 1, 1, 1, 1, 1, 1, 1 << 20, None),   # block 24
    lambda: L.align_blocks(1, 10, None, 0, 20000, 16, 1, 1, 1, 1, 1, 1, 1, 1 << 30, None),  # > max buckets
    lambda: L.align_blocks(1, 10, None, 0, 8, 16, 1, 1, 1, 1, 1, 1, 1, 4, None),         # tiny workspace
    lambda: L.tile_config(1, 0, 8, 0),
    lambda: L.tile_config(1, 1, 8, 7),
    lambda: L.tile_config(1, 1, 8, 9),                        # no format 9
]


@pytest.mark.parametrize("call", BAD_CALLS)
def test_bad_arguments_are_rejected_before_any_launch(lib, call):
    with pytest.raises(L.ScrError) as ei:
        call()
    assert ei.value.code in (L.SCR_EINVAL, L.SCR_ENOTSUP)


def test_bank_and_view_validation(lib):
    bank = L.BankDesc(0, 1, 8, 0, 1, 1, 1, 1, 1, 1, 1, 1, 16)        # S = 0
    with pytest.raises(L.ScrError):
        L.ensure_slots(bank, 0, 1, 0, 4, 0, 1, 1, 1, None)
    bank = L.BankDesc(16, 2, 8, 0, 1, 1, 1, 1, 1, 1, 1, 1, 16)
    with pytest.raises(L.ScrError):
        L.ensure_slots(bank, 2, 1, 0, 4, 0, 1, 1, 1, None)          # layer out of range
    with pytest.raises(L.ScrError):
        L.ensure_slots(bank, 0, 1, 0, 2000, 0, 1, 1, 1, None)       # width too large
    pool = L.HostPoolDesc(2, 8, 1, 1, 32)
    with pytest.raises(L.ScrError):
        L.copy_misses(bank, pool, 1, 1, 1, 4, None)                 # record sizes differ
    view = L.RoutedExperts(0, 8, 2, 192, 512, 0, 8, 1, 1)            # H not a multiple of 128
    with pytest.raises(L.ScrError):
        L.grouped_moe_forward(view, 1, 4, 1, 1, 1, 1, 1, 1, 0, 1, 1 << 30, None, None)
    view = L.RoutedExperts(0, 8, 2, 256, 128, 0, 8, 1, 1)
    with pytest.raises(L.ScrError):                                  # workspace too small
        L.grouped_moe_forward(view, 1, 4, 1, 1, 1, 1, 1, 1, 0, 1, 16, None, None)


def test_plan_chunk_validation(lib):
    bank = L.BankDesc(16, 2, 8, 0, 1, 1, 1, 1, 1, 1, 1, 1, 16)
    args = dict(ids=1, n=10, distinct=1, n_distinct=1, width=4, record_stats=0, miss_slot=1, miss_key=1,
                n_miss=1, n_total=1, block_size=16, sorted_routes=1, block_bucket=1, n_post_pad=1,
                active_buckets=1, active_block_begin=1, n_active=1, stream=None)

    def call(b, layer, **kw):
        a = dict(args, **kw)
        return L.plan_chunk(b, layer, a["ids"], a["n"], a["distinct"], a["n_distinct"], a["width"],
                            a["record_stats"], a["miss_slot"], a["miss_key"], a["n_miss"], a["n_total"],
                            a["block_size"], a["sorted_routes"], a["block_bucket"], a["n_post_pad"],
                            a["active_buckets"], a["active_block_begin"], a["n_active"], a["stream"])
    for kw in (dict(width=0), dict(width=2000), dict(n=0), dict(block_size=24), dict(ids=None)):
        with pytest.raises(L.ScrError):
            call(bank, 0, **kw)
    with pytest.raises(L.ScrError):
        call(bank, 2)                                                  # layer out of range
    # beyond one workgroup: reported as unsupported before any launch
    assert call(bank, 0, n=5000) is False
    big = L.BankDesc(9000, 2, 8, 0, 1, 1, 1, 1, 1, 1, 1, 1, 16)
    assert call(big, 0) is False


# bank states scr_bank_init must refuse (checked on the host, nothing enqueued):
# (slot keys, stamps, clock) of a bank with S = 4 slots, L = 2 layers, E = 8
BAD_BANK_STATES = [
    ([3, 3, -1, -1], [1, 2, 0, 0], 2),      # one key in two slots
    ([3, 16, -1, -1], [1, 2, 0, 0], 2),     # key beyond L * E
    ([3, -2, -1, -1], [1, 0, 0, 0], 2),     # key below -1
    ([3, 4, -1, -1], [1, 5, 0, 0], 4),      # a stamp after the clock
    ([3, 4, -1, -1], [1, 2, 7, 0], 9),      # an empty slot with a stamp
]


@pytest.mark.parametrize("keys,stamps,clock", BAD_BANK_STATES)
def test_bank_init_rejects_inconsistent_states(lib, keys, stamps, clock):
    bank = L.BankDesc(4, 2, 8, 0, 1, 1, 1, 1, 1, 1, 1, 1, 16)
    with pytest.raises(L.ScrError) as ei:
        L.bank_init(bank, keys, stamps, clock, None)
    assert ei.value.code == L.SCR_EINVAL
