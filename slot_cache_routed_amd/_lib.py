"""ctypes binding of libscr.so: the C ABI declared in include/scr.h, one
Python function per entry point, argument marshalling only.

Pointers are passed as integers (``tensor.data_ptr()``), streams as the raw
``hipStream_t`` handle.  Every wrapper raises ``ScrError`` on a non-zero
return code with the library's own error text.  Loading fails loudly when
the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libscr.so")

SCR_OK, SCR_EINVAL, SCR_ENOTSUP, SCR_ECAPACITY, SCR_EHIP = 0, -1, -2, -3, -4
SCR_ERR_CAPACITY = 1
SCR_W_BF16, SCR_W_NVFP4, SCR_W_FP8, SCR_W_MXFP4, SCR_W_MXFP4_A8, SCR_W_NVFP4_A4 = 0, 1, 2, 3, 4, 5
SCR_Y_F32, SCR_Y_BF16 = 0, 1
SCR_POLICY_LRU, SCR_POLICY_LRFU = 0, 1
SCR_MAX_TOPK = 32
SCR_MAX_EXPERTS = 4096
SCR_MAX_QUERY_WIDTH = 1024
SCR_MAX_SLOTS = 262144
SCR_MAX_BUCKETS = 16384

EXPORTS = (
    "scr_record_layout_of", "scr_route", "scr_dedup", "scr_ensure_slots", "scr_ensure_slots_batched",
    "scr_copy_misses", "scr_plan_chunk",
    "scr_align_capacity", "scr_align_workspace", "scr_align_blocks", "scr_align_blocks_noalloc", "scr_tile_config",
    "scr_moe_workspace", "scr_grouped_moe_forward", "scr_quantize_fp8", "scr_quantize_nvfp4", "scr_stream_layer_async",
    "scr_stage_plan",
    "scr_stage_rows_async", "scr_stage_rows_dma_async", "scr_fill_row_table", "scr_fill_staged_rows", "scr_bank_rebuild_map",
    "scr_bank_init",
    "scr_host_device_alias", "scr_prefill_on_demand", "scr_demand_capacity_ok", "scr_timer_create",
    "scr_timer_record", "scr_timer_elapsed_ms", "scr_timer_destroy", "scr_last_error", "scr_version",
)


class ScrError(RuntimeError):
    def __init__(self, fn, code, text):
        super().__init__(f"{fn} returned {code}: {text}")
        self.code = code


class RecordLayout(C.Structure):
    _fields_ = [("w13_off", C.c_uint64), ("w13_scale_off", C.c_uint64), ("w2_off", C.c_uint64),
                ("w2_scale_off", C.c_uint64), ("g13_off", C.c_uint64), ("g2_off", C.c_uint64),
                ("record_bytes", C.c_uint64)]


class BankDesc(C.Structure):
    _fields_ = [("S", C.c_int32), ("L", C.c_int32), ("E", C.c_int32), ("wdtype", C.c_int32),
                ("slot_key", C.c_void_p), ("slot_stamp", C.c_void_p), ("key_to_slot", C.c_void_p),
                ("clock", C.c_void_p), ("stats", C.c_void_p), ("decode_freq", C.c_void_p),
                ("err", C.c_void_p), ("rows", C.c_void_p), ("record_bytes", C.c_uint64),
                ("policy", C.c_int32), ("lrfu_decay", C.c_uint32), ("slot_crf", C.c_void_p),
                ("chunk_start", C.c_void_p)]


class HostPoolDesc(C.Structure):
    _fields_ = [("L", C.c_int32), ("E", C.c_int32), ("key_rows_dev", C.c_void_p),
                ("key_rows_host", C.c_void_p), ("record_bytes", C.c_uint64)]


class RoutedExperts(C.Structure):
    _fields_ = [("layer", C.c_int32), ("num_experts", C.c_int32), ("k", C.c_int32), ("H", C.c_int32),
                ("I", C.c_int32), ("wdtype", C.c_int32), ("num_buckets", C.c_int32),
                ("bucket_rows", C.c_void_p), ("input_scale", C.c_void_p), ("down_input_scale", C.c_void_p)]


class TileCfg(C.Structure):
    _fields_ = [("block_m", C.c_int32), ("m_chunk", C.c_int32), ("n_tile_gu", C.c_int32),
                ("n_tile_dn", C.c_int32), ("wdtype", C.c_int32)]

    def as_tuple(self):
        return (self.block_m, self.m_chunk, self.n_tile_gu, self.n_tile_dn, self.wdtype)


class Run(C.Structure):
    _fields_ = [("layer", C.c_int32), ("e_begin", C.c_int32), ("count", C.c_int32)]


_P = C.c_void_p
_I = C.c_int
_SZ = C.c_size_t

_SIGS = {
    "scr_record_layout_of": (_I, [_I, _I, _I, C.POINTER(RecordLayout)]),
    "scr_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "scr_dedup": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "scr_ensure_slots": (_I, [C.POINTER(BankDesc), _I, _P, _I, _I, _I, _P, _P, _P, _P]),
    "scr_ensure_slots_batched": (_I, [C.POINTER(BankDesc), _I, _P, _I, _I, _I, _P, _P, _P, _P, _P]),
    "scr_copy_misses": (_I, [C.POINTER(BankDesc), C.POINTER(HostPoolDesc), _P, _P, _P, _I, _P]),
    "scr_plan_chunk": (_I, [C.POINTER(BankDesc), _I, _P, _I, _P, _P, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P,
                            _P, _P, _P]),
    "scr_align_capacity": (_SZ, [_I, _I, _I]),
    "scr_align_workspace": (_I, [_I, _I, C.POINTER(_SZ)]),
    "scr_align_blocks": (_I, [_P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "scr_align_blocks_noalloc": (_I, [_P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "scr_tile_config": (_I, [_I, _I, _I, _I, C.POINTER(TileCfg)]),
    "scr_moe_workspace": (_I, [_I, _I, _I, _I, _I, C.POINTER(TileCfg), C.POINTER(_SZ)]),
    "scr_grouped_moe_forward": (_I, [C.POINTER(RoutedExperts), _P, _I, _P, _P, _P, _P, _P, _P, _I, _P,
                                     _SZ, C.POINTER(TileCfg), _P, _P, _P]),
    "scr_quantize_fp8": (_I, [_P, C.c_longlong, _I, _P, _I, _P, _P]),
    "scr_quantize_nvfp4": (_I, [_P, C.c_longlong, _I, _P, _I, _P, _P, _P]),
    "scr_stream_layer_async": (_I, [C.POINTER(HostPoolDesc), _I, _P, _P]),
    "scr_stage_plan": (_I, [C.POINTER(BankDesc), C.POINTER(HostPoolDesc), _I, _I, _P, C.POINTER(Run), _I,
                            C.POINTER(_I), _P]),
    "scr_stage_rows_async": (_I, [C.POINTER(HostPoolDesc), C.POINTER(Run), _I, _I, _P, _P, _P, _P]),
    "scr_stage_rows_dma_async": (_I, [C.POINTER(HostPoolDesc), C.POINTER(Run), _I, _I, _P, _P, _P, _P]),
    "scr_fill_row_table": (_I, [_P, _I, C.c_uint64, _P, _P]),
    "scr_fill_staged_rows": (_I, [C.POINTER(BankDesc), _I, _P, _P, _P]),
    "scr_bank_rebuild_map": (_I, [C.POINTER(BankDesc), _P]),
    "scr_bank_init": (_I, [C.POINTER(BankDesc), _P, _P, C.c_uint64, _P]),
    "scr_host_device_alias": (_I, [_P, C.POINTER(_P)]),
    "scr_prefill_on_demand": (_I, [_I, _I]),
    "scr_demand_capacity_ok": (_I, [_I, _I, _I, _I, _I]),
    "scr_timer_create": (_I, [C.POINTER(_P)]),
    "scr_timer_record": (_I, [_P, _P]),
    "scr_timer_elapsed_ms": (_I, [_P, _P, C.POINTER(C.c_float)]),
    "scr_timer_destroy": (_I, [_P]),
    "scr_last_error": (C.c_char_p, []),
    "scr_version": (C.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Loads libscr.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m slot_cache_routed_amd.build`")
    lib = C.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != SCR_OK:
        raise ScrError(fn, rc, load().scr_last_error().decode())


def _p(x):
    """Pointer of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


# ------------------------------------------------------------------ wrappers

def record_layout_of(wdtype: int, H: int, I: int) -> RecordLayout:
    out = RecordLayout()
    _check("scr_record_layout_of", load().scr_record_layout_of(wdtype, H, I, C.byref(out)))
    return out


def route(logits, T, E, k, topk_ids, topk_w, stream):
    _check("scr_route", load().scr_route(_p(logits), T, E, k, _p(topk_ids), _p(topk_w), stream))


def dedup(ids, n, E, distinct, n_distinct, inverse, stream):
    _check("scr_dedup", load().scr_dedup(_p(ids), n, E, _p(distinct), _p(n_distinct), _p(inverse), stream))


def ensure_slots(bank: BankDesc, layer, distinct, q_begin, width, record_stats, miss_slot, miss_key, n_miss,
                 stream):
    _check("scr_ensure_slots", load().scr_ensure_slots(C.byref(bank), layer, _p(distinct), q_begin, width,
                                                       int(record_stats), _p(miss_slot), _p(miss_key),
                                                       _p(n_miss), stream))


def plan_chunk(bank: BankDesc, layer, ids, n, distinct, n_distinct, width, record_stats, miss_slot, miss_key,
               n_miss, n_total, block_size, sorted_routes, block_bucket, n_post_pad, active_buckets,
               active_block_begin, n_active, stream) -> bool:
    """True when planned; False when the shape is beyond one workgroup (SCR_ENOTSUP)."""
    rc = load().scr_plan_chunk(C.byref(bank), layer, _p(ids), n, _p(distinct), _p(n_distinct), width,
                               int(record_stats), _p(miss_slot), _p(miss_key), _p(n_miss), _p(n_total), block_size,
                               _p(sorted_routes), _p(block_bucket), _p(n_post_pad), _p(active_buckets),
                               _p(active_block_begin), _p(n_active), stream)
    if rc == SCR_ENOTSUP:
        return False
    _check("scr_plan_chunk", rc)
    return True


def ensure_slots_batched(bank: BankDesc, layer, distinct, n, width, record_stats, miss_slot, miss_key, n_miss,
                         n_total, stream):
    _check("scr_ensure_slots_batched", load().scr_ensure_slots_batched(
        C.byref(bank), layer, _p(distinct), n, width, int(record_stats), _p(miss_slot), _p(miss_key), _p(n_miss),
        _p(n_total), stream))


def copy_misses(bank: BankDesc, pool: HostPoolDesc, miss_slot, miss_key, n_miss, max_miss, stream):
    _check("scr_copy_misses", load().scr_copy_misses(C.byref(bank), C.byref(pool), _p(miss_slot), _p(miss_key),
                                                     _p(n_miss), max_miss, stream))


def align_capacity(n, num_buckets, block_size) -> int:
    return int(load().scr_align_capacity(n, num_buckets, block_size))


def align_workspace(n, num_buckets) -> int:
    out = C.c_size_t(0)
    _check("scr_align_workspace", load().scr_align_workspace(n, num_buckets, C.byref(out)))
    return int(out.value)


def align_blocks(ids, n, id_to_bucket, num_ids, num_buckets, block_size, sorted_routes, block_bucket, n_post_pad,
                 active_buckets, active_block_begin, n_active, ws, ws_bytes, stream):
    _check("scr_align_blocks", load().scr_align_blocks(
        _p(ids), n, _p(id_to_bucket), num_ids, num_buckets, block_size, _p(sorted_routes), _p(block_bucket),
        _p(n_post_pad), _p(active_buckets), _p(active_block_begin), _p(n_active), _p(ws), ws_bytes, stream))


def align_blocks_noalloc(ids, n, id_to_bucket, num_ids, num_buckets, block_size, sorted_routes, block_bucket,
                         n_post_pad, active_buckets, active_block_begin, n_active, stream):
    _check("scr_align_blocks_noalloc", load().scr_align_blocks_noalloc(
        _p(ids), n, _p(id_to_bucket), num_ids, num_buckets, block_size, _p(sorted_routes), _p(block_bucket),
        _p(n_post_pad), _p(active_buckets), _p(active_block_begin), _p(n_active), stream))


def tile_config(T, k, E_layer, wdtype) -> TileCfg:
    cfg = TileCfg()
    _check("scr_tile_config", load().scr_tile_config(T, k, E_layer, wdtype, C.byref(cfg)))
    return cfg


def moe_workspace(T, k, E_layer, H, I, cfg: TileCfg) -> int:
    out = C.c_size_t(0)
    _check("scr_moe_workspace", load().scr_moe_workspace(T, k, E_layer, H, I, C.byref(cfg), C.byref(out)))
    return int(out.value)


def grouped_moe_forward(view: RoutedExperts, x, T, topk_w, sorted_routes, active_buckets, active_block_begin,
                        n_active, y, y_dtype, ws, ws_bytes, a_scale_out, stream, marks=None) -> TileCfg:
    """marks: None or a sequence of 5 raw hipEvent_t handles (ints)."""
    cfg = TileCfg()
    ev = None
    if marks is not None:
        ev = (C.c_void_p * 5)(*[int(m) if m else None for m in marks])
    _check("scr_grouped_moe_forward", load().scr_grouped_moe_forward(
        C.byref(view), _p(x), T, _p(topk_w), _p(sorted_routes), _p(active_buckets), _p(active_block_begin),
        _p(n_active), _p(y), y_dtype, _p(ws), ws_bytes, C.byref(cfg), _p(a_scale_out),
        None if ev is None else C.cast(ev, C.c_void_p), stream))
    return cfg


def quantize_fp8(x, rows, cols, scales, n_scales, codes, stream):
    _check("scr_quantize_fp8", load().scr_quantize_fp8(_p(x), rows, cols, _p(scales), n_scales, _p(codes), stream))


def quantize_nvfp4(x, rows, cols, scales, n_scales, codes, block_scales, stream):
    _check("scr_quantize_nvfp4", load().scr_quantize_nvfp4(_p(x), rows, cols, _p(scales), n_scales, _p(codes),
                                                           _p(block_scales), stream))


def stream_layer_async(pool: HostPoolDesc, layer, dst, stream):
    _check("scr_stream_layer_async", load().scr_stream_layer_async(C.byref(pool), layer, _p(dst), stream))


def stage_plan(bank: BankDesc, pool: HostPoolDesc, layer_begin, n_layers, host_map, runs, max_runs, stream) -> int:
    n = C.c_int(0)
    _check("scr_stage_plan", load().scr_stage_plan(C.byref(bank), C.byref(pool), layer_begin, n_layers,
                                                   _p(host_map), runs, max_runs, C.byref(n), stream))
    return int(n.value)


def stage_rows_async(pool: HostPoolDesc, runs, n_runs, layer, dst, side_stream, wait_on, done):
    _check("scr_stage_rows_async", load().scr_stage_rows_async(C.byref(pool), runs, n_runs, layer, _p(dst),
                                                               side_stream, wait_on, done))


def stage_rows_dma_async(pool: HostPoolDesc, runs, n_runs, layer, dst, side_stream, wait_on, done):
    _check("scr_stage_rows_dma_async", load().scr_stage_rows_dma_async(C.byref(pool), runs, n_runs, layer, _p(dst),
                                                                       side_stream, wait_on, done))


def fill_row_table(base, n, stride, bucket_rows, stream):
    _check("scr_fill_row_table", load().scr_fill_row_table(_p(base), n, stride, _p(bucket_rows), stream))


def fill_staged_rows(bank: BankDesc, layer, staging, bucket_rows, stream):
    _check("scr_fill_staged_rows", load().scr_fill_staged_rows(C.byref(bank), layer, _p(staging),
                                                               _p(bucket_rows), stream))


def bank_rebuild_map(bank: BankDesc, stream):
    _check("scr_bank_rebuild_map", load().scr_bank_rebuild_map(C.byref(bank), stream))


def bank_init(bank: BankDesc, slot_keys, stamps, clock: int, stream):
    """slot_keys: host int32 [S], stamps: host uint64 [S] (numpy, C-contiguous)."""
    import numpy as np
    sk = np.ascontiguousarray(slot_keys, dtype=np.int32)
    st = np.ascontiguousarray(stamps, dtype=np.uint64)
    _check("scr_bank_init", load().scr_bank_init(C.byref(bank), sk.ctypes.data, st.ctypes.data, int(clock), stream))


def host_device_alias(host_ptr: int) -> int:
    out = C.c_void_p(0)
    _check("scr_host_device_alias", load().scr_host_device_alias(host_ptr, C.byref(out)))
    return int(out.value or 0)


def prefill_on_demand(T, threshold) -> bool:
    return bool(load().scr_prefill_on_demand(T, threshold))


def demand_capacity_ok(T, k, E, S, half=False) -> bool:
    return bool(load().scr_demand_capacity_ok(T, k, E, S, int(half)))


class Timer:
    """A timing event of the library (no system-scope fence); .handle is the hipEvent_t."""

    def __init__(self):
        h = C.c_void_p(0)
        _check("scr_timer_create", load().scr_timer_create(C.byref(h)))
        self.handle = int(h.value)

    def record(self, stream: int):
        _check("scr_timer_record", load().scr_timer_record(self.handle, stream))

    def elapsed_ms(self, stop: "Timer") -> float:
        ms = C.c_float(0.0)
        _check("scr_timer_elapsed_ms", load().scr_timer_elapsed_ms(self.handle, stop.handle, C.byref(ms)))
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle and _lib is not None:
                _lib.scr_timer_destroy(self.handle)
        except Exception:
            pass


def version() -> str:
    return load().scr_version().decode()
