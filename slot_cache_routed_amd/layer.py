"""Layer drivers over libscr: the demand (slot) path, the whole-layer stream
path and the staged prefill path.

PyTorch is used here only to own device / pinned memory and to name streams
and events; every step of the path is a libscr entry point (HIP kernels).  The drivers keep every intermediate buffer so tests can compare each
step with the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import _lib as L

_DEV = "cuda"


def _stream(s=None) -> int:
    s = s if s is not None else torch.cuda.current_stream()
    return s.cuda_stream


def record_timer(t: L.Timer, stream=None):
    """Records a library timing event on the stream (default: torch's current stream)."""
    t.record(_stream(stream))


def _i32(n, fill=None):
    t = torch.empty(max(int(n), 1), dtype=torch.int32, device=_DEV)
    if fill is not None:
        t.fill_(fill)
    return t


# ------------------------------------------------------------------ records

def record_layout(wdtype: int, H: int, I: int) -> L.RecordLayout:
    return L.record_layout_of(wdtype, H, I)


# Tile-major record layout (include/scr.h): a weight tensor [N rows][K cols] is
# stored as tile-blocks (t, kb) of 16 rows x 128 columns, t-major then kb, each
# in the order the GEMM's lanes load it.  These are byte permutations only.

def tile_bf16(w_bits: np.ndarray) -> np.ndarray:
    """bf16 [N][K] -> tile-blocks [t][kb][step s][group g][row r][8 elements], k = 128 kb + 32 s + 8 g + e."""
    N, K = w_bits.shape
    w = np.ascontiguousarray(w_bits, np.uint16).reshape(N // 16, 16, K // 128, 4, 4, 8)
    return np.ascontiguousarray(w.transpose(0, 2, 3, 4, 1, 5)).view(np.uint8).reshape(-1)


def tile_fp4_codes(q: np.ndarray) -> np.ndarray:
    """packed e2m1 [N][K/2] -> [t][kb][group g][row r][16 bytes], codes 128 kb + 32 g + j (byte j/2)."""
    N, Kh = q.shape
    w = np.ascontiguousarray(q, np.uint8).reshape(N // 16, 16, Kh // 64, 4, 16)
    return np.ascontiguousarray(w.transpose(0, 2, 3, 1, 4)).reshape(-1)


def tile_fp4_scales(sc: np.ndarray) -> np.ndarray:
    """e4m3 scales [N][K/16] -> [t][kb][group g][row r][2], scale 8 kb + 2 g + h."""
    N, Ks = sc.shape
    w = np.ascontiguousarray(sc, np.uint8).reshape(N // 16, 16, Ks // 8, 4, 2)
    return np.ascontiguousarray(w.transpose(0, 2, 3, 1, 4)).reshape(-1)


def tile_fp8(q: np.ndarray) -> np.ndarray:
    """fp8 codes [N][K] -> [t][kb][half h][group g][row r][16 bytes], column 128 kb + 32 g + 16 h + j."""
    N, K = q.shape
    w = np.ascontiguousarray(q, np.uint8).reshape(N // 16, 16, K // 128, 4, 2, 16)
    return np.ascontiguousarray(w.transpose(0, 2, 4, 3, 1, 5)).reshape(-1)


def tile_mx_scales(sc: np.ndarray) -> np.ndarray:
    """e8m0 scales [N][K/32] -> [t][kb][group g][row r], scale 4 kb + g."""
    N, Ks = sc.shape
    w = np.ascontiguousarray(sc, np.uint8).reshape(N // 16, 16, Ks // 4, 4)
    return np.ascontiguousarray(w.transpose(0, 2, 3, 1)).reshape(-1)


def pack_record_bf16(lay: L.RecordLayout, w13_bits: np.ndarray, w2_bits: np.ndarray) -> np.ndarray:
    """Lays out one bf16 expert record (uint8 [record_bytes])."""
    rec = np.zeros(lay.record_bytes, np.uint8)
    a = tile_bf16(w13_bits)
    b = tile_bf16(w2_bits)
    rec[lay.w13_off:lay.w13_off + a.size] = a
    rec[lay.w2_off:lay.w2_off + b.size] = b
    return rec


def pack_record_nvfp4(lay: L.RecordLayout, d: dict) -> np.ndarray:
    """Lays out one NVFP4 expert record from codes, scale codes and global scales."""
    rec = np.zeros(lay.record_bytes, np.uint8)
    for key, off, fn in (("w13_q", lay.w13_off, tile_fp4_codes), ("w13_s", lay.w13_scale_off, tile_fp4_scales),
                         ("w2_q", lay.w2_off, tile_fp4_codes), ("w2_s", lay.w2_scale_off, tile_fp4_scales)):
        a = fn(d[key])
        rec[off:off + a.size] = a
    rec[lay.g13_off:lay.g13_off + 4] = np.array([d["g13"]], np.float32).view(np.uint8)
    rec[lay.g2_off:lay.g2_off + 4] = np.array([d["g2"]], np.float32).view(np.uint8)
    return rec


def pack_record_fp8(lay: L.RecordLayout, d: dict) -> np.ndarray:
    """Lays out one FP8 expert record from e4m3 codes and per-tensor scales."""
    rec = np.zeros(lay.record_bytes, np.uint8)
    for key, off in (("w13_q", lay.w13_off), ("w2_q", lay.w2_off)):
        a = tile_fp8(d[key])
        rec[off:off + a.size] = a
    rec[lay.g13_off:lay.g13_off + 4] = np.array([d["g13"]], np.float32).view(np.uint8)
    rec[lay.g2_off:lay.g2_off + 4] = np.array([d["g2"]], np.float32).view(np.uint8)
    return rec


def pack_record_mxfp4(lay: L.RecordLayout, d: dict) -> np.ndarray:
    """Lays out one MXFP4 expert record from e2m1 codes and e8m0 block scales."""
    rec = np.zeros(lay.record_bytes, np.uint8)
    for key, off, fn in (("w13_q", lay.w13_off, tile_fp4_codes), ("w13_s", lay.w13_scale_off, tile_mx_scales),
                         ("w2_q", lay.w2_off, tile_fp4_codes), ("w2_s", lay.w2_scale_off, tile_mx_scales)):
        a = fn(d[key])
        rec[off:off + a.size] = a
    return rec


# --------------------------------------------------------------------- bank

class Bank:
    """Device state of a slot bank plus its record rows (all caller-owned torch memory)."""

    def __init__(self, S: int, n_layers: int, E: int, wdtype: int, record_bytes: int, policy: int = L.SCR_POLICY_LRU,
                 lrfu_decay: int = 0):
        """policy SCR_POLICY_LRFU takes lrfu_decay = floor(2^32 * 2^-lambda), 0 < it < 2^32."""
        self.S, self.L, self.E, self.wdtype, self.rec = S, n_layers, E, wdtype, int(record_bytes)
        self.policy, self.lrfu_decay = int(policy), int(lrfu_decay)
        self.slot_key = _i32(S, -1)
        self.slot_stamp = torch.zeros(S, dtype=torch.int64, device=_DEV)
        self.key_to_slot = _i32(n_layers * E, -1)
        self.clock = torch.zeros(1, dtype=torch.int64, device=_DEV)
        self.stats = torch.zeros(4, dtype=torch.int64, device=_DEV)
        self.decode_freq = torch.zeros(n_layers * E, dtype=torch.int32, device=_DEV)
        self.err = torch.zeros(1, dtype=torch.int32, device=_DEV)
        self.rows = torch.zeros(S * self.rec, dtype=torch.uint8, device=_DEV)
        self.row_table = torch.zeros(S, dtype=torch.int64, device=_DEV)
        self.slot_crf = torch.zeros(S, dtype=torch.int32, device=_DEV)
        self.chunk_start = torch.zeros(1, dtype=torch.int64, device=_DEV)
        self.desc = L.BankDesc(S, n_layers, E, wdtype, self.slot_key.data_ptr(), self.slot_stamp.data_ptr(),
                               self.key_to_slot.data_ptr(), self.clock.data_ptr(), self.stats.data_ptr(),
                               self.decode_freq.data_ptr(), self.err.data_ptr(), self.rows.data_ptr(), self.rec,
                               self.policy, self.lrfu_decay, self.slot_crf.data_ptr(), self.chunk_start.data_ptr())
        L.fill_row_table(self.rows, S, self.rec, self.row_table, _stream())

    def load_fill(self, fill, stream=None):
        """Sets slot_key / slot_stamp / clock from a host BankFill (scr_bank_init:
        statistics cleared, key_to_slot rebuilt; synchronises the stream)."""
        L.bank_init(self.desc, fill.slot_key, fill.slot_stamp, int(fill.clock), _stream(stream))

    def snapshot(self) -> dict:
        torch.cuda.synchronize()
        return {
            "slot_key": self.slot_key.cpu().numpy().copy(),
            "slot_stamp": self.slot_stamp.cpu().numpy().astype(np.uint64),
            "key_to_slot": self.key_to_slot.cpu().numpy().copy(),
            "clock": int(self.clock.item()),
            "stats": self.stats.cpu().numpy().astype(np.uint64),
            "decode_freq": self.decode_freq.cpu().numpy().astype(np.uint32),
            "err": int(self.err.item()),
            "slot_crf": self.slot_crf.cpu().numpy().view(np.uint32).copy(),
            "chunk_start": int(self.chunk_start.item()),
        }

    def slot_record(self, s: int) -> torch.Tensor:
        return self.rows[s * self.rec:(s + 1) * self.rec]


# ---------------------------------------------------------------- host pool

class HostPool:
    """Pinned host records for keys (layer, expert); keys may alias payloads."""

    def __init__(self, n_layers: int, E: int, record_bytes: int, n_payloads: int, payload_of=None):
        self.L, self.E, self.rec, self.n_payloads = n_layers, E, int(record_bytes), n_payloads
        self.records = torch.empty(n_payloads * self.rec, dtype=torch.uint8, pin_memory=True)
        host_base = self.records.data_ptr()
        dev_base = L.host_device_alias(host_base)
        keys = np.arange(n_layers * E, dtype=np.int64)
        pay = keys if payload_of is None else np.asarray([payload_of(int(q)) for q in keys], np.int64)
        assert pay.min() >= 0 and pay.max() < n_payloads
        self.payload = pay
        self.key_rows_host = (host_base + pay * self.rec).astype(np.uint64)
        self.key_rows_dev = torch.from_numpy((dev_base + pay * self.rec).astype(np.int64)).to(_DEV)
        self.desc = L.HostPoolDesc(n_layers, E, self.key_rows_dev.data_ptr(), self.key_rows_host.ctypes.data,
                                   self.rec)

    def write_payload(self, p: int, record: np.ndarray):
        self.records[p * self.rec:(p + 1) * self.rec].copy_(torch.from_numpy(record))

    def key_record(self, key: int) -> torch.Tensor:
        p = int(self.payload[key])
        return self.records[p * self.rec:(p + 1) * self.rec]


# ----------------------------------------------------------------- buffers

@dataclass
class LayerBuffers:
    """Per-call device buffers of one routed layer."""
    T: int
    E: int
    k: int
    H: int
    I: int
    num_buckets: int
    wdtype: int
    width: int = 128
    y_dtype: int = L.SCR_Y_F32
    t: dict = field(default_factory=dict)

    def __post_init__(self):
        R = self.T * self.k
        self.R = R
        self.cfg = L.tile_config(self.T, self.k, self.E, self.wdtype)
        B = self.cfg.block_m
        self.lmax = min(R, self.E)
        self.n_queries = max(1, math.ceil(self.lmax / self.width))
        cap = L.align_capacity(R, self.num_buckets, B)
        m = min(R, self.num_buckets)
        self.t = {
            "topk_ids": _i32(R), "topk_w": torch.empty(max(R, 1), dtype=torch.float32, device=_DEV),
            "distinct": _i32(self.lmax), "n_distinct": _i32(1), "inverse": _i32(R),
            "miss_slot": _i32(self.n_queries * self.width, -1), "miss_key": _i32(self.n_queries * self.width, -1),
            "n_miss": _i32(self.n_queries, 0), "n_total": _i32(1, 0),
            "sorted_routes": _i32(cap), "block_bucket": _i32(max(cap // B, 1)), "n_post_pad": _i32(1),
            "active_buckets": _i32(m), "active_block_begin": _i32(m + 1), "n_active": _i32(1),
            "align_ws": torch.empty(L.align_workspace(R, self.num_buckets), dtype=torch.uint8, device=_DEV),
            "moe_ws": torch.empty(L.moe_workspace(self.T, self.k, self.E, self.H, self.I, self.cfg),
                                  dtype=torch.uint8, device=_DEV),
            "a_scale": torch.zeros(2, dtype=torch.float32, device=_DEV),
            "y": torch.empty((self.T, self.H), dtype=torch.float32 if self.y_dtype == L.SCR_Y_F32 else torch.bfloat16,
                             device=_DEV),
        }
        self.cap = cap

    def __getitem__(self, k):
        return self.t[k]


def make_view(layer, E, k, H, I, wdtype, num_buckets, bucket_rows: torch.Tensor, input_scale: torch.Tensor,
              down_input_scale: torch.Tensor | None = None):
    """The routed layer's view: bucket rows plus the layer's per-expert input
    scales (gate/up input, and down input for the activation-quantising
    formats; by default the same array serves both)."""
    ds = input_scale if down_input_scale is None else down_input_scale
    return L.RoutedExperts(layer, E, k, H, I, wdtype, num_buckets, bucket_rows.data_ptr(), input_scale.data_ptr(),
                           ds.data_ptr())


# ------------------------------------------------------------------ steps

def route_dedup(buf: LayerBuffers, logits: torch.Tensor, stream=None):
    s = _stream(stream)
    L.route(logits, buf.T, buf.E, buf.k, buf["topk_ids"], buf["topk_w"], s)
    L.dedup(buf["topk_ids"], buf.R, buf.E, buf["distinct"], buf["n_distinct"], buf["inverse"], s)


def admit(buf: LayerBuffers, bank: Bank, pool: HostPool, layer: int, record_stats: bool, stream=None,
          batched: bool = False):
    """Hands the distinct list to the LRU one query at a time, copying each
    query's misses before the next query runs (same stream, no host sync).
    batched=True plans every query in one launch and copies all final misses
    in one launch (the same slot decisions and bank contents under LRU)."""
    s = _stream(stream)
    W = buf.width
    if batched:
        n = buf.lmax
        L.ensure_slots_batched(bank.desc, layer, buf["distinct"], n, W, record_stats, buf["miss_slot"],
                               buf["miss_key"], buf["n_miss"], buf["n_total"], s)
        L.copy_misses(bank.desc, pool.desc, buf["miss_slot"], buf["miss_key"], buf["n_total"], n, s)
        return
    for q in range(buf.n_queries):
        q0 = q * W
        w = min(W, buf.lmax - q0)
        if w <= 0:
            break
        ms = buf["miss_slot"][q * W:(q + 1) * W]
        mk = buf["miss_key"][q * W:(q + 1) * W]
        nm = buf["n_miss"][q:q + 1]
        L.ensure_slots(bank.desc, layer, buf["distinct"], q0, w, record_stats, ms, mk, nm, s)
        L.copy_misses(bank.desc, pool.desc, ms, mk, nm, w, s)


def plan(buf: LayerBuffers, bank: Bank, pool: HostPool, layer: int, record_stats: bool, stream=None) -> bool:
    """Dedup, all LRU queries and the align of one chunk in one launch, then one
    copy of the final misses.  Needs the routed ids in buf (route first).
    False (nothing enqueued) when the shape is beyond the one-workgroup planner."""
    s = _stream(stream)
    ok = L.plan_chunk(bank.desc, layer, buf["topk_ids"], buf.R, buf["distinct"], buf["n_distinct"], buf.width,
                      record_stats, buf["miss_slot"], buf["miss_key"], buf["n_miss"], buf["n_total"],
                      buf.cfg.block_m, buf["sorted_routes"], buf["block_bucket"], buf["n_post_pad"],
                      buf["active_buckets"], buf["active_block_begin"], buf["n_active"], s)
    if ok:
        L.copy_misses(bank.desc, pool.desc, buf["miss_slot"], buf["miss_key"], buf["n_total"], buf.lmax, s)
    return ok


def align(buf: LayerBuffers, id_to_bucket, num_ids, stream=None):
    s = _stream(stream)
    L.align_blocks(buf["topk_ids"], buf.R, id_to_bucket, num_ids, buf.num_buckets, buf.cfg.block_m,
                   buf["sorted_routes"], buf["block_bucket"], buf["n_post_pad"], buf["active_buckets"],
                   buf["active_block_begin"], buf["n_active"], buf["align_ws"], buf["align_ws"].numel(), s)


def forward(buf: LayerBuffers, view: L.RoutedExperts, x: torch.Tensor, stream=None, marks=None) -> L.TileCfg:
    s = _stream(stream)
    return L.grouped_moe_forward(view, x, buf.T, buf["topk_w"], buf["sorted_routes"], buf["active_buckets"],
                                 buf["active_block_begin"], buf["n_active"], buf["y"], buf.y_dtype,
                                 buf["moe_ws"], buf["moe_ws"].numel(), buf["a_scale"], s, marks=marks)


def demand_layer(bank: Bank, pool: HostPool, layer: int, logits, x, input_scale, width=128, record_stats=False,
                 y_dtype=L.SCR_Y_F32, buf: LayerBuffers | None = None, stream=None, shape=None, batched=False,
                 fused=False, down_input_scale=None):
    """Demand (slot) path of one layer: route, dedup, per-query ensure + miss copy,
    align over the bank's slots through key_to_slot, grouped GEMM at the slots.
    fused=True plans the chunk (dedup, queries, align) in one launch when it fits."""
    T, E = logits.shape
    k, H, I = shape
    if buf is None:
        buf = LayerBuffers(T, E, k, H, I, bank.S, bank.wdtype, width=width, y_dtype=y_dtype)
    s = _stream(stream)
    if fused:
        L.route(logits, buf.T, buf.E, buf.k, buf["topk_ids"], buf["topk_w"], s)
        if not plan(buf, bank, pool, layer, record_stats, stream):
            L.dedup(buf["topk_ids"], buf.R, buf.E, buf["distinct"], buf["n_distinct"], buf["inverse"], s)
            admit(buf, bank, pool, layer, record_stats, stream, batched=True)
            align(buf, bank.key_to_slot.data_ptr() + layer * E * 4, E, stream)
    else:
        route_dedup(buf, logits, stream)
        admit(buf, bank, pool, layer, record_stats, stream, batched=batched)
        align(buf, bank.key_to_slot.data_ptr() + layer * E * 4, E, stream)
    view = make_view(layer, E, k, H, I, bank.wdtype, bank.S, bank.row_table, input_scale, down_input_scale)
    buf.cfg_used = forward(buf, view, x, stream)
    return buf


class DecodeStepGraph:
    """One decode step (the demand path of every listed layer) captured once
    as a HIP graph and replayed.

    The demand path holds no host sync (miss counts are read and the misses
    copied on the device, grids are fixed by the layer's shape), so capture
    enqueues nothing and every replay runs route, planning, miss copies and
    the grouped GEMM of each layer against the bank's current state.  Inputs
    are read from static tensors (``logits[i]`` f32 [T, E] and ``x[i]`` bf16
    bits [T, H] of the i-th listed layer) that the caller fills before each
    replay; layer i writes ``bufs[i]["y"]``."""

    def __init__(self, bank: Bank, pool: HostPool, layers, T: int, E: int, shape, input_scale: torch.Tensor,
                 width: int = 128, record_stats: bool = True, y_dtype: int = L.SCR_Y_BF16, fused: bool = False):
        k, H, I = shape
        self.layers = list(layers)
        n = len(self.layers)
        self.logits = torch.zeros((n, T, E), dtype=torch.float32, device=_DEV)
        self.x = torch.zeros((n, T, H), dtype=torch.int16, device=_DEV)
        self.bufs = [LayerBuffers(T, E, k, H, I, bank.S, bank.wdtype, width=width, y_dtype=y_dtype)
                     for _ in self.layers]
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(self.graph, stream=side):
                for i, layer in enumerate(self.layers):
                    demand_layer(bank, pool, layer, self.logits[i], self.x[i], input_scale, width=width,
                                 record_stats=record_stats, buf=self.bufs[i], shape=shape, batched=True,
                                 fused=fused)
        torch.cuda.current_stream().wait_stream(side)

    def replay(self):
        """Runs the captured step on the current stream."""
        self.graph.replay()


class LayerStreamBuffer:
    """A device buffer holding every expert record of one layer, plus its row table."""

    def __init__(self, E: int, record_bytes: int):
        self.E, self.rec = E, int(record_bytes)
        self.data = torch.empty(E * self.rec, dtype=torch.uint8, device=_DEV)
        self.row_table = torch.zeros(E, dtype=torch.int64, device=_DEV)
        L.fill_row_table(self.data, E, self.rec, self.row_table, _stream())


def stream_layer(pool: HostPool, layer: int, logits, x, input_scale, layer_buf: LayerStreamBuffer, wdtype,
                 y_dtype=L.SCR_Y_F32, buf: LayerBuffers | None = None, stream=None, shape=None, copy=True,
                 down_input_scale=None):
    """Whole-layer path: copy every expert of the layer, align over its experts,
    same grouped GEMM."""
    T, E = logits.shape
    k, H, I = shape
    if buf is None:
        buf = LayerBuffers(T, E, k, H, I, E, wdtype, y_dtype=y_dtype)
    s = _stream(stream)
    L.route(logits, T, E, k, buf["topk_ids"], buf["topk_w"], s)
    if copy:
        L.stream_layer_async(pool.desc, layer, layer_buf.data, s)
    align(buf, None, 0, stream)
    view = make_view(layer, E, k, H, I, wdtype, E, layer_buf.row_table, input_scale, down_input_scale)
    buf.cfg_used = forward(buf, view, x, stream)
    return buf


# ------------------------------------------------------------- staging

class StagedPrefill:
    """Prefill staging over consecutive layers.

    Layers take turns between a pair of device buffers that can each hold
    one full layer (vLLM fork PR #51, Details: prefill staging).  One host
    read-back per step (scr_stage_plan) fetches which experts of each layer
    are absent from the bank and groups them into runs; layer i+1's runs are
    copied by a copy kernel on a side stream while layer i computes, ordered with events
    (the copy into a buffer waits for the layer that last read it).  Each
    layer then runs route, align over its experts and the grouped GEMM on a
    view whose rows point into the bank (resident) or the staging buffer.
    """

    def __init__(self, bank: Bank, pool: HostPool, max_runs: int | None = None):
        self.bank, self.pool = bank, pool
        E, rec = bank.E, bank.rec
        self.staging = [torch.empty(E * rec, dtype=torch.uint8, device=_DEV) for _ in range(2)]
        self.tables = [torch.zeros(E, dtype=torch.int64, device=_DEV) for _ in range(2)]
        self.side = torch.cuda.Stream()          # default priority
        self.max_runs = max_runs or bank.L * E
        self.runs = (L.Run * self.max_runs)()
        self.host_map = torch.empty(bank.L * E, dtype=torch.int32, pin_memory=True)
        self.n_runs = 0

    def plan(self, layer_begin: int, n_layers: int, stream=None) -> int:
        self.n_runs = L.stage_plan(self.bank.desc, self.pool.desc, layer_begin, n_layers, self.host_map,
                                   self.runs, self.max_runs, _stream(stream))
        return self.n_runs

    def staged_bytes(self, layer: int) -> int:
        return sum(r.count for r in self.runs[:self.n_runs] if r.layer == layer) * self.bank.rec

    def run(self, layers, logits, x, input_scale, bufs, timers=None, stream=None):
        """Runs the layers in order; logits[i] is layer i's [T, E] router input,
        bufs[i] its LayerBuffers.  timers (optional) maps layer index to a
        LayerTimers-like dict of 5 library timers passed as forward marks."""
        comp = stream if stream is not None else torch.cuda.current_stream()
        n = len(layers)
        staged = [torch.cuda.Event() for _ in range(n)]
        done = [torch.cuda.Event() for _ in range(n)]
        for e in staged + done:              # creates the events
            e.record(comp)
        E, k, H, I = self.bank.E, bufs[0].k, bufs[0].H, bufs[0].I
        side = self.side.cuda_stream

        def stage(i):
            wait = done[i - 2].cuda_event if i >= 2 else None
            L.stage_rows_async(self.pool.desc, self.runs, self.n_runs, layers[i], self.staging[i % 2], side,
                               wait, staged[i].cuda_event)

        stage(0)
        for i, layer in enumerate(layers):
            if i + 1 < n:
                stage(i + 1)
            comp.wait_event(staged[i])
            b = bufs[i]
            s = comp.cuda_stream
            L.route(logits[i], b.T, E, k, b["topk_ids"], b["topk_w"], s)
            L.align_blocks(b["topk_ids"], b.R, None, 0, E, b.cfg.block_m, b["sorted_routes"], b["block_bucket"],
                           b["n_post_pad"], b["active_buckets"], b["active_block_begin"], b["n_active"],
                           b["align_ws"], b["align_ws"].numel(), s)
            L.fill_staged_rows(self.bank.desc, layer, self.staging[i % 2], self.tables[i % 2], s)
            view = make_view(layer, E, k, H, I, self.bank.wdtype, E, self.tables[i % 2], input_scale)
            marks = None if timers is None else [t.handle for t in timers[i]]
            b.cfg_used = forward(b, view, x, stream=comp, marks=marks)
            done[i].record(comp)
        return bufs
