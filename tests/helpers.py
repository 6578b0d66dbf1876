"""Shared set-up for the GPU tests: synthetic pools and banks from the seeded
generators, and the oracle's view of the same inputs (taken from the
generators, never from device buffers)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import workloads as W
from oracle.mlp import bf16_bits_to_f64
from oracle.nvfp4 import dequant_nvfp4
from oracle.lowbit import dequant_fp8, dequant_mxfp4

N_THREADS = min(16, os.cpu_count() or 4)


def flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_of_f32(a):
    return W.f32_to_bf16_bits(a)


class ExpertSource:
    """Generator-side expert weights of one workload, by payload id."""

    def __init__(self, seed, H, I, wdtype):
        # the activation-quantising formats read the records of their weight format
        wdtype = {"mxfp4_a8": "mxfp4", "nvfp4_a4": "nvfp4"}.get(wdtype, wdtype)
        self.seed, self.H, self.I, self.wdtype = seed, H, I, wdtype
        self._cache = {}

    def raw(self, payload):
        if self.wdtype == "nvfp4":
            return W.expert_nvfp4(self.seed, payload, self.H, self.I)
        if self.wdtype == "fp8":
            return W.expert_fp8(self.seed, payload, self.H, self.I)
        if self.wdtype == "mxfp4":
            return W.expert_mxfp4(self.seed, payload, self.H, self.I)
        if self.wdtype == "fp32":
            w13, w2 = W.expert_f32(self.seed, payload, self.H, self.I)
            return W.f32_to_bf16_bits(w13), W.f32_to_bf16_bits(w2)
        return W.expert_bf16(self.seed, payload, self.H, self.I)

    def f64(self, payload):
        """Decoded fp64 weights, exactly the values the device receives."""
        if payload in self._cache:
            return self._cache[payload]
        r = self.raw(payload)
        if self.wdtype == "nvfp4":
            out = (dequant_nvfp4(r["w13_q"], r["w13_s"], r["g13"]), dequant_nvfp4(r["w2_q"], r["w2_s"], r["g2"]))
        elif self.wdtype == "fp8":
            out = (dequant_fp8(r["w13_q"], r["g13"]), dequant_fp8(r["w2_q"], r["g2"]))
        elif self.wdtype == "mxfp4":
            out = (dequant_mxfp4(r["w13_q"], r["w13_s"]), dequant_mxfp4(r["w2_q"], r["w2_s"]))
        else:
            out = (bf16_bits_to_f64(r[0]), bf16_bits_to_f64(r[1]))
        if len(self._cache) < 64:
            self._cache[payload] = out
        return out

    def f32_original(self, payload):
        return W.expert_f32(self.seed, payload, self.H, self.I)


def fill_pool(pool, src: ExpertSource, lay, payloads):
    import slot_cache_routed_amd.layer as LY

    def one(p):
        r = src.raw(p)
        if src.wdtype == "nvfp4":
            rec = LY.pack_record_nvfp4(lay, r)
        elif src.wdtype == "fp8":
            rec = LY.pack_record_fp8(lay, r)
        elif src.wdtype == "mxfp4":
            rec = LY.pack_record_mxfp4(lay, r)
        else:
            rec = LY.pack_record_bf16(lay, r[0], r[1])
        pool.write_payload(p, rec)

    with ThreadPoolExecutor(N_THREADS) as ex:
        list(ex.map(one, payloads))


def wdtype_code(wd):
    import slot_cache_routed_amd._lib as L
    return {"nvfp4": L.SCR_W_NVFP4, "fp8": L.SCR_W_FP8, "mxfp4": L.SCR_W_MXFP4,
            "mxfp4_a8": L.SCR_W_MXFP4_A8, "nvfp4_a4": L.SCR_W_NVFP4_A4}.get(wd, L.SCR_W_BF16)


def rms(a):
    return float(np.sqrt(np.mean(np.square(np.asarray(a, np.float64)))))


def rel_max_err(y, ref):
    """max |y - ref| / rms(ref)"""
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref)) / rms(ref))
