"""CPU oracle for the routed-MoE-over-slot-cache path — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct restatement of what the path computes, written
from the pages that describe the method (FreeToken PR #676 "on-demand prefill
through the slot cache", gdevenyi's FreeToken PR #68, the vLLM fork's expert
pool PR #48 and its follow-up PR #51).  It shares no code with the HIP path and
imports nothing from it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never does.

Floating point is fp64 unless stated.  Parity status per function is in each
module's header; every function here is pinned by a ``-m "not gpu"`` test
against page-printed values, closed forms, library special cases or brute
force.
"""
from .route import route_topk_softmax
from .dedup import dedup_sorted
from .lru import SlotBankState, ensure_slots
from .align import align_blocks, align_capacity
from .nvfp4 import e2m1_value, e4m3_value, dequant_nvfp4
from .lowbit import e8m0_value, dequant_fp8, dequant_mxfp4, e4m3_encode
from .actquant import (layer_activation_scales, quantize_fp8_static, dequant_fp8_static, quantize_nvfp4_act,
                       dequant_nvfp4_act, e2m1_encode_array)
from .mlp import expert_mlp, moe_layer, moe_layer_tokens, moe_layer_w4a8, moe_layer_w4a4
from .dispatch import prefill_on_demand, demand_capacity_ok
