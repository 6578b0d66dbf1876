"""The host packing of expert records follows the tile-major layout that
include/scr.h documents (CPU; pure byte permutations)."""
import numpy as np

import slot_cache_routed_amd.layer as LY


def test_bf16_tiles_follow_the_documented_formula():
    g = np.random.default_rng(0)
    N, K = 48, 256
    w = g.integers(0, 65535, size=(N, K), dtype=np.uint16)
    t = LY.tile_bf16(w).view(np.uint16)
    nk = K // 128
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    tb, r, kb, kk = n // 16, n % 16, k // 128, k % 128
    s, gg, e = kk // 32, (kk % 32) // 8, kk % 8
    off = (tb * nk + kb) * 4096 + 1024 * s + 16 * (16 * gg + r) + 2 * e
    assert np.array_equal(t[off // 2], w)


def test_fp4_code_and_scale_tiles_follow_the_documented_formula():
    g = np.random.default_rng(1)
    N, K = 32, 384
    nk = K // 128
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    tq = LY.tile_fp4_codes(q)
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    tb, r, kb, kk = n // 16, n % 16, k // 128, k % 128
    gg, j = kk // 32, kk % 32
    byte = (tb * nk + kb) * 1024 + 16 * (16 * gg + r) + j // 2
    assert np.array_equal((tq[byte] >> (4 * (j % 2))) & 15, codes)
    sc = g.integers(0, 255, size=(N, K // 16), dtype=np.uint8)
    ts = LY.tile_fp4_scales(sc)
    n, b = np.meshgrid(np.arange(N), np.arange(K // 16), indexing="ij")
    tb, r, kb, bb = n // 16, n % 16, b // 8, b % 8
    assert np.array_equal(ts[(tb * nk + kb) * 128 + 2 * (16 * (bb // 2) + r) + bb % 2], sc)


def test_records_are_permutations_of_the_tensors():
    import slot_cache_routed_amd._lib as L
    import workloads as W
    lay = L.record_layout_of(L.SCR_W_NVFP4, 256, 128)
    d = W.expert_nvfp4(3, 0, 256, 128)
    rec = LY.pack_record_nvfp4(lay, d)
    assert rec.size == lay.record_bytes
    blk = rec[lay.w13_off:lay.w13_scale_off]
    assert np.array_equal(np.sort(blk), np.sort(d["w13_q"].reshape(-1)))
    assert rec[lay.g13_off:lay.g13_off + 4].view(np.float32)[0] == d["g13"]
    lay = L.record_layout_of(L.SCR_W_BF16, 256, 128)
    a, b = W.expert_bf16(3, 0, 256, 128)
    rec = LY.pack_record_bf16(lay, a, b)
    assert np.array_equal(np.sort(rec[lay.w2_off:].view(np.uint16)), np.sort(b.reshape(-1)))


def test_fp8_tiles_follow_the_documented_formula():
    g = np.random.default_rng(2)
    N, K = 32, 384
    nk = K // 128
    q = g.integers(0, 256, size=(N, K), dtype=np.uint8)
    t = LY.tile_fp8(q)
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    tb, r, kb, kk = n // 16, n % 16, k // 128, k % 128
    gg, j = kk // 32, kk % 32
    off = (tb * nk + kb) * 2048 + 1024 * (j // 16) + 16 * (16 * gg + r) + j % 16
    assert np.array_equal(t[off], q)


def test_mx_scale_tiles_follow_the_documented_formula():
    g = np.random.default_rng(3)
    N, K = 48, 256
    nk = K // 128
    sc = g.integers(0, 255, size=(N, K // 32), dtype=np.uint8)
    t = LY.tile_mx_scales(sc)
    n, b = np.meshgrid(np.arange(N), np.arange(K // 32), indexing="ij")
    tb, r, kb, gg = n // 16, n % 16, b // 4, b % 4
    assert np.array_equal(t[(tb * nk + kb) * 64 + 16 * gg + r], sc)


def test_fp8_and_mxfp4_records():
    import slot_cache_routed_amd._lib as L
    import workloads as W
    lay = L.record_layout_of(L.SCR_W_FP8, 256, 128)
    assert lay.w2_off == 2 * 128 * 256 and lay.g13_off == lay.w2_off + 256 * 128 and lay.g2_off == lay.g13_off + 4
    assert lay.record_bytes % 256 == 0 and lay.record_bytes >= lay.g2_off + 4
    d = W.expert_fp8(3, 0, 256, 128)
    rec = LY.pack_record_fp8(lay, d)
    assert np.array_equal(np.sort(rec[lay.w2_off:lay.g13_off]), np.sort(d["w2_q"].reshape(-1)))
    assert rec[lay.g2_off:lay.g2_off + 4].view(np.float32)[0] == d["g2"]
    lay = L.record_layout_of(L.SCR_W_MXFP4, 256, 128)
    assert lay.w13_scale_off == 128 * 256 and lay.w2_off == lay.w13_scale_off + 2 * 128 * 256 // 32
    assert lay.w2_scale_off == lay.w2_off + 256 * 128 // 2 and lay.g13_off == 0
    d = W.expert_mxfp4(3, 0, 256, 128)
    rec = LY.pack_record_mxfp4(lay, d)
    assert rec.size == lay.record_bytes
    assert np.array_equal(np.sort(rec[lay.w13_scale_off:lay.w2_off]), np.sort(d["w13_s"].reshape(-1)))
