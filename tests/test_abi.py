"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function include/qlora_nf4.h declares,
compute the same NF4 level table as the oracle (independently: Newton's method
on erfc in long double vs. the oracle's bisection), give thresholds whose
crossings are exactly the oracle's code boundaries, and reject bad arguments
with the documented status before touching the device.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_fine_amd as q
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(q.LIB_PATH),
                                reason="libqlora_nf4.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = q.lib()
    names = _declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(q.EXPORTED)


def test_level_table_matches_oracle_bitwise():
    got = np.array(q.qlora_nf4_levels(), dtype=np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), oracle.nf4_levels().view(np.uint32))


def test_thresholds_are_oracle_boundaries():
    """x > t_j  <=>  x >= boundary_{j+1}: the first float above t_j is the
    oracle's boundary, so counting thresholds reproduces nearest-level
    encoding on every float32 in [-1, 1]."""
    t = np.array(q.qlora_nf4_thresholds(), dtype=np.float32)
    nxt = np.nextafter(t, np.float32(2), dtype=np.float32)
    np.testing.assert_array_equal(nxt.view(np.uint32), oracle.code_boundaries().view(np.uint32))


@pytest.mark.parametrize("name", ["nf4", "int4", "fp4"])
def test_codebook_tables_match_oracle(name):
    """The library's level table of each codebook equals the oracle's bit for
    bit, and counting thresholds (code = #{j : x > t_j}) reproduces the
    oracle's nearest-level code at every threshold and the float above it,
    which fixes the step function on every float32 in [-1, 1]."""
    from oracle import codebooks as cb
    lv = np.array(q.qlora_q4_levels(name), dtype=np.float32)
    np.testing.assert_array_equal(lv.view(np.uint32), cb.levels(name).view(np.uint32))
    t = np.array(q.qlora_q4_thresholds(name), dtype=np.float32)
    assert np.all(np.diff(t.astype(np.float64)) >= 0)
    probes = np.concatenate([t, np.nextafter(t, np.float32(2), dtype=np.float32),
                             np.array([-1.0, 0.0, 1.0], np.float32)])
    rule = (probes[:, None] > t[None, :]).sum(axis=1)
    np.testing.assert_array_equal(rule, cb.encode_levels(probes, cb.levels(name)))
    if name == "nf4":
        np.testing.assert_array_equal(t, np.array(q.qlora_nf4_thresholds(), np.float32))


def test_q4_size_and_format_validation():
    L = q.lib()
    assert L.qlora_q4_scale_count(64, 1024, 1) == L.qlora_nf4_scale_count(64, 1024)
    assert L.qlora_q4_scale_count(64, 1024, 0) == 64 * 1024 // 64
    buf = (ctypes.c_float * 16)()
    assert L.qlora_q4_levels(3, buf) == q.QLORA_ERR_FORMAT
    assert L.qlora_q4_levels(-1, buf) == q.QLORA_ERR_FORMAT
    p = ctypes.c_void_p(4096)
    # unknown codebook / double_quant flag, before any other check
    assert L.qlora_q4_quantize(p, 4, 64, 5, 1, p, p, p, None) == q.QLORA_ERR_FORMAT
    assert L.qlora_q4_quantize(p, 4, 64, 0, 2, p, p, p, None) == q.QLORA_ERR_FORMAT
    # without double quantization absmax_q may be NULL, but fp32 constants
    # must be 16-byte aligned
    assert L.qlora_q4_quantize(p, 4, 100, 1, 0, p, None, p, None) == 2
    assert L.qlora_q4_quantize(p, 4, 64, 1, 1, p, None, p, None) == 1
    assert L.qlora_q4_quantize(p, 4, 64, 2, 0, p, None, ctypes.c_void_p(4100), None) == 4
    w = q._Q4Weight(4096, None, 4096, 64, 128, 1, 0)
    ws = L.qlora_linear_fwd_workspace_bytes(16, 64, 128, 16)
    assert L.qlora_q4_linear_fwd(None, 16, ctypes.byref(w), p, p, 16, 1.0, p, p, p, ws,
                                 None) == 1
    w.codebook = 7
    assert L.qlora_q4_linear_fwd(p, 16, ctypes.byref(w), p, p, 16, 1.0, p, p, p, ws,
                                 None) == q.QLORA_ERR_FORMAT
    w.codebook, w.double_quant = 2, 1   # double quantization needs absmax_q
    assert L.qlora_q4_linear_bwd(p, p, 16, ctypes.byref(w), p, p, 16, 1.0, None, p, p, p, p,
                                 ws, None) == 1


def test_size_helpers():
    L = q.lib()
    for N, K in [(1, 64), (1024, 1024), (11008, 4096), (3, 64 * 257)]:
        assert L.qlora_nf4_codes_bytes(N, K) == N * K // 2
        assert L.qlora_nf4_absmax_q_bytes(N, K) == N * K // 64
        assert L.qlora_nf4_scale_count(N, K) == -(-(N * K // 64) // 256)
        total = (L.qlora_nf4_codes_bytes(N, K) + L.qlora_nf4_absmax_q_bytes(N, K)
                 + 4 * L.qlora_nf4_scale_count(N, K))
        assert total == oracle.storage_bytes(N, K)
    assert L.qlora_nf4_codes_bytes(4, 100) == 0


def test_status_strings_and_version():
    L = q.lib()
    for s in range(9):
        assert L.qlora_status_string(s) != b"unknown status"
    assert L.qlora_status_string(99) == b"unknown status"
    assert L.qlora_version().decode().count(".") == 2


def _w(codes=16, aq=16, sc=16, N=64, K=64):
    return q._Nf4Weight(codes, aq, sc, N, K)


def test_quantize_validation_before_launch():
    L = q.lib()
    p = ctypes.c_void_p(4096)
    assert L.qlora_nf4_quantize(None, 4, 64, p, p, p, None) == 1
    assert L.qlora_nf4_quantize(p, 4, 100, p, p, p, None) == 2
    assert L.qlora_nf4_quantize(p, 0, 64, p, p, p, None) == 2
    assert L.qlora_nf4_quantize(ctypes.c_void_p(4100), 4, 64, p, p, p, None) == 4


def test_linear_validation_before_launch():
    L = q.lib()
    p = ctypes.c_void_p(4096)
    w = _w(4096, 4096, 4096, 64, 128)
    ws_need = L.qlora_linear_fwd_workspace_bytes(16, 64, 128, 16)
    assert ws_need > 0
    # null X
    assert L.qlora_linear_fwd(None, 16, ctypes.byref(w), p, p, 16, 1.0, p, p, p, ws_need, None) == 1
    # rank not a multiple of 8 / too large
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(w), p, p, 7, 1.0, p, p, p, ws_need, None) == 3
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(w), p, p, 264, 1.0, p, p, p, ws_need, None) == 3
    # r > 0 needs A, B and T
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(w), None, p, 16, 1.0, p, p, p, ws_need, None) == 1
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(w), p, p, 16, 1.0, p, None, p, ws_need, None) == 1
    # shapes
    assert L.qlora_linear_fwd(p, 0, ctypes.byref(w), p, p, 16, 1.0, p, p, p, ws_need, None) == 2
    bad_k = _w(4096, 4096, 4096, 64, 96)
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(bad_k), p, p, 16, 1.0, p, p, p, ws_need, None) == 2
    bad_n = _w(4096, 4096, 4096, 60, 128)
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(bad_n), p, p, 16, 1.0, p, p, p, ws_need, None) == 2
    # 32-bit tile offsets: N and K at most 2^22, N * K at most 2^32
    for n, k in ((64, (1 << 22) + 64), ((1 << 22) + 8, 64), (1 << 20, 1 << 13)):
        big = _w(4096, 4096, 4096, n, k)
        assert L.qlora_linear_fwd(p, 16, ctypes.byref(big), p, p, 16, 1.0, p, p, p, ws_need,
                                  None) == 2
        assert L.qlora_nf4_quantize(p, n, k, p, p, p, None) == 2
    # alignment
    assert L.qlora_linear_fwd(ctypes.c_void_p(4098), 16, ctypes.byref(w), p, p, 16, 1.0, p, p, p,
                              ws_need, None) == 4
    # workspace
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(w), p, p, 16, 1.0, p, p, p, ws_need - 1, None) == 6
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(w), p, p, 16, 1.0, p, p, None, ws_need, None) == 6
    # null weight struct / fields
    assert L.qlora_linear_fwd(p, 16, None, p, p, 16, 1.0, p, p, p, ws_need, None) == 1
    nw = _w(0, 4096, 4096, 64, 128)
    assert L.qlora_linear_fwd(p, 16, ctypes.byref(nw), p, p, 16, 1.0, p, p, p, ws_need, None) == 1


def test_bwd_validation_before_launch():
    L = q.lib()
    p = ctypes.c_void_p(4096)
    w = _w(4096, 4096, 4096, 64, 128)
    need = L.qlora_linear_bwd_workspace_bytes(16, 64, 128, 16)
    assert need > 0
    assert L.qlora_linear_bwd(None, p, 16, ctypes.byref(w), p, p, 16, 1.0, None, p, p, p, p,
                              need, None) == 1
    assert L.qlora_linear_bwd(p, p, 16, ctypes.byref(w), p, p, 16, 1.0, None, p, None, p, p,
                              need, None) == 1
    assert L.qlora_linear_bwd(p, p, 16, ctypes.byref(w), p, p, 12, 1.0, None, p, p, p, p,
                              need, None) == 3
    assert L.qlora_linear_bwd(p, p, 16, ctypes.byref(w), p, p, 16, 1.0, None, p, p, p, p,
                              need - 1, None) == 6
    assert L.qlora_linear_bwd(p, p, 16, ctypes.byref(w), p, p, 16, 1.0, None,
                              ctypes.c_void_p(4104), p, p, p, need, None) == 4
    # r = 0 needs no workspace and no adapters
    assert L.qlora_linear_bwd_workspace_bytes(16, 64, 128, 0) == 0


def test_profile_api_host_only():
    L = q.lib()
    assert L.qlora_profile_reset() == 0
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert L.qlora_profile_read(0, ctypes.byref(ms), ctypes.byref(n)) == 0
    assert n.value == 0 and ms.value == 0.0
    assert L.qlora_profile_read(9, None, None) == 2


def test_gemm_split_workspace_sizes():
    """The GEMMs split their reduction only when their tiles would leave most
    CUs idle; the workspace then holds one fp32 partial [M, N] (forward) or
    [M, K] (dX) per split, also for r = 0."""
    L = q.lib()
    # 2048 tokens, 4096 x 4096: 256 tiles of 128 x 256, no split
    assert L.qlora_linear_fwd_workspace_bytes(2048, 4096, 4096, 0) == 0
    assert L.qlora_linear_bwd_workspace_bytes(2048, 4096, 4096, 0) == 0
    # 256 tokens: 32 tiles, 8 splits of 8 chunks (64 chunks of 64)
    assert L.qlora_linear_fwd_workspace_bytes(256, 4096, 4096, 0) == 8 * 256 * 4096 * 4
    assert L.qlora_linear_bwd_workspace_bytes(256, 4096, 4096, 0) == 8 * 256 * 4096 * 4
    # with LoRA the partials of the rank products share those bytes
    assert L.qlora_linear_fwd_workspace_bytes(256, 4096, 4096, 64) >= 8 * 256 * 4096 * 4
    # few tokens take the decode path: no GEMM partials
    assert L.qlora_linear_fwd_workspace_bytes(16, 4096, 4096, 0) == 0


def test_noalloc_forward_refuses_calls_beyond_its_scratch():
    """qlora_linear_fwd_noalloc checks its fixed scratch before touching the
    device: a call whose workspace exceeds QLORA_NOALLOC_SCRATCH_BYTES gets
    QLORA_ERR_SCRATCH (the pointers are never read)."""
    L = q.lib()
    M, N, K, r = 1 << 18, 8, 64, 64          # T alone: M r fp32 = 64 MiB
    assert L.qlora_linear_fwd_workspace_bytes(M, N, K, r) > q.NOALLOC_SCRATCH_BYTES
    w = _w(N=N, K=K)
    st = L.qlora_linear_fwd_noalloc(16, M, ctypes.byref(w), 16, 16, r, 1.0, 16, 16, None)
    assert st == q.QLORA_ERR_SCRATCH
    assert b"scratch" in L.qlora_status_string(st)
    # the largest split-reduction partials of the GEMM (256 tiles' worth) fit
    assert L.qlora_linear_fwd_workspace_bytes(256, 4096, 4096, 64) <= q.NOALLOC_SCRATCH_BYTES
    assert L.qlora_linear_fwd_workspace_bytes(32768, 4096, 4096, 256) <= q.NOALLOC_SCRATCH_BYTES
    # argument errors come first, as in qlora_linear_fwd
    assert L.qlora_linear_fwd_noalloc(None, 4, ctypes.byref(w), 16, 16, 8, 1.0, 16, 16,
                                      None) == 1


def test_lora16_validation_before_launch():
    L = q.lib()
    p = ctypes.c_void_p(4096)
    ws = L.qlora_lora16_fwd_workspace_bytes(16, 64, 128, 16)
    assert ws > 0 and L.qlora_lora16_bwd_workspace_bytes(16, 64, 128, 16) > 0
    # null weight, K % 64, N % 8, N K above 2^30 (32-bit byte offsets below 2^31)
    assert L.qlora_lora16_fwd(p, 16, None, 64, 128, p, p, 16, 1.0, p, p, p, ws, None) == 1
    assert L.qlora_lora16_fwd(p, 16, p, 64, 100, p, p, 16, 1.0, p, p, p, ws, None) == 2
    assert L.qlora_lora16_fwd(p, 16, p, 60, 128, p, p, 16, 1.0, p, p, p, ws, None) == 2
    assert L.qlora_lora16_fwd(p, 16, p, 1 << 16, 1 << 15, p, p, 16, 1.0, p, p, p, ws, None) == 2
    assert L.qlora_lora16_fwd(p, 16, ctypes.c_void_p(4098), 64, 128, p, p, 16, 1.0, p, p, p, ws,
                              None) == 4
    # too small a workspace
    assert L.qlora_lora16_fwd(p, 16, p, 64, 128, p, p, 16, 1.0, p, p, p, 16, None) == 6
    assert L.qlora_lora16_bwd(p, p, 16, p, 64, 128, p, p, 7, 1.0, None, p, p, p, p, ws,
                              None) == 3


def test_adamw_and_paged_state_validation():
    L = q.lib()
    p = ctypes.c_void_p(4096)
    cfg = q._AdamWConfig(1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert L.qlora_adamw_step(None, p, p, p, 8, ctypes.byref(cfg), 1, None) == 1
    assert L.qlora_adamw_step(p, p, p, p, 8, None, 1, None) == 1
    assert L.qlora_adamw_step(p, p, p, p, 0, ctypes.byref(cfg), 1, None) == 2
    assert L.qlora_adamw_step(p, p, p, p, 8, ctypes.byref(cfg), 0, None) == 2
    bad = q._AdamWConfig(1e-3, 0.9, 1.0, 1e-8, 0.0)
    assert L.qlora_adamw_step(p, p, p, p, 8, ctypes.byref(bad), 1, None) == 2
    assert L.qlora_adamw_step(p, p, ctypes.c_void_p(4100), p, 8, ctypes.byref(cfg), 1, None) == 4
    h = ctypes.c_void_p()
    assert L.qlora_paged_state_create(0, 0, ctypes.byref(h)) == 2
    assert L.qlora_paged_state_create(8, 0, None) == 1
    assert L.qlora_paged_state_page_out(None, None) == 1
    assert L.qlora_paged_state_page_in(None, None) == 1
    assert L.qlora_paged_state_resident(None) == 0
    assert L.qlora_paged_state_destroy(None) == 0


def test_block_validation_before_launch():
    L = q.lib()
    p = ctypes.c_void_p(4096)
    w = _w(4096, 4096, 4096, 384, 128)
    ws = L.qlora_block_fwd_workspace_bytes(16, 3, 128, 128, 16)
    assert ws > 0
    # S r above 256, r = 0, segments not on 128-row tiles
    assert L.qlora_block_fwd(p, 16, ctypes.byref(w), 3, p, p, 96, 1.0, p, p, p, ws, None) == 3
    assert L.qlora_block_fwd(p, 16, ctypes.byref(w), 3, p, p, 0, 1.0, p, p, p, ws, None) == 3
    assert L.qlora_block_fwd(p, 16, ctypes.byref(w), 2, p, p, 16, 1.0, p, p, p, ws, None) == 2
