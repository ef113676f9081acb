"""CPU-only checks of the C-ABI library: it loads, exports every entry point
that include/mk.h declares, packs/unpacks the block layout losslessly, and
rejects bad arguments on the host before any GPU work (no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_weight_streaming_q4_amd as mk
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    L = mk.lib()
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n


def test_pack_unpack_round_trip_and_layout():
    W = synth.q4k_fields(0, 77, 150, 768)  # ragged: 150 rows = 2 tiles + 22
    blocks = mk.mk_q4k_pack(W)
    assert blocks.nbytes == mk.mk_q4k_bytes(150, 768) == 3 * 3 * 9216
    back = mk.mk_q4k_unpack(blocks, 150, 768)
    for k in ("d", "dmin", "sc", "m", "q"):
        assert np.array_equal(back[k], W[k]), k
    # layout spot check: code k of row r sits in unit (r//64, k//256), sub-block
    # j = (k%256)//32 at byte 16*(r%64) + 4*w + i (low nibble for the first four
    # of each 8, high nibble for the next four)
    r, k = 101, 3 * 256 - 256 + 77
    b, j, e = k // 256, (k % 256) // 32, k % 32
    w, i, hi = e // 8, e % 4, (e % 8) >= 4
    unit = (r // 64) * 3 + b
    byte = blocks[unit * 9216 + 1024 + j * 1024 + (r % 64) * 16 + 4 * w + i]
    assert (byte >> 4 if hi else byte & 15) == W["q"][r, k]
    # padding rows of the last tile are zero
    last = blocks[2 * 3 * 9216:].reshape(3, 9216)
    assert not last[:, 22 * 16:1024].any()


def test_pack_in_row_slices_matches_whole():
    W = synth.q4k_fields(0, 78, 192, 512)
    whole = mk.mk_q4k_pack(W)
    parts = []
    for r0 in (0, 64, 128):
        Wi = synth.q4k_fields(0, 78, 192, 512, r0, r0 + 64)
        Wi["n_out_total"] = 192
        parts.append(mk.mk_q4k_pack(Wi, r0, r0 + 64))
    assert np.array_equal(np.concatenate(parts), whole)


def test_pack_rejects_out_of_range_fields():
    W = synth.q4k_fields(0, 79, 64, 256)
    W["q"][3, 5] = 16
    with pytest.raises(mk.MkError) as e:
        mk.mk_q4k_pack(W)
    assert e.value.status == mk.MK_ERR_RANGE


def _q4k(ptr, n_out, n_in):
    return mk.mk_q4k(ptr, n_out, n_in)


def test_host_validation_before_any_gpu_work():
    L = mk.lib()
    fake = 1 << 20  # never dereferenced: validation fails first
    x = ctypes.c_void_p(fake)
    W = _q4k(fake, 64, 512)
    # T outside 1..16
    assert L.mk_qgemv_rows(ctypes.byref(W), x, 0, x, x, 1 << 30, None) == mk.MK_ERR_RANGE
    assert L.mk_qgemv_rows(ctypes.byref(W), x, 17, x, x, 1 << 30, None) == mk.MK_ERR_RANGE
    # n_in not a multiple of 256
    Wb = _q4k(fake, 64, 500)
    assert L.mk_qgemv_rows(ctypes.byref(Wb), x, 1, x, x, 1 << 30, None) == mk.MK_ERR_SHAPE
    # misaligned blocks
    Wm = _q4k(fake + 16, 64, 512)
    assert L.mk_qgemv_rows(ctypes.byref(Wm), x, 1, x, x, 1 << 30, None) == mk.MK_ERR_ALIGN
    # null input
    assert L.mk_qgemv_rows(ctypes.byref(W), None, 1, x, x, 1 << 30, None) == mk.MK_ERR_ARG
    # workspace too small
    assert L.mk_qgemv_rows(ctypes.byref(W), x, 1, x, x, 16, None) == mk.MK_ERR_WORKSPACE
    assert b"workspace" in L.mk_last_error()
    # dot4 engine is limited to T <= 8
    assert L.mk_qgemv_rows_ex(ctypes.byref(W), x, 9, x, mk.MK_PATH_DOT4, x, 1 << 30, None) == mk.MK_ERR_RANGE
    assert L.mk_qgemv_rows_ex(ctypes.byref(W), x, 4, x, 7, x, 1 << 30, None) == mk.MK_ERR_ARG
    # quantizer K % 32
    assert L.mk_quantize_rows(x, 2, 48, x, x, x, None) == mk.MK_ERR_SHAPE
    # FFN shapes must chain
    G = _q4k(fake, 512, 256)
    D = _q4k(fake, 256, 768)
    assert L.mk_ffn_rows(ctypes.byref(G), ctypes.byref(G), ctypes.byref(D), x, 1, x, None, x, 1 << 30,
                         None) == mk.MK_ERR_SHAPE
    # lm_head: bad groups, bad H
    gs = (ctypes.c_int32 * 3)(0, 3, 4)
    assert L.mk_lmhead_verify(x, 100, 512, x, 5, gs, 2, x, x, x, x, x, 1 << 30, None) == mk.MK_ERR_RANGE
    gs2 = (ctypes.c_int32 * 3)(0, 0, 5)
    assert L.mk_lmhead_verify(x, 100, 512, x, 5, gs2, 2, x, x, x, x, x, 1 << 30, None) == mk.MK_ERR_RANGE
    assert L.mk_lmhead_verify(x, 100, 500, x, 5, None, 1, x, x, x, x, x, 1 << 30, None) == mk.MK_ERR_SHAPE
    # deltanet: head size and T range
    dn = mk.mk_deltanet(fake, fake, fake, 4, 64, 128, 5)
    assert L.mk_deltanet_step(ctypes.byref(dn), 0, x, x, x, x, x, 1, x, None) == mk.MK_ERR_SHAPE
    dn = mk.mk_deltanet(fake, fake, fake, 4, 128, 128, 5)
    assert L.mk_deltanet_step(ctypes.byref(dn), 0, x, x, x, x, x, 6, x, None) == mk.MK_ERR_RANGE
    assert L.mk_status_string(mk.MK_ERR_WORKSPACE) == b"workspace too small"
    # sampling verify: top_k in 1..32, a positive finite temperature
    f = ctypes.c_float
    for k, tau in ((0, 0.6), (33, 0.6), (8, 0.0), (8, -1.0), (8, float("inf")), (8, float("nan"))):
        assert L.mk_lmhead_sample(x, 100, 512, x, 5, None, 1, x, k, f(tau), x, x, None, None, x, x, x, 1 << 30,
                                  None) == mk.MK_ERR_RANGE, (k, tau)
    assert L.mk_lmhead_sample(x, 100, 512, x, 5, None, 1, x, 8, f(0.6), None, x, None, None, x, x, x, 1 << 30,
                              None) == mk.MK_ERR_ARG
    assert L.mk_lmhead_sample(x, 100, 512, x, 5, None, 1, x, 8, f(0.6), x, x, None, None, x, x, x, 64,
                              None) == mk.MK_ERR_WORKSPACE
    # MTP draft loop: head shapes must chain, V_draft <= V, n_draft in 1..16
    fc, g_, u_, d_ = _q4k(fake, 512, 1024), _q4k(fake, 768, 512), _q4k(fake, 768, 512), _q4k(fake, 512, 768)
    head = mk.mk_mtp(fc, g_, u_, d_)
    bad = mk.mk_mtp(_q4k(fake, 512, 768), g_, u_, d_)
    assert L.mk_mtp_draft(ctypes.byref(bad), x, 1000, 300, x, 5, None, 1, x, x, 2, x, None, x, 1 << 30,
                          None) == mk.MK_ERR_SHAPE
    assert L.mk_mtp_draft(ctypes.byref(head), x, 1000, 1001, x, 5, None, 1, x, x, 2, x, None, x, 1 << 30,
                          None) == mk.MK_ERR_RANGE
    assert L.mk_mtp_draft(ctypes.byref(head), x, 1000, 300, x, 5, None, 1, x, x, 0, x, None, x, 1 << 30,
                          None) == mk.MK_ERR_RANGE
    assert L.mk_mtp_draft(ctypes.byref(head), x, 1000, 300, x, 5, None, 1, x, x, 2, x, None, x, 64,
                          None) == mk.MK_ERR_WORKSPACE
    assert mk.lib().mk_mtp_draft_workspace(ctypes.byref(head), 300, 5, 1) > 5 * 1024 * 4
    # the no-allocation GEMV refuses shapes whose workspace exceeds its array, before any device call
    Wbig = _q4k(fake, 32768, 32768)
    assert L.mk_qgemv_rows_noalloc(ctypes.byref(Wbig), x, 16, x, 0, None) == mk.MK_ERR_WORKSPACE


def test_workspace_queries_are_host_only():
    assert mk.mk_qgemv_rows_workspace(5, 5120, 5120) > 5 * 5120
    assert mk.mk_qgemv_rows_workspace(0, 5120, 5120) == 0
    assert mk.mk_ffn_rows_workspace(5, 5120, 17408) > 0
    assert mk.mk_lmhead_verify_workspace(151936, 5120, 5) > 151936 // 64 * 16 * 8
    assert mk.mk_lmhead_sample_workspace(151936, 5120, 12) > 12 * 151936 * 4
    assert mk.mk_q4k_bytes(5120, 5120) == 14_745_600


def test_attention_validation_and_workspace_on_the_host():
    """mk_attn_decode / mk_attn_decode_q8 reject bad shapes, ranges, pointers
    and workspaces before any GPU work; the workspace query is host-only,
    0 for invalid arguments and grows with the rows and the contexts."""
    L = mk.lib()
    fake = 1 << 20
    x = ctypes.c_void_p(fake)
    ctx = np.array([100, 7], np.int32)
    gs = np.array([0, 3, 6], np.int32)
    P = lambda a: a.ctypes.data

    def call(T=6, Hq=32, Hkv=8, d=128, cap=128, ctx_=ctx, gs_=gs, G=2, ws_bytes=1 << 30, q=x, ws=x):
        return L.mk_attn_decode(q, None, T, Hq, x, x, Hkv, d, cap, P(ctx_), P(gs_), G, x, ws, ws_bytes, None)

    assert call(d=64) == mk.MK_ERR_SHAPE
    assert call(cap=100) == mk.MK_ERR_SHAPE
    assert call(cap=mk.MK_ATTN_CAP_MAX + 64) == mk.MK_ERR_RANGE
    assert call(Hkv=3) == mk.MK_ERR_SHAPE
    assert call(T=17, gs_=np.array([0, 3, 17], np.int32)) == mk.MK_ERR_RANGE
    assert call(ctx_=np.array([126, 7], np.int32)) == mk.MK_ERR_RANGE          # 126 + 3 > cap
    assert call(T=17 - 1, gs_=np.array([0, 1, 16], np.int32), Hq=64) == mk.MK_ERR_RANGE  # 15 rows x 8 > 64
    assert call(gs_=np.array([0, 3, 5], np.int32)) == mk.MK_ERR_RANGE          # groups must end at T
    assert call(q=ctypes.c_void_p(fake + 4)) == mk.MK_ERR_ALIGN
    assert call(q=None) == mk.MK_ERR_ARG
    assert call(ws_bytes=16) == mk.MK_ERR_WORKSPACE
    assert L.mk_attn_decode_q8(x, None, 6, 32, None, x, x, x, 8, 128, 128, P(ctx), P(gs), 2, x, x, 1 << 30,
                               None) == mk.MK_ERR_ARG
    # workspace query
    W = lambda T, c, g: L.mk_attn_decode_workspace(T, 32, 8, P(np.array(c, np.int32)), P(np.array(g, np.int32)),
                                                   len(c))
    assert W(6, [100, 7], [0, 3, 6]) > 0
    assert W(6, [100, 7], [0, 3, 5]) == 0
    assert W(12, [32768] * 4, [0, 3, 6, 9, 12]) > W(12, [1024] * 4, [0, 3, 6, 9, 12])
    assert W(12, [4096] * 4, [0, 3, 6, 9, 12]) > W(4, [4096] * 4, [0, 1, 2, 3, 4])
