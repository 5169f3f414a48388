"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/stca.h declares, and rejects bad arguments with the
documented status codes before anything is enqueued."""
import ctypes as C
import os
import re

import pytest

from recsys_ultra_long_amd import stca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # 16-byte aligned, never dereferenced by host validation


def header_functions():
    src = open(os.path.join(ROOT, "include", "stca.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(stca_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_header_symbols():
    lib = stca.load()
    names = header_functions()
    assert set(names) == set(stca.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings():
    assert stca.status_string(0) == "STCA_OK"
    assert stca.status_string(-3) == "STCA_ERR_WORKSPACE"
    assert stca.load().stca_version() >= 100


def cfg(**over):
    c = dict(B=2, d=256, H=8, hidden=512, M=4, table_rows=1000, dtype=stca.BF16, score=0,
             qmode=0, path=0, flags=stca.FLAG_KV_LN, chunk_keys=0)
    c.update(over)
    return stca.Config(**c)


def batch(**over):
    b = dict(hist_offsets=FAKE, hist_ids=FAKE, tgt_offsets=FAKE, tgt_ids=FAKE, q0=None,
             table=FAKE, n_hist=1000, n_tgt=8, max_tgt_per_user=4)
    b.update(over)
    return stca.Batch(**b)


def ws_size(c, b):
    n = C.c_size_t(0)
    r = stca.load().stca_workspace_size(C.byref(c) if c is not None else None, C.byref(b), C.byref(n))
    return r, n.value


@pytest.mark.parametrize("over,code", [
    (dict(d=250), stca.ERR_INVALID_ARG),          # d % H
    (dict(H=16), stca.ERR_UNSUPPORTED),           # d_h = 16
    (dict(d=192, H=6), stca.ERR_UNSUPPORTED),     # bf16 d not in {128,256,512}
    (dict(hidden=500), stca.ERR_UNSUPPORTED),
    (dict(M=0), stca.ERR_INVALID_ARG),
    (dict(M=17), stca.ERR_INVALID_ARG),
    (dict(dtype=7), stca.ERR_INVALID_ARG),
    (dict(score=3), stca.ERR_INVALID_ARG),
    (dict(qmode=3), stca.ERR_INVALID_ARG),
    (dict(flags=64), stca.ERR_INVALID_ARG),
    (dict(chunk_keys=33), stca.ERR_INVALID_ARG),
    (dict(table_rows=0), stca.ERR_INVALID_ARG),
    (dict(B=-1), stca.ERR_INVALID_ARG),
    (dict(dtype=stca.F32, d=96, H=3, hidden=96), stca.OK),
    (dict(dtype=stca.F32, d=544, H=17, hidden=64), stca.ERR_UNSUPPORTED),
])
def test_config_validation(over, code):
    r, _ = ws_size(cfg(**over), batch())
    assert r == code, stca.last_error()
    if code != stca.OK:
        assert stca.last_error()


@pytest.mark.parametrize("over,code", [
    (dict(n_hist=1 << 31), stca.ERR_INVALID_ARG),
    (dict(n_tgt=-1), stca.ERR_INVALID_ARG),
    (dict(max_tgt_per_user=0), stca.ERR_INVALID_ARG),
    (dict(max_tgt_per_user=5000), stca.ERR_INVALID_ARG),
    (dict(table=None), stca.ERR_INVALID_ARG),
    (dict(hist_ids=None), stca.ERR_INVALID_ARG),
    (dict(tgt_ids=None), stca.ERR_INVALID_ARG),
    (dict(hist_offsets=FAKE + 4), stca.ERR_INVALID_ARG),   # misaligned
])
def test_batch_validation(over, code):
    r, _ = ws_size(cfg(), batch(**over))
    assert r == code, stca.last_error()


def test_null_config():
    n = C.c_size_t(0)
    b = batch()
    assert stca.load().stca_workspace_size(None, C.byref(b), C.byref(n)) == stca.ERR_INVALID_ARG


def test_workspace_grows_with_history_and_targets():
    _, a = ws_size(cfg(), batch(n_hist=1000))
    _, b = ws_size(cfg(), batch(n_hist=100_000))
    _, c = ws_size(cfg(), batch(n_hist=100_000, n_tgt=4000, max_tgt_per_user=64))
    assert 0 < a < b < c
    # staged K/V: M layers x (K and V) x padded tokens x d x 2 bytes at least
    assert b >= 4 * 2 * 100_000 * 256 * 2


def _weights(M=4, fusion=True, null=None):
    layers = (stca.Layer * M)()
    ffn = stca.Ffn(FAKE, FAKE, FAKE, FAKE, FAKE)
    for i in range(M):
        layers[i] = stca.Layer(ffn, ffn, FAKE, FAKE, FAKE, FAKE, FAKE if i > 0 else None, FAKE)
    if null == "wq":
        layers[1].wq = None
    if null == "wc":
        layers[2].wc = None
    return stca.Weights(layers, ffn, FAKE), layers


def _forward(c, b, w, out, ws_bytes):
    return stca.load().stca_forward(C.byref(c), C.byref(b), C.byref(w), C.byref(out), FAKE,
                                    ws_bytes, None)


def test_forward_rejects_before_enqueue():
    c, b = cfg(), batch()
    w, keep = _weights()
    out = stca.Outputs(z=FAKE)
    _, need = ws_size(c, b)
    assert _forward(c, b, w, out, need - 1) == stca.ERR_WORKSPACE
    assert "needed" in stca.last_error()
    assert _forward(c, b, w, stca.Outputs(), need) == stca.ERR_INVALID_ARG     # z required
    wq, k2 = _weights(null="wq")
    assert _forward(c, b, wq, out, need) == stca.ERR_INVALID_ARG
    wc, k3 = _weights(null="wc")
    assert _forward(c, b, wc, out, need) == stca.ERR_INVALID_ARG
    assert _forward(c, b, w, stca.Outputs(z=FAKE + 8), need) == stca.ERR_INVALID_ARG


def test_attention_validation():
    lib = stca.load()
    a = stca.AttnArgs(B=2, d=256, H=8, dtype=stca.BF16, score=0, chunk_keys=0,
                      hist_offsets=FAKE, tgt_offsets=FAKE, n_hist=100, n_tgt=4,
                      max_tgt_per_user=2, q=FAKE, k=FAKE, v=FAKE, attn=FAKE)
    n = C.c_size_t(0)
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.OK and n.value > 0
    a.H = 2
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.ERR_UNSUPPORTED
    a.H = 8
    a.k = None
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.ERR_INVALID_ARG
    a.k = FAKE
    assert lib.stca_attention(C.byref(a), FAKE, 0, None) == stca.ERR_WORKSPACE


# ------------------------------------------------------------------ fused path
@pytest.mark.parametrize("over,bover,code", [
    (dict(), dict(), stca.OK),                                   # d 256, d_h 32
    (dict(H=4), dict(), stca.OK),                                # d 256, d_h 64
    (dict(d=128, H=4, hidden=256), dict(), stca.OK),             # d 128, d_h 32
    (dict(d=128, H=2, hidden=256), dict(), stca.ERR_UNSUPPORTED),  # d 128, d_h 64
    (dict(d=512, H=8, hidden=1024), dict(), stca.ERR_UNSUPPORTED),
    (dict(dtype=stca.F32), dict(), stca.ERR_UNSUPPORTED),
    (dict(flags=0), dict(), stca.ERR_UNSUPPORTED),               # no LN after the history FFN
    (dict(), dict(max_tgt_per_user=65), stca.ERR_UNSUPPORTED),
    (dict(), dict(max_tgt_per_user=64), stca.OK),
])
def test_fused_validation(over, bover, code):
    r, _ = ws_size(cfg(path=1, **over), batch(**bover))
    assert r == code, stca.last_error()


def test_fused_workspace_does_not_grow_with_history():
    """The fused path keeps no K/V: beyond a bounded partial buffer (one slot
    per workgroup and user) its workspace does not depend on n_hist."""
    b = lambda n: batch(n_hist=n, n_tgt=64 * 32, max_tgt_per_user=64)
    _, f1 = ws_size(cfg(path=1, B=32), b(32 * 10_240))
    _, f2 = ws_size(cfg(path=1, B=32), b(32 * 100_000))
    _, f3 = ws_size(cfg(path=1, B=32), b(2**31 - 1))
    _, s1 = ws_size(cfg(path=0, B=32), b(32 * 10_240))
    assert f1 == f2 == f3
    # staged: 4 layers x K, V x 327,680 tokens x 256 x 2 bytes of K/V alone
    assert s1 >= 4 * 2 * 32 * 10_240 * 256 * 2
    assert f1 < s1 / 4


def test_fused_rejects_kv_dump():
    c, b = cfg(path=1), batch()
    w, keep = _weights()
    _, need = ws_size(c, b)
    out = stca.Outputs(z=FAKE, kv_dump=FAKE)
    assert _forward(c, b, w, out, need) == stca.ERR_UNSUPPORTED
    assert "staged" in stca.last_error()


# ------------------------------------------------------------------ id dedup
@pytest.mark.parametrize("over,code", [
    (dict(flags=stca.FLAG_KV_LN | stca.FLAG_DEDUP), stca.OK),
    (dict(flags=stca.FLAG_DEDUP), stca.OK),                                   # HyFormer-style, no LN
    (dict(flags=stca.FLAG_KV_LN | stca.FLAG_DEDUP, path=1), stca.ERR_UNSUPPORTED),
    (dict(flags=stca.FLAG_KV_LN | stca.FLAG_DEDUP, dtype=stca.F32), stca.ERR_UNSUPPORTED),
])
def test_dedup_validation(over, code):
    r, _ = ws_size(cfg(**over), batch())
    assert r == code, stca.last_error()


def test_dedup_workspace_and_x_dump():
    b = batch(n_hist=100_000, n_tgt=64, max_tgt_per_user=32)
    _, plain = ws_size(cfg(), b)
    _, dd = ws_size(cfg(flags=stca.FLAG_KV_LN | stca.FLAG_DEDUP), b)
    assert dd > plain          # hash set, maps and the unique rows' K/V
    c = cfg(flags=stca.FLAG_KV_LN | stca.FLAG_DEDUP)
    w, keep = _weights()
    out = stca.Outputs(z=FAKE, x_dump=FAKE)
    assert _forward(c, b, w, out, dd) == stca.ERR_UNSUPPORTED


# ----------------------------------------------------------------- HyFormer query mode
def _hy_cfg(**over):
    c = dict(B=2, d=512, H=8, hidden=1024, M=3, table_rows=1000, dtype=stca.BF16, score=0,
             qmode=stca.QMODE["hyformer"], path=0, flags=0, chunk_keys=0, n_ns=8, q_hidden=512)
    c.update(over)
    return stca.Config(**c)


def _hy_batch(**over):
    b = dict(hist_offsets=FAKE, hist_ids=FAKE, tgt_offsets=FAKE, tgt_ids=None, q0=None,
             table=FAKE, n_hist=1000, n_tgt=16, max_tgt_per_user=8, ns_feats=FAKE)
    b.update(over)
    return stca.Batch(**b)


@pytest.mark.parametrize("cover,bover,code", [
    ({}, {}, stca.OK),
    (dict(dtype=stca.F32), {}, stca.ERR_UNSUPPORTED),
    (dict(path=1), {}, stca.ERR_UNSUPPORTED),
    (dict(q_hidden=0), {}, stca.ERR_UNSUPPORTED),
    (dict(q_hidden=100), {}, stca.ERR_UNSUPPORTED),
    (dict(n_ns=-1), {}, stca.ERR_INVALID_ARG),
    ({}, dict(n_tgt=15), stca.ERR_INVALID_ARG),           # not B * m
    (dict(n_ns=5), {}, stca.ERR_UNSUPPORTED),             # m + n_ns = 13 does not divide d
    ({}, dict(ns_feats=None), stca.ERR_INVALID_ARG),
    (dict(n_ns=0), dict(ns_feats=None), stca.OK),          # no non-sequence tokens: none needed
])
def test_hyformer_validation(cover, bover, code):
    r, n = ws_size(_hy_cfg(**cover), _hy_batch(**bover))
    assert r == code, stca.last_error()
    if code == stca.OK:
        assert n > 0


def test_hyformer_forward_needs_query_weights():
    c, b = _hy_cfg(), _hy_batch()
    M = c.M
    layers = (stca.Layer * M)()
    ffn = stca.Ffn(FAKE, FAKE, FAKE, FAKE, FAKE)
    for i in range(M):
        layers[i] = stca.Layer(ffn, ffn, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE)
    out = stca.Outputs(z=FAKE)
    w = stca.Weights(layers, stca.Ffn(), None, None, FAKE, FAKE)      # qgen_w1 missing
    assert _forward(c, b, w, out, 1 << 40) == stca.ERR_INVALID_ARG
    assert "query-generation" in stca.last_error()
    w = stca.Weights(layers, stca.Ffn(), None, FAKE, FAKE, FAKE)
    layers[1].boost_w2 = None
    assert _forward(c, b, w, out, 1 << 40) == stca.ERR_INVALID_ARG
    assert "boosting" in stca.last_error()


# ----------------------------------------------------------------- Cross-Mask
def _map(vals):
    arr = (C.c_int32 * len(vals))(*vals)
    return arr, C.cast(arr, C.POINTER(C.c_int32))


@pytest.mark.parametrize("cover,bover,hmap,code", [
    ({}, dict(key_mask=FAKE), None, stca.OK),
    ({}, {}, [0, 0, 2, 2, 4, 4, 6, 6], stca.OK),
    (dict(flags=stca.FLAG_KV_LN | stca.FLAG_DEDUP), dict(key_mask=FAKE), [0, 1, 1, 3, 4, 5, 5, 7], stca.OK),
    (dict(path=1), dict(key_mask=FAKE), None, stca.ERR_UNSUPPORTED),          # fused path
    (dict(path=1), {}, [0] * 8, stca.ERR_UNSUPPORTED),
    (dict(dtype=stca.F32, d=64, H=2, hidden=64), dict(key_mask=FAKE), None, stca.ERR_UNSUPPORTED),
    ({}, dict(key_mask=FAKE + 4), None, stca.ERR_INVALID_ARG),                # misaligned
    ({}, {}, [0, 1, 2, 3, 4, 5, 6, 8], stca.ERR_INVALID_ARG),                 # outside [0, H)
    ({}, {}, [0, 1, 2, -1, 4, 5, 6, 7], stca.ERR_INVALID_ARG),
])
def test_cross_mask_validation(cover, bover, hmap, code):
    c = cfg(**cover)
    keep = None
    if hmap is not None:
        keep, c.head_map = _map(hmap)
    r, _ = ws_size(c, batch(**bover))
    assert r == code, stca.last_error()
    if code != stca.OK:
        assert "mask" in stca.last_error() or "head_map" in stca.last_error()


def test_cross_mask_attention_and_backward_validation():
    lib = stca.load()
    a = stca.AttnArgs(B=2, d=256, H=8, dtype=stca.BF16, score=0, chunk_keys=0,
                      hist_offsets=FAKE, tgt_offsets=FAKE, n_hist=100, n_tgt=4,
                      max_tgt_per_user=2, q=FAKE, k=FAKE, v=FAKE, attn=FAKE, key_mask=FAKE)
    n = C.c_size_t(0)
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.OK
    keep, a.head_map = _map([0, 0, 1, 1, 2, 2, 3, 9])
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.ERR_INVALID_ARG
    a.head_map = None
    a.dtype, a.d, a.H = stca.F32, 64, 2
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.ERR_UNSUPPORTED
    # the backward takes no masks: rejected before anything is enqueued
    c, b = cfg(), batch(key_mask=FAKE)
    w, keepw = _weights()
    g = stca.Grads()
    r = lib.stca_backward(C.byref(c), C.byref(b), C.byref(w), FAKE, C.byref(g), FAKE, 1 << 30, None)
    assert r == stca.ERR_UNSUPPORTED and "Cross-Mask" in stca.last_error()


@pytest.mark.parametrize("cover,bover,code", [
    ({}, dict(score_bias=FAKE), stca.OK),
    (dict(flags=stca.FLAG_KV_LN | stca.FLAG_DEDUP), dict(score_bias=FAKE, key_mask=FAKE), stca.OK),
    (dict(path=1), dict(score_bias=FAKE), stca.ERR_UNSUPPORTED),                # fused path
    (dict(dtype=stca.F32, d=64, H=2, hidden=64), dict(score_bias=FAKE), stca.ERR_UNSUPPORTED),
    ({}, dict(score_bias=FAKE + 4), stca.ERR_INVALID_ARG),                      # misaligned
    (dict(encoder=1, l_short=64), dict(score_bias=FAKE), stca.ERR_UNSUPPORTED),
])
def test_score_bias_validation(cover, bover, code):
    r, n = ws_size(cfg(**cover), batch(**bover))
    assert r == code, stca.last_error()
    if code == stca.OK:
        r0, n0 = ws_size(cfg(**cover), batch(**{k: v for k, v in bover.items() if k != "score_bias"}))
        assert n > n0            # the blocked copy of the bias lives in the workspace
    else:
        assert "bias" in stca.last_error() or "LONGER" in stca.last_error()


def test_score_bias_attention_and_backward_validation():
    lib = stca.load()
    a = stca.AttnArgs(B=2, d=256, H=8, dtype=stca.BF16, score=1, chunk_keys=0,
                      hist_offsets=FAKE, tgt_offsets=FAKE, n_hist=100, n_tgt=4,
                      max_tgt_per_user=2, q=FAKE, k=FAKE, v=FAKE, attn=FAKE, score_bias=FAKE)
    n = C.c_size_t(0)
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.OK
    a.score_bias = FAKE + 8
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.ERR_INVALID_ARG
    a.score_bias = FAKE
    a.dtype, a.d, a.H = stca.F32, 64, 2
    assert lib.stca_attention_workspace_size(C.byref(a), C.byref(n)) == stca.ERR_UNSUPPORTED
    c, b = cfg(), batch(score_bias=FAKE)
    w, keepw = _weights()
    g = stca.Grads()
    r = lib.stca_backward(C.byref(c), C.byref(b), C.byref(w), FAKE, C.byref(g), FAKE, 1 << 30, None)
    assert r == stca.ERR_UNSUPPORTED and "bias" in stca.last_error()


def test_noalloc_rejects_on_the_host_before_any_device_call():
    """stca_forward_noalloc validates and sizes the batch on the host first:
    invalid arguments and a workspace beyond the static scratch return at once
    (no GPU is touched, so this runs without one)."""
    lib = stca.load()
    w, keepw = _weights()
    out = stca.Outputs(z=FAKE)
    c = cfg()
    big = batch(n_hist=20_000_000, n_tgt=64, max_tgt_per_user=64)
    n = C.c_size_t(0)
    assert lib.stca_workspace_size(C.byref(c), C.byref(big), C.byref(n)) == stca.OK
    assert n.value > stca.NOALLOC_SCRATCH_BYTES
    r = lib.stca_forward_noalloc(C.byref(c), C.byref(big), C.byref(w), C.byref(out), None)
    assert r == stca.ERR_WORKSPACE and "static scratch" in stca.last_error()
    bad = cfg(H=7)
    r = lib.stca_forward_noalloc(C.byref(bad), C.byref(batch()), C.byref(w), C.byref(out), None)
    assert r == stca.ERR_INVALID_ARG


def test_peak_mfma_validation():
    lib = stca.load()
    assert lib.stca_peak_mfma_bf16(0, 10, C.c_void_p(FAKE), None, None) == stca.ERR_INVALID_ARG
    assert lib.stca_peak_mfma_bf16(4, 0, C.c_void_p(FAKE), None, None) == stca.ERR_INVALID_ARG
    assert lib.stca_peak_mfma_bf16(4, 10, None, None, None) == stca.ERR_INVALID_ARG


def test_peak_hbm_read_validation():
    lib = stca.load()
    for args in [(None, 1024, 4, FAKE), (FAKE, 0, 4, FAKE), (FAKE, 1000, 4, FAKE), (FAKE, 1024, 0, FAKE),
                 (FAKE, 1024, 4, None)]:
        buf, n, blocks, out = args
        assert lib.stca_peak_hbm_read(C.c_void_p(buf) if buf else None, n, blocks,
                                      C.c_void_p(out) if out else None, None) == stca.ERR_INVALID_ARG


def test_clock_ghz():
    # 2.3e6 shader cycles over 1e5 ticks of the 100 MHz counter = 2.3 GHz; a
    # row with no elapsed ticks (workgroup that did not exist) is ignored
    c = [[10, 1000, 10 + 2_300_000, 1000 + 100_000], [0, 0, 0, 0]]
    assert abs(stca.clock_ghz(c) - 2.3) < 1e-12


# ------------------------------------------------------- LONGER-style encoding
@pytest.mark.parametrize("over,bover,code", [
    (dict(encoder=1, l_short=256), {}, stca.OK),
    (dict(encoder=1, l_short=256, flags=0), {}, stca.OK),
    (dict(encoder=2), {}, stca.ERR_INVALID_ARG),
    (dict(encoder=1, l_short=0), {}, stca.ERR_INVALID_ARG),
    (dict(encoder=1, l_short=4097), {}, stca.ERR_INVALID_ARG),
    (dict(encoder=1, l_short=64, path=1), {}, stca.ERR_UNSUPPORTED),
    (dict(encoder=1, l_short=64, dtype=stca.F32), {}, stca.ERR_UNSUPPORTED),
    (dict(encoder=1, l_short=64, score=1), {}, stca.ERR_UNSUPPORTED),
    (dict(encoder=1, l_short=64, flags=stca.FLAG_DEDUP), {}, stca.ERR_UNSUPPORTED),
    (dict(encoder=1, l_short=64), dict(key_mask=FAKE), stca.ERR_UNSUPPORTED),
])
def test_longer_validation(over, bover, code):
    r, n = ws_size(cfg(**over), batch(**bover))
    assert r == code, stca.last_error()
    if code == stca.OK:
        assert n > 0


def test_longer_workspace_and_rejections():
    lib = stca.load()
    b = batch(n_hist=100_000, n_tgt=64, max_tgt_per_user=32)
    _, plain = ws_size(cfg(), b)
    _, lo = ws_size(cfg(encoder=1, l_short=256), b)
    # the raw K/V of one layer at a time, and every layer's B x l_short short rows
    assert lo > 2 * 100_000 * 256 * 2 + 4 * 2 * 256 * 256 * 2
    _, lo_small = ws_size(cfg(encoder=1, l_short=16), b)
    assert lo_small < lo
    c = cfg(encoder=1, l_short=256)
    w, keep = _weights()
    assert _forward(c, b, w, stca.Outputs(z=FAKE), lo) == stca.ERR_INVALID_ARG  # no encoder weights
    assert "encoder weight" in stca.last_error()
    for i in range(c.M):
        keep[i].enc_wq = keep[i].enc_wk = keep[i].enc_wv = keep[i].enc_wo = FAKE
    for f in ("x_dump", "kv_dump"):
        assert _forward(c, b, w, stca.Outputs(z=FAKE, **{f: FAKE}), lo) == stca.ERR_UNSUPPORTED
    assert _forward(c, b, w, stca.Outputs(z=FAKE), lo - 1) == stca.ERR_WORKSPACE
    n = C.c_size_t(0)
    assert lib.stca_backward_workspace_size(C.byref(c), C.byref(b), C.byref(n)) == stca.ERR_UNSUPPORTED
    assert "SwiGLU" in stca.last_error()


def test_forward_for_backward_rejects_on_the_host():
    """stca_forward_for_backward checks what the backward supports, z and the
    workspace before anything is enqueued; stca_backward with saved_forward
    refuses a z_out (z is the saving forward's output)."""
    lib = stca.load()
    w, keepw = _weights()
    b = batch()
    n = C.c_size_t(0)
    assert lib.stca_backward_workspace_size(C.byref(cfg()), C.byref(b), C.byref(n)) == stca.OK

    def ffb(c, z=FAKE, ws=FAKE, ws_bytes=None):
        return lib.stca_forward_for_backward(C.byref(c), C.byref(b), C.byref(w), z, None, ws,
                                             n.value if ws_bytes is None else ws_bytes, None)
    assert ffb(cfg(dtype=stca.F32, d=64, H=2, hidden=64)) == stca.ERR_UNSUPPORTED
    assert ffb(cfg(qmode=1)) == stca.ERR_UNSUPPORTED
    assert ffb(cfg(), z=None) == stca.ERR_INVALID_ARG and "z" in stca.last_error()
    assert ffb(cfg(), z=FAKE + 4) == stca.ERR_INVALID_ARG
    assert ffb(cfg(), ws_bytes=n.value - 1) == stca.ERR_WORKSPACE
    assert ffb(cfg(), ws=None) == stca.ERR_WORKSPACE
    lg = (stca.LayerGrad * 4)()
    fg = stca.FfnGrad(FAKE, FAKE, FAKE, FAKE, FAKE)
    for i in range(4):
        lg[i] = stca.LayerGrad(fg, fg, FAKE, FAKE, FAKE, FAKE, FAKE)
    g = stca.Grads(lg, fg, FAKE)
    g.z_out = FAKE
    g.saved_forward = 1
    r = lib.stca_backward(C.byref(cfg()), C.byref(b), C.byref(w), FAKE, C.byref(g), FAKE, n.value, None)
    assert r == stca.ERR_INVALID_ARG and "saved_forward" in stca.last_error()
