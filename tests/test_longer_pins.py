"""Pins for the oracle's LONGER-style sequence encoding (CPU only):
[HyFormer] §3.4.1 (ii) eq. (6), H_l = CrossAttn(S_short, S, S), followed by
eq. (8), K_l = H_l W_K, V_l = H_l W_V.

CrossAttn is checked against torch's multi-head attention in float64 (an
independent implementation of the same standard operation, with in- and
out-projections and no biases), with the short sequence taken as the user's
last min(L, L_H) rows -- the reading the oracle documents.  Closed forms pin
the degenerate cases (a zero query projection averages the values; one item
returns its value row; an empty history gives no rows), and a forward-level
closed form pins the encoder's place in the layer: with identity encoder
value/output projections and a zero query projection every short row is the
history mean, so every target's attention output is mean(X) W_V.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import stca_oracle as O
from recsys_ultra_long_amd import inputs as I


def _enc(rng, d):
    return {k: rng.normal(size=(d, d)) / np.sqrt(d) for k in ("wq", "wk", "wv", "wo")}


def _torch_cross_attention(X, enc, ls, H):
    """torch's multi-head attention, query = last ls rows of X, key = value = X."""
    d = X.shape[1]
    x = torch.from_numpy(X).unsqueeze(1)                       # [L, 1, d]
    q = x[X.shape[0] - ls:]
    w_in = torch.from_numpy(np.concatenate([enc["wq"].T, enc["wk"].T, enc["wv"].T]))
    out, _ = F.multi_head_attention_forward(
        q, x, x, d, H, w_in, None, None, None, False, 0.0,
        torch.from_numpy(enc["wo"].T), None, training=False, need_weights=False)
    return out[:, 0].numpy()


@pytest.mark.parametrize("L,l_short,H", [(40, 8, 4), (5, 8, 2), (8, 8, 4), (33, 1, 8)])
def test_cross_attention_matches_torch(L, l_short, H):
    rng = np.random.default_rng(L * 100 + l_short)
    d = 64
    X = rng.normal(size=(L, d))
    enc = _enc(rng, d)
    got = O.longer_encode(X, enc, l_short, H)
    ls = min(L, l_short)
    assert got.shape == (ls, d)
    np.testing.assert_allclose(got, _torch_cross_attention(X, enc, ls, H), rtol=1e-11, atol=1e-12)


def test_zero_query_projection_averages_the_values():
    rng = np.random.default_rng(1)
    d, H = 64, 4
    X = rng.normal(size=(30, d))
    enc = _enc(rng, d)
    enc["wq"] = np.zeros((d, d))
    got = O.longer_encode(X, enc, 6, H)
    want = (X @ enc["wv"]).mean(axis=0) @ enc["wo"]
    np.testing.assert_allclose(got, np.tile(want, (6, 1)), rtol=1e-12, atol=1e-13)


def test_one_item_returns_its_value_row_and_empty_gives_nothing():
    rng = np.random.default_rng(2)
    d, H = 64, 2
    x = rng.normal(size=(1, d))
    enc = _enc(rng, d)
    np.testing.assert_allclose(O.longer_encode(x, enc, 4, H), x @ enc["wv"] @ enc["wo"], rtol=1e-12)
    assert O.longer_encode(np.zeros((0, d)), enc, 4, H).shape == (0, d)


def test_short_rows_are_the_most_recent_items():
    # only the last row differs from the others: with L_H = 1 the single
    # query must be that row (a query from any other row would differ)
    rng = np.random.default_rng(3)
    d, H = 64, 4
    base = rng.normal(size=d)
    X = np.tile(base, (12, 1))
    X[-1] = rng.normal(size=d)
    enc = _enc(rng, d)
    got = O.longer_encode(X, enc, 1, H)
    np.testing.assert_allclose(got, _torch_cross_attention(X, enc, 1, H), rtol=1e-11)
    other = _torch_cross_attention(np.concatenate([X[-1:], X[:-1]]), enc, 1, H)
    assert np.abs(got - other).max() > 1e-3


def test_forward_decodes_the_encoded_rows():
    # identity encoder value / output projections and a zero query projection:
    # every short row is mean(X), so K and V rows are all equal and each
    # target's attention output is mean(X) W_V (softmax over equal keys)
    sp = replace(I.spec(2), B=3, L=None, L_max=200, L_min=16, M=2, table_rows=5000, m=3,
                 encoder="longer", l_short=12, dtype="bf16")
    p = I.make_problem(sp)
    layers, z, wz = O.weights_f64(p.layers, p.z, p.wz)
    d = sp.d
    for lw in layers:
        lw["enc"] = {"wq": np.zeros((d, d)), "wk": lw["enc"]["wk"], "wv": np.eye(d), "wo": np.eye(d)}
    cfg = dict(d=d, H=sp.H, M=sp.M, score="softmax", qmode=sp.qmode, kv_ln=sp.kv_ln, z_ln=sp.z_ln,
               encoder="longer", l_short=sp.l_short)
    rows = lambda ids: O.stored_to_f64(p.rows(ids))
    out = O.forward(cfg, p.hist_offsets, p.hist_ids, p.tgt_offsets, rows, layers, z, wz, tgt_ids=p.tgt_ids)
    for u in range(sp.B):
        X = rows(p.hist_ids[p.hist_offsets[u]:p.hist_offsets[u + 1]])
        for i in range(sp.M):
            want = X.mean(axis=0) @ layers[i]["wv"]
            for t in range(p.tgt_offsets[u], p.tgt_offsets[u + 1]):
                np.testing.assert_allclose(out["attn"][i, t], want, rtol=1e-10, atol=1e-12)
