"""Pins for the float64 backward oracle (CPU only).

The gradient oracle is tied to things other than itself:
* central finite differences of the float64 *forward* oracle (itself pinned in
  test_oracle_pins.py) along random directions, for every weight tensor and
  for the embedding rows, in softmax and ReLU mode, with and without the
  history LN and the z LN, on batches with repeated ids, an empty history and a
  user without targets;
* torch autograd (float64, CPU) of LayerNorm, of a SiLU-gated FFN and of
  scaled-dot-product attention: library derivatives of the same blocks;
* closed forms: one key under softmax has no key gradient and passes the
  upstream gradient straight to its value.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import stca_grad as G
from oracle import stca_oracle as O


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- blocks vs autograd
def test_ln_backward_matches_autograd():
    g = rng(1)
    x = g.normal(size=(7, 12)) * 2 + 0.5
    gam, bet, dy = g.normal(size=12), g.normal(size=12), g.normal(size=(7, 12))
    y, cache = G.ln_forward(x, gam, bet)
    dx, dg, db = G.ln_backward(dy, cache, gam)
    tx, tg, tb = (torch.tensor(a, requires_grad=True) for a in (x, gam, bet))
    ty = F.layer_norm(tx, (12,), tg, tb, eps=1e-5)
    ty.backward(torch.from_numpy(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_swiglu_backward_matches_autograd():
    g = rng(2)
    d, h = 6, 10
    x = g.normal(size=(5, d))
    w = {"w1": g.normal(size=(d, h)), "w3": g.normal(size=(d, h)), "w2": g.normal(size=(h, d))}
    dy = g.normal(size=(5, d))
    y, cache = G.swiglu_forward(x, w)
    dx, gw = G.swiglu_backward(dy, cache, w)
    tx = torch.tensor(x, requires_grad=True)
    tw = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    ty = (F.silu(tx @ tw["w1"]) * (tx @ tw["w3"])) @ tw["w2"]
    ty.backward(torch.from_numpy(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    for k in w:
        np.testing.assert_allclose(gw[k], tw[k].grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("m,L,H", [(1, 9, 2), (5, 17, 4), (3, 1, 1)])
def test_softmax_attention_backward_matches_autograd(m, L, H):
    g = rng(3 + m)
    d = 8 * H
    Q, K, V, dA = g.normal(size=(m, d)), g.normal(size=(L, d)), g.normal(size=(L, d)), g.normal(size=(m, d))
    dQ, dK, dV = G.attention_backward(Q, K, V, dA, H, "softmax")
    dh = d // H
    tq, tk, tv = (torch.tensor(a.reshape(a.shape[0], H, dh).transpose(1, 0, 2).copy(), requires_grad=True)
                  for a in (Q, K, V))
    ta = F.scaled_dot_product_attention(tq, tk, tv)               # [H, m, dh], scale 1/sqrt(dh)
    ta.backward(torch.from_numpy(dA.reshape(m, H, dh).transpose(1, 0, 2).copy()))
    back = lambda t: t.grad.numpy().transpose(1, 0, 2).reshape(-1, d)
    np.testing.assert_allclose(G.attention_forward(Q, K, V, H, "softmax"),
                               ta.detach().numpy().transpose(1, 0, 2).reshape(m, d), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dQ, back(tq), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dK, back(tk), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dV, back(tv), rtol=1e-9, atol=1e-12)


def test_single_key_softmax_closed_form():
    """One key: the weight is 1 whatever the score, so the key (and the query)
    get no gradient and the value gets the sum of the upstream gradients."""
    g = rng(4)
    Q, K, V, dA = g.normal(size=(4, 16)), g.normal(size=(1, 16)), g.normal(size=(1, 16)), g.normal(size=(4, 16))
    dQ, dK, dV = G.attention_backward(Q, K, V, dA, 2, "softmax")
    assert np.abs(dK).max() < 1e-15 and np.abs(dQ).max() < 1e-15
    np.testing.assert_allclose(dV[0], dA.sum(axis=0), rtol=1e-14)


def test_relu_attention_backward_matches_autograd():
    g = rng(5)
    m, L, H, d = 3, 11, 2, 16
    Q, K, V, dA = g.normal(size=(m, d)), g.normal(size=(L, d)), g.normal(size=(L, d)), g.normal(size=(m, d))
    dQ, dK, dV = G.attention_backward(Q, K, V, dA, H, "relu")
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    dh, outs = d // H, []
    for e in range(H):
        c = slice(e * dh, (e + 1) * dh)
        outs.append(torch.relu(tq[:, c] @ tk[:, c].T / math.sqrt(dh)) @ tv[:, c])
    torch.cat(outs, dim=1).backward(torch.from_numpy(dA))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------- whole chain vs finite differences
def _ffn(g, d, h, ln):
    w = {"w1": g.normal(size=(d, h)) / math.sqrt(d), "w3": g.normal(size=(d, h)) / math.sqrt(d),
         "w2": g.normal(size=(h, d)) / math.sqrt(h)}
    if ln:
        w["ln_g"] = 1.0 + 0.3 * g.normal(size=d)
        w["ln_b"] = 0.2 * g.normal(size=d)
    return w


def _model(seed, d=8, H=2, h=12, M=3, kv_ln=True, z_ln=False):
    g = rng(seed)
    layers = []
    for i in range(M):
        lw = {"kv": _ffn(g, d, h, True), "q": _ffn(g, d, h, True)}
        for k in ("wk", "wv", "wq", "wo"):
            lw[k] = g.normal(size=(d, d)) / math.sqrt(d)
        if i > 0:
            lw["wc"] = g.normal(size=((i + 1) * d, d)) / math.sqrt((i + 1) * d)
        layers.append(lw)
    z = _ffn(g, d, h, True)
    wz = g.normal(size=((M + 1) * d, d)) / math.sqrt((M + 1) * d)
    return layers, z, wz


def _batch(seed, d, N=20):
    g = rng(seed)
    table = g.normal(size=(N, d))
    hist_len = [5, 0, 3, 4]             # user 1: empty history
    tgt_len = [2, 1, 1, 0]              # user 3: no target
    ho = np.concatenate([[0], np.cumsum(hist_len)])
    to = np.concatenate([[0], np.cumsum(tgt_len)])
    hist_ids = g.integers(0, 6, size=ho[-1])         # few distinct ids: repeats
    hist_ids[2] = N + 3                               # out of range: a zero row
    tgt_ids = g.integers(0, N, size=to[-1])
    tgt_ids[0] = hist_ids[0]                          # a row read as target and history
    return table, ho, to, hist_ids, tgt_ids


def _rows(table):
    def f(ids):
        ids = np.asarray(ids, dtype=np.int64)
        out = np.zeros((len(ids), table.shape[1]))
        ok = (ids >= 0) & (ids < len(table))
        out[ok] = table[ids[ok]]
        return out
    return f


def _loss(cfg, table, ho, to, hist_ids, tgt_ids, layers, z, wz, dz):
    out = O.forward(cfg, ho, hist_ids, to, _rows(table), layers, z, wz, tgt_ids=tgt_ids,
                    want=("z",))
    return float(np.sum(out["z"] * dz))


def _leaves(layers, z, wz):
    """(getter path, array) for every weight tensor."""
    out = []
    for i, lw in enumerate(layers):
        for side in ("kv", "q"):
            for k in lw[side]:
                out.append((("layers", i, side, k), lw[side][k]))
        for k in ("wk", "wv", "wq", "wo", "wc"):
            if k in lw:
                out.append((("layers", i, k), lw[k]))
    for k in z:
        out.append((("z", k), z[k]))
    out.append((("wz",), wz))
    return out


def _get(grads, path):
    g = grads
    for p in path:
        g = g[p]
    return g


@pytest.mark.parametrize("score,kv_ln,z_ln", [("softmax", True, False), ("softmax", False, True),
                                              ("relu", True, True)])
def test_chain_gradient_matches_finite_differences(score, kv_ln, z_ln):
    d, H, M = 8, 2, 3
    layers, z, wz = _model(7, d=d, H=H, M=M, z_ln=z_ln)
    if not kv_ln:
        for lw in layers:
            lw["kv"].pop("ln_g")
            lw["kv"].pop("ln_b")
    if not z_ln:
        z.pop("ln_g")
        z.pop("ln_b")
    table, ho, to, hist_ids, tgt_ids = _batch(8, d)
    cfg = dict(d=d, H=H, M=M, score=score, qmode="fusion", kv_ln=kv_ln, z_ln=z_ln)
    g = rng(9)
    dz = g.normal(size=(to[-1], d))
    res = G.backward(cfg, ho, hist_ids, to, tgt_ids, _rows(table), layers, z, wz, dz)
    if score == "relu":
        # no score within reach of the kink at 0 for the step used below
        fw = O.forward(cfg, ho, hist_ids, to, _rows(table), layers, z, wz, tgt_ids=tgt_ids)
        smin = np.inf
        for u in range(len(ho) - 1):
            X = _rows(table)(hist_ids[ho[u]:ho[u + 1]])
            for i in range(M):
                K, _ = O.encode_history(X, layers[i], kv_ln)
                for t in range(to[u], to[u + 1]):
                    for e in range(H):
                        c = slice(e * d // H, (e + 1) * d // H)
                        if len(K):
                            smin = min(smin, np.abs(K[:, c] @ fw["qs"][i, t, c]).min())
        assert smin > 1e-4
    eps = 1e-6
    # z of the recomputed forward equals the forward oracle's
    fz = O.forward(cfg, ho, hist_ids, to, _rows(table), layers, z, wz, tgt_ids=tgt_ids)["z"]
    np.testing.assert_allclose(res["z"], fz, rtol=1e-12, atol=1e-12)
    for path, arr in _leaves(layers, z, wz):
        v = g.normal(size=arr.shape)
        saved = arr.copy()
        arr += eps * v
        lp = _loss(cfg, table, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)
        arr[...] = saved - eps * v
        lm = _loss(cfg, table, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)
        arr[...] = saved
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(_get(res["grads"], path) * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (path, fd, an)
    # embedding rows: the scatter-added table gradient
    gt = G.table_grad(len(table), d, hist_ids, tgt_ids, res["d_hist"], res["d_tgt"])
    for _ in range(3):
        v = g.normal(size=table.shape)
        lp = _loss(cfg, table + eps * v, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)
        lm = _loss(cfg, table - eps * v, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(gt * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (fd, an)
    # structure: the zero row read through an out-of-range id gets nothing in
    # the table, users without targets give zero rows
    assert np.all(res["d_hist"][ho[3]:ho[4]] == 0)


def test_per_token_gradient_single_coordinate():
    """One coordinate of one history row perturbed alone (a row used by a
    single token), against the per-token gradient."""
    d, H, M = 8, 2, 2
    layers, z, wz = _model(21, d=d, H=H, M=M)
    z.pop("ln_g")
    z.pop("ln_b")
    table, ho, to, hist_ids, tgt_ids = _batch(22, d, N=40)
    hist_ids = np.arange(len(hist_ids)) + 10           # every token its own row
    tgt_ids = np.arange(len(tgt_ids)) + 30
    cfg = dict(d=d, H=H, M=M, score="softmax", qmode="fusion", kv_ln=True, z_ln=False)
    dz = rng(23).normal(size=(to[-1], d))
    res = G.backward(cfg, ho, hist_ids, to, tgt_ids, _rows(table), layers, z, wz, dz)
    eps = 1e-6
    for tok, col in ((0, 3), (7, 5), (9, 0)):
        tp, tm = table.copy(), table.copy()
        tp[hist_ids[tok], col] += eps
        tm[hist_ids[tok], col] -= eps
        fd = (_loss(cfg, tp, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)
              - _loss(cfg, tm, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)) / (2 * eps)
        assert abs(fd - res["d_hist"][tok, col]) <= 1e-6 * max(1.0, abs(fd))
    for t, col in ((0, 1), (3, 7)):
        tp, tm = table.copy(), table.copy()
        tp[tgt_ids[t], col] += eps
        tm[tgt_ids[t], col] -= eps
        fd = (_loss(cfg, tp, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)
              - _loss(cfg, tm, ho, to, hist_ids, tgt_ids, layers, z, wz, dz)) / (2 * eps)
        assert abs(fd - res["d_tgt"][t, col]) <= 1e-6 * max(1.0, abs(fd))
