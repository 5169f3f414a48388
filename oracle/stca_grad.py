"""Float64 CPU oracle for the STCA backward pass (gradients of a training step).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``.  It shares no code with the HIP
implementation.

Training uses the same STCA forward as serving ([Review] "核心公式": the
single-layer attention, the inter-layer fusion, and the per-user RLB loss
L_u = (1/m) sum_k BCE(y_hat(u, t_k), y_k); [Notes] "短序列训练，长序列推理":
training on Beta-sampled lengths).  The prediction head that turns z into
y_hat (RankMixer, sigmoid) is outside this library, so the backward takes the
gradient of the loss with respect to z, dz [T, d], and returns the gradient of
every STCA weight and of every embedding row the forward read.

What it computes is the chain rule applied to the forward of
``stca_oracle.forward`` in float64, step by step in reverse order, per user,
with every activation recomputed from the inputs (nothing is shared with a
GPU run).  The only reading added to those of the forward: ReLU scores take
derivative 0 at s = 0 exactly (the subgradient of max(0, s) used by every
framework).  Gradients of the table are summed over every token and target
that reads a row; out-of-range ids (zero rows in the forward) get none.

Pins (``tests/test_grad_oracle_pins.py``): central finite differences of the
float64 forward oracle along random directions, for every weight tensor and
the table rows, in softmax and ReLU mode, with and without the history LN and
the z LN; closed forms for single-key softmax (zero key gradient, value
gradient = sum of the upstream gradients) and for all-positive ReLU scores
(linear attention).  Only fusion (STCA) query mode is covered.
"""
from __future__ import annotations

import math

import numpy as np

from .stca_oracle import LN_EPS, silu, stored_to_f64, weights_f64


# ---------------------------------------------------------------- blocks
def ln_forward(x, g, b, eps=LN_EPS):
    """LayerNorm over the last axis; returns (y, (xhat, rstd))."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    return xhat * g + b, (xhat, rstd)


def ln_backward(dy, cache, g):
    """d/dx of y = xhat * g + b with xhat = (x - mean) / sqrt(var + eps):
    dx = rstd * (gy - mean(gy) - xhat * mean(gy * xhat)), gy = dy * g;
    dg = sum_rows dy * xhat, db = sum_rows dy."""
    xhat, rstd = cache
    gy = dy * g
    dx = rstd * (gy - gy.mean(axis=-1, keepdims=True)
                 - xhat * (gy * xhat).mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def silu_grad(u):
    """d/du of u * sigmoid(u) = sigmoid(u) * (1 + u * (1 - sigmoid(u)))."""
    sg = 1.0 / (1.0 + np.exp(-u))
    return sg * (1.0 + u * (1.0 - sg))


def swiglu_forward(x, w):
    """(SiLU(x W1) * (x W3)) W2; returns (y, cache)."""
    h1 = x @ w["w1"]
    h3 = x @ w["w3"]
    gt = silu(h1) * h3
    return gt @ w["w2"], (x, h1, h3, gt)


def swiglu_backward(dy, cache, w):
    """Gradients of y = (SiLU(x W1) * (x W3)) W2 for row-stacked x."""
    x, h1, h3, gt = cache
    dg = dy @ w["w2"].T
    dh1 = dg * h3 * silu_grad(h1)
    dh3 = dg * silu(h1)
    grads = {"w1": x.T @ dh1, "w3": x.T @ dh3, "w2": gt.T @ dy}
    return dh1 @ w["w1"].T + dh3 @ w["w3"].T, grads


def ffn_ln_forward(x, w, ln):
    y, c1 = swiglu_forward(x, w)
    if not ln:
        return y, (c1, None)
    out, c2 = ln_forward(y, w["ln_g"], w["ln_b"])
    return out, (c1, c2)


def ffn_ln_backward(dout, cache, w, ln, grads):
    """Accumulates into ``grads`` (keys w1, w3, w2, ln_g, ln_b); returns dx."""
    c1, c2 = cache
    if ln:
        dy, dg, db = ln_backward(dout, c2, w["ln_g"])
        grads["ln_g"] += dg
        grads["ln_b"] += db
    else:
        dy = dout
    dx, g = swiglu_backward(dy, c1, w)
    for k in ("w1", "w3", "w2"):
        grads[k] += g[k]
    return dx


# ---------------------------------------------------------------- attention
def attention_backward(Qs, K, V, dA, H, score, scale=None):
    """All targets of one user against that user's keys, per head eta:
    s = scale * Q_eta K_eta^T ([m, L]);
    softmax: p = exp(s - max) / sum, a = p V_eta,
             dp = dA_eta V_eta^T, ds = p * (dp - rowsum(p * dp));
    relu:    p = max(0, s), a = p V_eta, dp = dA_eta V_eta^T, ds = dp * [s > 0];
    dV_eta = p^T dA_eta, dK_eta = scale ds^T Q_eta, dQ_eta = scale ds K_eta.
    ([Review] formula for alpha and o; [WeChat] §1.2 for the ReLU form.)
    Returns (dQ [m, d], dK [L, d], dV [L, d]) for Q = q W_Q before the scale."""
    m, d = Qs.shape
    L = K.shape[0]
    dh = d // H
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    dQ, dK, dV = np.zeros((m, d)), np.zeros((L, d)), np.zeros((L, d))
    if L == 0 or m == 0:
        return dQ, dK, dV
    for eta in range(H):
        cols = slice(eta * dh, (eta + 1) * dh)
        q, k, v, da = Qs[:, cols], K[:, cols], V[:, cols], dA[:, cols]
        s = scale * (q @ k.T)
        dp = da @ v.T
        if score == "softmax":
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        elif score == "relu":
            p = np.maximum(s, 0.0)
            ds = dp * (s > 0.0)
        else:
            raise ValueError(score)
        dV[:, cols] = p.T @ da
        dK[:, cols] = scale * (ds.T @ q)
        dQ[:, cols] = scale * (ds @ k)
    return dQ, dK, dV


def attention_forward(Qs, K, V, H, score, scale=None):
    """The forward of ``attention_backward`` for all targets of one user."""
    m, d = Qs.shape
    L = K.shape[0]
    dh = d // H
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    a = np.zeros((m, d))
    if L == 0:
        return a
    for eta in range(H):
        cols = slice(eta * dh, (eta + 1) * dh)
        s = scale * (Qs[:, cols] @ K[:, cols].T)
        if score == "softmax":
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
        else:
            p = np.maximum(s, 0.0)
        a[:, cols] = p @ V[:, cols]
    return a


# ---------------------------------------------------------------- whole model
def _zeros_like_ffn(w, ln):
    g = {k: np.zeros_like(w[k]) for k in ("w1", "w3", "w2")}
    if ln:
        g["ln_g"] = np.zeros_like(w["ln_g"])
        g["ln_b"] = np.zeros_like(w["ln_b"])
    return g


def zero_grads(cfg, layers, z, wz):
    M = cfg["M"]
    out = {"layers": [], "z": _zeros_like_ffn(z, cfg["z_ln"]), "wz": np.zeros_like(wz)}
    for i in range(M):
        lw = layers[i]
        g = {"kv": _zeros_like_ffn(lw["kv"], cfg["kv_ln"]), "q": _zeros_like_ffn(lw["q"], True),
             "wk": np.zeros_like(lw["wk"]), "wv": np.zeros_like(lw["wv"]),
             "wq": np.zeros_like(lw["wq"]), "wo": np.zeros_like(lw["wo"])}
        if i > 0:
            g["wc"] = np.zeros_like(lw["wc"])
        out["layers"].append(g)
    return out


def backward(cfg, hist_offsets, hist_ids, tgt_offsets, tgt_ids, rows_f64, layers, z, wz, dz,
             users=None):
    """Gradients of sum_t <dz_t, z_t> for the STCA forward (fusion mode).

    cfg: d, H, M, score, kv_ln, z_ln (qmode must be "fusion").
    rows_f64: callable ids -> float64 rows (zero rows for out-of-range ids).
    dz: [T, d] upstream gradient; targets of users outside ``users`` are
        ignored (their rows of the per-token outputs stay zero).
    Returns a dict: ``grads`` (same nesting as the weights: layers[i]["kv"|"q"]
    with w1, w3, w2, ln_g, ln_b; wk, wv, wq, wo, wc (i > 0); z; wz), ``d_hist``
    [n_hist, d] per history token, ``d_tgt`` [T, d] per target, and ``z`` [T, d]
    (the recomputed forward output).
    """
    if cfg.get("qmode", "fusion") != "fusion":
        raise ValueError("the backward oracle covers fusion (STCA) query mode")
    d, H, M, score = cfg["d"], cfg["H"], cfg["M"], cfg["score"]
    kv_ln, z_ln = cfg["kv_ln"], cfg["z_ln"]
    ho = np.asarray(hist_offsets, dtype=np.int64)
    to = np.asarray(tgt_offsets, dtype=np.int64)
    B = len(ho) - 1
    T = int(to[-1])
    grads = zero_grads(cfg, layers, z, wz)
    d_hist = np.zeros((int(ho[-1]), d))
    d_tgt = np.zeros((T, d))
    zout = np.zeros((T, d))
    dz = np.asarray(dz, dtype=np.float64)
    for u in (range(B) if users is None else users):
        h0, h1 = int(ho[u]), int(ho[u + 1])
        t0, t1 = int(to[u]), int(to[u + 1])
        if t1 == t0:
            continue                        # no target reads this history
        X = rows_f64(np.asarray(hist_ids[h0:h1])) if h1 > h0 else np.zeros((0, d))
        xt = rows_f64(np.asarray(tgt_ids[t0:t1]))
        # ---- forward, keeping what the chain rule needs
        hist = []
        for i in range(M):
            lw = layers[i]
            xtil, c = ffn_ln_forward(X, lw["kv"], kv_ln)
            hist.append((xtil, c, xtil @ lw["wk"], xtil @ lw["wv"]))
        q, qc = ffn_ln_forward(xt, layers[0]["q"], True)
        qside, outs, cats = [], [], []
        for i in range(M):
            lw = layers[i]
            Q = q @ lw["wq"]
            a = attention_forward(Q, hist[i][2], hist[i][3], H, score)
            o = a @ lw["wo"]
            qside.append((q, qc, Q, a))
            outs.append(o)
            if i + 1 < M:
                cat = np.concatenate(outs + [xt], axis=1)
                cats.append(cat)
                q, qc = ffn_ln_forward(cat @ layers[i + 1]["wc"], layers[i + 1]["q"], True)
        catz = np.concatenate(outs + [xt], axis=1)
        zz, zc = ffn_ln_forward(catz @ wz, z, z_ln)
        zout[t0:t1] = zz
        # ---- backward
        dcz = ffn_ln_backward(dz[t0:t1], zc, z, z_ln, grads["z"])
        grads["wz"] += catz.T @ dcz
        dcat = dcz @ wz.T
        do = [dcat[:, k * d:(k + 1) * d].copy() for k in range(M)]
        dxt = dcat[:, M * d:].copy()
        dX = np.zeros_like(X)
        for i in reversed(range(M)):
            lw, g = layers[i], grads["layers"][i]
            qi, qci, Q, a = qside[i]
            g["wo"] += a.T @ do[i]
            da = do[i] @ lw["wo"].T
            xtil, hc, K, V = hist[i]
            dQ, dK, dV = attention_backward(Q, K, V, da, H, score)
            g["wq"] += qi.T @ dQ
            dqi = dQ @ lw["wq"].T
            dc = ffn_ln_backward(dqi, qci, lw["q"], True, g["q"])
            if i > 0:
                g["wc"] += cats[i - 1].T @ dc
                dci = dc @ lw["wc"].T
                for k in range(i):
                    do[k] += dci[:, k * d:(k + 1) * d]
                dxt += dci[:, i * d:]
            else:
                dxt += dc
            # history side of layer i
            g["wk"] += xtil.T @ dK
            g["wv"] += xtil.T @ dV
            dxtil = dK @ lw["wk"].T + dV @ lw["wv"].T
            dX += ffn_ln_backward(dxtil, hc, lw["kv"], kv_ln, g["kv"])
        d_hist[h0:h1] = dX
        d_tgt[t0:t1] = dxt
    return {"grads": grads, "d_hist": d_hist, "d_tgt": d_tgt, "z": zout}


def table_grad(table_rows, d, hist_ids, tgt_ids, d_hist, d_tgt):
    """Scatter-add of the per-token and per-target row gradients into a dense
    [table_rows, d] gradient; out-of-range ids contribute nothing."""
    g = np.zeros((table_rows, d))
    for ids, rows in ((hist_ids, d_hist), (tgt_ids, d_tgt)):
        ids = np.asarray(ids, dtype=np.int64)
        ok = (ids >= 0) & (ids < table_rows)
        np.add.at(g, ids[ok], rows[ok])
    return g


def backward_problem(p, dz, users=None):
    """Convenience wrapper over a ``recsys_ultra_long_amd.inputs.Problem``."""
    sp = p.spec
    layers, z, wz = weights_f64(p.layers, p.z, p.wz)
    cfg = dict(d=sp.d, H=sp.H, M=sp.M, score=sp.score, qmode=sp.qmode,
               kv_ln=sp.kv_ln, z_ln=sp.z_ln)
    def rows(ids):
        ids = np.asarray(ids, dtype=np.int64)
        out = np.zeros((len(ids), sp.d))
        ok = (ids >= 0) & (ids < sp.table_rows)
        if ok.any():
            out[ok] = stored_to_f64(p.rows(ids[ok]))
        return out
    return backward(cfg, p.hist_offsets, p.hist_ids, p.tgt_offsets, p.tgt_ids, rows,
                    layers, z, wz, dz, users=users)
