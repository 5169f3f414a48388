"""Conditioning of the STCA forward: how far the end-to-end outputs move when
the exact float64 computation stores its intermediates at a lower precision.

``perturbed_forward`` composes the oracle's own steps (``oracle.stca_oracle``:
SwiGLU pieces, LayerNorm, the attention formulas of one head) and rounds
chosen intermediates to bf16 or fp32 before the next step reads them.  With
no rounding it is the oracle's forward.  The rounding points model where a
GPU implementation with bf16 (or fp32) storage and wide accumulation has to
store a value:

* ``kv``     the history keys and values K, V;
* ``hidden`` the SwiGLU gate product SiLU(x W1) * (x W3) before W2;
* ``ln``     the FFN(+LN) output that the next product reads (history X~,
             query q);
* ``pre``    the concat product [o_1 .. o_i | x_t] W_C (and W_Z) that the
             query-side FFN reads;
* ``q``      the scaled query rows Q = q W_Q / sqrt(d_h);
* ``w``      the attention weights of the value product (softmax p, ReLU
             max(0, s));
* ``attn``   the attention output that W_O reads;
* ``o``      the layer outputs as the concat of later layers reads them.

The deviation of the end-to-end outputs from the exact ones under such a
rounding is a property of the method on that input (its conditioning), not of
any implementation: it is the error an implementation that stores at that
precision cannot avoid in general.  Test infrastructure only; it shares no
code with the HIP path.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import stca_oracle as O

ALL_POINTS = ("kv", "hidden", "ln", "pre", "q", "w", "attn", "o")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest) -> bf16 (nearest, ties to even), as float64."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


ROUND = {"bf16": round_bf16, "f32": round_f32}


def _ffn(x, w, ln, rp):
    """(SiLU(x W1) * (x W3)) W2 [-> LN] with the hidden product rounded at
    ``hidden`` and the output at ``ln`` (the caller decides the latter)."""
    g = rp("hidden", O.silu(x @ w["w1"]) * (x @ w["w3"]))
    y = g @ w["w2"]
    return O.layer_norm(y, w["ln_g"], w["ln_b"]) if ln else y


def _attention(Q, K, V, H, score, rp, at, key_mask=None, head_map=None, bias=None):
    """One target, every head: the oracle's two-pass formulas, evaluated in
    the float type ``at``, with the value product's weights rounded at ``w``
    (Cross-Mask masks and maps and the score bias as in the oracle)."""
    Q, K, V = Q.astype(at), K.astype(at), V.astype(at)
    d = Q.shape[0]
    dh = d // H
    a = np.zeros(d, dtype=Q.dtype)
    if K.shape[0] == 0:
        return a
    for h in range(H):
        c = slice(h * dh, (h + 1) * dh)
        hq = h if head_map is None else int(head_map[h])
        cq = slice(hq * dh, (hq + 1) * dh)
        Kh, Vh = K, V
        bh = None if bias is None else bias[:, h].astype(at)
        if key_mask is not None:
            sel = ((np.asarray(key_mask, dtype=np.int64) >> h) & 1).astype(bool)
            if not sel.any():
                continue
            Kh, Vh = K[sel], V[sel]
            bh = None if bh is None else bh[sel]
        s = Kh[:, cq] @ Q[cq]
        if bh is not None:
            s = s + bh
        if score == "softmax":
            p = rp("w", np.exp(s - s.max())).astype(at)
            a[c] = (p @ Vh[:, c]) / p.sum()
        else:
            a[c] = rp("w", np.maximum(s, 0.0)).astype(at) @ Vh[:, c]
    return a


def perturbed_forward(p, precision: str = "bf16", points=ALL_POINTS, users=None, arith: str = "f64",
                      attn_arith=None):
    """The forward of ``p`` (fusion or linear query mode, SwiGLU history
    encoding) with the intermediates named in ``points`` rounded to
    ``precision``.  ``arith = "f32"`` evaluates the row steps (FFN, LN,
    products with the weights) in float32 arithmetic (numpy's float32
    products and reductions) instead of float64; ``attn_arith`` does the same
    for the attention's scores and sums (default: ``arith``).
    Returns {"z", "o", "attn"} indexed like the oracle's."""
    rnd = ROUND[precision]
    pts = set(points)
    ft = np.float32 if arith == "f32" else np.float64
    at = np.float32 if (attn_arith or arith) == "f32" else np.float64

    def rp(name, x):
        return rnd(x).astype(ft) if name in pts else x

    def cast(w):
        if isinstance(w, dict):
            return {k: cast(v) for k, v in w.items()}
        if isinstance(w, list):
            return [cast(v) for v in w]
        return None if w is None else np.asarray(w, ft)

    sp = p.spec
    d, H, M = sp.d, sp.H, sp.M
    dh = d // H
    layers, zw, wz = (cast(w) for w in O.weights_f64(p.layers, p.z, p.wz))
    scale = ft(1.0 / math.sqrt(dh))
    ho, to = p.hist_offsets.astype(np.int64), p.tgt_offsets.astype(np.int64)
    T = int(to[-1])
    out = {"z": np.zeros((T, d)), "o": np.zeros((M, T, d)), "attn": np.zeros((M, T, d))}
    km_all, hmap, sb_all = p.extra.get("key_mask"), p.extra.get("head_map"), p.extra.get("score_bias")
    for u in (range(sp.B) if users is None else users):
        ids = p.hist_ids[ho[u]:ho[u + 1]]
        km = None if km_all is None else np.asarray(km_all)[ho[u]:ho[u + 1]]
        sb = None if sb_all is None else np.asarray(sb_all, np.float64)[ho[u]:ho[u + 1]]
        X = (O.stored_to_f64(p.rows(ids)) if len(ids) else np.zeros((0, d))).astype(ft)
        KV = []
        for i in range(M):
            xt = rp("ln", _ffn(X, layers[i]["kv"], sp.kv_ln, rp))
            KV.append((rp("kv", xt @ layers[i]["wk"]), rp("kv", xt @ layers[i]["wv"])))
        for t in range(int(to[u]), int(to[u + 1])):
            if sp.qmode == "fusion":
                x_t = O.stored_to_f64(p.rows(np.asarray([p.tgt_ids[t]])))[0].astype(ft)
                q = rp("ln", _ffn(x_t, layers[0]["q"], True, rp))
            else:
                q = O.stored_to_f64(p.q0[t]).astype(ft)
            cat = []
            for i in range(M):
                Q = rp("q", (q @ layers[i]["wq"]) * scale)
                a = _attention(Q, KV[i][0], KV[i][1], H, sp.score, rp, at, km, hmap, sb)
                o = rp("attn", a).astype(ft) @ layers[i]["wo"]
                out["attn"][i, t], out["o"][i, t] = a, o
                cat.append(rp("o", o))
                if i + 1 < M:
                    if sp.qmode == "fusion":
                        pre = rp("pre", np.concatenate(cat + [x_t]) @ layers[i + 1]["wc"])
                        q = rp("ln", _ffn(pre, layers[i + 1]["q"], True, rp))
                    else:
                        q = cat[-1] @ layers[i]["r"]
            if sp.qmode == "fusion":
                pre = rp("pre", np.concatenate(cat + [x_t]) @ wz)
                out["z"][t] = _ffn(pre, zw, sp.z_ln, rp)
            else:
                out["z"][t] = out["o"][M - 1, t]
    return out


def row_rel(g: np.ndarray, o: np.ndarray) -> float:
    """max over rows of max_k |g - o| / max_k |o| (last axis = row)."""
    g = np.asarray(g, np.float64).reshape(-1, g.shape[-1])
    o = np.asarray(o, np.float64).reshape(-1, o.shape[-1])
    if g.size == 0:
        return 0.0
    den = np.abs(o).max(axis=1)
    return float((np.abs(g - o).max(axis=1) / np.where(den > 0, den, 1.0)).max())


def deviation(p, precision: str, points=ALL_POINTS, exact=None, keys=("z", "o", "attn"), arith="f64",
              users=None, attn_arith=None):
    """{key: end-to-end row-relative deviation} of ``perturbed_forward``
    from the exact forward (``exact``: the oracle's result, if at hand),
    over the targets of ``users`` (default: all)."""
    if exact is None:
        exact = O.forward_problem(p, users)
    pert = perturbed_forward(p, precision, points, users, arith, attn_arith)
    if users is not None:
        to = p.tgt_offsets
        rows = np.concatenate([np.arange(to[u], to[u + 1]) for u in users]).astype(np.int64)
        return {k: row_rel(pert[k][..., rows, :], exact[k][..., rows, :]) for k in keys}
    return {k: row_rel(pert[k], exact[k]) for k in keys}
