"""Float64 CPU oracle for the STCA forward hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``.  It shares no code, table or
constant with the HIP implementation; both sides only consume the seeded
arrays drawn by ``recsys_ultra_long_amd.inputs``.

What it computes is the plain definition of the method, evaluated in float64
per user and per target, with a two-pass softmax (max, then exp-sum) and no
splitting, blocking or online rescaling.  Page citations use these short
names for the pages this work is built from:

* [WeChat]   "视频号推荐超长序列技术演进：从端到端到 Cross-Mask Transformer"
* [Notes]    "超长序列建模 —— STCA 精读笔记" (STCA reading notes)
* [Review]   "Make It Long, Keep It Fast: End-to-End 10K Long User Behavior
             Sequence Modeling for Billion-Scale Douyin Recommendation"
             (paper review)
* [HyFormer] "HyFormer：重新审视序列建模和特征交互在 CTR 预测中的作用"
             (translation)

Readings taken where the pages are silent (each one is listed in the design doc):

* SwiGLU(x) = (SiLU(x W1) * (x W3)) W2 with SiLU(u) = u * sigmoid(u), no
  biases ([Notes] §STCA and [Review] §四 name the block but never define it).
* LN is LayerNorm over the model width, biased variance, eps = 1e-5, with a
  gain and a bias.
* History side, layer i: K = LN(SwiGLU_i(X)) W_K, V = LN(SwiGLU_i(X)) W_V, with
  X the raw embedding rows for every layer ([Notes] §STCA, layers i > 1).
  HyFormer mode drops the LN ([HyFormer] eq. (7), (8)).
* First query q1 = LN(SwiGLU_q1(x_t)) ([Notes] §STCA, first layer).
* Heads are column slices of width d_h of one d x d matrix; the score scale is
  1/sqrt(d_h) ([Review] architecture tree; the formula for alpha).
* Fusion: q_{i+1} = LN(SwiGLU_{i+1}([o_1 | ... | o_i | x_t] W_C^{i+1})) with
  o_k the post-W_O layer outputs ([Review] 核心公式, inter-layer fusion).
* Final: z = SwiGLU_Z([o_1 | ... | o_M | x_t] W_Z) ([Review] architecture
  tree), optionally followed by LN (the [Notes] wording: z is the last
  updated query).
* ReLU-scored variant: w_j = max(0, s_j), o = sum_j w_j v_j, and the active
  count is #{j : s_j > 0} ([WeChat] §1.2: a key is active when its score is
  above zero).
* Empty history: attention output 0, active count 0.
* An id outside [0, table rows) reads a zero row (no page covers invalid ids;
  this is the boundary's convention, which the library also flags).
* HyFormer linear mode: Q_{l+1} = O_l R_l, output O_M ([HyFormer] eq. (9),
  (16), with the boosting block replaced by a fixed linear map).
* Cross-Mask ([WeChat] §3.2-3.3): a vertical mask keeps, per head (one
  feature domain's column slice, its horizontal mask), only the history items
  its condition selects: softmax / ReLU over those items, 0 when none; heads
  sharing an attention map score with the same Q / K columns (a head map)
  under their own masks and V columns.
* Context-similarity score bias ([WeChat] §2.2.3, 上下文利用: the context
  similarity of two videos fine-tunes the target-attention score; the page
  gives no formula): an additive bias b[j, eta] per history item and head,
  added to the scaled score of every target of the user in every layer
  (all targets of one request share the user's current context), before the
  softmax or the ReLU.  Its values are the caller's.
* HyFormer query mode ([HyFormer] §3.3.2 eq. (3)-(4), §3.5 eq. (10)-(15),
  §3.6 eq. (16)-(17)): every "FFN" is the SwiGLU block above without LN; the
  N queries of a user are FFN_n(Concat(F_1, ..., F_M, MeanPool(Seq))) with
  Seq the user's raw history rows (zero for an empty history); each layer
  decodes them with the multi-head cross attention and W_O, then boosts
  [decoded queries | F_1 .. F_M] (T = N + M tokens) by the subspace token
  mixing, one FFN per mixed token and the residual; the first N boosted
  tokens are the next layer's queries (the non-sequence tokens re-enter from
  F at every layer) and, after the last layer, the output z.
* LONGER-style sequence encoding ([HyFormer] §3.4.1 (ii), eq. (6), then (8)):
  per layer, H_l = CrossAttn(S_short, S, S) is the standard multi-head
  softmax cross attention (its own W_Q, W_K, W_V, W_O per layer, heads as
  d_h-wide column slices, scale 1/sqrt(d_h), no residual, no LN) from the
  compact short sequence to the whole sequence, and K_l = H_l W_K,
  V_l = H_l W_V; the queries then decode these L_H rows.  S_short is the
  last min(L, L_H) rows of the user's history (the page does not say how the
  short sequence is formed; the most recent items are the plainest reading).
  The history FFN and its LN are not applied in this mode.

Parity pins: every function below is pinned by a closed form, an invariant,
a brute-force enumeration or an independent library routine in
``tests/test_oracle_pins.py``.  The absolute values of a whole multi-layer
forward (fusion chain, z) have no external anchor: they are pinned only
compositionally (parity unpinned as a whole; each step is pinned).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

LN_EPS = 1e-5


def stored_to_f64(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Stored values -> float64, exactly.  uint16 arrays hold raw bf16 bits."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        bits = a.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------- blocks
def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(u) = u * sigmoid(u) (the gate of the SwiGLU FFN)."""
    return x / (1.0 + np.exp(-x))


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis: biased variance, gain g, bias b."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def swiglu(x: np.ndarray, w: dict) -> np.ndarray:
    """Dimension-preserving SwiGLU FFN: (SiLU(x W1) * (x W3)) W2."""
    return (silu(x @ w["w1"]) * (x @ w["w3"])) @ w["w2"]


def ffn_ln(x: np.ndarray, w: dict, ln: bool) -> np.ndarray:
    y = swiglu(x, w)
    return layer_norm(y, w["ln_g"], w["ln_b"]) if ln else y


# ---------------------------------------------------------------- attention
def attention_target(Q: np.ndarray, K: np.ndarray, V: np.ndarray, H: int, score: str,
                     scale: Optional[float] = None, key_mask=None, head_map=None, score_bias=None):
    """One target (query row ``Q`` of width d, already multiplied by W_Q)
    against one user's keys K and values V ([L, d] each).

    Per head eta (columns eta*d_h .. (eta+1)*d_h):
      s_j   = Q_eta . K_{j,eta} / sqrt(d_h)
      softmax: a_eta = sum_j exp(s_j - max s) V_{j,eta} / sum_j exp(s_j - max s)
      relu:    a_eta = sum_j max(0, s_j) V_{j,eta};  cnt_eta = #{j : s_j > 0}
    ([Review] formula for alpha and o; [WeChat] §1.2 for the ReLU form.)

    ``scale`` defaults to 1/sqrt(d_h); pass 1.0 when ``Q`` already carries it.

    Cross-Mask ([WeChat] §3.2-3.3): ``key_mask`` [L] (ints) keeps, for head
    eta, only the keys whose bit eta is set (a head with none gives 0);
    ``head_map[eta]`` names the head whose Q / K columns give head eta's
    scores (V and the output stay head eta's columns).

    Context-similarity bias ([WeChat] §2.2.3): ``score_bias`` [L, H] is added
    to the scaled scores, s_j = Q_eta . K_{j,eta} * scale + b[j, eta], before
    the softmax or the ReLU.

    Returns (a [d], cnt [H], amb [H]) where ``amb`` counts the scores whose
    sign an fp32 evaluation of the same operands could flip:
    |s_j| <= d_h * 2^-23 * scale * sum_k |Q_k K_jk|  (plus 2^-23 (|s| + |b|)
    for the bias addition when a bias is given).
    """
    d = Q.shape[0]
    dh = d // H
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    a = np.zeros(d)
    cnt = np.zeros(H, dtype=np.int64)
    amb = np.zeros(H, dtype=np.int64)
    L = K.shape[0]
    if L == 0:
        return a, cnt, amb
    for eta in range(H):
        cols = slice(eta * dh, (eta + 1) * dh)
        qk = eta if head_map is None else int(head_map[eta])
        qcols = slice(qk * dh, (qk + 1) * dh)
        be = None if score_bias is None else np.asarray(score_bias, dtype=np.float64)[:, eta]
        if key_mask is None:
            Ke, Ve = K, V
        else:
            sel = ((np.asarray(key_mask, dtype=np.int64) >> eta) & 1).astype(bool)
            if not sel.any():
                continue                      # no visible key: output 0
            Ke, Ve = K[sel], V[sel]
            be = None if be is None else be[sel]
        q = Q[qcols]
        s = (Ke[:, qcols] @ q) * scale
        if be is not None:
            s = s + be
        if score == "softmax":
            p = np.exp(s - s.max())
            a[cols] = (p @ Ve[:, cols]) / p.sum()
        elif score == "relu":
            w = np.maximum(s, 0.0)
            a[cols] = w @ Ve[:, cols]
            cnt[eta] = int(np.count_nonzero(s > 0.0))
            bound = dh * 2.0 ** -23 * (np.abs(Ke[:, qcols]) @ np.abs(q)) * scale
            if be is not None:
                bound = bound + 2.0 ** -23 * (np.abs(s - be) + np.abs(be))
            amb[eta] = int(np.count_nonzero(np.abs(s) <= bound))
        else:
            raise ValueError(score)
    return a, cnt, amb


def attention_core(Qs: np.ndarray, K: np.ndarray, V: np.ndarray, H: int, score: str,
                   scale: Optional[float] = None, key_mask=None, head_map=None, score_bias=None):
    """Every target of one user: rows of ``Qs`` handled one at a time."""
    m, d = Qs.shape
    attn = np.zeros((m, d))
    cnt = np.zeros((m, H), dtype=np.int64)
    amb = np.zeros((m, H), dtype=np.int64)
    for t in range(m):
        attn[t], cnt[t], amb[t] = attention_target(Qs[t], K, V, H, score, scale, key_mask, head_map,
                                                   score_bias)
    return attn, cnt, amb


# ---------------------------------------------------------------- HyFormer queries
def mean_pool(X: np.ndarray) -> np.ndarray:
    """MeanPool(Seq) over the rows of a user's history (zero when empty)."""
    return X.mean(axis=0) if len(X) else np.zeros(X.shape[1])


def ffn_n(x: np.ndarray, w: dict, n: int) -> np.ndarray:
    """The n-th of a stack of SwiGLU FFNs (w1, w3 [n, in, h], w2 [n, h, d])."""
    return (silu(x @ w["w1"][n]) * (x @ w["w3"][n])) @ w["w2"][n]


def query_generation(F: np.ndarray, X: np.ndarray, qgen: dict) -> np.ndarray:
    """eq. (3)-(4): Q = [FFN_1(g), ..., FFN_N(g)], g = Concat(F_1..F_M, MeanPool(X))."""
    g = np.concatenate([F.reshape(-1), mean_pool(X)])
    return np.stack([ffn_n(g, qgen, n) for n in range(qgen["w1"].shape[0])])


def token_mix(Q: np.ndarray) -> np.ndarray:
    """eq. (11)-(13): token t is cut into T subspaces of width D / T; mixed
    token h is the concatenation over t of every token's h-th subspace."""
    T, D = Q.shape
    w = D // T
    out = np.empty_like(Q)
    for h in range(T):
        for t in range(T):
            out[h, t * w:(t + 1) * w] = Q[t, h * w:(h + 1) * w]
    return out


def query_boost(Qdec: np.ndarray, F: np.ndarray, boost: dict) -> np.ndarray:
    """eq. (10), (14), (15): Q = [Qdec | F], Q_boost = Q + PerToken-FFN(mix(Q))."""
    Q = np.concatenate([Qdec, F], axis=0)
    Qm = token_mix(Q)
    return Q + np.stack([ffn_n(Qm[h], boost, h) for h in range(Q.shape[0])])


# ---------------------------------------------------------------- weights
def weights_f64(layers, z=None, wz=None):
    """Upcast stored weights (bf16 bits or fp32) to float64 dictionaries."""
    def conv(w):
        if w is None:
            return None
        if isinstance(w, dict):
            return {k: conv(v) for k, v in w.items()}
        return stored_to_f64(w)
    return [conv(l) for l in layers], conv(z), conv(wz)


# ---------------------------------------------------------------- forward
def longer_encode(X: np.ndarray, enc: dict, l_short: int, H: int) -> np.ndarray:
    """[HyFormer] eq. (6): H_l = CrossAttn(S_short, S, S) over one user's
    raw rows X [L, d]: each of the last min(L, l_short) rows, projected by
    enc["wq"], attends (multi-head softmax) over all of X projected by
    enc["wk"], enc["wv"]; the head outputs, concatenated, go through
    enc["wo"].  Returns [min(L, l_short), d]."""
    L, d = X.shape
    ls = min(L, l_short)
    Ke, Ve = X @ enc["wk"], X @ enc["wv"]
    out = np.zeros((ls, d))
    for r in range(ls):
        a, _, _ = attention_target(X[L - ls + r] @ enc["wq"], Ke, Ve, H, "softmax")
        out[r] = a @ enc["wo"]
    return out


def encode_history(X: np.ndarray, lw: dict, kv_ln: bool, encoder: str = "swiglu", l_short: int = 0,
                   H: int = 0):
    """History side of one layer: K = Xt W_K, V = Xt W_V with
    Xt = LN(SwiGLU(X)) ([Notes] §STCA; [HyFormer] eq. (7)-(8) without LN), or,
    for the LONGER-style encoder, Xt = H_l of eq. (6) (``longer_encode``)."""
    if encoder == "longer":
        xt = longer_encode(X, lw["enc"], l_short, H)
    else:
        xt = ffn_ln(X, lw["kv"], kv_ln)
    return xt @ lw["wk"], xt @ lw["wv"]


def forward(cfg: dict, hist_offsets, hist_ids, tgt_offsets, rows_f64, layers, z=None, wz=None,
            tgt_ids=None, q0=None, users=None, want=("z", "o", "attn", "active", "q"), hy=None,
            key_mask=None, head_map=None, score_bias=None):
    """The STCA forward for the users in ``users`` (default: all).

    cfg: dict with d, H, M, score ("softmax"|"relu"), qmode ("fusion"|"linear"),
         kv_ln, z_ln; optionally encoder ("swiglu"|"longer") and l_short.
    rows_f64: callable ids -> float64 table rows [len(ids), d].
    layers/z/wz: float64 weights (see ``weights_f64``).
    Returns a dict of float64 arrays indexed by global target index:
      z [T, d], o [M, T, d], attn [M, T, d], active [M, T, H], amb [M, T, H],
      qs [M, T, d] (the query rows after W_Q, before the 1/sqrt(d_h) scale).
    Rows of targets whose user is not in ``users`` stay zero.
    """
    d, H, M = cfg["d"], cfg["H"], cfg["M"]
    score, qmode = cfg["score"], cfg["qmode"]
    ho = np.asarray(hist_offsets, dtype=np.int64)
    to = np.asarray(tgt_offsets, dtype=np.int64)
    B = len(ho) - 1
    T = int(to[-1])
    out = {"z": np.zeros((T, d)), "o": np.zeros((M, T, d)), "attn": np.zeros((M, T, d)),
           "active": np.zeros((M, T, H), dtype=np.int64), "amb": np.zeros((M, T, H), np.int64),
           "qs": np.zeros((M, T, d))}
    if users is None:
        users = range(B)
    for u in users:
        ids = np.asarray(hist_ids[ho[u]:ho[u + 1]])
        X = rows_f64(ids) if len(ids) else np.zeros((0, d))
        # Request Level Batching: the user's K/V of every layer is computed
        # once and serves all of the user's targets ([Notes] §RLB).
        KV = [encode_history(X, layers[i], cfg["kv_ln"], cfg.get("encoder", "swiglu"), cfg.get("l_short", 0), H)
              for i in range(M)]
        km = None if key_mask is None else np.asarray(key_mask)[ho[u]:ho[u + 1]]
        sb = None if score_bias is None else np.asarray(score_bias, dtype=np.float64)[ho[u]:ho[u + 1]]
        cm = dict(key_mask=km, head_map=head_map, score_bias=sb)
        if qmode == "hyformer":
            t0, t1 = int(to[u]), int(to[u + 1])
            F = hy["ns"][u]
            q = query_generation(F, X, hy["qgen"])        # [N, d]
            for i in range(M):
                K, V = KV[i]
                dec = np.zeros((t1 - t0, d))
                for n in range(t1 - t0):
                    Q = q[n] @ layers[i]["wq"]
                    a, c, amb = attention_target(Q, K, V, H, score, **cm)
                    dec[n] = a @ layers[i]["wo"]
                    out["qs"][i, t0 + n] = Q
                    out["attn"][i, t0 + n] = a
                    out["active"][i, t0 + n] = c
                    out["amb"][i, t0 + n] = amb
                    out["o"][i, t0 + n] = dec[n]
                q = query_boost(dec, F, layers[i]["boost"])[:t1 - t0]
            out["z"][t0:t1] = q
            continue
        for t in range(int(to[u]), int(to[u + 1])):
            if qmode == "fusion":
                x_t = rows_f64(np.asarray([tgt_ids[t]]))[0]
                q = ffn_ln(x_t, layers[0]["q"], True)
            else:
                q = np.asarray(q0[t], dtype=np.float64)
            outs = []
            for i in range(M):
                Q = q @ layers[i]["wq"]
                K, V = KV[i]
                a, c, amb = attention_target(Q, K, V, H, score, **cm)
                o = a @ layers[i]["wo"]
                outs.append(o)
                out["qs"][i, t] = Q
                out["attn"][i, t] = a
                out["active"][i, t] = c
                out["amb"][i, t] = amb
                out["o"][i, t] = o
                if i + 1 < M:
                    if qmode == "fusion":
                        cat = np.concatenate(outs + [x_t])
                        q = ffn_ln(cat @ layers[i + 1]["wc"], layers[i + 1]["q"], True)
                    else:
                        q = o @ layers[i]["r"]
            if qmode == "fusion":
                cat = np.concatenate(outs + [x_t])
                out["z"][t] = ffn_ln(cat @ wz, z, cfg["z_ln"])
            else:
                out["z"][t] = outs[-1]
    return out


def forward_problem(p, users=None):
    """Convenience wrapper over a ``recsys_ultra_long_amd.inputs.Problem``
    (a plain data container: only its arrays are read)."""
    sp = p.spec
    layers, z, wz = weights_f64(p.layers, p.z, p.wz)
    cfg = dict(d=sp.d, H=sp.H, M=sp.M, score=sp.score, qmode=sp.qmode,
               kv_ln=sp.kv_ln, z_ln=sp.z_ln, encoder=getattr(sp, "encoder", "swiglu"),
               l_short=getattr(sp, "l_short", 0))
    hy = None
    if sp.qmode == "hyformer":
        hy = {"ns": stored_to_f64(p.extra["ns"]),
              "qgen": {k: stored_to_f64(v) for k, v in p.extra["qgen"].items()}}
    def rows(ids):
        # an id outside [0, table_rows) reads a zero row (the boundary's
        # convention for invalid ids; the backward oracle's too)
        ids = np.asarray(ids, dtype=np.int64)
        out = np.zeros((len(ids), sp.d))
        ok = (ids >= 0) & (ids < sp.table_rows)
        if ok.any():
            out[ok] = stored_to_f64(p.rows(ids[ok]))
        return out
    return forward(cfg, p.hist_offsets, p.hist_ids, p.tgt_offsets,
                   rows, layers, z, wz,
                   tgt_ids=p.tgt_ids, q0=stored_to_f64(p.q0), users=users, hy=hy,
                   key_mask=p.extra.get("key_mask"), head_map=p.extra.get("head_map"),
                   score_bias=p.extra.get("score_bias"))
