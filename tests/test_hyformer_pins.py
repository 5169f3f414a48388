"""Pins for the oracle's HyFormer query mode (CPU only): query generation
([HyFormer] §3.3.2 eq. (3)-(4)), the subspace token mixing, per-token FFN
and residual of query boosting (§3.5 eq. (10)-(15)) and their composition
per layer (§3.6 eq. (16)-(17)).

Each step is tied to something other than the oracle itself: worked values
of the token mixing written out by hand, its involution property, closed
forms (zero FFN -> the residual alone; constant rows -> their mean), torch's
SiLU-gated FFN, and structural identities of the whole mode.
"""
import math
from dataclasses import replace

import numpy as np
import torch
import torch.nn.functional as F

from oracle import stca_oracle as O
from recsys_ultra_long_amd import inputs as I


def test_token_mix_worked_example():
    # T = 4 tokens of width D = 8 -> subspaces of width 2.  Token t holds the
    # values 10 t + j.  Mixed token h is [token0 sub h | token1 sub h | ...].
    Q = np.array([[10 * t + j for j in range(8)] for t in range(4)], dtype=float)
    M = O.token_mix(Q)
    np.testing.assert_array_equal(M[0], [0, 1, 10, 11, 20, 21, 30, 31])
    np.testing.assert_array_equal(M[1], [2, 3, 12, 13, 22, 23, 32, 33])
    np.testing.assert_array_equal(M[3], [6, 7, 16, 17, 26, 27, 36, 37])


def test_token_mix_is_an_involution_and_a_block_transpose():
    rng = np.random.default_rng(0)
    Q = rng.normal(size=(16, 512))
    np.testing.assert_array_equal(O.token_mix(O.token_mix(Q)), Q)
    # subspace (t, h) of Q becomes subspace (h, t) of the mix
    w = 32
    M = O.token_mix(Q)
    for t, h in [(0, 5), (7, 2), (15, 15), (3, 11)]:
        np.testing.assert_array_equal(M[h, t * w:(t + 1) * w], Q[t, h * w:(h + 1) * w])


def _ffn_stack(rng, n, din, hh, d, scale=1.0):
    return {"w1": rng.normal(size=(n, din, hh)) * scale / math.sqrt(din),
            "w3": rng.normal(size=(n, din, hh)) * scale / math.sqrt(din),
            "w2": rng.normal(size=(n, hh, d)) * scale / math.sqrt(hh)}


def test_ffn_stack_matches_torch():
    rng = np.random.default_rng(1)
    w = _ffn_stack(rng, 3, 12, 10, 8)
    x = rng.normal(size=12)
    for n in range(3):
        t = lambda a: torch.from_numpy(a)
        ref = ((F.silu(t(x) @ t(w["w1"][n])) * (t(x) @ t(w["w3"][n]))) @ t(w["w2"][n])).numpy()
        np.testing.assert_allclose(O.ffn_n(x, w, n), ref, rtol=1e-12, atol=1e-14)


def test_boost_with_zero_ffn_is_the_residual():
    rng = np.random.default_rng(2)
    N, Fn, d = 3, 5, 16
    Qdec, Fns = rng.normal(size=(N, d)), rng.normal(size=(Fn, d))
    w = _ffn_stack(rng, N + Fn, d, 8, d)
    w["w2"][:] = 0.0
    np.testing.assert_array_equal(O.query_boost(Qdec, Fns, w), np.concatenate([Qdec, Fns]))


def test_boost_adds_the_ffn_of_the_mixed_token_at_its_position():
    """Q_boost[t] = Q[t] + FFN_t(mix(Q)[t]): with every FFN but FFN_k zero,
    only row k changes, by FFN_k of the k-th mixed token."""
    rng = np.random.default_rng(3)
    N, Fn, d = 2, 2, 8
    Qdec, Fns = rng.normal(size=(N, d)), rng.normal(size=(Fn, d))
    w = _ffn_stack(rng, N + Fn, d, 6, d)
    k = 2
    for n in range(N + Fn):
        if n != k:
            w["w2"][n] = 0.0
    Q = np.concatenate([Qdec, Fns])
    out = O.query_boost(Qdec, Fns, w)
    mixed_k = np.concatenate([Q[t, k * 2:(k + 1) * 2] for t in range(4)])  # width D / T = 2
    for t in range(4):
        expect = Q[t] + (O.ffn_n(mixed_k, w, k) if t == k else 0.0)
        np.testing.assert_allclose(out[t], expect, rtol=1e-13, atol=1e-15)


def test_mean_pool_closed_forms():
    X = np.tile(np.arange(6.0), (7, 1))
    np.testing.assert_array_equal(O.mean_pool(X), np.arange(6.0))
    np.testing.assert_array_equal(O.mean_pool(np.zeros((0, 6))), np.zeros(6))
    X = np.array([[1.0, 2.0], [3.0, 6.0]])
    np.testing.assert_array_equal(O.mean_pool(X), [2.0, 4.0])


def test_query_generation_orders_the_global_info():
    """g = [F_1 .. F_M | MeanPool]: an FFN that reads only the last d inputs
    (W1 = W3 = 0 elsewhere) sees the pooled history alone, one that reads
    only the first d sees F_1."""
    rng = np.random.default_rng(4)
    d, Fn, hh = 4, 2, 5
    Fns = rng.normal(size=(Fn, d))
    X = rng.normal(size=(9, d))
    w = _ffn_stack(rng, 2, (Fn + 1) * d, hh, d)
    w["w1"][0, :Fn * d] = 0.0
    w["w3"][0, :Fn * d] = 0.0
    w["w1"][1, d:] = 0.0
    w["w3"][1, d:] = 0.0
    q = O.query_generation(Fns, X, w)
    sub = lambda n, lo, hi: {k: v[n:n + 1, lo:hi] if k != "w2" else v[n:n + 1] for k, v in w.items()}
    np.testing.assert_allclose(q[0], O.ffn_n(X.mean(axis=0), sub(0, Fn * d, (Fn + 1) * d), 0), rtol=1e-12)
    np.testing.assert_allclose(q[1], O.ffn_n(Fns[0], sub(1, 0, d), 0), rtol=1e-12)


def test_hyformer_forward_composition():
    """The mode end to end equals its steps composed by hand: generation,
    per-query decoding (the linear mode's attention and W_O), boosting, and
    the first N boosted tokens as the next queries / output."""
    sp = replace(I.spec(5)["feed"], qmode="hyformer", n_ns=3, B=2, L=40, m=5, d=64, H=2, hidden=64,
                 M=2, table_rows=500, hy_hidden=48)
    p = I.make_problem(sp)
    out = O.forward_problem(p)
    layers, _, _ = O.weights_f64(p.layers)
    ns = O.stored_to_f64(p.extra["ns"])
    qgen = {k: O.stored_to_f64(v) for k, v in p.extra["qgen"].items()}
    for u in range(sp.B):
        X = O.stored_to_f64(p.rows(p.hist_ids[p.hist_offsets[u]:p.hist_offsets[u + 1]]))
        q = O.query_generation(ns[u], X, qgen)
        for i in range(sp.M):
            K, V = O.encode_history(X, layers[i], False)
            a, _, _ = O.attention_core(q @ layers[i]["wq"], K, V, sp.H, "softmax")
            dec = a @ layers[i]["wo"]
            t0 = p.tgt_offsets[u]
            np.testing.assert_allclose(out["o"][i, t0:t0 + sp.m], dec, rtol=1e-12, atol=1e-16)
            q = O.query_boost(dec, ns[u], layers[i]["boost"])[:sp.m]
        np.testing.assert_allclose(out["z"][p.tgt_offsets[u]:p.tgt_offsets[u + 1]], q, rtol=1e-12, atol=1e-16)
