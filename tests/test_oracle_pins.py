"""Pins for the float64 oracle (CPU only).

Each test ties one oracle function to something other than the oracle itself:
a library routine (torch's SiLU, LayerNorm, scaled-dot-product attention), a
closed form, an invariant of the method, or a constructed special case whose
answer is known.  Page names as in the oracle header: [Review] is the "Make It
Long, Keep It Fast" paper review, [Notes] the STCA reading notes, [WeChat] the
WeChat Channels long-sequence post, [HyFormer] the HyFormer translation.
"""
import math
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import stca_oracle as O
from recsys_ultra_long_amd import inputs as I

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def rng(seed=0):
    return np.random.default_rng(seed)


def small_spec(**over):
    base = dict(name="pin", B=3, d=16, H=2, hidden=32, M=3, table_rows=200, dtype="f32",
                L=7, m=3, ids="uniform", ln_random=True, seed=11)
    base.update(over)
    return I.Spec(**base)


def weights(p):
    return O.weights_f64(p.layers, p.z, p.wz)


# ----------------------------------------------------------------- blocks
def test_silu_matches_torch():
    x = rng(1).normal(size=1000) * 6
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-15)


def test_layer_norm_matches_torch():
    g = rng(2)
    x = g.normal(size=(9, 24)) * 3 + 1
    gam, bet = g.normal(size=24), g.normal(size=24)
    ref = F.layer_norm(torch.from_numpy(x), (24,), torch.from_numpy(gam), torch.from_numpy(bet),
                       eps=1e-5).numpy()
    np.testing.assert_allclose(O.layer_norm(x, gam, bet), ref, rtol=1e-12, atol=1e-12)


def test_swiglu_constructed_case():
    # W1 = 2I, W3 = I, W2 = cyclic shift P: y = (SiLU(2x) * x) P.  A swapped
    # W1/W3 gives SiLU(x) * 2x and a transposed W2 shifts the other way.
    d = 6
    P = np.roll(np.eye(d), 1, axis=1)
    w = {"w1": 2 * np.eye(d), "w3": np.eye(d), "w2": P}
    x = np.array([0.3, -1.2, 2.0, 0.0, 4.5, -0.7])
    silu2 = 2 * x / (1 + np.exp(-2 * x))
    expect = np.roll(silu2 * x, 1)
    np.testing.assert_allclose(O.swiglu(x, w), expect, rtol=1e-14, atol=1e-15)
    # asymmetric h != d shapes go through as row vectors: [d]x[d,h] -> [h]x[h,d]
    g = rng(3)
    w2 = {"w1": g.normal(size=(4, 10)), "w3": g.normal(size=(4, 10)), "w2": g.normal(size=(10, 4))}
    assert O.swiglu(g.normal(size=(5, 4)), w2).shape == (5, 4)


# ----------------------------------------------------------------- attention core
@pytest.mark.parametrize("H,dh,L,m", [(1, 8, 5, 1), (2, 16, 33, 4), (4, 32, 200, 3)])
def test_softmax_attention_matches_sdpa(H, dh, L, m):
    g = rng(H * 100 + L)
    d = H * dh
    Q, K, V = g.normal(size=(m, d)), g.normal(size=(L, d)), g.normal(size=(L, d))
    attn, _, _ = O.attention_core(Q, K, V, H, "softmax")
    tq = torch.from_numpy(Q).reshape(m, H, dh).transpose(0, 1)[None]
    tk = torch.from_numpy(K).reshape(L, H, dh).transpose(0, 1)[None]
    tv = torch.from_numpy(V).reshape(L, H, dh).transpose(0, 1)[None]
    ref = F.scaled_dot_product_attention(tq, tk, tv)          # scale 1/sqrt(dh)
    ref = ref[0].transpose(0, 1).reshape(m, d).numpy()
    np.testing.assert_allclose(attn, ref, rtol=1e-12, atol=1e-13)


def test_two_key_closed_form():
    # softmax over two keys: weight of key 1 = sigmoid((s1 - s2)), s = q.k/sqrt(dh)
    dh = 9
    q = np.zeros(dh); q[0] = 2.0
    K = np.zeros((2, dh)); K[0, 0] = 1.5; K[1, 0] = -0.5
    V = np.zeros((2, dh)); V[0, 1] = 1.0; V[1, 2] = 1.0
    a, _, _ = O.attention_target(q, K, V, 1, "softmax")
    delta = (2.0 * 1.5 - 2.0 * -0.5) / 3.0
    w1 = 1.0 / (1.0 + math.exp(-delta))
    np.testing.assert_allclose(a[1:3], [w1, 1 - w1], rtol=1e-14)
    assert a[0] == 0 and np.all(a[3:] == 0)


def test_single_key_returns_v():                                  # P1
    g = rng(5)
    d, H = 16, 4
    Q, K, V = g.normal(size=(3, d)), g.normal(size=(1, d)), g.normal(size=(1, d))
    attn, _, _ = O.attention_core(Q, K, V, H, "softmax")
    assert np.array_equal(attn, np.repeat(V, 3, axis=0))
    a_r, cnt, _ = O.attention_core(Q, K, V, H, "relu")
    dh = d // H
    for t in range(3):
        for e in range(H):
            c = slice(e * dh, (e + 1) * dh)
            s = Q[t, c] @ K[0, c] / math.sqrt(dh)
            np.testing.assert_allclose(a_r[t, c], max(s, 0) * V[0, c], rtol=1e-14, atol=0)
            assert cnt[t, e] == (1 if s > 0 else 0)


def test_equal_keys_give_mean_v():                                # P2
    g = rng(6)
    d, H, L = 12, 3, 50
    Q, V = g.normal(size=(4, d)), g.normal(size=(L, d))
    K = np.tile(g.normal(size=(1, d)), (L, 1))
    attn, _, _ = O.attention_core(Q, K, V, H, "softmax")
    np.testing.assert_allclose(attn, np.tile(V.mean(0), (4, 1)), rtol=1e-13, atol=1e-14)
    a_r, cnt, _ = O.attention_core(Q, np.zeros((L, d)), V, H, "relu")
    assert np.all(a_r == 0) and np.all(cnt == 0)


def test_relu_constructed_keys():                                 # P7
    g = rng(7)
    d, H, L = 8, 1, 40
    q = g.normal(size=d)
    c = g.normal(size=L)
    c[5] = 0.0                                   # s = 0 is inactive (strict)
    K = c[:, None] * q[None, :]
    V = g.normal(size=(L, d))
    a, cnt, _ = O.attention_target(q, K, V, H, "relu")
    s = c * (q @ q) / math.sqrt(d)
    np.testing.assert_allclose(a, (np.maximum(s, 0)[:, None] * V).sum(0), rtol=1e-12)
    assert cnt[0] == int((c > 0).sum())
    # keys along +q: every key active; W_Q = 0: none active
    _, cnt_all, _ = O.attention_target(q, (np.abs(c) + 0.1)[:, None] * q[None, :], V, H, "relu")
    assert cnt_all[0] == L
    _, cnt0, _ = O.attention_target(np.zeros(d), K, V, H, "relu")
    assert cnt0[0] == 0


# ----------------------------------------------------------------- ambiguity band
# The bit-exact active-count contract is stated on shared operands: where a
# score lies so close to zero that an fp32 evaluation of the same d_h-term
# dot product could give it the other sign, the count may differ.  The
# oracle reports those keys (``amb``) with the bound
#     |s| <= d_h 2^-23 scale sum_k |Q_k K_k|,
# twice the classical forward-error bound of a recursively summed dot
# product, gamma_n sum |x_k y_k| with gamma_n = n u / (1 - n u) and
# u = 2^-24 for fp32 round to nearest (Higham, "Accuracy and Stability of
# Numerical Algorithms", section 3.1); the factor two covers any summation
# order and fused or unfused products.


def _fp32_scores(q, k):
    """q.k in float32 arithmetic: sequential, reversed, pairwise, blocked by 8."""
    q32, k32 = q.astype(np.float32), k.astype(np.float32)
    p = q32 * k32
    out = []
    for order in (p, p[::-1]):
        acc = np.float32(0)
        for x in order:
            acc = np.float32(acc + x)
        out.append(float(acc))
    v = p.copy()
    while len(v) > 1:
        if len(v) % 2:
            v = np.append(v, np.float32(0))
        v = (v[0::2] + v[1::2]).astype(np.float32)
    out.append(float(v[0]))
    out.append(float(np.float32(sum(np.float32(p[i:i + 8].sum(dtype=np.float32)) for i in range(0, len(p), 8)))))
    return out


def _amb_case(dh, s_over_bound, seed):
    """One head of width dh, one key whose exact score is s_over_bound times
    the oracle's ambiguity bound."""
    g = rng(seed)
    q = g.normal(size=dh)
    k = g.normal(size=dh)
    k -= (k @ q) / (q @ q) * q          # exactly orthogonal up to float64 rounding
    scale = 1.0 / math.sqrt(dh)
    # add t q so that s = t |q|^2 scale; the bound grows with |k| only slowly
    for _ in range(50):
        bound = dh * 2.0 ** -23 * scale * (np.abs(q) @ np.abs(k))
        t = s_over_bound * bound / ((q @ q) * scale) - (k @ q) / (q @ q)
        k = k + t * q
    return q, k


@pytest.mark.parametrize("dh", [32, 64])
def test_amb_constant(dh):
    """A key just inside the bound is ambiguous, one just outside is not, for
    either sign: this fixes the constant (a doubled or halved bound fails)."""
    for i, (r, want) in enumerate([(0.9, 1), (1.1, 0), (-0.9, 1), (-1.1, 0), (0.55, 1), (1.9, 0)]):
        q, k = _amb_case(dh, r, seed=31 * dh + i)
        _, cnt, amb = O.attention_target(q, k[None, :], np.ones((1, dh)), 1, "relu")
        assert amb[0] == want, (r, amb)
        assert cnt[0] == (1 if r > 0 else 0)


def test_amb_exact_zero_score():
    q = np.zeros(32)
    q[0] = 1.0
    k = np.zeros(32)
    k[1] = 3.0                                   # s = 0 exactly, bound = 0
    _, cnt, amb = O.attention_target(q, k[None, :], np.ones((1, 32)), 1, "relu")
    assert cnt[0] == 0 and amb[0] == 1


def test_amb_far_scores_are_exact():
    g = rng(5)
    d, H, L = 64, 2, 200
    Q = g.normal(size=d)
    K = g.normal(size=(L, d))
    _, cnt, amb = O.attention_target(Q, K, np.ones((L, d)), H, "relu")
    dh = d // H
    s = np.stack([K[:, h * dh:(h + 1) * dh] @ Q[h * dh:(h + 1) * dh] for h in range(H)], 1) / math.sqrt(dh)
    bound = np.stack([np.abs(K[:, h * dh:(h + 1) * dh]) @ np.abs(Q[h * dh:(h + 1) * dh]) for h in range(H)], 1) \
        * dh * 2.0 ** -23 / math.sqrt(dh)
    assert np.all(np.abs(s) > 10 * bound)        # random scores sit far from the band
    assert np.all(amb == 0) and np.array_equal(cnt, (s > 0).sum(0))


def test_amb_bounds_every_fp32_evaluation():
    """For near-cancelling dot products (exact scores within a few bounds of
    zero) every fp32 evaluation order stays within the bound of the exact
    score, so a key outside the band keeps its sign under any of them."""
    worst = 0.0
    for seed in range(400):
        dh = (32, 64)[seed % 2]
        q, k = _amb_case(dh, rng(1000 + seed).uniform(-3, 3), seed=2000 + seed)
        s = q @ k                                  # scale 1: the bound's own units
        b = dh * 2.0 ** -23 * (np.abs(q) @ np.abs(k))
        for s32 in _fp32_scores(q, k):
            worst = max(worst, abs(s32 - s) / b)
    assert worst <= 1.0, worst
    assert worst > 1e-3                          # the cases do exercise rounding


def test_amb_flags_a_key_fp32_gets_wrong():
    """A key whose exact score is positive but which a sequential fp32
    evaluation rounds to zero is counted active by the oracle and marked
    ambiguous, so the GPU's count may differ by it."""
    q = np.zeros(32)
    q[:3] = 1.0
    k = np.zeros(32)
    k[:3] = [1.0, 2.0 ** -25, -1.0]
    assert min(abs(s) for s in _fp32_scores(q, k)[:1]) == 0.0   # 1 + 2^-25 rounds to 1
    _, cnt, amb = O.attention_target(q, k[None, :], np.ones((1, 32)), 1, "relu")
    assert cnt[0] == 1 and amb[0] == 1


def test_empty_history():
    a, cnt, amb = O.attention_target(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)), 2, "softmax")
    assert np.all(a == 0) and np.all(cnt == 0)


def test_split_merge_identity():                                  # P6
    """Merging (max, sum, acc) partials over any partition of the keys gives
    the unsplit softmax attention (the identity the GPU's split-L relies on)."""
    g = rng(8)
    d, H, L = 16, 2, 97
    dh = d // H
    Q, K, V = g.normal(size=(1, d)) * 3, g.normal(size=(L, d)), g.normal(size=(L, d))
    ref, _, _ = O.attention_core(Q, K, V, H, "softmax")
    for trial in range(5):
        cuts = np.sort(g.choice(np.arange(1, L), size=trial + 1, replace=False))
        bounds = [0, *cuts.tolist(), L]
        for e in range(H):
            c = slice(e * dh, (e + 1) * dh)
            parts = []
            for a, b in zip(bounds[:-1], bounds[1:]):
                s = K[a:b, c] @ Q[0, c] / math.sqrt(dh)
                mx = s.max()
                p = np.exp(s - mx)
                parts.append((mx, p.sum(), p @ V[a:b, c]))
            M = max(x[0] for x in parts)
            l = sum(x[1] * math.exp(x[0] - M) for x in parts)
            acc = sum(x[2] * math.exp(x[0] - M) for x in parts)
            np.testing.assert_allclose(acc / l, ref[0, c], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- full forward
def run(p, users=None):
    return O.forward_problem(p, users)


@pytest.mark.parametrize("score", ["softmax", "relu"])
def test_permutation_invariance(score):                           # P3
    p = I.make_problem(small_spec(score=score, L=None, L_max=30, L_min=1))
    q = I.make_problem(small_spec(score=score, L=None, L_max=30, L_min=1))
    g = rng(9)
    for u in range(p.spec.B):
        a, b = q.hist_offsets[u], q.hist_offsets[u + 1]
        q.hist_ids[a:b] = q.hist_ids[a:b][g.permutation(b - a)]
    r1, r2 = run(p), run(q)
    for k in ("z", "o", "attn"):
        np.testing.assert_allclose(r1[k], r2[k], rtol=1e-10, atol=1e-12)
    assert np.array_equal(r1["active"], r2["active"])


@pytest.mark.parametrize("qmode", ["fusion", "linear"])
def test_rlb_equals_independent_targets(qmode):                   # P4 / P8
    p = I.make_problem(small_spec(qmode=qmode, m=4, kv_ln=(qmode == "fusion")))
    full = run(p)
    # split every user into m single-target users sharing the same history
    B, m = p.spec.B, p.spec.m
    ho, to = p.hist_offsets, p.tgt_offsets
    hid, hoff, toff = [], [0], [0]
    for u in range(B):
        for t in range(to[u], to[u + 1]):
            hid.append(p.hist_ids[ho[u]:ho[u + 1]])
            hoff.append(hoff[-1] + ho[u + 1] - ho[u])
            toff.append(toff[-1] + 1)
    q = I.Problem(replace(p.spec, B=B * m, m=1), np.asarray(hoff, np.int32),
                  np.concatenate(hid).astype(np.int32), np.asarray(toff, np.int32),
                  p.tgt_ids, p.q0, p.table, p.layers, p.z, p.wz)
    single = run(q)
    for k in ("z", "o", "attn", "active"):
        assert np.array_equal(full[k], single[k]), k


def test_layer_uses_raw_history_and_concat_order():
    """Layer 2 built as a copy of layer 1 with W_C^(2) = [0 ; I] (o_1 block
    zero, x_t block identity) must reproduce layer 1 exactly: this holds only
    if the history FFN of every layer reads the raw rows X and x_t is the last
    block of the concatenation ([Notes] §STCA; [Review] fusion formula)."""
    p = I.make_problem(small_spec(M=2))
    d = p.spec.d
    l0, l1 = p.layers
    for k in ("kv", "q", "wk", "wv", "wq", "wo"):
        l1[k] = l0[k]
    wc = np.zeros((2 * d, d), np.float32)
    wc[d:] = np.eye(d, dtype=np.float32)
    l1["wc"] = wc
    r = run(p)
    np.testing.assert_allclose(r["attn"][1], r["attn"][0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["o"][1], r["o"][0], rtol=1e-13, atol=1e-14)
    # the swapped order ([x_t ; o_1]) must not reproduce it
    wc2 = np.zeros((2 * d, d), np.float32)
    wc2[:d] = np.eye(d, dtype=np.float32)
    l1["wc"] = wc2
    r2 = run(p)
    assert np.abs(r2["attn"][1] - r2["attn"][0]).max() > 1e-3


@pytest.mark.parametrize("block", ["x_t", "o_last"])
def test_final_z_concat(block):
    p = I.make_problem(small_spec(M=2))
    d, M = p.spec.d, p.spec.M
    wz = np.zeros(((M + 1) * d, d), np.float32)
    if block == "x_t":
        wz[M * d:] = np.eye(d, dtype=np.float32)
    else:
        wz[(M - 1) * d:M * d] = np.eye(d, dtype=np.float32)
    p.wz = wz
    r = run(p)
    layers, z, _ = weights(p)
    if block == "x_t":
        src = O.stored_to_f64(p.rows(p.tgt_ids))
    else:
        src = r["o"][M - 1]
    # W1 = W3 = W2 = I gives SwiGLU(x) = SiLU(x) * x elementwise
    expect = O.swiglu(src, z)
    np.testing.assert_allclose(r["z"], expect, rtol=1e-12, atol=1e-14)
    p.spec = replace(p.spec, z_ln=True)
    r_ln = run(p)
    expect_ln = O.layer_norm(expect, z["ln_g"], z["ln_b"])
    np.testing.assert_allclose(r_ln["z"], expect_ln, rtol=1e-10, atol=1e-12)


def test_output_projection_identity():
    p = I.make_problem(small_spec(M=1))
    p.layers[0]["wo"] = np.eye(p.spec.d, dtype=np.float32)
    r = run(p)
    np.testing.assert_array_equal(r["o"][0], r["attn"][0])


def test_linear_mode_zero_map_gives_mean_v():
    """HyFormer linear mode with R_1 = 0: the next layer's queries are zero,
    so its softmax is uniform and the output is the mean of V^(2)."""
    p = I.make_problem(small_spec(qmode="linear", kv_ln=False, M=2))
    p.layers[0]["r"] = np.zeros((p.spec.d, p.spec.d), np.float32)
    r = run(p)
    layers, _, _ = weights(p)
    for u in range(p.spec.B):
        ids = p.hist_ids[p.hist_offsets[u]:p.hist_offsets[u + 1]]
        X = O.stored_to_f64(p.rows(ids))
        _, V = O.encode_history(X, layers[1], False)
        for t in range(p.tgt_offsets[u], p.tgt_offsets[u + 1]):
            np.testing.assert_allclose(r["attn"][1, t], V.mean(0), rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(r["z"][p.tgt_offsets[u]:p.tgt_offsets[u + 1]],
                                      r["o"][1, p.tgt_offsets[u]:p.tgt_offsets[u + 1]])


def test_history_encoding_without_ln_matches_torch_modules():
    """K/V of one layer against an independent torch float64 evaluation built
    from library modules (nn.Linear without bias, SiLU, LayerNorm)."""
    g = rng(12)
    d, h, L = 16, 40, 23
    X = g.normal(size=(L, d)) * 0.5
    w = {"w1": g.normal(size=(d, h)), "w3": g.normal(size=(d, h)), "w2": g.normal(size=(h, d)),
         "ln_g": g.normal(size=d), "ln_b": g.normal(size=d)}
    lw = {"kv": w, "wk": g.normal(size=(d, d)), "wv": g.normal(size=(d, d))}
    for ln in (True, False):
        K, V = O.encode_history(X, lw, ln)
        lin = lambda W: torch.nn.Linear(W.shape[0], W.shape[1], bias=False, dtype=torch.float64)
        l1, l3, l2, lk, lv = (lin(lw["kv"]["w1"]), lin(lw["kv"]["w3"]), lin(lw["kv"]["w2"]),
                              lin(lw["wk"]), lin(lw["wv"]))
        with torch.no_grad():
            for mod, W in ((l1, w["w1"]), (l3, w["w3"]), (l2, w["w2"]), (lk, lw["wk"]), (lv, lw["wv"])):
                mod.weight.copy_(torch.from_numpy(W.T.copy()))
            x = torch.from_numpy(X)
            y = l2(torch.nn.SiLU()(l1(x)) * l3(x))
            if ln:
                norm = torch.nn.LayerNorm(d, eps=1e-5, dtype=torch.float64)
                norm.weight.copy_(torch.from_numpy(w["ln_g"]))
                norm.bias.copy_(torch.from_numpy(w["ln_b"]))
                y = norm(y)
            np.testing.assert_allclose(K, lk(y).numpy(), rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(V, lv(y).numpy(), rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------- generator
def test_bf16_rounding_matches_torch():
    x = rng(13).normal(size=4096).astype(np.float32) * 10
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]          # ties to even
    ours = I.bf16_bits_to_f32(I.f32_to_bf16_bits(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_generator_determinism_and_rows():
    sp = small_spec(table_rows=70_000, dtype="bf16")
    a, b = I.make_problem(sp), I.make_problem(sp)
    assert np.array_equal(a.table, b.table) and np.array_equal(a.hist_ids, b.hist_ids)
    rows = np.array([0, 5, 65_535, 65_536, 69_999])
    assert np.array_equal(I.table_rows(sp, rows), a.table[rows])


def test_workload_shapes():
    s3 = I.spec(3)
    assert (s3.B, s3.L, s3.m, s3.d, s3.H, s3.hidden, s3.M) == (32, 10_240, 64, 256, 8, 512, 4)
    p4 = I.make_problem(replace(I.spec(4), table_rows=1000), with_table=False)
    lens = np.diff(p4.hist_offsets)
    assert lens.min() >= 16 and lens.max() <= 10_240
    assert abs(lens.mean() / 10_240 - 2 / 3) < 0.05          # Beta(2,1) mean
    ids = I.sample_ids(rng(1), 200_000, 4_000_000, "zipf", 1.1)
    assert 0.1 < len(np.unique(ids)) / len(ids) < 0.4        # ~a quarter unique
