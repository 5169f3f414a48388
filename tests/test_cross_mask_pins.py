"""Pins for the oracle's Cross-Mask attention ([WeChat] §3.2-3.3): vertical
masks per head and heads that share an attention map, and the additive
context-similarity score bias ([WeChat] §2.2.3) (CPU only).

Each is tied to something other than the masked code path: the unmasked
oracle on explicitly selected rows (brute force), identities (all-visible
mask, identity map), a constructed equivalent (copying one head's Q / K
columns into another's), and the all-masked closed form.
"""
import math

import numpy as np
import pytest

from oracle import stca_oracle as O


def _ops(seed, L=23, H=4, dh=8):
    g = np.random.default_rng(seed)
    d = H * dh
    return g.normal(size=d), g.normal(size=(L, d)), g.normal(size=(L, d)), H, dh


@pytest.mark.parametrize("score", ["softmax", "relu"])
def test_all_visible_mask_and_identity_map_change_nothing(score):
    Q, K, V, H, _ = _ops(1)
    a0, c0, _ = O.attention_target(Q, K, V, H, score)
    a1, c1, _ = O.attention_target(Q, K, V, H, score, key_mask=np.full(len(K), (1 << H) - 1),
                                   head_map=list(range(H)))
    np.testing.assert_array_equal(a0, a1)
    np.testing.assert_array_equal(c0, c1)


@pytest.mark.parametrize("score", ["softmax", "relu"])
def test_masked_head_equals_attention_over_selected_rows(score):
    Q, K, V, H, dh = _ops(2)
    g = np.random.default_rng(3)
    mask = g.integers(0, 1 << H, size=len(K))
    a, c, _ = O.attention_target(Q, K, V, H, score, key_mask=mask)
    for eta in range(H):
        rows = [j for j in range(len(K)) if (mask[j] >> eta) & 1]
        ref, rc, _ = O.attention_target(Q, K[rows], V[rows], H, score)
        cols = slice(eta * dh, (eta + 1) * dh)
        np.testing.assert_allclose(a[cols], ref[cols], rtol=1e-12, atol=1e-15)
        if score == "relu":
            assert c[eta] == rc[eta]


def test_head_map_equals_copied_columns():
    """Head 1 scoring with head 0's Q / K columns is the plain attention on
    operands whose head-1 Q / K columns are a copy of head 0's."""
    Q, K, V, H, dh = _ops(4)
    hmap = [0, 0, 2, 2]
    a, _, _ = O.attention_target(Q, K, V, H, "softmax", head_map=hmap)
    Q2, K2 = Q.copy(), K.copy()
    for eta, src in enumerate(hmap):
        Q2[eta * dh:(eta + 1) * dh] = Q[src * dh:(src + 1) * dh]
        K2[:, eta * dh:(eta + 1) * dh] = K[:, src * dh:(src + 1) * dh]
    ref, _, _ = O.attention_target(Q2, K2, V, H, "softmax")
    np.testing.assert_allclose(a, ref, rtol=1e-13, atol=1e-15)
    # heads 0 and 1 share one map: with V's head-1 columns equal to head 0's
    # they give the same output
    V2 = V.copy()
    V2[:, dh:2 * dh] = V[:, :dh]
    b, _, _ = O.attention_target(Q, K, V2, H, "softmax", head_map=hmap)
    np.testing.assert_allclose(b[:dh], b[dh:2 * dh], rtol=1e-13)


@pytest.mark.parametrize("score", ["softmax", "relu"])
def test_head_without_visible_keys_gives_zero(score):
    Q, K, V, H, dh = _ops(5)
    mask = np.full(len(K), (1 << H) - 1) & ~(1 << 2)          # head 2 sees nothing
    a, c, _ = O.attention_target(Q, K, V, H, score, key_mask=mask)
    assert np.all(a[2 * dh:3 * dh] == 0) and c[2] == 0
    ref, _, _ = O.attention_target(Q, K, V, H, score)
    np.testing.assert_array_equal(a[:2 * dh], ref[:2 * dh])


def test_single_visible_key_returns_its_value():
    Q, K, V, H, dh = _ops(6)
    mask = np.zeros(len(K), dtype=np.int64)
    mask[7] = 1 << 1
    a, _, _ = O.attention_target(Q, K, V, H, "softmax", key_mask=mask)
    np.testing.assert_allclose(a[dh:2 * dh], V[7, dh:2 * dh], rtol=1e-14)


# ----------------------------------------------------------------- score bias
# The context-similarity bias of [WeChat] §2.2.3 (no formula on the page) is
# read as an additive per-(item, head) term on the scaled score.


def test_constant_bias_changes_nothing_under_softmax():
    Q, K, V, H, _ = _ops(7)
    a0, _, _ = O.attention_target(Q, K, V, H, "softmax")
    bias = np.tile(np.array([3.0, -7.5, 0.25, 12.0]), (len(K), 1))   # one constant per head
    a1, _, _ = O.attention_target(Q, K, V, H, "softmax", score_bias=bias)
    np.testing.assert_allclose(a1, a0, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("score", ["softmax", "relu"])
def test_large_negative_bias_is_a_mask(score):
    """A bias of -1e4 on an item drives its softmax weight to exactly 0 in
    float64 and its ReLU score below 0: the same as masking it out."""
    Q, K, V, H, dh = _ops(8)
    g = np.random.default_rng(9)
    mask = g.integers(0, 1 << H, size=len(K))
    mask[0] = (1 << H) - 1                    # every head keeps at least one item
    bias = np.where(((mask[:, None] >> np.arange(H)) & 1) == 1, 0.0, -1e4)
    a, c, _ = O.attention_target(Q, K, V, H, score, score_bias=bias)
    ref, rc, _ = O.attention_target(Q, K, V, H, score, key_mask=mask)
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-15)
    if score == "relu":
        np.testing.assert_array_equal(c, rc)


def test_bias_matches_sdpa_additive_mask():
    """Softmax with a per-item bias is torch's scaled-dot-product attention
    with that bias as its additive float mask (float64, every head)."""
    import torch
    import torch.nn.functional as F
    g = np.random.default_rng(10)
    H, dh, L, m = 3, 16, 29, 5
    d = H * dh
    Q = g.normal(size=(m, d))
    K, V = g.normal(size=(L, d)), g.normal(size=(L, d))
    bias = g.normal(size=(L, H)) * 2.0
    a, _, _ = O.attention_core(Q, K, V, H, "softmax", score_bias=bias)
    t = lambda x: torch.from_numpy(x)
    for h in range(H):
        c = slice(h * dh, (h + 1) * dh)
        ref = F.scaled_dot_product_attention(t(Q[:, c])[None], t(K[:, c])[None], t(V[:, c])[None],
                                             attn_mask=t(np.tile(bias[:, h], (m, 1)))[None])[0].numpy()
        np.testing.assert_allclose(a[:, c], ref, rtol=1e-12, atol=1e-14)


def test_single_item_bias_scales_its_weight():
    """A bias b on one item multiplies its softmax weight by e^b: with two
    items of equal score and values e1, e2, the output is
    (e^b e1 + e2) / (e^b + 1)."""
    H, dh = 1, 4
    Q = np.array([1.0, 0.0, 0.0, 0.0])
    K = np.array([[0.5, 1.0, 0.0, 0.0], [0.5, -1.0, 0.0, 0.0]])   # equal scores
    V = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])
    for b in (-2.0, 0.0, 0.7, 5.0):
        a, _, _ = O.attention_target(Q, K, V, H, "softmax", score_bias=np.array([[b], [0.0]]))
        e = math.exp(b)
        np.testing.assert_allclose(a, [e / (e + 1), 1 / (e + 1), 0, 0], rtol=1e-14, atol=1e-16)


def test_relu_bias_shifts_the_threshold():
    """ReLU: an item whose score is exactly 0 becomes active with weight b
    under a bias b > 0; a bias below -max(s) switches every item off."""
    H, dh = 1, 4
    Q = np.array([1.0, 0.0, 0.0, 0.0])
    K = np.array([[0.0, 1.0, 0.0, 0.0], [2.0, 0.0, 0.0, 0.0]])     # scores 0 and 1 (scale 1/2)
    V = np.array([[0.0, 0.0, 1.0, 0.0], [0.0, 0.0, 0.0, 1.0]])
    a, c, _ = O.attention_target(Q, K, V, H, "relu", score_bias=np.array([[0.25], [0.0]]))
    np.testing.assert_allclose(a, [0, 0, 0.25, 1.0], rtol=1e-15)
    assert c[0] == 2
    a, c, _ = O.attention_target(Q, K, V, H, "relu", score_bias=np.array([[-0.5], [-1.5]]))
    assert np.all(a == 0) and c[0] == 0


def test_bias_follows_the_mask_rows():
    """With a mask, item j's bias stays item j's: masking then biasing equals
    biasing the explicitly selected rows."""
    Q, K, V, H, dh = _ops(11)
    g = np.random.default_rng(12)
    mask = g.integers(1, 1 << H, size=len(K))
    bias = g.normal(size=(len(K), H))
    a, _, _ = O.attention_target(Q, K, V, H, "softmax", key_mask=mask, score_bias=bias)
    for eta in range(H):
        rows = [j for j in range(len(K)) if (mask[j] >> eta) & 1]
        ref, _, _ = O.attention_target(Q, K[rows], V[rows], H, "softmax", score_bias=bias[rows])
        cols = slice(eta * dh, (eta + 1) * dh)
        np.testing.assert_allclose(a[cols], ref[cols], rtol=1e-12, atol=1e-15)
