"""Pins for the oracle's Cross-Mask attention ([WeChat] §3.2-3.3): vertical
masks per head and heads that share an attention map (CPU only).

Each is tied to something other than the masked code path: the unmasked
oracle on explicitly selected rows (brute force), identities (all-visible
mask, identity map), a constructed equivalent (copying one head's Q / K
columns into another's), and the all-masked closed form.
"""
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
