"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (row-normalised max error, see parity_util.row_rel_err): 1e-5 for
the fp32 configuration, 2e-2 for bf16 storage with fp32 accumulation.  Gather
rows and active-key counts on shared operands are compared bit-exactly.
"""
from dataclasses import replace

import numpy as np
import pytest

from oracle import stca_oracle as O
from recsys_ultra_long_amd import inputs as I

from parity_util import TOL, compare_forward, end_to_end_bar, gpu_run, oracle_run, row_rel_err, stepwise_errors

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # the gpu marker selects these tests; fail loudly on a CPU machine
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU visible")]


def _stca():
    from recsys_ultra_long_amd import stca
    stca.load()
    return stca


# ------------------------------------------------------------------ attention core
def _attn_case(dtype, score, dh, H, lens, ms, seed=0, scale_q=1.0):
    g = np.random.default_rng(seed)
    d = dh * H
    ho = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    to = np.concatenate([[0], np.cumsum(ms)]).astype(np.int32)
    n, T = int(ho[-1]), int(to[-1])
    q = (g.standard_normal((T, d)) * scale_q / np.sqrt(dh)).astype(np.float32)
    k = g.standard_normal((n, d)).astype(np.float32)
    v = g.standard_normal((n, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (I.f32_to_bf16_bits(x) for x in (q, k, v))
    return ho, to, q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("score", ["softmax", "relu"])
@pytest.mark.parametrize("dh,H", [(32, 8), (64, 4)])
def test_attention_core_shared_operands(dtype, score, dh, H):
    # 70 targets for one user: two target groups (bf16: one wave per group)
    _check_core(dtype, score, dh, H, [0, 1, 31, 32, 33, 200, 1000, 5], [3, 1, 17, 64, 70, 2, 33, 0], dh + H)


@pytest.mark.parametrize("score", ["softmax", "relu"])
@pytest.mark.parametrize("dh,H", [(32, 8), (64, 8)])
@pytest.mark.parametrize("ms", [[256, 3, 130, 0, 200, 64], [300, 3, 130, 0, 200, 64]])
def test_attention_core_many_targets(score, dh, H, ms):
    # up to 256 targets per user (four groups, one per wave, K/V read once
    # per workgroup), and 300 (five groups, the waves split the keys)
    _check_core("bf16", score, dh, H, [700, 40, 1, 300, 0, 2049], ms, 7 + dh)


def _check_core(dtype, score, dh, H, lens, ms, seed):
    stca = _stca()
    print(f"[core] {dtype} {score} dh={dh} H={H} lens={lens} ms={ms}", flush=True)
    ho, to, q, k, v = _attn_case(dtype, score, dh, H, lens, ms, seed=seed)
    dev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    attn, active, st = stca.attention(dev(q), dev(k), dev(v), dev(ho), dev(to), H, score,
                                      chunk_keys=64)
    torch.cuda.synchronize()
    attn = attn.cpu().numpy()
    assert int(st.cpu()[0]) == 0
    Q, K, V = O.stored_to_f64(q), O.stored_to_f64(k), O.stored_to_f64(v)
    for u in range(len(lens)):
        a, b = ho[u], ho[u + 1]
        t0, t1 = to[u], to[u + 1]
        if t1 == t0:
            continue
        ref, cnt, amb = O.attention_core(Q[t0:t1], K[a:b], V[a:b], H, score, scale=1.0)
        err = row_rel_err(attn[t0:t1], ref)
        assert err <= TOL[dtype], (u, err)
        if score == "relu":
            gc = active.cpu().numpy()[t0:t1]
            exact = amb == 0
            assert np.array_equal(gc[exact], cnt[exact]), u
            band = np.abs(gc - cnt) <= amb
            assert np.all(band), u
        if b - a == 0:
            assert np.all(attn[t0:t1] == 0)


def test_attention_split_invariance():
    """Different split-L chunk sizes give the same result within tolerance and
    the same chunk size gives bit-identical results (fixed-order merge)."""
    stca = _stca()
    ho, to, q, k, v = _attn_case("bf16", "softmax", 32, 8, [5000, 77, 1], [64, 9, 1], seed=5)
    dev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    args = (dev(q), dev(k), dev(v), dev(ho), dev(to), 8, "softmax")
    outs = [stca.attention(*args, chunk_keys=ck)[0].cpu().numpy() for ck in (32, 128, 1024, 0)]
    again = stca.attention(*args, chunk_keys=128)[0].cpu().numpy()
    assert np.array_equal(outs[1], again)
    for o in outs[1:]:
        assert row_rel_err(o, outs[0]) < 1e-2


def test_attention_split_invariance_four_groups():
    """The same with 256 targets for the long user (one wave per target group)."""
    stca = _stca()
    ho, to, q, k, v = _attn_case("bf16", "softmax", 64, 4, [5000, 77, 1], [256, 9, 1], seed=6)
    dev = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    args = (dev(q), dev(k), dev(v), dev(ho), dev(to), 4, "softmax")
    outs = [stca.attention(*args, chunk_keys=ck)[0].cpu().numpy() for ck in (32, 128, 1024, 0)]
    again = stca.attention(*args, chunk_keys=128)[0].cpu().numpy()
    assert np.array_equal(outs[1], again)
    for o in outs[1:]:
        assert row_rel_err(o, outs[0]) < 1e-2


# ------------------------------------------------------------------ full forward
def _small(k, **over):
    base = {
        1: {},
        2: dict(B=4, L=300, table_rows=5000),
        3: dict(B=2, L=700, m=64, table_rows=20000),
        4: dict(B=6, L_max=1200, table_rows=20000),
    }[k]
    base.update(over)
    return I.spec(k, **base)


def _check(p, path="staged", chunk_keys=0, keys=("z", "o", "attn")):
    g = gpu_run(p, path=path, chunk_keys=chunk_keys)
    o = oracle_run(p)
    errs = compare_forward(g, o, p.spec.dtype, keys=keys)
    tol = TOL[p.spec.dtype]
    assert all(e <= tol for e in errs.values()), errs
    assert int(g["status"][0]) == 0
    return g, o, errs


def test_config1_full_fp32():
    p = I.make_problem(I.spec(1))
    _check(p)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_configs_reduced_bf16(k):
    p = I.make_problem(_small(k))
    _check(p)


def _check_stepwise(p):
    """Every step within tolerance at the operands the GPU fed it; active
    counts exact where no score lies within rounding of zero; and end to end
    within ``end_to_end_bar``: the tolerance for softmax, for the ReLU-scored
    chain max(tol, 2 D) with D its measured conditioning on these inputs."""
    g = gpu_run(p, dumps=("q", "kv"))
    errs, cnt_exact, cnt_band = stepwise_errors(p, g)
    tol = TOL[p.spec.dtype]
    assert all(e <= tol for e in errs.values()), errs
    assert cnt_exact and cnt_band
    assert int(g["status"][0]) == 0
    o = oracle_run(p)
    e2e = compare_forward(g, o, p.spec.dtype)
    bar = end_to_end_bar(p, exact=o)
    print("stepwise", {k: f"{v:.1e}" for k, v in errs.items()},
          "end-to-end", {k: f"{v:.1e}" for k, v in e2e.items()},
          "bar", {k: f"{v:.1e}" for k, v in bar.items()}, flush=True)
    assert all(e2e[k] <= bar[k] for k in e2e), (e2e, bar)
    return g, o


def test_config4_relu_counts():
    p = I.make_problem(_small(4, score="relu"))
    g, o = _check_stepwise(p)
    # first layer: both sides start from the same table rows, so the counts
    # agree up to scores that sit within rounding of zero
    diff = np.abs(g["active"][0].astype(np.int64) - o["active"][0])
    assert diff.mean() < 0.02 * max(1.0, o["active"][0].mean())


@pytest.mark.parametrize("k", [2, 3, 4])
def test_stepwise_softmax(k):
    _check_stepwise(I.make_problem(_small(k, B=3)))


def test_config5_linear_no_kv_ln():
    sp = I.spec(5)["feed"]
    p = I.make_problem(replace(sp, B=3, L=400, table_rows=5000))
    _check(p)
    sp = I.spec(5)["search"]
    p = I.make_problem(replace(sp, B=3, L=150, table_rows=5000))
    _check(p)


@pytest.mark.parametrize("z_ln,ln_random", [(True, True), (False, True)])
def test_ln_affine_and_z_ln(z_ln, ln_random):
    p = I.make_problem(_small(2, z_ln=z_ln, ln_random=ln_random, B=3, L=100))
    _check(p)


def test_fp32_ragged_relu_multilayer():
    p = I.make_problem(I.spec(1, L=None, L_max=300, L_min=1, B=5, M=3, m=5, score="relu",
                              ln_random=True))
    _check_stepwise(p)


def test_fp32_ragged_softmax_multilayer():
    p = I.make_problem(I.spec(1, L=None, L_max=300, L_min=1, B=5, M=3, m=5, ln_random=True))
    _check(p)


def test_config5_stepwise():
    sp = I.spec(5)["feed"]
    _check_stepwise(I.make_problem(replace(sp, B=2, L=300, table_rows=5000)))


def test_gather_dump_bitwise():
    p = I.make_problem(_small(4, B=3))
    g = gpu_run(p, dumps=("x",))
    assert np.array_equal(g["x"], p.table[p.hist_ids])


def test_single_key_returns_v_exactly():
    """P1 on the device: a one-item history returns V exactly (softmax weight 1)."""
    p = I.make_problem(_small(3, B=2, L=1, m=5))
    g = gpu_run(p, dumps=("kv",))
    M, T, d = g["attn"].shape
    for i in range(M):
        V = O.stored_to_f64(g["kv"][i, 1])               # [n_hist, d]
        for u in range(p.spec.B):
            v = V[p.hist_offsets[u]]
            for t in range(p.tgt_offsets[u], p.tgt_offsets[u + 1]):
                assert np.array_equal(g["attn"][i, t], v.astype(np.float32))


def test_equal_keys_give_mean_v():
    """P2 on the device: W_K = 0 makes every score 0, so attention = mean(V)."""
    p = I.make_problem(_small(2, B=3, L=150))
    for l in p.layers:
        l["wk"] = np.zeros_like(l["wk"])
    g = gpu_run(p, dumps=("kv",))
    for i in range(p.spec.M):
        V = O.stored_to_f64(g["kv"][i, 1])
        for u in range(p.spec.B):
            mv = V[p.hist_offsets[u]:p.hist_offsets[u + 1]].mean(0)
            for t in range(p.tgt_offsets[u], p.tgt_offsets[u + 1]):
                assert row_rel_err(g["attn"][i, t][None], mv[None]) < 1e-2


def test_permutation_invariance_gpu():
    p = I.make_problem(_small(4, B=4))
    q = I.make_problem(_small(4, B=4))
    rng = np.random.default_rng(3)
    for u in range(q.spec.B):
        a, b = q.hist_offsets[u], q.hist_offsets[u + 1]
        q.hist_ids[a:b] = q.hist_ids[a:b][rng.permutation(b - a)]
    g1, g2 = gpu_run(p), gpu_run(q)
    assert row_rel_err(g2["z"], g1["z"]) < TOL["bf16"]


def test_rlb_equals_single_target_runs():
    """P4 on the device: m targets sharing a user's K/V equal m single-target
    users with the same history.  The K/V side and the first layer's queries
    are computed identically (bitwise).  The persistent attention grid cuts a
    user's history into partials according to the whole batch; each partial
    scales its probabilities against its own running max before they are
    rounded to bf16 for the PV product, so first-layer attention agrees at that
    quantisation level (2^-9 per weight, a few 1e-4 per row), not bitwise.
    Deeper layers carry the difference through bf16 roundings of attn and o, so
    end to end the bar is the bf16 tolerance."""
    p = I.make_problem(_small(3, B=2, L=500, m=20))
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
    g1 = gpu_run(p, chunk_keys=128, dumps=("kv", "q"))
    g2 = gpu_run(q, chunk_keys=128, dumps=("kv", "q"))
    for i in range(p.spec.M):
        for u in range(B):
            a, b = ho[u], ho[u + 1]
            for t in range(to[u], to[u + 1]):
                assert np.array_equal(g1["kv"][i, :, a:b], g2["kv"][i, :, hoff[t]:hoff[t + 1]])
    assert np.array_equal(g1["q"][0], g2["q"][0])
    assert row_rel_err(g2["attn"][0], g1["attn"][0]) < 2e-3
    for k in ("z", "o", "attn"):
        assert row_rel_err(g2[k], g1[k]) < TOL["bf16"], k


def test_deterministic_rerun():
    p = I.make_problem(_small(3, B=2, L=900))
    g1, g2 = gpu_run(p), gpu_run(p)
    for k in ("z", "o", "attn"):
        assert np.array_equal(g1[k], g2[k]), k


def test_out_of_range_id_flags_and_zero_row():
    stca = _stca()
    p = I.make_problem(_small(2, B=2, L=64))
    p.hist_ids[3] = p.spec.table_rows + 5
    p.hist_ids[70] = -2
    g = gpu_run(p, dumps=("x",))
    assert int(g["status"][0]) & stca.DEV_BAD_ID
    assert np.all(g["x"][3] == 0) and np.all(g["x"][70] == 0)
    assert np.isfinite(g["z"]).all()


def test_bad_offsets_flagged_not_faulting():
    stca = _stca()
    p = I.make_problem(_small(2, B=3, L=64))
    p.hist_offsets = p.hist_offsets.copy()
    p.hist_offsets[1] = p.hist_offsets[2] + 5        # not monotone
    g = gpu_run(p)
    assert int(g["status"][0]) & stca.DEV_BAD_HIST_OFFSETS
    assert np.all(g["attn"] == 0)                      # every user treated as empty


def test_empty_histories_give_zero_attention():
    p = I.make_problem(_small(2, B=3, L=64))
    p.hist_offsets = np.array([0, 0, 64, 64], np.int32)
    p.hist_ids = p.hist_ids[:64].copy()
    g = gpu_run(p)
    o = oracle_run(p)
    assert np.all(g["attn"][:, 0] == 0) and np.all(g["attn"][:, 2] == 0)
    assert row_rel_err(g["z"], o["z"]) <= TOL["bf16"]
