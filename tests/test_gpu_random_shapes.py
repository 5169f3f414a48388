"""GPU parity over a seeded random sweep of small problem shapes.

Each case draws, from its own seed: the model width and head width (d 128,
256 or 512; d_h 32 or 64), the hidden width (d or 2d), the number of layers
(1-3), the number of users (1-5) with fixed or Beta-ragged lengths, some
users' histories emptied, the targets per user (1-64), LN after the history
FFN on or off, a random LN affine, LN on z, a small Zipf table (so that ids
repeat), the path (staged, or fused where it applies) and unique-id dedup on
the staged path.  z, every layer's o and attention output are compared with
the float64 oracle row by row at the bf16 bar (2e-2), the same bar as the
reduced workload tests; softmax scores only (ReLU chains are held to their
conditioning bar elsewhere).  A second sweep does the same on the fp32 path at
its bar (1e-5) over the widths it takes (any d = 32 H or 64 H up to 512, hidden
a multiple of 32) and both query modes (the W_C fusion chain, and the linear
next-query map).  The sweeps look for the shape corner the fixed cases miss: a
tail tile, an empty user at a tile boundary, a width or layer count
combination no named workload uses.  A third sweep mixes the modes (bf16,
staged): softmax or ReLU scores (ReLU held to its conditioning bar), the
fusion, linear or HyFormer query modes, the LONGER-style encoding, Cross-Mask
key masks and head maps, the context-similarity score bias and dedup, in the
combinations the library accepts.
"""
import numpy as np
import pytest

from parity_util import TOL, compare_forward, end_to_end_bar, gpu_run, oracle_run
from recsys_ultra_long_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU visible")]

N_CASES = 24


def _drop_histories(p, users):
    """The problem with the histories of ``users`` emptied (ids removed)."""
    ho = p.hist_offsets.astype(np.int64)
    keep = np.ones(int(ho[-1]), dtype=bool)
    lens = np.diff(ho)
    for u in users:
        keep[ho[u]:ho[u + 1]] = False
        lens[u] = 0
    p.hist_ids = p.hist_ids[keep]
    p.hist_offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return p


def _case(i):
    r = np.random.default_rng(1000 + i)
    d, H = [(128, 4), (256, 8), (256, 4), (512, 8), (512, 16)][r.integers(5)]
    B = int(r.integers(1, 6))
    ragged = bool(r.integers(2))
    sp = I.spec(3, name=f"random-{i}", B=B, d=d, H=H, hidden=int(d * r.choice([1, 2])), M=int(r.integers(1, 4)),
                table_rows=int(r.choice([3000, 20000])), m=int(r.choice([1, 3, 16, 40, 64])),
                L=None if ragged else int(r.integers(1, 700)), L_max=int(r.integers(40, 700)) if ragged else None,
                kv_ln=bool(r.integers(4) > 0), z_ln=bool(r.integers(2)), ln_random=bool(r.integers(2)),
                seed=5000 + i)
    fused_ok = sp.kv_ln and sp.m <= 64 and ((d == 256 and d // H in (32, 64)) or (d == 128 and d // H == 32))
    path = "fused" if fused_ok and r.integers(3) == 0 else "staged"
    dedup = path == "staged" and bool(r.integers(2))
    drop = [u for u in range(B) if B > 1 and r.integers(4) == 0]
    return sp, path, dedup, drop


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    sp, path, dedup, drop = _case(i)
    p = I.make_problem(sp)
    if drop:
        p = _drop_histories(p, drop)
    print(f"[random {i}] d={sp.d} H={sp.H} hidden={sp.hidden} M={sp.M} B={sp.B} m={sp.m} "
          f"n_hist={p.n_hist} kv_ln={sp.kv_ln} z_ln={sp.z_ln} ln_random={sp.ln_random} "
          f"path={path} dedup={dedup} empty={drop}", flush=True)
    g = gpu_run(p, path=path, dedup=dedup)
    o = oracle_run(p)
    errs = compare_forward(g, o, sp.dtype)
    print(f"[random {i}] errors {errs}", flush=True)
    assert int(g["status"][0]) == 0
    assert all(e <= TOL[sp.dtype] for e in errs.values()), errs


def _case_f32(i):
    r = np.random.default_rng(3000 + i)
    dh = int(r.choice([32, 64]))
    H = int(r.integers(1, 512 // dh + 1))
    d = dh * H
    ragged = bool(r.integers(2))
    linear = bool(r.integers(3) == 0)
    sp = I.spec(1, name=f"random-f32-{i}", B=int(r.integers(1, 6)), d=d, H=H, hidden=int(32 * r.integers(1, 17)),
                M=int(r.integers(1, 4)), table_rows=int(r.choice([3000, 20000])), m=int(r.choice([1, 3, 16, 40, 64])),
                L=None if ragged else int(r.integers(1, 500)), L_max=int(r.integers(40, 500)) if ragged else None,
                qmode="linear" if linear else "fusion", kv_ln=bool(r.integers(4) > 0) and not linear,
                z_ln=bool(r.integers(2)), ln_random=bool(r.integers(2)), ids="zipf", seed=6000 + i)
    drop = [u for u in range(sp.B) if sp.B > 1 and r.integers(4) == 0]
    return sp, drop


@pytest.mark.parametrize("i", range(16))
def test_random_shape_f32_matches_oracle(i):
    sp, drop = _case_f32(i)
    p = I.make_problem(sp)
    if drop:
        p = _drop_histories(p, drop)
    print(f"[random-f32 {i}] d={sp.d} H={sp.H} hidden={sp.hidden} M={sp.M} B={sp.B} m={sp.m} "
          f"n_hist={p.n_hist} qmode={sp.qmode} kv_ln={sp.kv_ln} z_ln={sp.z_ln} empty={drop}", flush=True)
    g = gpu_run(p)
    o = oracle_run(p)
    errs = compare_forward(g, o, sp.dtype)
    print(f"[random-f32 {i}] errors {errs}", flush=True)
    assert int(g["status"][0]) == 0
    assert all(e <= TOL[sp.dtype] for e in errs.values()), errs


def _case_modes(i):
    r = np.random.default_rng(4000 + i)
    d, H = [(128, 4), (256, 8), (256, 4), (512, 8), (512, 16)][r.integers(5)]
    longer = r.integers(4) == 0
    qmode = ["fusion", "linear", "hyformer"][r.integers(3)]
    score = "softmax" if longer or r.integers(2) else "relu"
    ragged = bool(r.integers(2))
    over = dict(name=f"random-modes-{i}", B=int(r.integers(1, 6)), d=d, H=H, hidden=int(d * r.choice([1, 2])),
                M=int(r.integers(1, 4)), table_rows=int(r.choice([3000, 20000])), m=int(r.choice([1, 3, 16, 40])),
                L=None if ragged else int(r.integers(1, 600)), L_max=int(r.integers(40, 600)) if ragged else None,
                score=score, qmode=qmode, kv_ln=bool(r.integers(4) > 0), z_ln=bool(r.integers(2)),
                ln_random=bool(r.integers(2)), seed=8000 + i)
    if qmode == "hyformer":  # the token mixing splits d into m + n_ns equal parts
        ok = [n for n in range(0, 25) if d % (over["m"] + n) == 0]
        if ok:
            over["n_ns"] = int(r.choice(ok))
        else:
            over["qmode"] = "fusion"
    if longer:
        over.update(encoder="longer", l_short=int(r.integers(1, 600)))
    sp = I.spec(3, **over)
    mask = not longer and r.integers(3) == 0
    hmap = [int(x) for x in r.integers(0, H, size=H)] if mask and H <= 16 and r.integers(2) else None
    bias = not longer and r.integers(3) == 0
    dedup = not longer and bool(r.integers(2))
    drop = [u for u in range(sp.B) if sp.B > 1 and r.integers(5) == 0]
    return sp, mask, hmap, bias, dedup, drop


@pytest.mark.parametrize("i", range(20))
def test_random_modes_match_oracle(i):
    sp, mask, hmap, bias, dedup, drop = _case_modes(i)
    p = I.make_problem(sp)
    if drop:
        p = _drop_histories(p, drop)
    if mask:
        p.extra["key_mask"] = I.cross_mask(sp, p.n_hist, sorted({1 % sp.H, (sp.H - 1)}), 0.5, seed=i)
    if hmap is not None:
        p.extra["head_map"] = hmap
    if bias:
        p.extra["score_bias"] = I.score_bias(sp, p.n_hist)
    print(f"[random-modes {i}] d={sp.d} H={sp.H} hidden={sp.hidden} M={sp.M} B={sp.B} m={sp.m} "
          f"n_hist={p.n_hist} score={sp.score} qmode={sp.qmode} n_ns={sp.n_ns} encoder={sp.encoder} "
          f"l_short={sp.l_short} kv_ln={sp.kv_ln} mask={bool(mask)} map={hmap} bias={bool(bias)} "
          f"dedup={dedup} empty={drop}", flush=True)
    g = gpu_run(p, dedup=dedup)
    o = oracle_run(p)
    errs = compare_forward(g, o, sp.dtype)
    bar = end_to_end_bar(p, exact=o)
    print(f"[random-modes {i}] errors {errs} bar {bar}", flush=True)
    assert int(g["status"][0]) == 0
    assert all(errs[k] <= bar[k] for k in errs), (errs, bar)
