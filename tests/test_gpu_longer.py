"""GPU parity of the LONGER-style sequence encoding (STCA_ENC_LONGER):
[HyFormer] §3.4.1 (ii), eq. (6) H_l = CrossAttn(S_short, S, S) with S_short
the user's last min(L_u, l_short) rows, then eq. (8) K_l = H_l W_K,
V_l = H_l W_V; the targets decode over the short rows.  Checked end to end
against the float64 oracle at the bf16 tolerance.

Cases: the three query modes (HyFormer, fusion, linear) at reduced sizes with
ragged histories, so that some users have fewer than l_short items and their
short sequence is the whole history; d = 128 / 256 / 512 (d_h 32 and 64);
l_short = 1; 65..256 short rows (one wave per target group in the
encoder attention); users with an empty history; and the HyFormer feed workload at
full size (64 users x 8192 items, l_short = 256) in the bench's launch
configuration, checked on sampled users.
"""
from dataclasses import replace

import numpy as np
import pytest

from recsys_ultra_long_amd import inputs as I

from parity_util import TOL, compare_forward, gpu_run, oracle_run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU visible")]


def _hy(seq="feed", **over):
    sp = replace(I.spec(5)[seq], qmode="hyformer", n_ns=8, encoder="longer", l_short=256)
    return replace(sp, **over)


def _check(p, users=None):
    sp = p.spec
    print(f"[longer] {sp.name} qmode={sp.qmode} d={sp.d} H={sp.H} B={sp.B} n_hist={p.n_hist} "
          f"n_tgt={p.n_tgt} l_short={sp.l_short}", flush=True)
    g = gpu_run(p)
    o = oracle_run(p, users)
    ut = None
    if users is not None:
        ut = np.concatenate([np.arange(p.tgt_offsets[u], p.tgt_offsets[u + 1]) for u in users])
    errs = compare_forward(g, o, sp.dtype, users_t=ut)
    print(f"[longer] errors {errs}", flush=True)
    assert int(g["status"][0]) == 0
    assert all(e <= TOL[sp.dtype] for e in errs.values()), errs
    return g, o


CASES = {
    "hyformer-feed": lambda: _hy(B=4, L=700, table_rows=20000, l_short=64),
    "hyformer-search-short": lambda: _hy("search", B=3, L=None, L_max=300, L_min=5, table_rows=20000,
                                         n_ns=0, M=2, l_short=512, seed=78),
    "fusion-ragged": lambda: replace(I.spec(3), B=3, L=None, L_max=1500, L_min=20, m=8, M=2,
                                     table_rows=20000, encoder="longer", l_short=900, seed=31),
    "linear-d128": lambda: replace(I.spec(4), B=6, L_max=1200, m=4, M=2, table_rows=20000,
                                   qmode="linear", encoder="longer", l_short=40, seed=41),
    "fusion-lshort1": lambda: replace(I.spec(2), B=4, L=300, M=2, table_rows=20000, m=3,
                                      encoder="longer", l_short=1, seed=21),
    # 65..256 short rows: one wave per group of 64 in the encoder attention
    "fusion-3groups-dh32": lambda: replace(I.spec(3), B=3, L=None, L_max=1500, L_min=20, m=8, M=2,
                                           table_rows=20000, encoder="longer", l_short=130, seed=32),
    "hyformer-4groups-ragged": lambda: _hy(B=5, L=None, L_max=900, L_min=60, beta_a=0.7, table_rows=20000,
                                           M=2, l_short=250, seed=53),
}


@pytest.mark.parametrize("case", list(CASES))
def test_longer_matches_oracle(case):
    _check(I.make_problem(CASES[case]()))


def test_longer_empty_history_users():
    sp = _hy(B=4, L=200, table_rows=20000, M=2, l_short=32)
    p = I.make_problem(sp)
    lens = np.diff(p.hist_offsets).copy()
    lens[[1, 3]] = 0
    p.hist_ids = np.concatenate([p.hist_ids[p.hist_offsets[u]:p.hist_offsets[u] + lens[u]]
                                 for u in range(sp.B)]).astype(np.int32)
    p.hist_offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g, _ = _check(p)
    for u in (1, 3):
        assert np.all(g["attn"][:, p.tgt_offsets[u]:p.tgt_offsets[u + 1]] == 0)


def test_longer_fullsize_feed_sampled():
    sp = _hy()
    p = I.make_problem(sp, threads=16)
    _check(p, users=sorted({0, sp.B // 2, sp.B - 1}))


def _fusion(**over):
    sp = replace(I.spec(3), B=3, L=300, m=4, M=2, table_rows=20000, encoder="longer", l_short=64, seed=33)
    return replace(sp, **over)


@pytest.mark.parametrize("mode", ["hyformer", "fusion"])
def test_longer_all_histories_empty(mode):
    sp = _hy(B=3, L=100, table_rows=20000, M=2, l_short=16) if mode == "hyformer" else _fusion(L=100)
    p = I.make_problem(sp)
    p.hist_offsets = np.zeros(sp.B + 1, np.int32)
    p.hist_ids = p.hist_ids[:0].copy()
    g, _ = _check(p)
    assert np.all(g["attn"] == 0)


def test_longer_no_targets():
    p = I.make_problem(_fusion())
    p.tgt_offsets = np.zeros(p.spec.B + 1, np.int32)
    p.tgt_ids = p.tgt_ids[:0].copy()
    print(f"[longer] no targets: n_hist={p.n_hist}", flush=True)
    g = gpu_run(p)
    assert int(g["status"][0]) == 0
    assert g["z"].shape[0] == 0


def test_longer_bad_offsets_flagged_not_faulting():
    from recsys_ultra_long_amd import stca
    p = I.make_problem(_fusion(L=200))
    p.hist_offsets = p.hist_offsets.copy()
    p.hist_offsets[1] = p.hist_offsets[2] + 5        # not monotone
    print("[longer] bad offsets", flush=True)
    g = gpu_run(p)
    assert int(g["status"][0]) & stca.DEV_BAD_HIST_OFFSETS
    assert np.all(g["attn"] == 0)                      # every user treated as empty
