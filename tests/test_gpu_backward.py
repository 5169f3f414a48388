"""GPU parity of the backward pass (``stca_backward``): gradients of <dz, z>
for every weight and embedding row against the float64 backward oracle.

Checks:
* end to end on reduced workloads (d 256 with d_h 64 / 32, d 128 ragged, the
  training workload's Beta(1/4, 1) lengths, random LN affine and z-LN): the
  per-item and per-target row gradients and the table gradient on every row a
  history item or target touched, row by row (each row's largest error over
  its largest magnitude) within the bf16 bar 2e-2; every weight gradient
  within 2e-2 relative Frobenius and, row by row (each input feature's row of
  an [in, out] gradient), within WEIGHT_ROW_TOL of max(its own largest
  magnitude, the median row's).  Row r of a weight gradient is
  sum_t x_t[r] g_t over tokens or targets: a feature r that is small for
  every token makes a row far below the others, and its error comes from the
  forward's error in x_t[r], which is relative to the whole row x_t, not to
  x_t[r] -- hence the median floor.  The largest row error of bf16 rounding
  noise sits 2-4x above its Frobenius level (measured on these workloads:
  Frobenius <= 1.2e-2, floored rows <= 3.7e-2), hence 5e-2; a wrong, swapped
  or missing row is off by the order of the row scale itself;
* the attention backward stepwise, softmax and ReLU: dQ, dK, dV against the
  oracle evaluated at the operands the GPU actually used (its Q, K, V rows
  and its upstream gradient of the attention output);
* invariants: dz = 0 gives exactly zero gradients; a second call accumulates
  exactly the same weight gradients again; users without history or targets;
* full size (training workload, every user present): dz nonzero for a few
  sampled users only, so the weight gradients equal those users' own
  contributions, which the oracle computes;
* unique-id dedup (STCA_FLAG_DEDUP): the history backward once per distinct
  id on the summed dK | dV of its items -- against the oracle on every
  workload above, bitwise repeatable, with out-of-range ids, with rows whose
  items fill one, just over one and several 128-item spans, and at full
  size.
"""
import numpy as np
import pytest

from oracle import stca_grad as OG
from oracle import stca_oracle as O
from recsys_ultra_long_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU visible")]

TOL = 2e-2
WEIGHT_ROW_TOL = 5e-2


def row_err(g, o, floor=0.0, info=False):
    """max over rows of max_k |g - o| / max(max_k |o|, floor * median row max)
    (rows along the last axis; a 1-D array is one row); an all-zero reference
    row is compared absolutely.  ``info``: also return (row, its max, the
    median row max) of the worst row."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if o.size == 0:
        return (0.0, None) if info else 0.0
    g = g.reshape(-1, o.shape[-1])
    o = o.reshape(-1, o.shape[-1])
    rm = np.abs(o).max(axis=1)
    med = float(np.median(rm))
    den = np.maximum(rm, floor * med)
    r = np.abs(g - o).max(axis=1) / np.where(den > 0, den, 1.0)
    w = int(r.argmax())
    return (float(r[w]), (w, float(rm[w]), med)) if info else float(r[w])


def rel_fro(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    den = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / den) if den > 0 else float(np.linalg.norm(g))


def gpu_backward(p, dz, outputs=("table", "d_hist", "d_tgt", "z"), dumps=(), calls=1, zero=True, dedup=False):
    from recsys_ultra_long_amd import stca
    dp = stca.upload(p, dedup=dedup)
    if dedup:
        outputs = tuple(o for o in outputs if o != "d_hist")
    dzt = torch.from_numpy(np.ascontiguousarray(dz, dtype=np.float32)).cuda()
    bw = stca.Backward(dp, dzt, outputs=outputs, dumps=dumps)
    if zero:
        bw.zero()
    for _ in range(calls):
        bw()
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.detach().cpu().numpy()
    tree = lambda g: ({k: tree(v) for k, v in g.items()} if isinstance(g, dict)
                      else [tree(v) for v in g] if isinstance(g, list) else cpu(g))
    out = {"grads": tree(bw.grads), "table": cpu(bw.table), "d_hist": cpu(bw.d_hist),
           "d_tgt": cpu(bw.d_tgt), "z": cpu(bw.z_out), "dq": cpu(bw.dq_dump), "da": cpu(bw.da_dump),
           "dkv": None if bw.dkv_dump is None else stca.to_numpy_stored(bw.dkv_dump),
           "status": int(bw.status[0].item())}
    return out


def leaves(grads, prefix=()):
    if isinstance(grads, dict):
        for k, v in grads.items():
            yield from leaves(v, prefix + (k,))
    elif isinstance(grads, list):
        for i, v in enumerate(grads):
            yield from leaves(v, prefix + (i,))
    elif grads is not None:
        yield prefix, grads


def get(tree, path):
    for k in path:
        tree = tree[k]
    return tree


def touched_rows(p, users=None):
    """Valid table rows read by the history items or targets (of ``users``)."""
    ho, to = p.hist_offsets, p.tgt_offsets
    us = range(p.spec.B) if users is None else users
    ids = np.concatenate([p.hist_ids[ho[u]:ho[u + 1]] for u in us] + [p.tgt_ids[to[u]:to[u + 1]] for u in us])
    ids = ids.astype(np.int64)
    return np.unique(ids[(ids >= 0) & (ids < p.spec.table_rows)])


def compare_all(p, g, ref, tol=TOL, table=True, users=None):
    """Row gradients (items, targets, table rows) row by row within ``tol``;
    weight gradients within ``tol`` relative Frobenius and, row by row with
    the median floor, within WEIGHT_ROW_TOL (see the module docstring)."""
    errs, fro = {}, {}
    pairs = [("/".join(map(str, path)), get(g["grads"], path), o) for path, o in leaves(ref["grads"])]
    n_weights = len(pairs)
    rows_t = None if users is None else np.concatenate(
        [np.arange(p.tgt_offsets[u], p.tgt_offsets[u + 1]) for u in users])
    rows_h = None if users is None else np.concatenate(
        [np.arange(p.hist_offsets[u], p.hist_offsets[u + 1]) for u in users])
    if g["d_hist"] is not None:
        pairs.append(("d_hist", g["d_hist"] if rows_h is None else g["d_hist"][rows_h],
                      ref["d_hist"] if rows_h is None else ref["d_hist"][rows_h]))
    pairs.append(("d_tgt", g["d_tgt"] if rows_t is None else g["d_tgt"][rows_t],
                  ref["d_tgt"] if rows_t is None else ref["d_tgt"][rows_t]))
    if table:
        sp = p.spec
        tg = OG.table_grad(sp.table_rows, sp.d, p.hist_ids, p.tgt_ids, ref["d_hist"], ref["d_tgt"])
        rows = touched_rows(p)
        pairs.append(("table", g["table"][rows], tg[rows]))
    bad = {}
    for i, (name, a, b) in enumerate(pairs):
        fro[name] = rel_fro(a, b)
        if i < n_weights:
            errs[name] = row_err(a, b, floor=1.0)
            if not (errs[name] <= WEIGHT_ROW_TOL and fro[name] <= tol):
                bad[name] = (errs[name], fro[name])
        else:
            errs[name] = row_err(a, b)
            if not errs[name] <= tol:
                bad[name] = errs[name]
    worst = max(errs, key=errs.get)
    print(f"[bwd] {p.spec.name}: worst row error {worst} {errs[worst]:.3e}; "
          + " ".join(f"{k}={v:.1e}/{fro[k]:.1e}" for k, v in sorted(errs.items())), flush=True)
    assert not bad, bad
    return errs


def _small(k, **over):
    base = {
        2: dict(B=4, L=300, table_rows=5000, ln_random=True),                       # d_h 64, m 1
        3: dict(B=3, L=500, m=24, M=3, table_rows=20000, ln_random=True, z_ln=True),  # d_h 32
        4: dict(B=6, L_max=700, m=8, table_rows=20000, ln_random=True),             # d 128 ragged
        6: dict(B=8, L_max=1500, m=16, M=2, table_rows=30000, ln_random=True),      # Beta(1/4,1)
    }[k]
    base.update(over)
    return I.spec(k, **base)


@pytest.mark.parametrize("k", [2, 3, 4, 6])
def test_backward_matches_oracle(k):
    p = I.make_problem(_small(k))
    dz = I.upstream_grad(p.spec, p.n_tgt)
    print(f"[bwd] workload {k}: B={p.spec.B} n_hist={p.n_hist} n_tgt={p.n_tgt}", flush=True)
    g = gpu_backward(p, dz)
    ref = OG.backward_problem(p, dz)
    assert g["status"] == 0
    compare_all(p, g, ref)
    # the recomputed forward's z is the forward's
    zo = O.forward_problem(p)["z"]
    assert row_err(g["z"], zo) < TOL


@pytest.mark.parametrize("over", [dict(kv_ln=False), dict(hidden=128), dict(hidden=256, M=2),
                                  dict(hidden=384, B=2, L=650)])
@pytest.mark.parametrize("dedup", [False, True])
def test_backward_history_shapes(over, dedup):
    """The d = 256 history backward runs as one launch per layer over hidden
    chunks of 128: without the LN after the encoder, one to three chunks, and
    row counts that leave a ragged last tile."""
    sp = _small(3, **over)  # m = 24: enough targets for the query side's weight-gradient rows
    p = I.make_problem(sp)
    dz = I.upstream_grad(sp, p.n_tgt)
    print(f"[bwd] history shapes {over} dedup={dedup}: n_hist={p.n_hist}", flush=True)
    g = gpu_backward(p, dz, outputs=("table", "d_tgt") if dedup else ("table", "d_hist", "d_tgt"), dedup=dedup)
    ref = OG.backward_problem(p, dz)
    assert g["status"] == 0
    compare_all(p, g, ref)


@pytest.mark.parametrize("dedup", [False, True])
def test_backward_with_saved_forward_equals_the_recompute(dedup):
    """stca_forward_for_backward + stca_backward(saved_forward) is the same
    computation as stca_backward's own recompute: z, every weight gradient and
    the target rows bit for bit, a second saved step the same again; the table
    gradient up to the order of its fp32 atomic adds (rows read more than once)."""
    from recsys_ultra_long_amd import stca
    p = I.make_problem(_small(6, B=6, score="relu") if dedup else _small(3, B=3))
    dz = I.upstream_grad(p.spec, p.n_tgt)
    ref = gpu_backward(p, dz, outputs=("table", "d_tgt", "z"), dedup=dedup)
    dp = stca.upload(p, dedup=dedup)
    dzt = torch.from_numpy(np.ascontiguousarray(dz, dtype=np.float32)).cuda()
    bw = stca.Backward(dp, dzt, outputs=("table", "d_tgt"))
    z = torch.empty((p.n_tgt, p.spec.d), dtype=torch.float32, device="cuda")
    for step in range(2):
        bw.zero()
        z.fill_(float("nan"))
        bw.forward_for_backward(z)
        bw(saved_forward=True)
        torch.cuda.synchronize()
        assert int(bw.status[0].item()) == 0
        assert np.array_equal(z.cpu().numpy(), ref["z"]), step
        for path, v in leaves(ref["grads"]):
            assert np.array_equal(get(bw.grads, path).cpu().numpy(), v), (step, path)
        assert np.array_equal(bw.d_tgt.cpu().numpy(), ref["d_tgt"])
        tab = bw.table.cpu().numpy()
        scale = np.abs(ref["table"]).max(axis=1, keepdims=True)
        assert np.all(np.abs(tab - ref["table"]) <= 1e-5 * np.maximum(scale, 1e-30))


@pytest.mark.parametrize("score", ["softmax", "relu"])
def test_attention_backward_stepwise(score):
    """dQ, dK, dV of every layer at the operands the GPU used: its scaled Q,
    its K/V rows (the forward's dumps; the recompute inside the backward is
    the same deterministic forward) and its dA."""
    from recsys_ultra_long_amd import stca
    p = I.make_problem(_small(4, score=score, B=5))
    sp = p.spec
    dz = I.upstream_grad(sp, p.n_tgt, seed=1)
    g = gpu_backward(p, dz, dumps=("dq", "da", "dkv"))
    f = stca.Forward(stca.upload(p), want=(), dumps=("q", "kv"))
    f()
    torch.cuda.synchronize()
    qd = O.stored_to_f64(stca.to_numpy_stored(f.q_dump))
    kvd = O.stored_to_f64(stca.to_numpy_stored(f.kv_dump))
    dkv = O.stored_to_f64(g["dkv"])
    ho, to = p.hist_offsets, p.tgt_offsets
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for i in range(sp.M):
        dq_ref = np.zeros((p.n_tgt, sp.d))
        dk_ref = np.zeros((p.n_hist, sp.d))
        dv_ref = np.zeros((p.n_hist, sp.d))
        for u in range(sp.B):
            a, b, t0, t1 = ho[u], ho[u + 1], to[u], to[u + 1]
            dQ, dK, dV = OG.attention_backward(qd[i, t0:t1], kvd[i, 0, a:b], kvd[i, 1, a:b],
                                               g["da"][i, t0:t1].astype(np.float64), sp.H, score, scale=1.0)
            dq_ref[t0:t1], dk_ref[a:b], dv_ref[a:b] = dQ, dK, dV
        worst["dq"] = max(worst["dq"], row_err(g["dq"][i], dq_ref))
        worst["dk"] = max(worst["dk"], row_err(dkv[i, :, :sp.d], dk_ref))
        worst["dv"] = max(worst["dv"], row_err(dkv[i, :, sp.d:], dv_ref))
    print(f"[bwd] attention stepwise {score}: {worst}", flush=True)
    assert all(v <= TOL for v in worst.values()), worst  # row by row, at the GPU's own operands


def test_backward_zero_upstream_gives_zero():
    p = I.make_problem(_small(3, B=2, L=200, m=8))
    g = gpu_backward(p, np.zeros((p.n_tgt, p.spec.d), np.float32))
    for path, v in leaves(g["grads"]):
        assert np.all(v == 0), path
    assert np.all(g["table"] == 0) and np.all(g["d_hist"] == 0) and np.all(g["d_tgt"] == 0)


def test_backward_accumulates_exactly():
    """Weight gradients are accumulated (+=) and computed in a fixed order:
    two calls give exactly twice one call."""
    p = I.make_problem(_small(3, B=2, L=300, m=8))
    dz = I.upstream_grad(p.spec, p.n_tgt)
    g1 = gpu_backward(p, dz, outputs=(), calls=1)
    g2 = gpu_backward(p, dz, outputs=(), calls=2)
    for path, v in leaves(g1["grads"]):
        assert np.array_equal(get(g2["grads"], path), 2 * v), path


def test_backward_empty_users_and_no_targets():
    sp = _small(4, B=7, L_max=300, m=6)
    p = I.make_problem(sp)
    ho = np.diff(p.hist_offsets).copy()
    to = np.diff(p.tgt_offsets).copy()
    ho[[1, 4]] = 0          # empty histories
    to[[2, 4]] = 0          # users without targets
    p.hist_ids = np.concatenate([p.hist_ids[p.hist_offsets[u]:p.hist_offsets[u] + ho[u]]
                                 for u in range(sp.B)]).astype(np.int32)
    p.tgt_ids = np.concatenate([p.tgt_ids[p.tgt_offsets[u]:p.tgt_offsets[u] + to[u]]
                                for u in range(sp.B)]).astype(np.int32)
    p.hist_offsets = np.concatenate([[0], np.cumsum(ho)]).astype(np.int32)
    p.tgt_offsets = np.concatenate([[0], np.cumsum(to)]).astype(np.int32)
    dz = I.upstream_grad(sp, int(p.tgt_offsets[-1]))
    g = gpu_backward(p, dz)
    ref = OG.backward_problem(p, dz)
    compare_all(p, g, ref)
    # the history of a user without targets receives no gradient
    u = 2
    assert np.all(g["d_hist"][p.hist_offsets[u]:p.hist_offsets[u + 1]] == 0)


def test_backward_fullsize_training_sampled():
    """The training workload at full size (128 users, 281K history items,
    2,048 targets) in the launch configuration the bench times; dz is zero
    except for three users (the first, the longest and the shortest), so
    every weight gradient is those users' contribution alone."""
    sp = I.spec(6)
    p = I.make_problem(sp, threads=16)
    L = np.diff(p.hist_offsets)
    users = sorted({0, int(np.argmax(L)), int(np.argmin(L))})
    dz = np.zeros((p.n_tgt, sp.d), np.float32)
    full = I.upstream_grad(sp, p.n_tgt)
    for u in users:
        dz[p.tgt_offsets[u]:p.tgt_offsets[u + 1]] = full[p.tgt_offsets[u]:p.tgt_offsets[u + 1]]
    print(f"[bwd] full size: n_hist={p.n_hist} users {users} lengths {[int(L[u]) for u in users]}", flush=True)
    g = gpu_backward(p, dz, outputs=("d_hist", "d_tgt"))
    ref = OG.backward_problem(p, dz, users=users)
    assert g["status"] == 0
    compare_all(p, g, ref, table=False, users=users)


@pytest.mark.parametrize("k", [2, 3, 4, 6])
def test_backward_dedup_matches_oracle(k):
    p = I.make_problem(_small(k))
    dz = I.upstream_grad(p.spec, p.n_tgt)
    print(f"[bwd-dedup] workload {k}: n_hist={p.n_hist} unique={len(np.unique(p.hist_ids))}", flush=True)
    g = gpu_backward(p, dz, dedup=True)
    ref = OG.backward_problem(p, dz)
    assert g["status"] == 0
    compare_all(p, g, ref)


@pytest.mark.parametrize("k,over", [(3, dict(L=700)), (4, dict(L_max=1400)),
                                    (3, dict(L=700, d=512, H=8, hidden=1024))], ids=["d256", "d128", "d512"])
def test_backward_dedup_rows_spanning_spans(k, over):
    """Unique rows of exactly one 128-item span's length, one item more, two
    spans and one, and several spans (their partial sums folded in span
    order), scattered over the users, beside rows of one or a few items, at
    d = 256 (the fused row pass), 128 (half of each lane group idle in the
    sums) and 512 (two 512-value blocks per row): against the oracle."""
    p = I.make_problem(_small(k, **over))
    rng = np.random.default_rng(17)
    pos = rng.permutation(p.n_hist)
    hot = [10, 11, 12, 13]
    p.hist_ids[np.isin(p.hist_ids, hot)] = 14  # the hot rows get only the items below
    for ident, (a, b) in zip(hot, ((0, 128), (128, 257), (257, 514), (514, 1114))):
        p.hist_ids[pos[a:b]] = ident
    dz = I.upstream_grad(p.spec, p.n_tgt)
    counts = np.bincount(p.hist_ids[p.hist_ids >= 0], minlength=14)[10:14]
    print(f"[bwd-dedup] rows spanning spans: items per hot row {counts.tolist()}", flush=True)
    assert counts.tolist() == [128, 129, 257, 600]
    g = gpu_backward(p, dz, dedup=True)
    ref = OG.backward_problem(p, dz)
    assert g["status"] == 0
    compare_all(p, g, ref)


def test_backward_dedup_repeatable_and_close_to_plain():
    """Fixed-order sums: two dedup runs are bitwise equal; against the plain
    path the gradients differ only by where bf16 rounding happens."""
    p = I.make_problem(_small(6, B=6))
    dz = I.upstream_grad(p.spec, p.n_tgt)
    g1 = gpu_backward(p, dz, outputs=(), dedup=True)
    g2 = gpu_backward(p, dz, outputs=(), dedup=True)
    g0 = gpu_backward(p, dz, outputs=())
    worst = 0.0
    for path, v in leaves(g1["grads"]):
        assert np.array_equal(get(g2["grads"], path), v), path
        worst = max(worst, rel_fro(v, get(g0["grads"], path)))
    print(f"[bwd-dedup] dedup vs plain: worst {worst:.2e}", flush=True)
    assert worst < 1e-2


def test_backward_dedup_out_of_range_ids():
    p = I.make_problem(_small(3, B=2, L=300, m=8))
    p.hist_ids[[5, 77, 78]] = p.spec.table_rows + 11      # one bad id, three items
    dz = I.upstream_grad(p.spec, p.n_tgt)
    from recsys_ultra_long_amd import stca
    g = gpu_backward(p, dz, dedup=True)
    assert g["status"] & stca.DEV_BAD_ID
    ref = OG.backward_problem(p, dz)
    compare_all(p, g, ref)


def test_backward_dedup_fullsize_training_sampled():
    sp = I.spec(6)
    p = I.make_problem(sp, threads=16)
    L = np.diff(p.hist_offsets)
    users = sorted({0, int(np.argmax(L)), int(np.argmin(L))})
    dz = np.zeros((p.n_tgt, sp.d), np.float32)
    full = I.upstream_grad(sp, p.n_tgt)
    for u in users:
        dz[p.tgt_offsets[u]:p.tgt_offsets[u + 1]] = full[p.tgt_offsets[u]:p.tgt_offsets[u + 1]]
    g = gpu_backward(p, dz, outputs=("d_tgt", "table"), dedup=True)
    ref = OG.backward_problem(p, dz, users=users)
    assert g["status"] == 0
    # the table gradient of the sampled users' rows (other rows get nothing)
    tg = np.zeros((sp.table_rows, sp.d))
    for u in users:
        ids = p.hist_ids[p.hist_offsets[u]:p.hist_offsets[u + 1]]
        np.add.at(tg, ids, ref["d_hist"][p.hist_offsets[u]:p.hist_offsets[u + 1]])
        tids = p.tgt_ids[p.tgt_offsets[u]:p.tgt_offsets[u + 1]]
        np.add.at(tg, tids, ref["d_tgt"][p.tgt_offsets[u]:p.tgt_offsets[u + 1]])
    rows = touched_rows(p, users)
    err_t = row_err(g["table"][rows], tg[rows])
    print(f"[bwd-dedup] full size table rows err {err_t:.2e}", flush=True)
    assert err_t <= TOL
    compare_all(p, g, ref, table=False, users=users)
