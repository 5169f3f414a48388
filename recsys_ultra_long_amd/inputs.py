"""Seeded synthetic workloads for the STCA forward.

This module only draws numbers: ids, lengths, tables, weights and queries.
It contains none of the method's arithmetic, so both the float64 oracle
(``oracle/``) and the HIP path (``recsys_ultra_long_amd.stca``) can consume its
output without sharing any computation.

Workload shapes follow the pages (cited by page title):

* "Make It Long, Keep It Fast" review, section 六 (model configuration):
  4 layers, d = 256, 8 heads; inference length 10K.
* STCA reading notes, "短序列训练，长序列推理" and the review's length
  sampling formula: lengths drawn from a Beta(alpha, 1) law.
* HyFormer translation, section 3.8.1: only about a quarter of the ids in a
  long sequence are unique, which a bounded Zipf(1.1) id law reproduces.

Distributions (readings of the workload descriptions, restated in the design doc):

* table rows i.i.d. N(0, 0.02^2); every weight matrix i.i.d. N(0, 1/d);
  LayerNorm gain 1 and bias 0 unless ``ln_random`` is set (tests use random
  gain/bias so that a dropped affine term is caught);
* ids: uniform on [0, N) or bounded Zipf, P(k) proportional to (k+1)^-s;
* ragged lengths: L_u = max(16, ceil(L_max * beta)), beta ~ Beta(alpha, 1),
  sampled as U^(1/alpha) (alpha = 2 for the ragged inference workload;
  alpha = 1/4 for the training workload, whose mean length L_max / 5 = 2K is
  the training length the reading notes give for 10K inference);
* the upstream gradient of z for the backward: i.i.d. N(0, 1);
* context-similarity score bias (Cross-Mask page): i.i.d. N(0, 0.5^2) per
  history item and head;
* HyFormer query mode: n_ns non-sequence feature tokens per user i.i.d.
  N(0, 0.02^2) like table rows; the query-generation FFNs (input
  (n_ns + 1) d) and the per-token boosting FFNs i.i.d. N(0, 1/fan_in), drawn
  from a stream of their own so the other arrays are unchanged;
* bf16 storage is produced by round-to-nearest-even from float32.

Storage convention: a bf16 array is a ``numpy.uint16`` array of raw bf16
bits; an fp32 array is ``numpy.float32``.  ``to_f64`` upcasts either one
exactly.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

TABLE_STD = 0.02
_BLOCK_ROWS = 1 << 16          # table rows per independently seeded block


# --------------------------------------------------------------------------
# storage helpers (data plumbing, not method arithmetic)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Exact upcast of stored values (bf16 bits or float32) to float64."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


# --------------------------------------------------------------------------
# configuration
# --------------------------------------------------------------------------
@dataclass
class Spec:
    """Shape and mode of one STCA problem (one sequence)."""
    name: str
    B: int
    d: int
    H: int
    hidden: int
    M: int
    table_rows: int
    dtype: str = "bf16"                 # "bf16" | "f32"
    score: str = "softmax"              # "softmax" | "relu"
    qmode: str = "fusion"               # "fusion" (STCA W_C chain) | "linear" (Q' = O R)
                                        # | "hyformer" (generated queries + boosting)
    kv_ln: bool = True                  # LN after the history FFN
    z_ln: bool = False                  # LN on the final z
    L: Optional[int] = None             # fixed history length
    L_max: Optional[int] = None         # ragged: max(L_min, ceil(L_max * Beta(beta_a, 1)))
    L_min: int = 16
    beta_a: float = 2.0
    n_ns: int = 0                       # hyformer: non-sequence feature tokens per user
    hy_hidden: Optional[int] = None     # hyformer: hidden width of the query FFNs (default d)
    encoder: str = "swiglu"             # history encoding: "swiglu" (FFN [+LN]) | "longer"
    l_short: int = 0                    # longer: length L_H of the short query sequence
    m: int = 1                          # targets (or queries) per user
    ids: str = "zipf"                   # "zipf" | "uniform"
    zipf_s: float = 1.1
    ln_random: bool = False
    seed: int = 0

    @property
    def d_h(self) -> int:
        return self.d // self.H


# The five workloads (full size).  configs 1-4 are one sequence each;
# workload 5 is two independent sequences (feed and search).
def spec(k: int, **over) -> Spec | dict:
    if k == 1:
        s = Spec("tiny-f32", B=4, d=64, H=2, hidden=128, M=1, table_rows=10_000,
                 dtype="f32", L=256, m=1, ids="uniform", seed=1)
    elif k == 2:
        s = Spec("single-target-bf16", B=64, d=256, H=4, hidden=512, M=2,
                 table_rows=1_000_000, L=2048, m=1, seed=2)
    elif k == 3:
        s = Spec("rlb-long-bf16", B=32, d=256, H=8, hidden=512, M=4,
                 table_rows=4_000_000, L=10_240, m=64, seed=3)
    elif k == 4:
        s = Spec("ragged-bf16", B=256, d=128, H=4, hidden=256, M=3,
                 table_rows=4_000_000, L_max=10_240, m=16, seed=4)
    elif k == 5:
        feed = Spec("hyformer-feed", B=64, d=512, H=8, hidden=1024, M=3,
                    table_rows=2_000_000, L=8192, m=8, qmode="linear", kv_ln=False,
                    seed=51)
        search = replace(feed, name="hyformer-search", L=1024, seed=52)
        return {"feed": replace(feed, **over), "search": replace(search, **over)}
    elif k == 6:
        # training: the RLB long model on Beta(1/4, 1) lengths (mean 2K of 10K)
        s = Spec("rlb-train-bf16", B=128, d=256, H=8, hidden=512, M=4,
                 table_rows=4_000_000, L_max=10_240, beta_a=0.25, m=16, seed=6)
    else:
        raise ValueError(f"unknown workload {k}")
    return replace(s, **over)


def cross_mask(sp: Spec, n_hist: int, masked_heads, keep: float = 0.5, seed: int = 0) -> np.ndarray:
    """Seeded Cross-Mask vertical masks [n_hist] (uint32): every head sees
    every item except the heads in ``masked_heads``, which see an item with
    probability ``keep`` (a stand-in for a per-item feature condition such as
    "action = complete")."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([sp.seed, 0x4D41, seed])))
    m = np.full(n_hist, (1 << sp.H) - 1, dtype=np.uint64)
    for h in masked_heads:
        off = g.random(n_hist) >= keep
        m[off] &= ~np.uint64(1 << h)
    return m.astype(np.uint32)


def score_bias(sp: Spec, n_hist: int, std: float = 0.5, seed: int = 0) -> np.ndarray:
    """Seeded context-similarity score bias [n_hist, H] (float32), i.i.d.
    N(0, std^2): a stand-in for the per-item, per-head similarity between an
    item's context and the request's, which the pages name but do not define."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([sp.seed, 0x4249, seed])))
    return (g.standard_normal((n_hist, sp.H), dtype=np.float32) * np.float32(std)).astype(np.float32)


def upstream_grad(sp: Spec, n_tgt: int, seed: int = 0) -> np.ndarray:
    """Seeded upstream gradient dL/dz [n_tgt, d] (float32) for the backward."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([sp.seed, 7919, seed])))
    return g.standard_normal((n_tgt, sp.d), dtype=np.float32)


# --------------------------------------------------------------------------
# samplers
# --------------------------------------------------------------------------
_ZIPF_CDF_CACHE: dict = {}


def _zipf_cdf(n: int, s: float) -> np.ndarray:
    key = (n, s)
    c = _ZIPF_CDF_CACHE.get(key)
    if c is None:
        w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(w)
        c /= c[-1]
        if len(_ZIPF_CDF_CACHE) > 4:
            _ZIPF_CDF_CACHE.clear()
        _ZIPF_CDF_CACHE[key] = c
    return c


def sample_ids(rng: np.random.Generator, n: int, rows: int, law: str, s: float) -> np.ndarray:
    if law == "uniform":
        return rng.integers(0, rows, size=n, dtype=np.int64).astype(np.int32)
    cdf = _zipf_cdf(rows, s)
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, rows - 1).astype(np.int32)


def sample_lengths(rng: np.random.Generator, sp: Spec) -> np.ndarray:
    if sp.L is not None:
        return np.full(sp.B, sp.L, dtype=np.int64)
    u = rng.random(sp.B)
    beta = np.sqrt(u) if sp.beta_a == 2.0 else u ** (1.0 / sp.beta_a)   # Beta(a, 1)
    return np.maximum(sp.L_min, np.ceil(sp.L_max * beta)).astype(np.int64)


def _table_block(seed: int, blk: int, nrows: int, d: int, dtype: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7, blk])))
    x = g.standard_normal((nrows, d), dtype=np.float32) * np.float32(TABLE_STD)
    return _store(x, dtype)


def make_table(sp: Spec, threads: int = 8) -> np.ndarray:
    """Full embedding table; row blocks are seeded independently so any row
    can be regenerated alone (``table_rows``)."""
    n, d = sp.table_rows, sp.d
    out = np.empty((n, d), dtype=np.uint16 if sp.dtype == "bf16" else np.float32)
    nblk = (n + _BLOCK_ROWS - 1) // _BLOCK_ROWS

    def work(b):
        r0 = b * _BLOCK_ROWS
        r1 = min(n, r0 + _BLOCK_ROWS)
        out[r0:r1] = _table_block(sp.seed, b, r1 - r0, d, sp.dtype)

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            list(ex.map(work, range(nblk)))
    return out


def table_rows(sp: Spec, rows: np.ndarray) -> np.ndarray:
    """Rows ``rows`` of ``make_table(sp)``, regenerated without the full table."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), sp.d), dtype=np.uint16 if sp.dtype == "bf16" else np.float32)
    for b in np.unique(rows // _BLOCK_ROWS):
        r0 = int(b) * _BLOCK_ROWS
        r1 = min(sp.table_rows, r0 + _BLOCK_ROWS)
        blk = _table_block(sp.seed, int(b), r1 - r0, sp.d, sp.dtype)
        sel = (rows // _BLOCK_ROWS) == b
        out[sel] = blk[rows[sel] - r0]
    return out


# --------------------------------------------------------------------------
# problem
# --------------------------------------------------------------------------
@dataclass
class Problem:
    spec: Spec
    hist_offsets: np.ndarray          # int32 [B+1]
    hist_ids: np.ndarray              # int32 [n_hist]
    tgt_offsets: np.ndarray           # int32 [B+1]
    tgt_ids: Optional[np.ndarray]     # int32 [n_tgt]   (fusion mode)
    q0: Optional[np.ndarray]          # [n_tgt, d]       (linear mode)
    table: Optional[np.ndarray]       # [N, d]; None when generated lazily
    layers: list                      # per layer dict, see _make_weights
    z: Optional[dict] = None          # final SwiGLU (fusion mode)
    wz: Optional[np.ndarray] = None   # [(M+1) d, d]
    extra: dict = field(default_factory=dict)

    @property
    def n_hist(self) -> int:
        return int(self.hist_offsets[-1])

    @property
    def n_tgt(self) -> int:
        return int(self.tgt_offsets[-1])

    def rows(self, ids: np.ndarray) -> np.ndarray:
        """Table rows for ``ids`` (stored dtype)."""
        if self.table is not None:
            return self.table[np.asarray(ids, dtype=np.int64)]
        return table_rows(self.spec, ids)


def _ffn(g: np.random.Generator, sp: Spec, ln: bool) -> dict:
    d, h = sp.d, sp.hidden
    std = np.float32(1.0 / math.sqrt(d))
    w = {
        "w1": _store(g.standard_normal((d, h), dtype=np.float32) * std, sp.dtype),
        "w3": _store(g.standard_normal((d, h), dtype=np.float32) * std, sp.dtype),
        "w2": _store(g.standard_normal((h, d), dtype=np.float32) * std, sp.dtype),
    }
    if ln:
        if sp.ln_random:
            w["ln_g"] = (1.0 + 0.2 * g.standard_normal(d)).astype(np.float32)
            w["ln_b"] = (0.1 * g.standard_normal(d)).astype(np.float32)
        else:
            w["ln_g"] = np.ones(d, np.float32)
            w["ln_b"] = np.zeros(d, np.float32)
    return w


def _mat(g: np.random.Generator, sp: Spec, rows: int, cols: int) -> np.ndarray:
    std = np.float32(1.0 / math.sqrt(sp.d))
    return _store(g.standard_normal((rows, cols), dtype=np.float32) * std, sp.dtype)


def _make_weights(g: np.random.Generator, sp: Spec):
    d = sp.d
    layers = []
    for i in range(sp.M):
        lw = {"kv": _ffn(g, sp, ln=sp.kv_ln),
              "wk": _mat(g, sp, d, d), "wv": _mat(g, sp, d, d),
              "wq": _mat(g, sp, d, d), "wo": _mat(g, sp, d, d)}
        if sp.qmode == "fusion":
            lw["q"] = _ffn(g, sp, ln=True)
            lw["wc"] = None if i == 0 else _mat(g, sp, (i + 1) * d, d)
        else:
            lw["r"] = _mat(g, sp, d, d)
        layers.append(lw)
    if sp.qmode == "fusion":
        z = _ffn(g, sp, ln=True)
        wz = _mat(g, sp, (sp.M + 1) * d, d)
    else:
        z, wz = None, None
    return layers, z, wz


def make_problem(sp: Spec, *, with_table: bool = True, threads: int = 8) -> Problem:
    """Draw one seeded problem.  Independent streams (lengths, history ids,
    target ids, weights, queries) are spawned from SeedSequence(seed)."""
    ss = np.random.SeedSequence(sp.seed)
    s_len, s_hist, s_tgt, s_w, s_q = ss.spawn(5)
    lens = sample_lengths(np.random.Generator(np.random.PCG64(s_len)), sp)
    hist_offsets = np.zeros(sp.B + 1, dtype=np.int64)
    hist_offsets[1:] = np.cumsum(lens)
    g_hist = np.random.Generator(np.random.PCG64(s_hist))
    hist_ids = sample_ids(g_hist, int(hist_offsets[-1]), sp.table_rows, sp.ids, sp.zipf_s)
    tgt_offsets = (np.arange(sp.B + 1, dtype=np.int64) * sp.m)
    n_tgt = int(tgt_offsets[-1])
    tgt_ids, q0 = None, None
    extra = {}
    if sp.qmode == "fusion":
        tgt_ids = sample_ids(np.random.Generator(np.random.PCG64(s_tgt)), n_tgt,
                             sp.table_rows, sp.ids, sp.zipf_s)
    elif sp.qmode == "hyformer":
        extra = _make_hyformer(sp)
    else:
        gq = np.random.Generator(np.random.PCG64(s_q))
        q0 = _store(gq.standard_normal((n_tgt, sp.d), dtype=np.float32), sp.dtype)
    layers, z, wz = _make_weights(np.random.Generator(np.random.PCG64(s_w)), sp)
    if sp.qmode == "hyformer":
        for i, l in enumerate(layers):
            l["boost"] = extra["boost"][i]
    if sp.encoder == "longer":  # the encoder's own projections, from a stream of their own
        ge = np.random.Generator(np.random.PCG64(np.random.SeedSequence([sp.seed, 0x4C4E])))
        for l in layers:
            l["enc"] = {k: _mat(ge, sp, sp.d, sp.d) for k in ("wq", "wk", "wv", "wo")}
    table = make_table(sp, threads) if with_table else None
    return Problem(sp, hist_offsets.astype(np.int32), hist_ids, tgt_offsets.astype(np.int32),
                   tgt_ids, q0, table, layers, z, wz,
                   {k: v for k, v in extra.items() if k != "boost"})


def _make_hyformer(sp: Spec) -> dict:
    """Non-sequence tokens [B, n_ns, d], the m query-generation FFNs
    (w1, w3 [m, (n_ns+1) d, hh], w2 [m, hh, d]) and, per layer, the m + n_ns
    per-token boosting FFNs (w1, w3 [T, d, hh], w2 [T, hh, d])."""
    d, hh, N, F = sp.d, sp.hy_hidden or sp.d, sp.m, sp.n_ns
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([sp.seed, 0x4859])))
    ns = _store(g.standard_normal((sp.B, F, d), dtype=np.float32) * np.float32(TABLE_STD), sp.dtype)

    def ffn(n, din):
        return {"w1": _store(g.standard_normal((n, din, hh), dtype=np.float32) / np.float32(math.sqrt(din)), sp.dtype),
                "w3": _store(g.standard_normal((n, din, hh), dtype=np.float32) / np.float32(math.sqrt(din)), sp.dtype),
                "w2": _store(g.standard_normal((n, hh, d), dtype=np.float32) / np.float32(math.sqrt(hh)), sp.dtype)}
    qgen = ffn(N, (F + 1) * d)
    boost = [ffn(N + F, d) for _ in range(sp.M)]
    return {"ns": ns, "qgen": qgen, "boost": boost}


def subset_users(p: Problem, users) -> Problem:
    """The same problem restricted to ``users`` (CSR rebuilt, weights shared)."""
    users = [int(u) for u in users]
    ho, to = p.hist_offsets.astype(np.int64), p.tgt_offsets.astype(np.int64)
    hid, tid, q0 = [], [], []
    hoff, toff = [0], [0]
    for u in users:
        hid.append(p.hist_ids[ho[u]:ho[u + 1]])
        hoff.append(hoff[-1] + int(ho[u + 1] - ho[u]))
        if p.tgt_ids is not None:
            tid.append(p.tgt_ids[to[u]:to[u + 1]])
        if p.q0 is not None:
            q0.append(p.q0[to[u]:to[u + 1]])
        toff.append(toff[-1] + int(to[u + 1] - to[u]))
    sp = replace(p.spec, B=len(users))
    cat = (lambda xs, dt: np.concatenate(xs).astype(dt) if xs else np.zeros(0, dt))
    return Problem(sp, np.asarray(hoff, np.int32), cat(hid, np.int32),
                   np.asarray(toff, np.int32),
                   cat(tid, np.int32) if p.tgt_ids is not None else None,
                   (np.concatenate(q0) if q0 else None) if p.q0 is not None else None,
                   p.table, p.layers, p.z, p.wz,
                   {**p.extra, **({"ns": p.extra["ns"][users]} if "ns" in p.extra else {}),
                    **({"key_mask": np.concatenate([p.extra["key_mask"][ho[u]:ho[u + 1]] for u in users])
                        .astype(np.uint32)} if "key_mask" in p.extra else {}),
                    **({"score_bias": np.concatenate([p.extra["score_bias"][ho[u]:ho[u + 1]] for u in users])
                        .astype(np.float32)} if "score_bias" in p.extra else {})})
