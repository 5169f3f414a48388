"""GPU parity of the backward pass over a seeded random sweep of small shapes.

Each case draws, from its own seed: d 128 / 256 / 512 with d_h 32 or 64, the
hidden width (d or 2d), 1-3 layers, 1-5 users of fixed or Beta-ragged length,
1-64 targets per user, LN after the history FFN on or off, a random LN affine,
LN on z, a small Zipf table (repeated ids) and unique-id dedup on or off.
Every gradient is compared with the float64 backward oracle with the bars of
the fixed-shape backward tests (rows of items, targets and touched table rows
within 2e-2; weight gradients within 2e-2 relative Frobenius and, row by row
with the median floor, within 5e-2).
"""
import numpy as np
import pytest

from oracle import stca_grad as OG
from recsys_ultra_long_amd import inputs as I
from test_gpu_backward import compare_all, gpu_backward

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU visible")]

N_CASES = 12


def _case(i):
    r = np.random.default_rng(2000 + i)
    d, H = [(128, 4), (256, 8), (256, 4), (512, 8), (512, 16)][r.integers(5)]
    ragged = bool(r.integers(2))
    sp = I.spec(3, name=f"random-bwd-{i}", B=int(r.integers(1, 6)), d=d, H=H, hidden=int(d * r.choice([1, 2])),
                M=int(r.integers(1, 4)), table_rows=int(r.choice([3000, 20000])), m=int(r.choice([1, 3, 16, 40, 64])),
                L=None if ragged else int(r.integers(16, 500)), L_max=int(r.integers(40, 500)) if ragged else None,
                kv_ln=bool(r.integers(4) > 0), z_ln=bool(r.integers(2)), ln_random=True, seed=7000 + i)
    return sp, bool(r.integers(2))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_backward_matches_oracle(i):
    sp, dedup = _case(i)
    p = I.make_problem(sp)
    print(f"[random-bwd {i}] d={sp.d} H={sp.H} hidden={sp.hidden} M={sp.M} B={sp.B} m={sp.m} "
          f"n_hist={p.n_hist} kv_ln={sp.kv_ln} z_ln={sp.z_ln} dedup={dedup}", flush=True)
    dz = I.upstream_grad(sp, p.n_tgt)
    g = gpu_backward(p, dz, dedup=dedup)
    ref = OG.backward_problem(p, dz)
    assert g["status"] == 0
    compare_all(p, g, ref)
