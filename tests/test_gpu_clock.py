"""The clock counters the library exposes as a measurement aid: the MFMA-only
peak kernel and the optional clock probe of the d = 256 history launch each
report {s_memtime, s_memrealtime} pairs, from which the shader clock during
the launch follows.  Checks: counters advance, the clock lies in the range the
chip can run at, the probe leaves the forward's outputs unchanged (bitwise),
and rows of workgroups that do not exist stay untouched."""
import numpy as np
import pytest

from recsys_ultra_long_amd import inputs as I
from recsys_ultra_long_amd import stca

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU visible")]


def test_peak_kernel_clock():
    rate, ghz = stca.peak_mfma_bf16(blocks=512, iters=2000, repeats=1)
    assert 100.0 < rate < 3000.0
    assert 0.3 < ghz < 3.0


def test_hbm_read_stream():
    # 256 MB: the rate is only sanity-checked here (the bench streams 2 GiB)
    rate = stca.peak_hbm_read(nbytes=256 << 20, blocks=512, repeats=2)
    assert 500.0 < rate < 20000.0


@pytest.mark.parametrize("k", [3, 4])
def test_history_launch_clock_probe(k):
    # d = 256 and d = 128: 3 users of 300 items: 1,024 padded rows = 8
    # workgroups of 128 rows; a sentinel row past them must stay untouched
    sp = I.spec(k, B=3, L=300, L_max=None, m=8, table_rows=20000)
    p = I.make_problem(sp)
    dp = stca.upload(p, path="staged")
    f = stca.Forward(dp, want=(), dumps=())
    f()
    torch.cuda.synchronize()
    z0 = f.z.clone()
    clk = torch.full((9, 4), -1, dtype=torch.int64, device="cuda")
    f.out.clock_probe = clk.data_ptr()
    f()
    torch.cuda.synchronize()
    c = clk.cpu().numpy()
    assert (c[-1] == -1).all()                      # no workgroup 8
    rows = c[:-1][(c[:-1] != -1).all(axis=1)]
    assert len(rows) >= 1
    assert (rows[:, 2] > rows[:, 0]).all() and (rows[:, 3] >= rows[:, 1]).all()
    ghz = stca.clock_ghz(rows)
    assert ghz != ghz or 0.3 < ghz < 3.0            # nan if the launch took < 10 ns
    assert torch.equal(f.z, z0)
