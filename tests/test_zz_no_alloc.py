"""stca_forward_noalloc: the forward with its workspace in the library's
static device scratch (for callers that cannot allocate).  Every output
must equal stca_forward's with a caller workspace bit for bit (the same
kernels and the same workspace layout at another address), on two calls in a
row whose second input is smaller, so that contents the first call left in
the shared scratch cannot leak into the second; with the unique-id dedup
(its hash set lives in the workspace) and with ReLU scores (active counts)."""
import numpy as np
import pytest

from recsys_ultra_long_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU visible")]


def _run(p, noalloc, dedup=False):
    from recsys_ultra_long_amd import stca
    dp = stca.upload(p, dedup=dedup)
    f = stca.Forward(dp, want=("o", "attn", "active"), dumps=("q",), noalloc=noalloc)
    assert (f.ws is None) == noalloc
    f()
    torch.cuda.synchronize()
    return {k: stca.to_numpy_stored(v) for k, v in f.results().items()}


def _same(p, dedup=False):
    print(f"[noalloc] {p.spec.name} B={p.spec.B} n_hist={p.n_hist} n_tgt={p.n_tgt} dedup={dedup}", flush=True)
    a = _run(p, noalloc=False, dedup=dedup)
    b = _run(p, noalloc=True, dedup=dedup)
    assert set(a) == set(b)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert int(b["status"][0]) == 0


@pytest.mark.parametrize("dedup", [False, True])
def test_noalloc_equals_forward_two_calls_second_smaller(dedup):
    from recsys_ultra_long_amd import stca
    big = I.make_problem(I.spec(3, B=3, L=2000, m=64, table_rows=20000))
    small = I.make_problem(I.spec(4, B=5, L_max=400, m=7, table_rows=20000, score="relu"))
    assert stca.workspace_bytes(stca.upload(small)) < stca.workspace_bytes(stca.upload(big))
    _same(big, dedup)
    _same(small, dedup)


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    from recsys_ultra_long_amd import stca
    p = I.make_problem(I.spec(3, B=8, L=10240, m=64, table_rows=20000))
    dp = stca.upload(p)
    assert stca.workspace_bytes(dp) > stca.NOALLOC_SCRATCH_BYTES
    f = stca.Forward(dp, noalloc=True)
    with pytest.raises(stca.StcaError) as e:
        f()
    assert e.value.code == stca.ERR_WORKSPACE and "static scratch" in str(e.value)
