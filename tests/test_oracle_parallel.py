"""oracle.parallel runs the oracle per (batch, head) slice on spawned worker
processes and reassembles the CSR row order; on batch-2, 3-head grids its
results must equal the oracle called on the whole tensors.  CPU only."""
import numpy as np
import pytest

import lcsa_inputs as li
import oracle
from oracle.parallel import OraclePool


@pytest.mark.parametrize("name", ["tiny_window", "small_edges"])
def test_pool_equals_whole_tensor_oracle(name):
    desc = dict(li.CONFIGS[name], batch=2, heads=3)
    inp = li.generate(desc, seed=11)
    g = oracle.geometry(desc)
    q, k, v = (li.bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
    rp, ci, s = oracle.select(g, q, k)
    o_ref, lse_ref = oracle.attend(g, q, k, v, rp, ci)
    with OraclePool(desc, inp.q, inp.k, inp.v, workers=3) as pool:
        rp2, ci2, s2, _ = pool.select()
        o2, lse2, _ = pool.attend(rp, ci)
        rows = [5, 0, len(rp) - 2, 17, 5]
        part = pool.attend_rows(rp, ci, rows)
    assert np.array_equal(rp2, rp) and np.array_equal(ci2, ci)
    fin = np.isfinite(s)
    assert np.array_equal(np.isfinite(s2), fin)
    assert np.abs(s2[fin] - s[fin]).max() <= 1e-15 * np.abs(s[fin]).max()
    assert np.array_equal(o2, o_ref) and np.array_equal(lse2, lse_ref)
    whole = oracle.attend_rows(g, q, k, v, rp, ci, rows)
    for (b, h, qt, orow, lrow), (b2, h2, qt2, orow2, lrow2) in zip(whole, part):
        assert (b, h) == (b2, h2) and np.array_equal(qt, qt2)
        assert np.array_equal(orow, orow2) and np.array_equal(lrow, lrow2)
