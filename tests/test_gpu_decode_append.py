"""Decode-time tail append after the phase-1 reorder (TriAxialKV, key design 4: the
tokens a decode step produces are written as INT4 at the tail of the table).

Each case builds a small cache through the library and through the oracle, reorders
it, then runs decode steps that append 1, 17 and 40 new tokens per table with
kvq_quantize_append (the first step continues a reordered, partly filled INT4 page
where a table ends on one), re-plans, and decodes with the step's query.  After every
step: pools and tables bit-exact, attention rows within 2e-3 of the oracle."""
import numpy as np
import pytest
import torch

import synth
from harness import DeviceRun, OracleRun, row_metric
from test_gpu_parity import TOL, _pools_equal, _say

pytestmark = pytest.mark.gpu
STEPS = (1, 17, 40)

CASES = {
    "qwen3_8b 2x2048": lambda: synth.qwen3_8b(batch=2, n_tokens=2048),
    "agentic 2x9000-12000": lambda: synth.qwen3_vl_agentic(batch=2, lo=9000, hi=12000, chunk=4096),
    "hybrid 2x4096": lambda: synth.hybrid_anchor(batch=2, n_tokens=4096),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_tail_append_steps(name):
    make = lambda: synth.reserve_tail(CASES[name](), sum(STEPS))  # noqa: E731
    wg, wo = make(), make()
    gpu, orc = DeviceRun(wg), OracleRun(wo)
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0
    _pools_equal(gpu, orc)
    assert np.array_equal(gpu.tables.cpu().numpy(), orc.tables)
    ends_partial = 0
    for t in range(wg.n_tables):
        n = int(wg.alloc.n_entries[t])
        last = int(orc.tables[t, n - 1])
        e = int(np.flatnonzero(wo.alloc.tables[t, :n] == last)[0])
        ends_partial += int(wo.alloc.entry_cls[t][e] == synth.INT4 and wo.alloc.fill[t][e] < synth.PAGE)
    _say(f"{name}: {ends_partial} of {wg.n_tables} tables end on a partly filled INT4 page")
    for i, n_new in enumerate(STEPS):
        k, v, q = synth.tail_rows(wg, i, n_new)
        a_g = gpu.append_tail(k, v, q)
        a_o = orc.append_tail(k, v, q)
        assert all(np.array_equal(a_g[x], a_o[x]) for x in ("rows4", "slots4"))
        torch.cuda.synchronize()
        assert int(gpu.err.item()) == 0, f"device error bits {int(gpu.err.item())}"
        _pools_equal(gpu, orc)
        assert np.array_equal(gpu.tables.cpu().numpy(), orc.tables)
        assert np.array_equal(gpu.ranges, orc.ranges)
        ref, ref_lse = orc.attend()
        splits, offsets = gpu.plan(target_bytes=1 << 17)
        out, lse, _, _ = gpu.decode(splits, offsets)
        assert int(gpu.err.item()) == 0
        err = row_metric(ref, out.cpu().numpy())
        _say(f"  step {i}: +{n_new} tokens per table, {splits.shape[0]} splits, row error {err:.2e}")
        assert err <= TOL, f"{name} step {i}: row error {err:.3e} > {TOL}"
        assert np.allclose(lse.cpu().numpy(), ref_lse, atol=1e-3, rtol=1e-4)
