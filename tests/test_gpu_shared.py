"""GPU parity of the shared-window decode (kvq_decode_attn_shared): the workers of a
(table, head, class) range take its 32-token windows from a counter, each writing the
softmax partial of the windows it took, merged by kvq_lse_merge as split partials.
Outputs within 2e-3 of the oracle by the per-row metric on every call; the counters
back at zero after every call.  Repeated calls are not bit-identical: the windows a
worker takes vary from call to call, and with them the running maximum its fp16
weights are rounded against."""
import numpy as np
import pytest
import torch

import synth
from harness import DeviceRun, OracleRun, row_metric

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _say(*a):
    print("[gpu-shared]", *a, flush=True)


def _shared_case(name, make, workers_per_head, calls=2, out_dtype=torch.float32):
    _say(name, f"workers per head {workers_per_head}")
    gpu, orc = DeviceRun(make()), OracleRun(make())
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0
    ref, ref_lse = orc.attend()
    workers, groups, n_groups, offsets = gpu.plan_workers(workers_per_head)
    work, first = None, None
    for c in range(calls):
        out, lse, _, _, work = gpu.decode_shared(workers, groups, n_groups, offsets, out_dtype=out_dtype, work=work)
        assert int(gpu.err.item()) == 0, f"device error bits {int(gpu.err.item())}"
        assert not work.any().item(), "work counters not reset"
        got = out.float().cpu().numpy()
        err = row_metric(ref, got)
        _say(f"  {name} call {c}: {workers.shape[0]} workers in {n_groups} groups, row error {err:.2e}")
        assert err <= (TOL if out_dtype == torch.float32 else TOL + 2.0 ** -8)  # bf16: + half an ulp
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse.cpu().numpy()))
        assert np.allclose(lse.cpu().numpy()[fin], ref_lse[fin], atol=1e-3, rtol=1e-4)
        if first is None:
            first = got
        else:
            _say(f"  {name} call {c}: differs from call 0 by {row_metric(first, got):.1e}")
    return gpu, orc


def test_shared_tiny():
    _shared_case("tiny", synth.tiny, 3)


@pytest.mark.parametrize("wph", [1, 2, 7, 40])
def test_shared_qwen3_8b_small(wph):
    """One worker per range (no sharing), a few, more workers than windows of the INT4
    range (capped), and many."""
    _shared_case("qwen3_8b 2x2048", lambda: synth.qwen3_8b(batch=2, n_tokens=2048), wph, calls=3)


def test_shared_ragged_lengths_g8():
    """g = 8 over tagged contexts appended in chunks: INT4 ranges broken by each call's
    partially filled page, so a (table, head) has several INT4 groups."""
    make = lambda: synth.qwen3_vl_agentic(batch=2, lo=9000, hi=12000, chunk=4096)  # noqa: E731
    _shared_case("qwen3_vl_agentic 2 x ~10K", make, 9)


def test_shared_hybrid_anchor_small():
    """INT4 prefix shared, the FP16 anchor ranges one worker each (their kernel reads a
    range whole)."""
    _shared_case("hybrid 2x4096", lambda: synth.hybrid_anchor(batch=2, n_tokens=4096), 6)


def test_shared_bf16_output():
    _shared_case("qwen3_8b bf16 out", lambda: synth.qwen3_8b(batch=1, n_tokens=1024), 5, out_dtype=torch.bfloat16)


def test_shared_full_size_qwen3_8b_sampled():
    """The benchmark's workload (16 x 32768 tokens, g = 4) with its shared plan (the
    resident workers shared per (request, head) by cost), two requests against the
    oracle, twice."""
    _say("full-size qwen3_8b shared: generating on the GPU")
    w = synth.qwen3_8b(device="cuda")
    gpu = DeviceRun(w)
    per_cu, n_cu = gpu.kvq.decode_occupancy(w.g, gpu.kvq.TABLE_PAGES)
    workers, groups, n_groups, offsets = gpu.plan_workers(per_cu * n_cu // (w.batch * w.hkv))
    outs = []
    work = None
    for _ in range(2):
        out, _, _, _, work = gpu.decode_shared(workers, groups, n_groups, offsets, work=work)
        assert int(gpu.err.item()) == 0 and not work.any().item()
        outs.append(out.cpu().numpy())
    del gpu
    orc = OracleRun(synth.subset(synth.qwen3_8b(device="cuda"), [3, 11]))
    ref, _ = orc.attend()
    for got in outs:
        err = row_metric(ref, got[[3, 11]])
        _say(f"  {workers.shape[0]} workers; sampled row error {err:.2e}")
        assert err <= TOL
    _say(f"  the two calls differ by {row_metric(outs[0], outs[1]):.1e}")


def test_shared_rejects_slot_maps_and_g16():
    from mixed_precision_quantized_amd import kvq
    cache = kvq.Cache(1, (0, 16, 0), "cuda")
    z = torch.zeros((4, 5), dtype=torch.int32, device="cuda")
    g = torch.zeros(4, dtype=torch.int32, device="cuda")
    work = kvq.decode_work(1)
    po, pl = torch.empty((4, 16, 128), device="cuda"), torch.empty((4, 16), device="cuda")
    tables = torch.zeros((1, 16), dtype=torch.int32, device="cuda")
    q4 = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_shared(cache, q4, 1, tables, kvq.TABLE_SLOTS, z, g, 1, work, po, pl)
    assert e.value.status == -2
    q16 = torch.zeros((1, 16, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_shared(cache, q16, 1, tables, kvq.TABLE_PAGES, z, g, 1, work, po, pl)
    assert e.value.status == -2
