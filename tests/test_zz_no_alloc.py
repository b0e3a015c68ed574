"""The no-allocation shared-window decode (kvq_decode_attn_shared_noalloc, counters in
the library's own device array) through the C ABI against the entry point it varies
(kvq_decode_attn_shared with a caller's workspace) and the oracle: two calls in a row,
the second on a smaller workload, both within the 2e-3 row-error bar."""
import numpy as np
import pytest
import torch

import synth
from harness import DeviceRun, OracleRun, row_metric

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _run(make, wph):
    from mixed_precision_quantized_amd import kvq
    gpu, orc = DeviceRun(make()), OracleRun(make())
    ref, _ = orc.attend()
    workers, groups, n_groups, offsets = gpu.plan_workers(wph)
    w = gpu.w
    shared, _, _, _, work = gpu.decode_shared(workers, groups, n_groups, offsets)
    n = workers.shape[0]
    wk = torch.as_tensor(workers, device="cuda").contiguous()
    gr = torch.as_tensor(groups, device="cuda").contiguous()
    part_o = torch.empty((n, w.g, 128), dtype=torch.float32, device="cuda")
    part_lse = torch.empty((n, w.g), dtype=torch.float32, device="cuda")
    out = torch.empty((w.batch, w.hq, 128), dtype=torch.float32, device="cuda")
    kvq.decode_attn_shared_noalloc(gpu.cache, gpu.q, w.hkv, gpu.tables, kvq.TABLE_PAGES, wk, gr, n_groups,
                                   part_o, part_lse, dev_err=gpu.err)
    kvq.lse_merge(part_o, part_lse, n, torch.as_tensor(offsets, device="cuda"), w.batch, w.hq, w.hkv, out)
    torch.cuda.synchronize()
    assert int(gpu.err.item()) == 0
    got = out.cpu().numpy()
    e_entry, e_oracle = row_metric(shared.cpu().numpy(), got), row_metric(ref, got)
    print(f"[no-alloc] {w.note}: {n} workers, {n_groups} groups; vs kvq_decode_attn_shared {e_entry:.2e}, "
          f"vs oracle {e_oracle:.2e}", flush=True)
    assert e_entry <= TOL and e_oracle <= TOL


def test_no_alloc_two_calls_second_smaller():
    _run(lambda: synth.qwen3_8b(batch=2, n_tokens=2048), 7)
    _run(lambda: synth.qwen3_8b(batch=1, n_tokens=1024), 3)


def test_no_alloc_rejects_too_many_groups():
    from mixed_precision_quantized_amd import kvq
    cache = kvq.Cache(1, (0, 16, 0), "cuda")
    z = torch.zeros((1, 5), dtype=torch.int32, device="cuda")
    g = torch.zeros(1, dtype=torch.int32, device="cuda")
    po, pl = torch.empty((1, 4, 128), device="cuda"), torch.empty((1, 4), device="cuda")
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros((1, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_shared_noalloc(cache, q, 1, tables, kvq.TABLE_PAGES, z, g, 16385, po, pl)
    assert e.value.status == -3
