"""GPU prefill attention with an INT8 prefix (HyQuant, the core method's fused operator
and Algorithm 2: the query as given, the prefix's K and V through per-tile INT8) through
the C ABI against the oracle: K and V codes and tile scales bit-exact (both sides divide
in IEEE fp32), outputs within 2e-3 by the per-row metric (rows = (request, position,
query head) below the request's length)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _say(*a):
    print("[gpu-prefill]", *a, flush=True)


def _codes_equal(ws, ref):
    """ws: the binding's (k_codes, k_scales, v_codes, v_scales, ...); ref: the oracle's
    (k_codes, k_scales, v_codes, v_scales)."""
    for got, want, what in zip(ws[:4], ref, ("K codes", "K scales", "V codes", "V scales")):
        assert np.array_equal(got.cpu().numpy(), want), what


def _case(name, batch, n_max, hq, hkv, lengths, window, vl_frac=0.05, with_cls=True, seed=7):
    from mixed_precision_quantized_amd import kvq
    from oracle import oracle
    from harness import row_metric
    _say(name)
    q, k, v, lens, cls = synth.prefill_qkv(seed, batch, n_max, hq, hkv, lengths, vl_frac)
    dev = "cuda"
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    c_dev = torch.as_tensor(cls, device=dev).contiguous() if with_cls else None
    ws = kvq.prefill_attn(q.to(dev), k.to(dev), v.to(dev), torch.as_tensor(lens, device=dev), c_dev,
                          window=window, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref, *rcodes = oracle.prefill_attend(q.float().numpy(), k.float().numpy(), v.float().numpy(), lens,
                                         cls if with_cls else None, window)
    _codes_equal(ws, rcodes)
    got = ws[5].cpu().numpy()
    rows_ref, rows_got = [], []
    for b in range(batch):
        rows_ref.append(ref[b, : lens[b]].reshape(-1, 128))
        rows_got.append(got[b, : lens[b]].reshape(-1, 128))
        assert not got[b, lens[b]:].any()
    e = row_metric(np.concatenate(rows_ref), np.concatenate(rows_got))
    _say(f"  {name}: row error {e:.2e}")
    assert e <= TOL
    return e


def test_small_mixed_segments():
    _case("b2 n256 g4 W64", 2, 256, 8, 2, [256, 150], window=64)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (16, 2), (16, 1)])
def test_gqa_ratios(hq, hkv):
    """Every supported g: a work group holds 256 / g positions of all g heads."""
    _case(f"g={hq // hkv}", 1, 192, hq, hkv, [181], window=32)


def test_many_stages():
    """Several work groups per head, INT8 stages before and across the window edge,
    more than one 64-entry stage of vertical lines, a ragged second request."""
    _case("b2 n1024 g4 W128", 2, 1024, 8, 2, [1024, 701], window=128, vl_frac=0.1, seed=11)


def test_limits():
    """Window covering the whole prompt (all full precision); no window and no vertical
    line (all INT8); every position a vertical line."""
    _case("all full precision", 1, 128, 4, 2, [128], window=128)
    _case("all INT8", 1, 128, 4, 2, [120], window=0, with_cls=False)
    _case("all vertical lines", 1, 128, 4, 2, [128], window=0, vl_frac=1.0)


def test_bad_length_is_reported():
    from mixed_precision_quantized_amd import kvq
    q, k, v, lens, cls = synth.prefill_qkv(1, 2, 64, 4, 2)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    *_, out = kvq.prefill_attn(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(np.array([64, 65], np.int32),
                               device="cuda"), None, window=16, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == kvq.DEVERR_RANGE and not out[1].any()


def test_full_size_sampled():
    """The benchmarked workload (1 x 16384 positions, Hq 32 / Hkv 8, 5 % lines, window
    128) in the benchmarked launch: codes and tile scales bit-exact in full; twelve
    positions (all 32 query heads each; tile and window edges, the last position)
    against the oracle's rows."""
    from mixed_precision_quantized_amd import kvq
    from oracle import oracle
    from harness import row_metric
    n, hq, hkv = 16384, 32, 8
    _say("full size 1 x 16384, Hq 32 / Hkv 8")
    q, k, v, lens, cls = synth.prefill_qkv(seed=8, batch=1, n_max=n, hq=hq, hkv=hkv, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvq.prefill_attn(q, k, v, torch.as_tensor(lens, device="cuda"),
                          torch.as_tensor(cls, device="cuda").contiguous(), window=128, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    pos = [0, 1, 63, 64, 127, 128, 129, 4095, 8191, 12000, 16320, 16383]
    ref, *rcodes = oracle.prefill_attend_rows(q.float().cpu().numpy(), k.float().cpu().numpy(),
                                              v.float().cpu().numpy(), lens, cls, 128, [(0, t) for t in pos])
    _codes_equal(ws, rcodes)
    got = ws[5][0, pos].cpu().numpy()
    e = row_metric(ref, got)
    _say(f"  full size: row error {e:.2e} over {len(pos)} positions x {hq} heads")
    assert e <= TOL


def test_empty_and_single_token_requests_and_window_class():
    """A request of length 0, one of length 1 and a ragged one in one batch; class flags
    holding 2 (the FREEZE window class the selection writes) besides 0 and 1: only 1
    marks a vertical line."""
    from mixed_precision_quantized_amd import kvq
    from oracle import oracle
    from harness import row_metric
    _say("lengths 0 / 1 / 200, classes 0 / 1 / 2")
    batch, n_max, hq, hkv = 3, 256, 8, 2
    q, k, v, _, _ = synth.prefill_qkv(13, batch, n_max, hq, hkv)
    lens = np.array([0, 1, 200], np.int32)
    cls = np.random.default_rng(13).integers(0, 3, (batch, hkv, n_max)).astype(np.uint8)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvq.prefill_attn(q.cuda(), k.cuda(), v.cuda(), torch.as_tensor(lens, device="cuda"),
                          torch.as_tensor(cls, device="cuda"), window=32, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref, *rcodes = oracle.prefill_attend(q.float().numpy(), k.float().numpy(), v.float().numpy(), lens, cls, 32)
    _codes_equal(ws, rcodes)
    got = ws[5].cpu().numpy()
    assert not got[0].any() and not got[1, 1:].any() and not got[2, 200:].any()
    e = row_metric(np.concatenate([ref[1, :1].reshape(-1, 128), ref[2, :200].reshape(-1, 128)]),
                   np.concatenate([got[1, :1].reshape(-1, 128), got[2, :200].reshape(-1, 128)]))
    _say(f"  edge batch: row error {e:.2e}")
    assert e <= TOL
