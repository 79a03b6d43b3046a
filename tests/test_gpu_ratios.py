"""GPU parity at every compression ratio the operator accepts (2 .. 128; the
overlapping channel sets only at ratio 4), through the C ABI against the
fp64 oracle: packed varlen prefill continuing from state, decode, and
prefill == the same tokens fed one per call through decode.

Every case prints its name before it touches the GPU.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import compressor_oracle as O
from compare import assert_out, assert_states

pytestmark = pytest.mark.gpu

RATIOS = [2, 8, 16, 32, 64]


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _spec(name, ratio, **kw):
    base = dict(ratio=ratio, head_dim=512, hidden=1024, rotate=False, block_size=16, batch=4,
                lengths=("uniform", 1, 900), start_pos=("uniform", 1, 3 * ratio),
                tables="perm", separate_kv_table=True)
    base.update(kw)
    return workloads.Spec(name, **base)


def _prefill_case(harness, w):
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    res = O.compressor(w)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    return mx, mae


@pytest.mark.parametrize("ratio", RATIOS)
def test_prefill_varlen_continuation(harness, ratio, tile_rows):
    """Ragged requests continuing from state: prefix rows from the ring,
    edge and interior GEMM tiles, live state rows written back."""
    _announce(f"prefill varlen r={ratio} tile rows {tile_rows}")
    w = workloads.build(_spec(f"ratio{ratio}_varlen", ratio, rotate=ratio in (2, 32)),
                        workloads.SEED_BASE + 300 + ratio)
    mx, mae = _prefill_case(harness, w)
    print(f"r={ratio}: max scaled err {mx:.2e}, MAE {mae:.2e}")


@pytest.mark.parametrize("ratio,batch", [(4, 33), (4, 64), (128, 64)])
def test_decode_more_than_32_requests(harness, ratio, batch):
    """One token per request with 33..64 requests (the 64-row GEMV): every
    other request closes a window, every fifth is inactive (seqused 0), so
    output rows are packed over the active ones."""
    _announce(f"decode r={ratio} batch={batch}")
    spec = _spec(f"ratio{ratio}_decode_b{batch}", ratio, hidden=2048, batch=batch, lengths=(1,),
                 start_pos=("uniform", 0, 65535), block_size=64, separate_kv_table=False,
                 out_rows=batch)
    w = workloads.build(spec, workloads.SEED_BASE + 380 + ratio + batch)
    sp = w["start_pos"].astype(np.int64)
    sp[::2] = sp[::2] - sp[::2] % ratio + ratio - 1
    used = np.ones(batch, np.int32)
    used[::5] = 0
    w = dict(w, start_pos=sp.astype(np.int32), seqused=used)
    case = harness.DeviceCase(w)
    case.decode()
    torch.cuda.synchronize()
    res = O.compressor(w)
    assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    assert int(res.plan.nwin.sum()) == int(np.sum(used * ((sp + 1) % ratio == 0)))


@pytest.mark.parametrize("ratio", [2, 16])
def test_prefill_aligned_long_and_padded(harness, ratio):
    """Window-aligned starts and long requests (interior tiles, no prefix),
    padded slots with seqused, head_dim 128."""
    _announce(f"prefill aligned/padded r={ratio}")
    spec = _spec(f"ratio{ratio}_aligned", ratio, head_dim=128, batch=3, lengths=(1500, 777, 256),
                 start_pos=(0, 4 * ratio, 128 * ratio), pad_rows=3, block_size=8,
                 rotate=True)
    w = workloads.build(spec, workloads.SEED_BASE + 320 + ratio)
    _prefill_case(harness, w)


@pytest.mark.parametrize("ratio", RATIOS)
@pytest.mark.parametrize("emit", [False, True])
def test_decode(harness, ratio, emit):
    _announce(f"decode r={ratio} emit_all={emit}")
    spec = _spec(f"ratio{ratio}_decode", ratio, hidden=2048, batch=32, lengths=(1,),
                 start_pos=("uniform", 0, 65535), block_size=64, separate_kv_table=False,
                 out_rows=32)
    w = workloads.build(spec, workloads.SEED_BASE + 340 + ratio + (7 if emit else 0))
    if emit:
        sp = w["start_pos"].astype(np.int64)
        w = dict(w, start_pos=(sp - sp % ratio + ratio - 1).astype(np.int32))
    case = harness.DeviceCase(w)
    case.decode()
    torch.cuda.synchronize()
    res = O.compressor(w)
    assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    if emit:
        assert int(res.plan.nwin.sum()) == w["batch"]


@pytest.mark.parametrize("ratio,rotate", [(2, True), (16, True), (2, False), (32, False)])
def test_prefill_equals_token_by_token_decode(harness, ratio, rotate):
    """The same tokens through one prefill call and through one decode call
    per token (state carried over): every window's output within the
    tolerance, the live state rows equal within fp32 rounding."""
    _announce(f"prefill vs decode r={ratio} rotate={rotate}")
    spec = _spec(f"ratio{ratio}_stream", ratio, batch=3, lengths=(3 * ratio + 1, 2 * ratio, 5),
                 start_pos=(0, ratio - 1, 1), block_size=8, separate_kv_table=False,
                 rotate=rotate)
    w = workloads.build(spec, workloads.SEED_BASE + 360 + ratio)
    case = harness.DeviceCase(w)
    case.prefill()
    res = O.compressor(w)
    full = {(b, wi): case.out_bits()[row] for b, wi, row in res.window_rows}
    plan = res.plan
    B, r = w["batch"], ratio
    d = harness.DeviceCase(dict(w, x=w["x"][:B], T=B, out_rows=B, cos=w["cos"][:B],
                                sin=w["sin"][:B], seqused=None))
    n = plan.ntok
    got = {}
    for t in range(int(n.max())):
        active = (n > t).astype(np.int32)
        rows = np.array([plan.row0[b] + min(t, max(n[b] - 1, 0)) for b in range(B)])
        pos = (plan.start + t).astype(np.int32)
        d.x.copy_(torch.from_numpy(w["x"][rows].view(np.int16)).to(d.dev).view(torch.bfloat16))
        # rope rows: decode row o_b carries the prefill row of the same window
        cos = np.zeros((B, 64), np.uint16)
        sin = np.zeros((B, 64), np.uint16)
        o = np.cumsum(active) - active
        for b in range(B):
            if active[b] and (pos[b] + 1) % r == 0:
                k = (pos[b] + 1) // r - 1 - plan.start[b] // r
                cos[o[b]] = w["cos"][plan.out0[b] + k]
                sin[o[b]] = w["sin"][plan.out0[b] + k]
        d.cos.copy_(torch.from_numpy(cos.view(np.int16)).to(d.dev).view(torch.bfloat16))
        d.sin.copy_(torch.from_numpy(sin.view(np.int16)).to(d.dev).view(torch.bfloat16))
        d.decode(start_pos=torch.from_numpy(pos).to(d.dev),
                 seqused=torch.from_numpy(active).to(d.dev))
        bits = d.out_bits()
        for b in range(B):
            if active[b] and (pos[b] + 1) % r == 0:
                got[(b, (pos[b] + 1) // r - 1)] = bits[o[b]].copy()
            elif active[b]:
                assert np.all(bits[o[b]] == 0)
        assert d.device_error() == 0
    assert set(got) == set(full)
    worst = 0.0
    for key in full:
        a = O.bf16_to_f64(full[key])
        b_ = O.bf16_to_f64(got[key])
        rms = np.sqrt(np.mean(a * a))
        worst = max(worst, float(np.max(np.abs(a - b_) / np.maximum(np.abs(a), rms))))
    assert worst <= 2e-2, worst
    kvp, scp = case.states()
    kvd, scd = d.states()
    for b in range(B):
        for p in O.live_positions(int(plan.start[b]), int(plan.end[b]), r, 1):
            q = p % r
            blk = w["state_block_table"][b, q // w["block_size"]]
            off = q % w["block_size"]
            assert np.allclose(kvp[blk, off], kvd[blk, off], rtol=1e-3, atol=1e-3)
            assert np.allclose(scp[blk, off], scd[blk, off], rtol=1e-3, atol=1e-3)
