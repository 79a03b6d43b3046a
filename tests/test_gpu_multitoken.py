"""GPU parity of multi-token decode (up to 4 tokens per request per call,
packed with cu_seqlens) through the decode entry point, against the fp64
oracle; and a prefill == a sequence of multi-token decode calls.

Every case prints its name before it touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import compressor_oracle as O
from compare import assert_out, assert_states

pytestmark = pytest.mark.gpu


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
    base = dict(ratio=ratio, head_dim=512, hidden=2048, rotate=False, block_size=16, batch=16,
                lengths=("uniform", 0, 4), start_pos=("uniform", 0, 5000), tables="perm",
                separate_kv_table=True)
    base.update(kw)
    return workloads.Spec(name, **base)


@pytest.mark.parametrize("ratio,pad,rotate", [(2, 0, False), (4, 0, True), (4, 2, False),
                                              (8, 1, False), (128, 0, False)])
def test_multitoken_decode(harness, ratio, pad, rotate):
    _announce(f"multi-token decode r={ratio} pad={pad} rotate={rotate}")
    w = workloads.build(_spec(f"mtp_r{ratio}", ratio, pad_rows=pad, rotate=rotate,
                              batch=64 // (4 + pad)),
                        workloads.SEED_BASE + 400 + ratio + pad)
    assert w["T"] <= 64
    case = harness.DeviceCase(w)
    case.decode(cu_seqlens=case.cu_seqlens)
    torch.cuda.synchronize()
    res = O.compressor(w)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    print(f"r={ratio}: {int(res.plan.nwin.sum())} windows, max scaled err {mx:.2e}, MAE {mae:.2e}")


def test_multitoken_decode_rejects_five_tokens(harness):
    _announce("multi-token decode, 5 tokens in a request")
    w = workloads.build(_spec("mtp_five", 4, batch=2, lengths=(5, 3), start_pos=(3, 9)),
                        workloads.SEED_BASE + 431)
    case = harness.DeviceCase(w)
    case.decode(cu_seqlens=case.cu_seqlens)
    torch.cuda.synchronize()
    assert case.device_error() & 4       # CMP_DEVERR_SEQLEN


@pytest.mark.parametrize("ratio,step", [(4, 3), (2, 4), (16, 2)])
def test_prefill_equals_multitoken_decode_steps(harness, ratio, step):
    """The tokens of one prefill call fed `step` at a time per request through
    the decode entry point, state carried over: same windows within the
    tolerance, same live state rows."""
    _announce(f"prefill vs {step}-token decode steps r={ratio}")
    w = workloads.build(_spec(f"mtp_stream_r{ratio}", ratio, batch=4,
                              lengths=(3 * ratio + 2, 2 * ratio + 1, 7, 1),
                              start_pos=(0, ratio - 1, 5, 2), block_size=8, rotate=True,
                              separate_kv_table=False),
                        workloads.SEED_BASE + 440 + ratio)
    case = harness.DeviceCase(w)
    case.prefill()
    res = O.compressor(w)
    full = {(b, wi): case.out_bits()[row] for b, wi, row in res.window_rows}
    plan = res.plan
    B = w["batch"]
    n = plan.ntok
    maxrows = B * step
    zeros = np.zeros((maxrows, 64), np.uint16)
    d = harness.DeviceCase(dict(w, x=w["x"][:maxrows], T=maxrows, out_rows=maxrows,
                                cos=zeros, sin=zeros, seqused=None,
                                cu_seqlens=np.arange(B + 1, dtype=np.int32) * step))
    got = {}
    for t0 in range(0, int(n.max()), step):
        take = np.clip(n - t0, 0, step).astype(np.int32)
        pos = (plan.start + t0).astype(np.int32)
        xs = np.zeros((maxrows, w["hidden"]), np.uint16)
        for b in range(B):
            for j in range(take[b]):
                xs[b * step + j] = w["x"][plan.row0[b] + t0 + j]
        d.x.copy_(torch.from_numpy(xs.view(np.int16)).to(d.dev).view(torch.bfloat16))
        # output rows of this call: request b owns ceil(take_b / r) rows from
        # o_b; its k-th window gets the rotary row of the prefill's window
        cos = np.zeros((maxrows, 64), np.uint16)
        sin = np.zeros((maxrows, 64), np.uint16)
        u = (take + ratio - 1) // ratio
        o = np.cumsum(u) - u
        wins = []
        for b in range(B):
            if take[b] == 0:
                continue
            s, e = int(pos[b]), int(pos[b]) + int(take[b])
            for k, wi in enumerate(range(s // ratio, e // ratio)):
                kk = wi - plan.start[b] // ratio
                cos[o[b] + k] = w["cos"][plan.out0[b] + kk]
                sin[o[b] + k] = w["sin"][plan.out0[b] + kk]
                wins.append((b, wi, o[b] + k))
        d.cos.copy_(torch.from_numpy(cos.view(np.int16)).to(d.dev).view(torch.bfloat16))
        d.sin.copy_(torch.from_numpy(sin.view(np.int16)).to(d.dev).view(torch.bfloat16))
        d.decode(cu_seqlens=d.cu_seqlens, start_pos=torch.from_numpy(pos).to(d.dev),
                 seqused=torch.from_numpy(take).to(d.dev))
        bits = d.out_bits()
        for b, wi, row in wins:
            got[(b, wi)] = bits[row].copy()
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
    coff = O.coff_of(ratio)
    for b in range(B):
        for p in O.live_positions(int(plan.start[b]), int(plan.end[b]), ratio, coff):
            if p < 0:
                continue
            q = p % (coff * ratio)
            blk = w["state_block_table"][b, q // w["block_size"]]
            off = q % w["block_size"]
            assert np.allclose(kvp[blk, off], kvd[blk, off], rtol=1e-3, atol=1e-3)
            assert np.allclose(scp[blk, off], scd[blk, off], rtol=1e-3, atol=1e-3)
