"""The full variable-length continuation workload (C4A, rotate, H = 4096,
D = 512, 8 requests of up to 16384 tokens resuming partial windows from the
paged state) run twice on the GPU: as one packed prefill call, and with the
same tokens fed one per request per call through the decode entry point,
state carried over.  Every completed window must agree (within the output
tolerance: the GEMM and the GEMV sum K in different orders), every decode
row of a request that completes nothing must be zero, and the live state
rows must agree at the end.  The property holds at any size, so it is
checked at the full size here.

Every decode call's inputs (token rows, positions, active flags, rotary
rows) are gathered on the device beforehand and every call writes its own
slice of one output buffer, so the loop only enqueues.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import compressor_oracle as O

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


def test_full_varlen_prefill_equals_token_by_token_decode(harness):
    _announce("varlen_c4a full size: prefill vs token-by-token decode")
    w = workloads.build_named("varlen_c4a")
    B, r, D = w["batch"], w["ratio"], w["head_dim"]
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    assert case.device_error() == 0
    full = case.out_bits()
    plan = O.make_plan(r, B, w["T"], w["cu_seqlens"], w["seqused"], w["start_pos"])
    n = plan.ntok
    steps = int(n.max())
    dev = case.dev
    # per call t: request b feeds its token t (active while t < n_b)
    t_idx = np.arange(steps)[:, None]
    active = (n[None, :] > t_idx).astype(np.int32)                         # [steps, B]
    rows = plan.row0[None, :] + np.minimum(t_idx, np.maximum(n - 1, 0)[None, :])
    pos = (plan.start[None, :] + t_idx).astype(np.int32)
    o = np.cumsum(active, axis=1) - active                                 # decode out row
    emits = (active == 1) & ((pos + 1) % r == 0)
    k = (pos + 1) // r - 1 - (plan.start // r)[None, :]                    # window index
    cos = np.zeros((steps, B, 64), np.uint16)
    sin = np.zeros((steps, B, 64), np.uint16)
    tt, bb = np.nonzero(emits)
    cos[tt, o[tt, bb]] = w["cos"][plan.out0[bb] + k[tt, bb]]
    sin[tt, o[tt, bb]] = w["sin"][plan.out0[bb] + k[tt, bb]]
    x_dec = case.x.index_select(0, torch.from_numpy(rows.reshape(-1)).to(dev)).view(steps, B, -1)
    pos_d = torch.from_numpy(pos).to(dev)
    act_d = torch.from_numpy(active).to(dev)
    cos_d = torch.from_numpy(cos.view(np.int16)).to(dev).view(torch.bfloat16)
    sin_d = torch.from_numpy(sin.view(np.int16)).to(dev).view(torch.bfloat16)
    out_d = torch.zeros((steps, B, D), dtype=torch.bfloat16, device=dev)

    d = harness.DeviceCase(dict(w, x=w["x"][:B], T=B, out_rows=B, cos=w["cos"][:B],
                                sin=w["sin"][:B], seqused=None))
    for t in range(steps):
        d.decode(x=x_dec[t], start_pos=pos_d[t], seqused=act_d[t], cos=cos_d[t], sin=sin_d[t],
                 out=out_d[t])
        if t % 2048 == 2047 or t == steps - 1:
            assert d.device_error() == 0, t
    torch.cuda.synchronize()
    got = out_d.view(torch.int16).cpu().numpy().view(np.uint16)

    # rows of active requests that complete nothing are zero
    quiet = (active == 1) & ~emits
    qt, qb = np.nonzero(quiet)
    assert not got[qt, o[qt, qb]].any()
    # every completed window agrees with the prefill's row
    assert int(emits.sum()) == int(plan.nwin.sum())
    a = O.bf16_to_f64(full[plan.out0[bb] + k[tt, bb]])
    g = O.bf16_to_f64(got[tt, o[tt, bb]])
    rms = np.sqrt(np.mean(a * a, axis=1, keepdims=True))
    worst = float(np.max(np.abs(a - g) / np.maximum(np.abs(a), rms)))
    same = int(np.all(full[plan.out0[bb] + k[tt, bb]] == got[tt, o[tt, bb]], axis=1).sum())
    print(f"{len(tt)} windows over {steps} decode calls: {same} bit-identical to the prefill's "
          f"rows, max scaled difference {worst:.2e}")
    assert worst <= 2e-2, worst
    # live state rows agree
    kvp, scp = case.states()
    kvd, scd = d.states()
    bs = w["block_size"]
    sdiff = 0.0
    nrows = 0
    for b in range(B):
        for p in O.live_positions(int(plan.start[b]), int(plan.end[b]), r, 2):
            q = p % (2 * r)
            kb = w["kv_block_table"][b, q // bs]
            sb = w["state_block_table"][b, q // bs]
            assert np.allclose(kvp[kb, q % bs], kvd[kb, q % bs], rtol=1e-3, atol=1e-3)
            assert np.allclose(scp[sb, q % bs], scd[sb, q % bs], rtol=1e-3, atol=1e-3)
            for pa, pb in ((kvp[kb, q % bs], kvd[kb, q % bs]), (scp[sb, q % bs], scd[sb, q % bs])):
                fin = np.isfinite(pa)
                if fin.any():
                    sdiff = max(sdiff, float(np.max(np.abs(pa[fin].astype(np.float64) - pb[fin]))))
            nrows += 1
    print(f"{nrows} live state rows: max |prefill - decode| {sdiff:.2e}")
