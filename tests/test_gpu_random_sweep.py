"""Seeded sweep of small random configurations through the C ABI against the
oracle: every ratio, D = 128 and 512, H multiples of 512, with and without
rotation, block sizes that do and do not divide the ring, padded slots,
empty requests, separate or shared kv / score tables, prefill (continuing
from state) and decode (one token per request, or packed steps of up to 4).

Half of the prefill cases force 256-row projection tiles.  Every case
prints its parameters before it touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import compressor_oracle as O
from compare import assert_out, assert_states

pytestmark = pytest.mark.gpu

N_CASES = 512
# cases from this index on run their prefill with 256-row projection tiles
# (short calls otherwise take 128-row tiles)
FORCE_256_FROM = 256


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _draw(i):
    rng = np.random.default_rng(workloads.SEED_BASE + 900 + i)
    ratio = int(rng.choice([2, 4, 8, 16, 32, 64, 128]))
    D = int(rng.choice([128, 512]))
    H = int(rng.choice([1024, 1536, 2048, 3072, 4096, 7168]))
    rotate = bool(rng.integers(0, 2))
    bs = int(rng.choice([1, 3, 8, 16, 64]))
    mode = ["prefill", "decode1", "decode_packed"][i % 3]
    if mode == "prefill":
        B = int(rng.integers(1, 6))
        lengths = ("uniform", 0, int(rng.choice([40, 300])))
        pad = int(rng.choice([0, 3]))
    elif mode == "decode1":
        B = int(rng.integers(1, 33))
        lengths = (1,)
        pad = 0
    else:
        B = int(rng.integers(1, 13))
        lengths = ("uniform", 0, 4)
        pad = int(rng.choice([0, 1]))
    spec = workloads.Spec(f"sweep{i}", ratio=ratio, head_dim=D, hidden=H, rotate=rotate,
                          block_size=bs, batch=B, lengths=lengths,
                          start_pos=("uniform", 0, 1000), pad_rows=pad, tables="perm",
                          separate_kv_table=bool(rng.integers(0, 2)), spare_blocks=2)
    w = workloads.build(spec, workloads.SEED_BASE + 950 + i)
    if mode == "decode1":
        # a third of the requests close a window in this step
        sp = w["start_pos"].astype(np.int64)
        sp[::3] = sp[::3] - sp[::3] % ratio + (ratio - 1)
        w["start_pos"] = sp.astype(np.int32)
    if mode == "decode_packed" and w["T"] > 64:
        return None
    return mode, w


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(harness, i):
    drawn = _draw(i)
    if drawn is None:
        pytest.skip("more packed rows than one decode call takes")
    mode, w = drawn
    _announce(f"sweep {i}: {mode} r={w['ratio']} D={w['head_dim']} H={w['hidden']} "
              f"rotate={w['rotate']} bs={w['block_size']} B={w['batch']} T={w['T']}")
    case = harness.DeviceCase(w)
    if mode == "prefill":
        import long_context_kv_wkv_amd as cmp
        cmp.compressor_set_prefill_tile_rows(256 if i >= FORCE_256_FROM else 0)
        try:
            case.prefill()
        finally:
            cmp.compressor_set_prefill_tile_rows(0)
    elif mode == "decode1":
        case.decode()
    else:
        case.decode(cu_seqlens=case.cu_seqlens)
    torch.cuda.synchronize()
    res = O.compressor(w)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    print(f"sweep {i}: {int(res.plan.nwin.sum())} windows, max scaled err {mx:.2e}, MAE {mae:.2e}")
