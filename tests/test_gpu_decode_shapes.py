"""GPU parity of the decode entry point at hidden sizes that are multiples of
512 but not of 1024 (the K split must cover every k-step), at both GEMV
widths (T <= 32 and 33..64 packed rows), and with rotation matrices that are
not symmetric (the tail's product is out = y @ Had, not y @ Had^T).

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


def _decode_case(name, ratio, hidden, packed, seed, D=512, rotate=False):
    """32 single-token requests (T = 32), or 14 requests of 3 tokens packed
    with cu_seqlens (T = 42 > 32: the two-row-block GEMV)."""
    if packed:
        spec = workloads.Spec(name, ratio=ratio, head_dim=D, hidden=hidden, rotate=rotate,
                              block_size=16, batch=14, lengths=(3,),
                              start_pos=("uniform", 0, 3000), tables="perm",
                              separate_kv_table=True)
    else:
        spec = workloads.Spec(name, ratio=ratio, head_dim=D, hidden=hidden, rotate=rotate,
                              block_size=64, batch=32, lengths=(1,),
                              start_pos=("uniform", 0, 65535), tables="perm",
                              separate_kv_table=False, spare_blocks=0, out_rows=32)
    w = workloads.build(spec, seed)
    # half of the requests close a window in this step (the single token
    # sits on a window's last position; of three tokens, the second does)
    r = w["ratio"]
    sp = w["start_pos"].astype(np.int64)
    sp[::2] = sp[::2] - sp[::2] % r + (r - 2 if packed else r - 1)
    w["start_pos"] = sp.astype(np.int32)
    return w


def _run_decode(harness, w, packed):
    case = harness.DeviceCase(w)
    if packed:
        case.decode(cu_seqlens=case.cu_seqlens)
    else:
        case.decode()
    torch.cuda.synchronize()
    res = O.compressor(w)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    return res, mx, mae


@pytest.mark.parametrize("hidden", [1536, 2560, 5632, 8704, 1024, 10240])
@pytest.mark.parametrize("ratio", [4, 128])
@pytest.mark.parametrize("packed", [False, True], ids=["T32", "T42"])
def test_decode_hidden_sizes(harness, hidden, ratio, packed):
    _announce(f"decode H={hidden} ratio={ratio} packed={packed}")
    w = _decode_case(f"dec_h{hidden}_r{ratio}", ratio, hidden, packed,
                     workloads.SEED_BASE + 600 + hidden // 512 + ratio + 7 * packed)
    assert w["T"] == (42 if packed else 32)
    res, mx, mae = _run_decode(harness, w, packed)
    nwin = int(res.plan.nwin.sum())
    assert nwin > 0
    print(f"H={hidden} r={ratio} T={w['T']}: {nwin} windows, max scaled err {mx:.2e}, MAE {mae:.2e}")


@pytest.mark.parametrize("D", [512, 128])
@pytest.mark.parametrize("packed", [False, True], ids=["T32", "T42"])
def test_decode_random_rotation_matrix(harness, D, packed):
    """A random D x D matrix (not symmetric): the decode tails must compute
    y @ Had with Had's rows indexed by y's channels."""
    _announce(f"decode with a random rotation matrix, D={D}, packed={packed}")
    w = _decode_case(f"dec_had_{D}", 4, 2048, packed, workloads.SEED_BASE + 650 + D + packed,
                     D=D, rotate=True)
    rng = np.random.default_rng(workloads.SEED_BASE + 651)
    m = (rng.standard_normal((D, D)) / np.sqrt(D)).astype(np.float32)
    w = dict(w, hadamard=workloads.f32_to_bf16_bits(m))
    hb = O.bf16_to_f64(w["hadamard"])
    assert not np.allclose(hb, hb.T)
    res, mx, mae = _run_decode(harness, w, packed)
    assert int(res.plan.nwin.sum()) > 0
    print(f"D={D} packed={packed}: max scaled err {mx:.2e}, MAE {mae:.2e}")
