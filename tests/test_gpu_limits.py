"""GPU parity at the limits the C header states, against the fp64 oracle:

* prefill at the largest hidden size (H = 10240) and at one that is a
  multiple of 512 but not of 1024 (H = 1536), D = 128 and 512, both tile
  heights, continuing from state with padded slots;
* block size 1024 (one block holds a request's whole ring and more);
* prefill with many short requests (48, of 0 to 60 tokens: most tiles hold
  one request's few windows, some requests are empty), and with 600 (more
  than the plan's 256 threads);
* single-token decode at the largest batch (64 requests: the two-row-block
  GEMV with one row per request), half of them closing a window.

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


# name, ratio, D, H, block size, rotate
PREFILL = [
    ("lim_h10240_c4a", 4, 512, 10240, 16, True),
    ("lim_h10240_c128a", 128, 512, 10240, 128, False),
    ("lim_h1536_c4a_bs1024", 4, 128, 1536, 1024, True),
    ("lim_h1536_c128a_bs1024", 128, 128, 1536, 1024, False),
]


def _check(case, w, res, label):
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    print(f"{label}: {int(res.plan.nwin.sum())} windows, max scaled err {mx:.2e}, MAE {mae:.2e}")


@pytest.mark.parametrize("cfg", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_limits(harness, cfg, tile_rows):
    name, ratio, D, H, bs, rotate = cfg
    spec = workloads.Spec(name, ratio=ratio, head_dim=D, hidden=H, rotate=rotate, block_size=bs,
                          batch=3, lengths=("uniform", 150, 700), start_pos=("uniform", 0, 2000),
                          pad_rows=2, tables="perm", separate_kv_table=True, spare_blocks=2)
    w = workloads.build(spec, workloads.SEED_BASE + 1300 + PREFILL.index(cfg))
    _announce(f"{name} T={w['T']} tile rows {tile_rows}")
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    _check(case, w, O.compressor(w), f"{name} bm{tile_rows}")


@pytest.mark.parametrize("ratio", [4, 16])
def test_prefill_many_short_requests(harness, ratio, tile_rows):
    name = f"lim_many_requests_r{ratio}"
    spec = workloads.Spec(name, ratio=ratio, head_dim=128, hidden=1024, rotate=True, block_size=8,
                          batch=48, lengths=("uniform", 0, 60), start_pos=("uniform", 0, 500),
                          pad_rows=1, tables="perm", separate_kv_table=False, spare_blocks=2)
    w = workloads.build(spec, workloads.SEED_BASE + 1320 + ratio)
    _announce(f"{name} B=48 T={w['T']} tile rows {tile_rows}")
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    _check(case, w, O.compressor(w), f"{name} bm{tile_rows}")


@pytest.mark.parametrize("ratio", [4, 128])
def test_prefill_more_requests_than_plan_threads(harness, ratio):
    """600 requests: the plan walks them in chunks of its 256 threads with a
    carried offset, and the staging of earlier positions runs one workgroup
    per request and ring slot."""
    name = f"lim_600_requests_r{ratio}"
    spec = workloads.Spec(name, ratio=ratio, head_dim=128, hidden=1024, rotate=False,
                          block_size=16, batch=600, lengths=("uniform", 0, 12),
                          start_pos=("uniform", 0, 400), pad_rows=0, tables="perm",
                          separate_kv_table=True, spare_blocks=2)
    w = workloads.build(spec, workloads.SEED_BASE + 1380 + ratio)
    _announce(f"{name} B=600 T={w['T']}")
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    _check(case, w, O.compressor(w), name)


@pytest.mark.parametrize("ratio", [4, 128])
def test_decode_largest_batch(harness, ratio):
    name = f"lim_decode_b64_r{ratio}"
    spec = workloads.Spec(name, ratio=ratio, head_dim=512, hidden=7168, rotate=False,
                          block_size=64, batch=64, lengths=(1,), start_pos=("uniform", 0, 65535),
                          tables="perm", separate_kv_table=True, spare_blocks=0, out_rows=64)
    w = workloads.build(spec, workloads.SEED_BASE + 1340 + ratio)
    # every other request closes a window with this step's token
    sp = w["start_pos"].astype(np.int64)
    sp[::2] = sp[::2] - sp[::2] % ratio + (ratio - 1)
    w["start_pos"] = sp.astype(np.int32)
    _announce(f"{name} B=64 T={w['T']}")
    case = harness.DeviceCase(w)
    case.decode()
    torch.cuda.synchronize()
    _check(case, w, O.compressor(w), name)


@pytest.mark.parametrize("kind", ["random_rotation", "no_rotation"])
def test_post_rows_per_workgroup(harness, kind):
    """9001 output rows: more than one 32-row post workgroup per CU, so the
    post kernel runs its 32-row workgroups (shorter calls take 16-row ones,
    which every smaller test covers); with a random rotation matrix (the
    matrix-product path) and without rotation."""
    rotate = kind == "random_rotation"
    spec = workloads.Spec(f"lim_post_{kind}", ratio=4, head_dim=128, hidden=1024, rotate=rotate,
                          block_size=16, batch=1, lengths=(36003,), start_pos=(5,),
                          tables="perm", separate_kv_table=True, spare_blocks=2)
    w = workloads.build(spec, workloads.SEED_BASE + 1360 + rotate)
    if rotate:
        rng = np.random.default_rng(workloads.SEED_BASE + 1362)
        m = (rng.standard_normal((128, 128)) / np.sqrt(128)).astype(np.float32)
        w = dict(w, hadamard=workloads.f32_to_bf16_bits(m))
    assert w["out_rows"] > 32 * 256
    _announce(f"lim_post_{kind} T={w['T']} out_rows={w['out_rows']}")
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    _check(case, w, O.compressor(w), f"lim_post_{kind}")
