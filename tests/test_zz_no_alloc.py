"""compressor_decode_noalloc (decode in the library's per-device scratch, no
workspace) against compressor_decode on the same inputs, through the C ABI:
two calls in a row, the second with a smaller batch, outputs and states bit
for bit; then its caller error word on a bad table entry.

Every case prints its name before it touches the GPU.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads

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


def _both(harness, w, packed=False):
    import long_context_kv_wkv_amd as cmp
    case = harness.DeviceCase(w)
    over = dict(cu_seqlens=case.cu_seqlens) if packed else {}
    case.decode(**over)
    torch.cuda.synchronize()
    ref_out = case.out_bits().copy()
    ref_kv, ref_sc = case.states()
    assert case.device_error() == 0
    case.reset_state()
    case.out.fill_(0x7F7F)
    err = torch.zeros(1, dtype=torch.int32, device=case.dev)
    args = case._args(True, workspace=None, **over)
    cmp.compressor_decode_noalloc(case.shape, args, device_error=err)
    torch.cuda.synchronize()
    assert np.array_equal(case.out_bits(), ref_out)
    kv, sc = case.states()
    assert np.array_equal(kv.view(np.uint32), ref_kv.view(np.uint32))
    assert np.array_equal(sc.view(np.uint32), ref_sc.view(np.uint32))
    assert int(err.item()) == 0


def test_noalloc_decode_equals_decode_twice(harness):
    _announce("noalloc decode: 32-request C4A step, then an 8-request C128A step")
    _both(harness, workloads.build_named("decode_c4a_all"))
    spec = dataclasses.replace(workloads.DECODE_C128A, name="noalloc_small", batch=8, out_rows=8)
    w = workloads.build(spec, workloads.SEED_BASE + 880)
    r = w["ratio"]
    sp = w["start_pos"].astype(np.int64)
    sp[::2] = sp[::2] - sp[::2] % r + (r - 1)          # half of them close a window
    _both(harness, dict(w, start_pos=sp.astype(np.int32)))


def test_noalloc_decode_packed_and_error_word(harness):
    import long_context_kv_wkv_amd as cmp
    _announce("noalloc decode: packed multi-token step, then a bad table entry")
    spec = workloads.Spec("noalloc_mtp", ratio=4, head_dim=512, hidden=2048, rotate=True,
                          block_size=16, batch=12, lengths=(3,), start_pos=("uniform", 0, 900),
                          tables="perm", separate_kv_table=True)
    w = workloads.build(spec, workloads.SEED_BASE + 881)
    _both(harness, w, packed=True)
    bad = w["state_block_table"].copy()
    bad[3, 0] = w["num_blocks"] + 9                      # outside the pool: skipped, reported
    case = harness.DeviceCase(dict(w, state_block_table=bad))
    err = torch.zeros(1, dtype=torch.int32, device=case.dev)
    args = case._args(True, workspace=None, cu_seqlens=case.cu_seqlens)
    cmp.compressor_decode_noalloc(case.shape, args, device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
