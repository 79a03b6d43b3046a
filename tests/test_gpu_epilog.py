"""GPU parity of compressor_epilog (the FP8 cache write after the operator)
against the oracle: codes and scales bit for bit (both sides take the
quantisation decision in fp32 and round to E4M3 to nearest even), rows the
slot mapping does not name unchanged, and the error bit for slots outside
the cache.

Every case prints its name before it touches the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle import epilog_oracle as E

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_kv_wkv_amd as cmp
    return cmp


def _run(cmp, rows_bits, slots, cache, cscale):
    dev = "cuda:0"
    r = torch.from_numpy(np.ascontiguousarray(rows_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    s = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).to(dev)
    c = torch.from_numpy(np.ascontiguousarray(cache)).to(dev)
    sc = torch.from_numpy(np.ascontiguousarray(cscale)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    cmp.compressor_epilog(r, s, c, sc, err)
    torch.cuda.synchronize()
    return c.cpu().numpy(), sc.cpu().numpy(), int(err.item())


def _check(rows_bits, slots, cache, cscale, got):
    want_c, want_s, want_err = E.epilog(W.bf16_bits_to_f32(rows_bits), slots, cache, cscale)
    gc, gs, gerr = got
    assert gerr == want_err
    diff = np.nonzero((gc != want_c).any(axis=1))[0]
    if diff.size:
        r = diff[0]
        col = np.nonzero(gc[r] != want_c[r])[0][:8]
        raise AssertionError(f"{diff.size} cache rows differ; row {r} cols {col}: "
                             f"got {gc[r, col]} want {want_c[r, col]}")
    assert np.array_equal(gs.view(np.uint32), want_s.view(np.uint32))


@pytest.mark.parametrize("spec", [W.EPILOG_INDEXER, W.EPILOG_RAGGED, W.EPILOG_C4A],
                         ids=lambda s: s.name)
def test_epilog_parity(lib, spec):
    _announce(spec.name)
    w = W.build_epilog(spec, W.SEED_BASE + 710)
    got = _run(lib, w["rows"], w["slot_mapping"], w["cache"], w["cache_scale"])
    _check(w["rows"], w["slot_mapping"], w["cache"], w["cache_scale"], got)


def _special_rows():
    """Blocks (D = 128, one per row) whose q values hit the rounding cases:
    with 448 in the block, 448 / amax = 1 and q = x exactly."""
    ties = [(1 + (2 * k + 1) / 16) * 2.0 ** e for e in range(-6, 8) for k in range(8)]
    r0 = [448.0] + ties + [-t for t in ties[:15]]
    sub = [(2 * k + 1) * 2.0 ** -10 for k in range(8)]            # subnormal midpoints
    r1 = ([448.0] + sub + [-v for v in sub] + [m * 2.0 ** -9 for m in range(8)]
          + [2.0 ** -11, -2.0 ** -11, 2.0 ** -10 * (1 + 2.0 ** -4), 2.0 ** -10 * (1 - 2.0 ** -5)])
    eps = [t * (1 + 2.0 ** -7) for t in ties[::4]] + [t * (1 - 2.0 ** -8) for t in ties[1::4]]
    r2 = [448.0] + eps
    r3 = [0.0] * 128                                               # amax 0
    r4 = [-0.0] * 127 + [5.0]                                      # signed zeros
    r5 = [-448.0, 447.0, 200.0, -3.25, 1e-30]                      # negative amax
    rows = []
    for r in (r0, r1, r2, r3, r4, r5):
        r = list(r)[:128]
        rows.append(r + [0.0] * (128 - len(r)))
    x = np.array(rows, dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    # the tie, subnormal and signed-zero rows are exact in bf16
    assert np.array_equal(W.bf16_bits_to_f32(bits)[[0, 1, 3, 4]], x[[0, 1, 3, 4]])
    return bits


def test_epilog_rounding_cases(lib):
    _announce("epilog_rounding_cases")
    bits = _special_rows()
    n = bits.shape[0]
    slots = np.arange(n, dtype=np.int32)[::-1].copy()
    cache = np.full((n, 128), 0x55, np.uint8)
    cscale = np.full((n, 1), 7.0, np.float32)
    got = _run(lib, bits, slots, cache, cscale)
    _check(bits, slots, cache, cscale, got)
    # the ties went to the even code and the signed zeros kept their sign
    assert got[0][n - 1 - 4][0] == 0x80 and got[0][n - 1 - 3][0] == 0x00


def test_epilog_of_prefill_output(lib):
    """The cache write of the rows a prefill call produced (the step the
    epilog follows), placed in reverse order."""
    _announce("epilog_of_prefill_output c4li_small")
    import gpu_harness
    w = W.build_named("c4li_small")
    case = gpu_harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    out = case.out_bits()
    n, d = out.shape
    slots = np.arange(n, dtype=np.int32)[::-1].copy()
    cache = np.zeros((n, d), np.uint8)
    cscale = np.zeros((n, d // 128), np.float32)
    got = _run(lib, out, slots, cache, cscale)
    _check(out, slots, cache, cscale, got)


def test_epilog_graph_replay_matches_eager(lib):
    """A captured call (one kernel, no memset, no allocation) replays to the
    eager result; every replay is checked, with eager work and a
    synchronisation between replays."""
    _announce("epilog graph replay")
    w = W.build_epilog(W.EPILOG_INDEXER, W.SEED_BASE + 711)
    dev = "cuda:0"
    rows = torch.from_numpy(w["rows"].view(np.int16)).to(dev).view(torch.bfloat16)
    slots = torch.from_numpy(w["slot_mapping"]).to(dev)
    cache0 = torch.from_numpy(w["cache"]).to(dev)
    scale0 = torch.from_numpy(w["cache_scale"]).to(dev)
    cache, scale = cache0.clone(), scale0.clone()
    lib.compressor_epilog(rows, slots, cache, scale)
    torch.cuda.synchronize()
    want_c, want_s = cache.cpu().numpy(), scale.cpu().numpy()
    gc, gs = cache0.clone(), scale0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.compressor_epilog(rows, slots, gc, gs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.compressor_epilog(rows, slots, gc, gs)
    for rep in range(3):
        gc.copy_(cache0)
        gs.copy_(scale0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gc.cpu().numpy(), want_c), rep
        assert np.array_equal(gs.cpu().numpy().view(np.uint32), want_s.view(np.uint32)), rep
        lib.compressor_epilog(rows, slots, cache, scale)        # eager work in between
