"""GPU tests of the state cache entry points and of state carried across
calls:

* compressor_state_init fills every slot of both pools with kv +0 and score
  -inf, bit for bit (the padding values of the first window, [PyPTO] page
  "CANN PyPTO 算子实战：Compressor 长序列 KV Cache 压缩算子的原理、参数与调用方法",
  section 压缩窗口与状态更新);
* compressor_state_reset refills exactly the blocks the named table rows
  address (separate kv and score tables) and leaves every other block
  bit-identical; bad row indices and table entries are skipped and reported;
* a prefill that resumes from reset rows equals the oracle on pools holding
  those values, and the same prefill on a freshly initialised pool;
* requests change batch positions between consecutive calls (prefill,
  prefill, decode), their table rows moving with them and their state
  carried in the pools ([Triton] article: request positions change between
  calls and the mapping table finds each request's state; its validation
  runs request swaps over several consecutive calls).

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

NEG_INF_BITS = np.uint32(0xFF800000)


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _varlen(name, seed, B=5, max_len=300, ratio=4, rotate=True, bs=4):
    spec = dataclasses.replace(workloads.VARLEN_C4A, name=name, batch=B,
                               lengths=("uniform", 1, max_len), ratio=ratio, rotate=rotate,
                               block_size=bs, spare_blocks=4)
    return workloads.build(spec, seed)


@pytest.mark.parametrize("ratio,bs", [(4, 4), (128, 64)])
def test_state_init_fills_zero_and_minus_inf(harness, ratio, bs):
    _announce(f"state init r={ratio} bs={bs}")
    import long_context_kv_wkv_amd as cmp
    w = _varlen(f"init_r{ratio}", workloads.SEED_BASE + 700 + ratio, ratio=ratio, bs=bs)
    case = harness.DeviceCase(w)
    cmp.compressor_state_init(case.shape, case.kv_state, case.score_state)
    kv, sc = case.states()
    assert kv.shape == w["kv_state"].shape
    assert np.all(kv.view(np.uint32) == 0), "kv slots must be +0.0"
    assert np.all(sc.view(np.uint32) == NEG_INF_BITS), "score slots must be -inf"


def _expected_reset(w, rows, table_rows):
    """Host copy of the pools after a reset of table rows `rows` (rows
    outside the table skipped; entries outside the pools skipped)."""
    r, coff, bs = w["ratio"], w["coff"], w["block_size"]
    used = -(-coff * r // bs)
    st = w["state_block_table"]
    kvt = st if w["kv_block_table"] is None else w["kv_block_table"]
    kv = w["kv_state"].copy()
    sc = w["score_state"].copy()
    nb = kv.shape[0]
    for row in rows:
        if not 0 <= row < table_rows:
            continue
        for j in range(used):
            if 0 <= kvt[row, j] < nb:
                kv[kvt[row, j]] = 0.0
            if 0 <= st[row, j] < nb:
                sc[st[row, j]] = -np.inf
    return kv, sc


@pytest.mark.parametrize("ratio,bs", [(4, 4), (4, 16), (128, 64)])
def test_state_reset_only_named_blocks(harness, ratio, bs):
    _announce(f"state reset r={ratio} bs={bs}")
    import long_context_kv_wkv_amd as cmp
    w = _varlen(f"reset_r{ratio}_{bs}", workloads.SEED_BASE + 710 + ratio + bs, ratio=ratio, bs=bs)
    assert w["kv_block_table"] is not None            # separate kv and score tables
    case = harness.DeviceCase(w)
    rows = np.array([3, 0], np.int32)
    cmp.compressor_state_reset(case.shape, case.kv_state, case.score_state, case.kv_table,
                               case.st_table, torch.from_numpy(rows).to(case.dev))
    kv, sc = case.states()
    ekv, esc = _expected_reset(w, rows, w["batch"])
    assert np.array_equal(kv.view(np.uint32), ekv.view(np.uint32))
    assert np.array_equal(sc.view(np.uint32), esc.view(np.uint32))
    # the reset touched something and left some blocks alone
    assert not np.array_equal(kv, w["kv_state"]) and np.any(kv == w["kv_state"])


def test_state_reset_bad_rows_and_entries_are_skipped(harness):
    _announce("state reset with a bad row index and a bad table entry")
    import long_context_kv_wkv_amd as cmp
    w = _varlen("reset_bad", workloads.SEED_BASE + 730)
    st = w["state_block_table"].copy()
    st[2, 0] = w["num_blocks"] + 5                    # outside the pool
    w = dict(w, state_block_table=st)
    case = harness.DeviceCase(w)
    err = torch.zeros(1, dtype=torch.int32, device=case.dev)
    rows = np.array([1, w["batch"] + 3, 2, -1], np.int32)    # two rows outside the table
    cmp.compressor_state_reset(case.shape, case.kv_state, case.score_state, case.kv_table,
                               case.st_table, torch.from_numpy(rows).to(case.dev),
                               device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    kv, sc = case.states()
    ekv, esc = _expected_reset(w, rows, w["batch"])
    assert np.array_equal(kv.view(np.uint32), ekv.view(np.uint32))
    assert np.array_equal(sc.view(np.uint32), esc.view(np.uint32))


def test_prefill_after_reset(harness):
    """Reset requests 0 and 2, then resume every request from its start
    position: equals the oracle on host pools holding the reset values, and
    (for the reset requests' windows) the same call on pools that
    compressor_state_init filled."""
    _announce("prefill resuming from reset rows")
    import long_context_kv_wkv_amd as cmp
    w = _varlen("reset_prefill", workloads.SEED_BASE + 740, max_len=120)
    case = harness.DeviceCase(w)
    rows = np.array([0, 2], np.int32)
    cmp.compressor_state_reset(case.shape, case.kv_state, case.score_state, case.kv_table,
                               case.st_table, torch.from_numpy(rows).to(case.dev))
    case.prefill()
    torch.cuda.synchronize()
    ekv, esc = _expected_reset(w, rows, w["batch"])
    wr = dict(w, kv_state=ekv, score_state=esc)
    res = O.compressor(wr)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, wr, res)
    assert case.device_error() == 0
    got = case.out_bits().copy()
    # the same call on freshly initialised pools
    fresh = harness.DeviceCase(w)
    cmp.compressor_state_init(fresh.shape, fresh.kv_state, fresh.score_state)
    fresh.prefill()
    torch.cuda.synchronize()
    fb = fresh.out_bits()
    for b, _, row in res.window_rows:
        if b in rows:
            assert np.array_equal(got[row], fb[row]), (b, row)
    print(f"prefill after reset: max scaled err {mx:.2e}, MAE {mae:.2e}")


def _gpu_pools(case):
    kv, sc = case.states()
    return kv.copy(), sc.copy()


def test_requests_change_batch_position_between_calls(harness):
    """Call 1: prefill of 6 requests.  Call 2: their next tokens, batch order
    permuted, table rows moved with the requests.  Call 3: one decode token
    each in a third order.  Each call against the oracle run on the same
    inputs with the oracle's own state carried over."""
    _announce("request swaps across prefill, prefill, decode")
    B = 6
    w1 = _varlen("swap1", workloads.SEED_BASE + 750, B=B, max_len=90)
    rng = np.random.default_rng(workloads.SEED_BASE + 751)
    res1 = O.compressor(w1)
    c1 = harness.DeviceCase(w1)
    c1.prefill()
    torch.cuda.synchronize()
    assert_out(c1.out_bits(), res1)
    kv1, sc1 = _gpu_pools(c1)
    assert_states(kv1, sc1, w1, res1)
    end1 = res1.plan.end.copy()

    # call 2: new tokens, permuted batch
    perm2 = rng.permutation(B)
    w2n = _varlen("swap2", workloads.SEED_BASE + 752, B=B, max_len=70)
    keep = ("wkv", "wgate", "ape", "weight", "hadamard", "num_blocks", "table_stride")
    w2 = dict(w2n, **{k: w1[k] for k in keep})
    w2["start_pos"] = end1[perm2].astype(np.int32)
    w2["state_block_table"] = w1["state_block_table"][perm2].copy()
    w2["kv_block_table"] = w1["kv_block_table"][perm2].copy()
    w2_oracle = dict(w2, kv_state=res1.kv_state, score_state=res1.score_state)
    res2 = O.compressor(w2_oracle)
    c2 = harness.DeviceCase(dict(w2, kv_state=kv1, score_state=sc1))
    c2.prefill()
    torch.cuda.synchronize()
    mx2, _ = assert_out(c2.out_bits(), res2)
    kv2, sc2 = _gpu_pools(c2)
    assert_states(kv2, sc2, dict(w2, kv_state=kv1, score_state=sc1), res2)
    assert c2.device_error() == 0
    end2 = np.empty(B, np.int64)
    end2[perm2] = res2.plan.end          # by original request

    # call 3: one decode token per request, a third order
    perm3 = rng.permutation(B)
    x3 = workloads.normal_bf16(rng, (B, w1["hidden"]), 1.0)
    cos3, sin3 = workloads.rope_tables(np.arange(B) + 11.0)
    w3 = dict(w1, x=x3, T=B, batch=B, cu_seqlens=np.arange(B + 1, dtype=np.int32), seqused=None,
              start_pos=end2[perm3].astype(np.int32),
              state_block_table=w1["state_block_table"][perm3].copy(),
              kv_block_table=w1["kv_block_table"][perm3].copy(), out_rows=B, cos=cos3, sin=sin3)
    res3 = O.compressor(dict(w3, kv_state=res2.kv_state, score_state=res2.score_state))
    c3 = harness.DeviceCase(dict(w3, kv_state=kv2, score_state=sc2))
    c3.decode()
    torch.cuda.synchronize()
    mx3, _ = assert_out(c3.out_bits(), res3)
    kv3, sc3 = _gpu_pools(c3)
    assert_states(kv3, sc3, dict(w3, kv_state=kv2, score_state=sc2), res3)
    assert c3.device_error() == 0
    print(f"swaps: call 2 max scaled err {mx2:.2e}, call 3 {mx3:.2e}, "
          f"{int(res3.plan.nwin.sum())} decode windows")
