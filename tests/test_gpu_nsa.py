"""GPU parity of the NSA KV-compression operator (NsaCompressWithCache)
through the C ABI against the fp64 oracle: paged and packed layouts, bf16
and fp16, every allowed window / stride / page size, untouched slots, and
device errors for bad slots and block tables.

Every case prints its name before it touches the GPU.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import nsa_oracle as N

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


def _check(case, w):
    kw = dict(cbs=w["cbs"], stride=w["stride"], page_block_size=w["page"], dtype=w["dtype"])
    args = (w["input"], w["weight"], w["slot_mapping"], w["act_seq_len"], w["block_table"],
            w["output_cache"])
    exact, new, written = N.nsa_compress(*args, **kw)
    mag = N.nsa_compress(*args, absolute=True, **kw)[0]
    got = case.out_bits()
    written_slots = {s for _, s in written}
    # slots no batch writes are untouched, bit for bit
    for s in range(w["result_len"]):
        if s not in written_slots:
            assert np.array_equal(got[s], w["output_cache"][s]), s
    # written slots: the method sums in fp32 ([NSA] kernel notes) and rounds
    # once: within one output ulp of the exact sum plus the fp32 summation
    # bound cbs * 2^-24 * sum |token * weight|
    for s in written_slots:
        g = N.decode_dtype(got[s], w["dtype"])
        o = N.decode_dtype(new[s], w["dtype"])
        ulp = np.abs(N.decode_dtype(new[s] + np.uint16(1), w["dtype"]) - o)
        bound = ulp + w["cbs"] * 2.0 ** -24 * mag[s]
        assert np.all(np.abs(g - exact[s]) <= bound), (s, float(np.max(np.abs(g - exact[s]) / bound)))
        assert np.mean(g == o) > 0.99
    assert case.device_error() == 0
    return len(written_slots)


CASES = [
    # (head_num, head_dim, cbs, stride, page, dtype, layout)
    (32, 128, 32, 16, 128, "bf16", "paged"),
    (64, 256, 64, 64, 64, "f16", "paged"),
    (52, 16, 48, 48, 64, "bf16", "tnd"),
    (7, 64, 16, 16, 128, "f16", "tnd"),
    (3, 32, 64, 32, 128, "bf16", "paged"),
]


@pytest.mark.parametrize("case", CASES)
def test_nsa_parity(harness, case):
    N_, D, cbs, stride, page, dtype, layout = case
    _announce(f"nsa {case}")
    spec = workloads.NsaSpec("nsa_case", head_num=N_, head_dim=D, cbs=cbs, stride=stride,
                             page=page, dtype=dtype, layout=layout, batch=24,
                             max_len=3 * page, fire_fraction=0.6)
    w = workloads.build_nsa(spec, workloads.SEED_BASE + 500 + N_ + D + cbs)
    c = harness.NsaCase(w)
    c.run()
    n = _check(c, w)
    assert n > 0


def test_nsa_decode_config(harness):
    _announce("nsa_decode (the benchmark configuration)")
    w = workloads.build_nsa(workloads.NSA_DECODE, workloads.SEED_BASE + 560)
    c = harness.NsaCase(w)
    c.run()
    assert _check(c, w) == w["batch"]


def test_nsa_device_errors(harness):
    _announce("nsa device errors")
    spec = workloads.NsaSpec("nsa_err", head_num=4, head_dim=32, cbs=32, stride=16, page=64,
                             dtype="bf16", layout="paged", batch=6, max_len=100,
                             fire_fraction=1.0)
    w = workloads.build_nsa(spec, workloads.SEED_BASE + 570)
    # batch 0 writes past the cache, batch 1 reads a block that does not exist
    slots = w["slot_mapping"].copy()
    slots[0] = w["result_len"] + 5
    table = w["block_table"].copy()
    table[1, :] = w["input"].shape[0] + 9
    w2 = dict(w, slot_mapping=slots, block_table=table)
    c = harness.NsaCase(w2)
    c.run()
    got = c.out_bits()
    import long_context_kv_wkv_amd as cmp
    err = c.device_error()
    assert err & cmp.NSA_DEVERR_SLOT and err & cmp.NSA_DEVERR_TABLE
    # the other batches match the oracle of the unmodified call, and the two
    # bad batches wrote nothing
    ref = N.nsa_compress(w["input"], w["weight"], w["slot_mapping"], w["act_seq_len"],
                         w["block_table"], w["output_cache"], cbs=32, stride=16,
                         page_block_size=64, dtype="bf16")[1]
    good = range(2, 6)
    for b in good:
        s = int(slots[b])
        o = N.decode_dtype(ref[s], "bf16")
        assert np.abs(N.decode_dtype(got[s], "bf16") - o).max() <= np.abs(o).max() * 2 ** -7
    untouched = set(range(w["result_len"])) - {int(slots[b]) for b in good}
    for s in untouched:
        assert np.array_equal(got[s], w["output_cache"][s])
