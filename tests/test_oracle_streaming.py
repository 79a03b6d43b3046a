"""Invariants of the oracle's state handling (streaming, paging, batch order).

* one prefill == the same tokens cut at random points and streamed through
  repeated calls with the state carried over == one token per call;
* permuting the physical blocks (tables and pool contents together) changes
  nothing;
* reordering the requests of a batch permutes the output rows accordingly.
"""
import numpy as np
import pytest

import workloads
from oracle import compressor_oracle as O
from test_oracle_pins import small_random


def window_outputs(w, res):
    """{(b, window): fp64 output row} of one call."""
    return {(b, wi): res.out[row] for b, wi, row in res.window_rows}


def live_rows(w, res, ends):
    """{(b, position): (kv, score)} of every live position after a call that
    ended request b at position ends[b]."""
    r, coff, bs = w["ratio"], w["coff"], w["block_size"]
    st = w["state_block_table"]
    kvt = st if w["kv_block_table"] is None else w["kv_block_table"]
    out = {}
    for b, e in enumerate(ends):
        for p in O.live_positions(0, int(e), r, coff):
            if p < 0:
                continue
            q = O.ring_slot(p, r, coff)
            kb, ko = O.state_location(kvt, b, q, bs)
            sb, so = O.state_location(st, b, q, bs)
            out[(b, p)] = (res.kv_state[kb, ko].copy(), res.score_state[sb, so].copy())
    return out


def run_split(w, chunks):
    """Feed request b's tokens in pieces chunks[b] (lists of lengths) through
    successive calls, carrying the pools.  Returns window outputs and the last
    result.  Each call's rope rows carry the angles of the full call's row for
    the same window."""
    r, B = w["ratio"], w["batch"]
    full_plan = O.make_plan(r, B, w["T"], w["cu_seqlens"], w["seqused"], w["start_pos"])
    ncalls = max(len(c) for c in chunks)
    s0 = full_plan.start.copy()
    offs = np.zeros(B, np.int64)                  # tokens consumed so far
    kv_state, score_state = w["kv_state"], w["score_state"]
    outs = {}
    cos_full, sin_full = w["cos"], w["sin"]
    res = None
    for call in range(ncalls):
        n = np.array([c[call] if call < len(c) else 0 for c in chunks], np.int64)
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        rows = np.concatenate([full_plan.row0[b] + offs[b] + np.arange(n[b]) for b in range(B)]
                              ).astype(np.int64)
        T = int(cu[-1])
        start = (s0 + offs).astype(np.int32)
        out_rows = max(1, min(T, T // r + B))
        plan = O.make_plan(r, B, T, cu, None, start)
        cos = np.zeros((out_rows, cos_full.shape[1]), np.uint16)
        sin = np.zeros_like(cos)
        for b in range(B):
            for k in range(int(plan.nwin[b])):
                wi = int(plan.start[b] // r) + k
                kfull = wi - int(full_plan.start[b] // r)
                cos[plan.out0[b] + k] = cos_full[full_plan.out0[b] + kfull]
                sin[plan.out0[b] + k] = sin_full[full_plan.out0[b] + kfull]
        wc = dict(w, x=w["x"][rows] if T else np.zeros((0, w["hidden"]), np.uint16),
                  T=T, cu_seqlens=cu, seqused=None, start_pos=start,
                  kv_state=kv_state, score_state=score_state, out_rows=out_rows,
                  cos=cos, sin=sin)
        res = O.compressor(wc)
        outs.update(window_outputs(wc, res))
        kv_state, score_state = res.kv_state, res.score_state
        offs += n
    return outs, res


def random_chunks(rng, n, max_pieces):
    if n == 0:
        return [0]
    k = int(rng.integers(1, max_pieces + 1))
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(k - 1, n - 1), replace=False)) if n > 1 else []
    edges = np.concatenate([[0], cuts, [n]]).astype(int)
    return list(np.diff(edges))


@pytest.mark.parametrize("ratio", [4, 128, 8, 2])
def test_prefill_equals_random_splits_and_token_by_token(ratio):
    rng = np.random.default_rng(100 + ratio)
    lengths = (int(rng.integers(1, 3 * ratio)), int(rng.integers(1, 3 * ratio)), 3)
    w = small_random(ratio, D=64, H=48, lengths=lengths,
                     start_pos=[int(v) for v in rng.integers(0, 2 * ratio, 3)],
                     seed=ratio, bs=4, rotate=False, perm=True)
    full = O.compressor(w)
    ref = window_outputs(w, full)
    ends = full.plan.end
    ref_live = live_rows(w, full, ends)
    for mode in ("random", "tokens"):
        if mode == "random":
            chunks = [random_chunks(rng, n, 4) for n in lengths]
        else:
            chunks = [[1] * n for n in lengths]
        outs, last = run_split(w, chunks)
        assert set(outs) == set(ref)
        for key in ref:
            # the split path passes rows through fp32 state; allow that rounding
            assert np.allclose(outs[key], ref[key], rtol=2e-6, atol=2e-6), (mode, key)
        live = live_rows(w, last, ends)
        assert set(live) == set(ref_live)
        for key in ref_live:
            assert np.array_equal(live[key][0], ref_live[key][0])
            assert np.array_equal(live[key][1], ref_live[key][1])


def test_block_permutation_invariance():
    w = small_random(4, D=64, H=32, lengths=(13, 7), start_pos=[5, 2], seed=7, bs=2, perm=False)
    base = O.compressor(w)
    nb = w["kv_state"].shape[0]
    pi = np.random.default_rng(8).permutation(nb)
    w2 = dict(w)
    w2["state_block_table"] = pi[w["state_block_table"]].astype(np.int32)
    kvt = w["state_block_table"] if w["kv_block_table"] is None else w["kv_block_table"]
    w2["kv_block_table"] = pi[kvt].astype(np.int32)
    kv2 = np.empty_like(w["kv_state"])
    sc2 = np.empty_like(w["score_state"])
    kv2[pi] = w["kv_state"]
    sc2[pi] = w["score_state"]
    w2["kv_state"], w2["score_state"] = kv2, sc2
    res = O.compressor(w2)
    assert np.array_equal(res.out, base.out)
    assert np.array_equal(res.kv_state[pi], base.kv_state)
    assert np.array_equal(res.score_state[pi], base.score_state)
    assert np.array_equal(res.kv_written[pi], base.kv_written)


def test_batch_reorder_permutes_rows():
    w = small_random(4, D=64, H=32, lengths=(9, 14, 6), start_pos=[3, 0, 6], seed=9, bs=8,
                     perm=True)
    base = O.compressor(w)
    order = [2, 0, 1]
    B = 3
    cu = w["cu_seqlens"]
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order])
    n = np.array([cu[b + 1] - cu[b] for b in order])
    w2 = dict(w, x=w["x"][rows], cu_seqlens=np.concatenate([[0], np.cumsum(n)]).astype(np.int32),
              start_pos=w["start_pos"][order],
              state_block_table=w["state_block_table"][order],
              kv_block_table=w["kv_block_table"][order])
    # rope rows follow their windows
    p1 = base.plan
    p2 = O.make_plan(4, B, w["T"], w2["cu_seqlens"], None, w2["start_pos"])
    cos, sin = np.zeros_like(w["cos"]), np.zeros_like(w["sin"])
    for nb_, b in enumerate(order):
        for k in range(int(p1.nrows[b])):
            cos[p2.out0[nb_] + k] = w["cos"][p1.out0[b] + k]
            sin[p2.out0[nb_] + k] = w["sin"][p1.out0[b] + k]
    w2["cos"], w2["sin"] = cos, sin
    res = O.compressor(w2)
    for nb_, b in enumerate(order):
        u = int(p1.nrows[b])
        assert np.array_equal(res.out[p2.out0[nb_]:p2.out0[nb_] + u],
                              base.out[p1.out0[b]:p1.out0[b] + u])
    assert np.array_equal(res.kv_state, base.kv_state)
    assert np.array_equal(res.score_state, base.score_state)


def test_padding_rows_and_seqused_are_ignored():
    """Rows after seqused inside a cu_seqlens slot never influence anything."""
    w = small_random(4, D=64, H=32, lengths=(11, 6), start_pos=[1, 3], seed=12, bs=8, pad=3)
    base = O.compressor(w)
    w2 = dict(w)
    x2 = w["x"].copy()
    cu = w["cu_seqlens"]
    for b in range(2):
        x2[cu[b] + w["seqused"][b]:cu[b + 1]] = workloads.f32_to_bf16_bits(
            np.full((cu[b + 1] - cu[b] - w["seqused"][b], w["hidden"]), 1e4, np.float32))
    w2["x"] = x2
    res = O.compressor(w2)
    assert np.array_equal(res.out, base.out)
    assert np.array_equal(res.kv_state, base.kv_state)


def test_stale_pool_rows_are_not_read_for_window_zero():
    """Window 0 of C4A pads its a set by position; whatever the ring holds
    there is ignored."""
    w = small_random(4, D=64, H=32, lengths=(10,), start_pos=[0], seed=13, bs=8)
    base = O.compressor(w)
    w2 = dict(w, kv_state=w["kv_state"] * 0 + 1e6, score_state=w["score_state"] * 0 + 50.0)
    res = O.compressor(w2)
    assert np.array_equal(res.out, base.out)


def test_written_mask_matches_closed_form_intervals():
    w = small_random(4, D=64, H=32, lengths=(13, 2, 5), start_pos=[2, 3, 8], seed=14, bs=2,
                     perm=True)
    res = O.compressor(w)
    expect = np.zeros_like(res.score_written)
    for b, (s, n) in enumerate(zip(w["start_pos"], (13, 2, 5))):
        e = int(s) + n
        lo = max(int(s), 4 * (e // 4) - 4)
        for p in range(lo, e):
            q = p % 8
            expect[w["state_block_table"][b, q // 2], q % 2] = True
    assert np.array_equal(res.score_written, expect)
