"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

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


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def harness():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_harness
    return gpu_harness


def _run_prefill(harness, w, rows=None, project_all=True):
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    res = O.compressor(w, windows=rows, project_all=project_all)
    return case, res


SMALL = ["c4li_small", "c128a_8192", "c128a_8269", "p1_comp_128", "p1_comp_4", "p1_comp_indexer"]


@pytest.mark.parametrize("name", SMALL)
def test_prefill_config(harness, name, tile_rows):
    _announce(f"{name} tile rows {tile_rows}")
    w = workloads.build_named(name)
    case, res = _run_prefill(harness, w)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    print(f"{name}: max scaled err {mx:.2e}, MAE {mae:.2e}")


@pytest.mark.parametrize("name", ["decode_c4a", "decode_c128a", "decode_c4a_all",
                                  "decode_c128a_all"])
def test_decode_config(harness, name):
    _announce(name)
    w = workloads.build_named(name)
    case = harness.DeviceCase(w)
    case.decode()
    torch.cuda.synchronize()
    res = O.compressor(w)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    nwin = int(res.plan.nwin.sum())
    print(f"{name}: {nwin} windows, max scaled err {mx:.2e}, MAE {mae:.2e}")
    if name.endswith("_all"):
        assert nwin == w["batch"]


def _varlen_small(seed_name, max_len, pad=0, rotate=True, B=8):
    spec = dataclasses.replace(workloads.VARLEN_C4A, name=seed_name,
                               lengths=("uniform", 1, max_len), pad_rows=pad, batch=B,
                               rotate=rotate)
    return workloads.build(spec, workloads.SEED_BASE + 40 + max_len + pad)


@pytest.mark.parametrize("max_len,pad", [(700, 0), (513, 5)])
def test_varlen_reduced(harness, max_len, pad, tile_rows):
    _announce(f"varlen max_len={max_len} pad={pad} tile rows {tile_rows}")
    w = _varlen_small("varlen_small", max_len, pad)
    case, res = _run_prefill(harness, w)
    assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0


@pytest.mark.parametrize("D", [512, 128])
@pytest.mark.parametrize("kind", ["random", "one_entry_flipped", "sylvester_times_minus_2"])
def test_prefill_hadamard_matrix_kinds(harness, kind, D):
    """The rotation matrix is an input: a scaled Sylvester matrix (any sign
    or scale) takes the in-register transform, anything else the matrix
    product; both against the oracle's plain product with the same matrix."""
    _announce(f"prefill with a {kind} rotation matrix, D={D}")
    if D == 512:
        w = _varlen_small(f"varlen_had_{kind}", 300, rotate=True, B=3)
    else:
        # the indexer shape (D = 128) from position 2: every request closes a window
        spec = dataclasses.replace(workloads.P1_COMP_INDEXER, name=f"indexer_had_{kind}",
                                   start_pos=(2,))
        w = workloads.build(spec, workloads.SEED_BASE + 93)
    assert w["head_dim"] == D
    D = w["head_dim"]
    syl = workloads.bf16_bits_to_f32(w["hadamard"])
    if kind == "random":
        rng = np.random.default_rng(workloads.SEED_BASE + 91)
        m = (rng.standard_normal((D, D)) / np.sqrt(D)).astype(np.float32)
    elif kind == "one_entry_flipped":
        m = syl.copy()
        m[D // 2 + 3, 5] = -m[D // 2 + 3, 5]
    else:
        m = syl * np.float32(-2.0)
    w = dict(w, hadamard=workloads.f32_to_bf16_bits(m))
    case, res = _run_prefill(harness, w)
    assert_out(case.out_bits(), res)
    assert case.device_error() == 0


def test_varlen_mid_size(harness, tile_rows):
    """About 20K packed tokens (8 requests): enough tiles that each XCD's
    run has a fixed part (every workgroup's first two tiles) and a queued
    part, at either tile height."""
    _announce(f"varlen mid size, tile rows {tile_rows}")
    w = _varlen_small("varlen_mid", 5000, pad=3)
    assert w["T"] > 12000
    case, res = _run_prefill(harness, w)
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    print(f"varlen mid T={w['T']} tile rows {tile_rows}: max scaled err {mx:.2e}, MAE {mae:.2e}")


# oracle results of the full-size workloads, computed once for both tile heights
_FULL = {}


def _full_oracle(name):
    if name not in _FULL:
        w = workloads.build_named(name)
        _FULL[name] = (w, O.compressor(w))
    return _FULL[name]


@pytest.mark.parametrize("name", ["varlen_c4a", "c4a_128k"])
def test_full_size_every_row(harness, name, tile_rows):
    """Every output row (windows and the exact +0 rows) and every state slot
    of the full-size packed variable-length prefill (8 requests, 88826
    tokens, H = 4096, resuming partial windows) and of the 128K-token C4A
    prefill (H = 7168, Hadamard) against the oracle; a second call on the
    same inputs is bit-identical."""
    _announce(f"{name} full size, every row, tile rows {tile_rows}")
    w, res = _full_oracle(name)
    case = harness.DeviceCase(w)
    case.prefill()
    torch.cuda.synchronize()
    mx, mae = assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)
    assert case.device_error() == 0
    # the GEMM hands most tiles out through per-XCD queues, so which CU runs
    # a tile changes from call to call; the results must not
    first = case.out_bits().copy()
    kv, sc = kv.copy(), sc.copy()
    case.reset_state()
    case.out.view(torch.int16).fill_(-1)          # every row must be written again
    case.prefill()
    torch.cuda.synchronize()
    assert np.array_equal(first, case.out_bits())
    kv2, sc2 = case.states()
    assert np.array_equal(kv.view(np.uint32), kv2.view(np.uint32))
    assert np.array_equal(sc.view(np.uint32), sc2.view(np.uint32))
    nwin = len(res.window_rows)
    print(f"{name} tile rows {tile_rows}: {nwin} windows of {w['out_rows']} rows, "
          f"max scaled err {mx:.2e}, MAE {mae:.2e}")
    del case
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------
def test_empty_and_zero_length_requests(harness):
    _announce("zero-length requests")
    w = _varlen_small("varlen_zero", 60, rotate=False, B=5)
    # requests 1 and 3 carry no token this call
    n = np.diff(w["cu_seqlens"]).astype(np.int64)
    n[1] = 0
    n[3] = 0
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    rows = np.concatenate([np.arange(w["cu_seqlens"][b], w["cu_seqlens"][b] + n[b])
                           for b in range(5)]).astype(np.int64)
    w = dict(w, x=w["x"][rows], T=int(cu[-1]), cu_seqlens=cu)
    case, res = _run_prefill(harness, w)
    assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)


def test_no_tokens_only_zero_fill(harness):
    _announce("T == 0")
    w = _varlen_small("varlen_t0", 10, rotate=False, B=2)
    w = dict(w, x=np.zeros((0, w["hidden"]), np.uint16), T=0,
             cu_seqlens=np.zeros(3, np.int32), out_rows=3,
             cos=w["cos"][:3], sin=w["sin"][:3])
    case = harness.DeviceCase(w)
    case.out.fill_(1.0)
    case.prefill()
    torch.cuda.synchronize()
    assert np.all(case.out_bits() == 0)
    kv, sc = case.states()
    assert np.array_equal(kv, w["kv_state"]) and np.array_equal(sc, w["score_state"])


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_no_tokens_no_output_rows(harness, mode):
    """Every request empty and out_rows = 0: out, sin and cos are then NULL
    (empty tensors) and the call succeeds, sets no error bit and changes no
    state row."""
    _announce(f"T == 0, out_rows == 0 ({mode})")
    w = _varlen_small("varlen_t0r0", 10, rotate=False, B=2)
    w = dict(w, x=np.zeros((0, w["hidden"]), np.uint16), T=0,
             cu_seqlens=np.zeros(3, np.int32), out_rows=0,
             cos=w["cos"][:0], sin=w["sin"][:0])
    case = harness.DeviceCase(w)
    if mode == "prefill":
        case.prefill()
    else:
        case.decode(cu_seqlens=case.cu_seqlens)
    torch.cuda.synchronize()
    assert case.device_error() == 0
    kv, sc = case.states()
    assert np.array_equal(kv, w["kv_state"]) and np.array_equal(sc, w["score_state"])


def test_block_size_one_and_trailing_rows(harness):
    _announce("block_size 1, extra out rows")
    spec = dataclasses.replace(workloads.VARLEN_C4A, name="bs1", block_size=1, batch=3,
                               lengths=("uniform", 1, 90), rotate=False)
    w = workloads.build(spec, 777)
    w = dict(w, out_rows=w["out_rows"] + 5)
    w["cos"], w["sin"] = workloads.rope_tables(np.arange(w["out_rows"]))
    case, res = _run_prefill(harness, w)
    assert_out(case.out_bits(), res)
    kv, sc = case.states()
    assert_states(kv, sc, w, res)


def test_device_error_flags_without_fault(harness):
    _announce("device error flags")
    w = _varlen_small("varlen_err", 50, rotate=False, B=3)
    bad = w["state_block_table"].copy()
    bad[1, 0] = w["num_blocks"] + 7          # out of range
    case = harness.DeviceCase(dict(w, state_block_table=bad))
    case.prefill()
    code = case.device_error()
    assert code & 1, code
    sp = w["start_pos"].copy()
    sp[2] = -5
    case2 = harness.DeviceCase(dict(w, start_pos=sp))
    case2.prefill()
    assert case2.device_error() & 2
    # a clean call on the same workspace clears the word
    case2.start_pos.copy_(torch.from_numpy(w["start_pos"]).to(case2.dev))
    case2.prefill()
    assert case2.device_error() == 0


@pytest.mark.parametrize("name", ["decode_c4a_all", "decode_c128a_all"])
def test_decode_device_errors_leave_other_requests(harness, name):
    """Single-token decode where every request closes a window: request 3's
    ring blocks are out of range in the table (its window's ring slots and
    its token's slot) and request 5 has a negative start position.  The call
    sets the table and start-position bits without a fault; every other
    request's output row and every other ring block equal those of the clean
    call bit for bit (request 5 is inactive, so the rows after it, and their
    rotary rows, move up by one)."""
    _announce(f"{name}: device errors in the pre-pooled windows")
    w = workloads.build_named(name)
    clean = harness.DeviceCase(w)
    clean.decode()
    torch.cuda.synchronize()
    assert clean.device_error() == 0
    tab = w["state_block_table"].copy()
    tab[3, :] = w["num_blocks"] + 5
    sp = w["start_pos"].copy()
    sp[5] = -1
    # rows after the inactive request move up by one: their rotary rows move
    # with them, so that the rows stay bit-identical
    cos, sin = w["cos"].copy(), w["sin"].copy()
    cos[5:-1], sin[5:-1] = w["cos"][6:], w["sin"][6:]
    bad = harness.DeviceCase(dict(w, state_block_table=tab, start_pos=sp, cos=cos, sin=sin))
    bad.decode()
    torch.cuda.synchronize()
    code = bad.device_error()
    assert code & 1 and code & 2, code
    a, b = clean.out_bits(), bad.out_bits()
    B = w["batch"]
    for r in range(B):
        if r in (3, 5):
            continue
        rb = r if r < 5 else r - 1
        assert np.array_equal(a[r], b[rb]), r
    assert np.all(b[B - 1:] == 0)                # the inactive request's row is not used
    ka, sa = clean.states()
    kb, sb = bad.states()
    keep = np.ones(w["num_blocks"], bool)
    keep[w["state_block_table"][[3, 5]].ravel()] = False
    assert np.array_equal(ka[keep].view(np.uint32), kb[keep].view(np.uint32))
    assert np.array_equal(sa[keep].view(np.uint32), sb[keep].view(np.uint32))
    # request 3's blocks: nothing was written through the bad entries
    k0, s0 = w["kv_state"], w["score_state"]
    for blk in w["state_block_table"][3]:
        assert np.array_equal(kb[blk].view(np.uint32), k0[blk].view(np.uint32))
        assert np.array_equal(sb[blk].view(np.uint32), s0[blk].view(np.uint32))


def test_host_side_errors(harness):
    _announce("host-side argument errors")
    import long_context_kv_wkv_amd as cmp
    w = workloads.build_named("c4li_small")
    case = harness.DeviceCase(w)
    small = torch.empty(16, dtype=torch.uint8, device=case.dev)
    with pytest.raises(cmp.CompressorError) as ei:
        case.prefill(workspace=small)
    assert ei.value.status == 4
    with pytest.raises(cmp.CompressorError) as ei:
        case.decode()                 # no cu_seqlens needs one row per request
    assert ei.value.status == 2
    # more than 64 packed rows is beyond the decode entry point
    spec = dataclasses.replace(workloads.C4LI_SMALL, name="decode_rows", batch=2, lengths=(40, 40),
                               tables="perm", spare_blocks=2, out_rows=20)
    big = harness.DeviceCase(workloads.build(spec, workloads.SEED_BASE + 77))
    with pytest.raises(cmp.CompressorError) as ei:
        big.decode(cu_seqlens=big.cu_seqlens)
    assert ei.value.status == 3


# --------------------------------------------------------------------------
# invariants on the GPU
# --------------------------------------------------------------------------
def test_determinism_bitwise(harness):
    _announce("determinism")
    w = _varlen_small("varlen_det", 400)
    case = harness.DeviceCase(w)
    case.prefill()
    a = case.out_bits().copy()
    ka, sa = case.states()
    case.reset_state()
    case.prefill()
    assert np.array_equal(a, case.out_bits())
    kb, sb = case.states()
    assert np.array_equal(ka.view(np.uint32), kb.view(np.uint32))
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    wd = workloads.build_named("decode_c4a_all")
    d = harness.DeviceCase(wd)
    d.decode()
    a = d.out_bits().copy()
    d.reset_state()
    d.decode()
    assert np.array_equal(a, d.out_bits())


@pytest.mark.parametrize("name,exact", [("c128a_8269", True), ("varlen_c4a", False)])
def test_tile_heights_agree(harness, name, exact):
    """The same call with 128-row and 256-row projection tiles.  The state
    rows come straight from the accumulators, whose K order does not depend
    on the tile height: bit-identical.  At ratio 128 every window lies in
    one tile at either height and is pooled by the same code: outputs
    bit-identical.  At ratio 4 the windows split between two tiles differ
    with the height (merged by the post kernel instead of in the epilogue):
    outputs within the output tolerance of each other."""
    import long_context_kv_wkv_amd as cmp
    _announce(f"tile heights agree: {name}")
    got = []
    for rows in (128, 256):
        cmp.compressor_set_prefill_tile_rows(rows)
        try:
            case = harness.DeviceCase(workloads.build_named(name))
            case.prefill()
            torch.cuda.synchronize()
            assert case.device_error() == 0
            got.append((case.out_bits().copy(), case.states()))
        finally:
            cmp.compressor_set_prefill_tile_rows(0)
    (o1, (k1, s1)), (o2, (k2, s2)) = got
    assert np.array_equal(k1.view(np.uint32), k2.view(np.uint32))
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    if exact:
        assert np.array_equal(o1, o2)
    else:
        a, g = O.bf16_to_f64(o1), O.bf16_to_f64(o2)
        rms = np.sqrt(np.mean(a * a, axis=1, keepdims=True))
        worst = float(np.max(np.abs(a - g) / np.maximum(np.maximum(np.abs(a), rms), 1e-30)))
        print(f"{name}: {int((o1 != o2).any(axis=1).sum())} rows differ, max scaled {worst:.2e}")
        assert worst <= 2e-2, worst


@pytest.mark.parametrize("rotate", [True, False])
def test_prefill_equals_token_by_token_decode(harness, rotate):
    """Config-4 style: packed varlen prefill vs the same tokens fed one per
    request per call through the decode entry point, state carried over."""
    _announce(f"prefill vs token-by-token decode, rotate={rotate}")
    w = _varlen_small(f"varlen_dec_{int(rotate)}", 40, rotate=rotate, B=6)
    case = harness.DeviceCase(w)
    case.prefill()
    res = O.compressor(w)
    full = {(b, wi): case.out_bits()[row] for b, wi, row in res.window_rows}
    plan = res.plan
    B, r = w["batch"], 4
    # decode loop
    d = harness.DeviceCase(dict(w, x=w["x"][:B], T=B, out_rows=B, cos=w["cos"][:B],
                                sin=w["sin"][:B], seqused=None))
    n = plan.ntok
    got = {}
    for t in range(int(n.max())):
        active = (n > t).astype(np.int32)
        rows = np.array([plan.row0[b] + min(t, max(n[b] - 1, 0)) for b in range(B)])
        pos = (plan.start + t).astype(np.int32)
        d.x.copy_(torch.from_numpy(w["x"][rows].view(np.int16)).to(d.dev).view(torch.bfloat16))
        # rope rows: decode row o_b carries the prefill row of the same window
        cos = np.zeros((B, 64), np.uint16)
        sin = np.zeros((B, 64), np.uint16)
        o = np.cumsum(active) - active
        for b in range(B):
            if active[b] and (pos[b] + 1) % r == 0:
                k = (pos[b] + 1) // r - 1 - plan.start[b] // r
                cos[o[b]] = w["cos"][plan.out0[b] + k]
                sin[o[b]] = w["sin"][plan.out0[b] + k]
        d.cos.copy_(torch.from_numpy(cos.view(np.int16)).to(d.dev).view(torch.bfloat16))
        d.sin.copy_(torch.from_numpy(sin.view(np.int16)).to(d.dev).view(torch.bfloat16))
        sp = torch.from_numpy(pos).to(d.dev)
        su = torch.from_numpy(active).to(d.dev)
        d.decode(start_pos=sp, seqused=su)
        bits = d.out_bits()
        for b in range(B):
            if active[b] and (pos[b] + 1) % r == 0:
                got[(b, (pos[b] + 1) // r - 1)] = bits[o[b]].copy()
            elif active[b]:
                assert np.all(bits[o[b]] == 0)
        assert d.device_error() == 0
    assert set(got) == set(full)
    worst = 0.0
    for key in full:
        a = O.bf16_to_f64(full[key])
        b_ = O.bf16_to_f64(got[key])
        rms = np.sqrt(np.mean(a * a))
        worst = max(worst, float(np.max(np.abs(a - b_) / np.maximum(np.abs(a), rms))))
    assert worst <= 2e-2, worst
    # live state rows agree
    kvp, scp = case.states()
    kvd, scd = d.states()
    for b in range(B):
        for p in O.live_positions(0, int(plan.end[b]), r, 2):
            if p < 0:
                continue
            q = p % 8
            kb = w["kv_block_table"][b, q // w["block_size"]]
            sb = w["state_block_table"][b, q // w["block_size"]]
            off = q % w["block_size"]
            assert np.allclose(kvp[kb, off], kvd[kb, off], rtol=1e-3, atol=1e-3)
            assert np.allclose(scp[sb, off], scd[sb, off], rtol=1e-3, atol=1e-3)


# --------------------------------------------------------------------------
# HIP graph capture: no host sync, allocation or memset inside a call, so a
# captured call replays to the eager result.  Every replay is checked, with
# eager work and synchronisation between replays.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,entry", [("decode_c4a_all", "decode"),
                                        ("decode_c128a_all", "decode"),
                                        ("c4li_small", "prefill")])
def test_graph_replay_matches_eager(harness, name, entry):
    _announce(f"graph replay {name} {entry}")
    w = workloads.build_named(name)
    case = harness.DeviceCase(w)
    call = getattr(case, entry)
    call()
    torch.cuda.synchronize()
    ref_out = case.out_bits().copy()
    ref_kv, ref_sc = case.states()
    case.reset_state()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                    # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        case.reset_state()                        # eager work between replays
        case.out.fill_(0x7F7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(case.out_bits(), ref_out), f"replay {rep}: output differs"
        kv, sc = case.states()
        assert np.array_equal(kv.view(np.uint32), ref_kv.view(np.uint32)), f"replay {rep}: kv"
        assert np.array_equal(sc.view(np.uint32), ref_sc.view(np.uint32)), f"replay {rep}: score"
    assert case.device_error() == 0
