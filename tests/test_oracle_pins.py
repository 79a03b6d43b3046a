"""Pins of the fp64 oracle against things other than itself.

Each test checks an oracle function against a closed form worked by hand, a
textbook or library routine, an identity of the mathematics, or the rule the
pages print.  A plausible slip in the oracle (a dropped term, a wrong sign,
an off-by-one window, swapped channel sets) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import compressor_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers: hand-built inputs with controlled values
# --------------------------------------------------------------------------
def bf(a):
    return workloads.f32_to_bf16_bits(np.asarray(a, np.float32))


def make_inputs(*, ratio, D, H, x, wkv, wgate, ape, gamma=None, lengths, start_pos=None,
                block_size=None, cos=None, sin=None, had=None, out_rows=None,
                kv_state=None, score_state=None, tables=None, kv_tables=None, seqused=None,
                cu=None):
    coff = O.coff_of(ratio)
    B = len(lengths)
    if cu is None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    bs = block_size or coff * ratio
    stride = -(-coff * ratio // bs)
    if tables is None:
        tables = np.arange(B * stride, dtype=np.int32).reshape(B, stride)
    nb = int(max(np.max(tables), -1 if kv_tables is None else np.max(kv_tables))) + 1
    if kv_state is None:
        kv_state = np.zeros((nb, bs, coff * D), np.float32)
        score_state = np.full((nb, bs, coff * D), -np.inf, np.float32)
    if out_rows is None:
        out_rows = min(T, T // ratio + B)
    if cos is None:
        cos = np.ones((out_rows, 64), np.float32)
        sin = np.zeros((out_rows, 64), np.float32)
    return dict(ratio=ratio, coff=coff, head_dim=D, hidden=H, rotate=had is not None, rope_dim=64,
                block_size=bs, batch=B, T=T, x=bf(x), wkv=bf(wkv), wgate=bf(wgate),
                ape=np.asarray(ape, np.float32),
                weight=bf(np.ones(D) if gamma is None else gamma),
                hadamard=None if had is None else bf(had),
                start_pos=None if start_pos is None else np.asarray(start_pos, np.int32),
                cu_seqlens=cu, seqused=seqused,
                kv_block_table=kv_tables, state_block_table=np.asarray(tables, np.int32),
                kv_state=np.asarray(kv_state, np.float32),
                score_state=np.asarray(score_state, np.float32),
                out_rows=out_rows, cos=bf(cos), sin=bf(sin),
                num_blocks=nb, table_stride=stride)


def small_random(ratio, D=128, H=96, lengths=(37,), start_pos=None, seed=0, bs=None,
                 rotate=False, pools="random", perm=False, pad=0):
    """Random small inputs drawn with workloads' generator conventions."""
    rng = np.random.default_rng(seed)
    coff = O.coff_of(ratio)
    B = len(lengths)
    slot = np.asarray(lengths) + pad
    cu = np.concatenate([[0], np.cumsum(slot)]).astype(np.int32)
    T = int(cu[-1])
    bs = bs or 8
    stride = -(-coff * ratio // bs)
    nb = B * stride + 2
    tables = (rng.permutation(nb)[:B * stride] if perm else np.arange(B * stride)).reshape(B, stride)
    kvt = (rng.permutation(nb)[:B * stride].reshape(B, stride) if perm else None)
    kv_state = rng.standard_normal((nb, bs, coff * D)).astype(np.float32)
    score_state = rng.standard_normal((nb, bs, coff * D)).astype(np.float32)
    out_rows = min(T, T // ratio + B)
    cos, sin = workloads.rope_tables(np.arange(out_rows) * 3.0 + 1.0)
    w = make_inputs(ratio=ratio, D=D, H=H, x=rng.standard_normal((T, H)),
                    wkv=rng.standard_normal((coff * D, H)) / math.sqrt(H),
                    wgate=rng.standard_normal((coff * D, H)) / math.sqrt(H),
                    ape=rng.standard_normal((ratio, coff * D)) * 0.3,
                    gamma=1 + 0.2 * rng.standard_normal(D), lengths=list(lengths),
                    start_pos=start_pos, block_size=bs,
                    cos=workloads.bf16_bits_to_f32(cos), sin=workloads.bf16_bits_to_f32(sin),
                    had=(workloads.bf16_bits_to_f32(workloads.sylvester_hadamard_bf16(D))
                         if rotate else None),
                    kv_state=kv_state, score_state=score_state, tables=tables, kv_tables=kvt,
                    cu=cu, seqused=(np.asarray(lengths, np.int32) if pad else None))
    return w


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------
def test_bf16_rounding_matches_bit_trick_on_f32_values():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    assert np.array_equal(O.f64_to_bf16(v.astype(np.float64)), workloads.f32_to_bf16_bits(v))


def test_bf16_rounding_ties_and_double_rounding():
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing at 1
    # exact halfway cases round to even
    assert O.f64_to_bf16(one + ulp / 2) == 0x3F80          # 1.0 (even)
    assert O.f64_to_bf16(one + 3 * ulp / 2) == 0x3F82      # 1 + 2ulp (even)
    # just above halfway by less than an fp32 ulp: fp64 must round up; a
    # double rounding through fp32 would tie and go to even (down)
    assert O.f64_to_bf16(one + ulp / 2 + 2.0 ** -40) == 0x3F81
    assert O.f64_to_bf16(-0.0) == 0x8000 and O.f64_to_bf16(0.0) == 0
    assert O.f64_to_bf16(np.inf) == 0x7F80 and O.f64_to_bf16(1e39) == 0x7F80
    # every bf16 code round-trips
    codes = np.arange(0, 0x7F80, dtype=np.uint16)
    assert np.array_equal(O.f64_to_bf16(O.bf16_to_f64(codes)), codes)


# --------------------------------------------------------------------------
# pooling: closed forms
# --------------------------------------------------------------------------
def test_pool_hand_worked_weights():
    # 8 slots, one score at ln 3, seven at 0, kv one-hot: weights 3/10, 1/10
    kv = np.eye(8)
    z = np.zeros((8, 8))
    z[0, :] = math.log(3.0)
    c = O.softmax_pool(kv, z)
    assert np.allclose(c, [0.3] + [0.1] * 7, rtol=0, atol=1e-15)
    # padded first window: four -inf slots get zero weight; 3/6 and 1/6
    z2 = np.full((8, 8), -np.inf)
    z2[4:, :] = 0.0
    z2[4, :] = math.log(3.0)
    c2 = O.softmax_pool(kv, z2)
    assert np.allclose(c2, [0, 0, 0, 0, 0.5, 1 / 6, 1 / 6, 1 / 6], rtol=0, atol=1e-15)


def test_pool_against_torch_softmax():
    rng = np.random.default_rng(2)
    kv = rng.standard_normal((128, 40))
    z = rng.standard_normal((128, 40)) * 4
    ref = (torch.softmax(torch.from_numpy(z), dim=0) * torch.from_numpy(kv)).sum(0).numpy()
    assert np.allclose(O.softmax_pool(kv, z), ref, rtol=1e-13, atol=1e-14)


def test_pool_saturation_and_shift():
    rng = np.random.default_rng(3)
    kv = rng.standard_normal((8, 16))
    z = rng.standard_normal((8, 16))
    z_sat = z.copy()
    z_sat[5] += 80.0
    assert np.allclose(O.softmax_pool(kv, z_sat), kv[5], rtol=0, atol=1e-25 + 1e-30)
    shift = rng.standard_normal(16) * 50
    assert np.allclose(O.softmax_pool(kv, z + shift), O.softmax_pool(kv, z), rtol=1e-13)


# --------------------------------------------------------------------------
# full pipeline, hand-worked C4A example
# --------------------------------------------------------------------------
def test_c4a_pipeline_hand_worked():
    """8 tokens, ratio 4: x one-hot, Wkv puts token p on channel p of both
    channel sets, Wgate = 0 and Ape sets one a-set score to ln 3.

    window 0: a set padded (-inf), b set = tokens 0..3 with equal scores
              -> C = (e0+e1+e2+e3)/4
    window 1: a set = tokens 0..3 with scores (ln 3, 0, 0, 0), b set = tokens
              4..7 with score 0 -> weights 3/10 (token 0) and 1/10 (others)
    """
    D, H, r = 128, 8, 4
    x = np.eye(8)
    wkv = np.zeros((2 * D, H))
    for p in range(8):
        wkv[p, p] = 1.0          # a set, channel p
        wkv[D + p, p] = 1.0      # b set, channel p
    wgate = np.zeros((2 * D, H))
    ape = np.zeros((4, 2 * D), np.float32)
    ape[0, :D] = np.float32(math.log(3.0))
    w = make_inputs(ratio=r, D=D, H=H, x=x, wkv=wkv, wgate=wgate, ape=ape, lengths=[8])
    res = O.compressor(w)
    assert res.out.shape == (min(8, 8 // 4 + 1), D)
    c0 = np.zeros(D)
    c0[:4] = 0.25
    e3 = math.exp(float(np.float32(math.log(3.0))))     # ape is fp32
    c1 = np.zeros(D)
    c1[0] = e3 / (e3 + 7)
    c1[1:8] = 1 / (e3 + 7)
    for row, c in ((0, c0), (1, c1)):
        y = c / math.sqrt(np.mean(c * c) + 1e-6)
        assert np.allclose(res.out[row], y, rtol=1e-12, atol=1e-12)
        assert np.array_equal(res.out_bf16[row], O.f64_to_bf16(y))
    assert np.all(res.out[2] == 0)      # third row: no window


def test_uniform_scores_give_plain_mean():
    """Wgate = 0 and Ape = 0: each window's output is RMSNorm of the plain mean
    of its valid slots (C4A: the a half of the 4 previous rows and the b half
    of the 4 current ones; window 0 only the 4 b rows; every other ratio its
    own r rows)."""
    rng = np.random.default_rng(4)
    for ratio, T in ((4, 20), (128, 300), (2, 11), (16, 50)):
        coff = O.coff_of(ratio)
        D, H = 64, 16
        x = rng.standard_normal((T, H))
        wkv = rng.standard_normal((coff * D, H))
        w = make_inputs(ratio=ratio, D=D, H=H, x=x, wkv=wkv, wgate=np.zeros((coff * D, H)),
                        ape=np.zeros((ratio, coff * D)), lengths=[T])
        res = O.compressor(w)
        xb, wb = O.bf16_to_f64(w["x"]), O.bf16_to_f64(w["wkv"])
        # brute-force projection by explicit dot products
        kv = np.array([[sum(xb[p, h] * wb[c, h] for h in range(H)) for c in range(coff * D)]
                       for p in range(T)])
        for k in range(T // ratio):
            if coff == 1:
                c = kv[k * ratio:(k + 1) * ratio].mean(0)
            else:
                b_rows = kv[k * 4:(k + 1) * 4, D:]
                if k == 0:
                    c = b_rows.mean(0)
                else:
                    c = np.concatenate([kv[(k - 1) * 4:k * 4, :D], b_rows]).mean(0)
            y = c / math.sqrt(np.mean(c * c) + 1e-6)
            assert np.allclose(res.out[k], y, rtol=1e-10, atol=1e-12), (ratio, k)


def test_ape_rows_follow_position_and_channel_set():
    """A large Ape entry at (row j, a-set channel c) makes window w >= 1 pick
    token (w-1)*4 + j's a-set kv on channel c; at (row j, b-set channel c) it
    picks token w*4 + j's b-set kv."""
    rng = np.random.default_rng(5)
    D, H, T = 64, 8, 16
    x = rng.standard_normal((T, H))
    wkv = rng.standard_normal((2 * D, H))
    for j, cset, c in ((2, 0, 7), (1, 1, 9)):
        ape = np.zeros((4, 2 * D), np.float32)
        ape[j, cset * D + c] = 200.0
        w = make_inputs(ratio=4, D=D, H=H, x=x, wkv=wkv, wgate=np.zeros((2 * D, H)), ape=ape,
                        lengths=[T], gamma=np.ones(D))
        res = O.compressor(w)
        kv = O.bf16_to_f64(w["x"]) @ O.bf16_to_f64(w["wkv"]).T
        for k in range(1, T // 4):
            tok = (k - 1) * 4 + j if cset == 0 else k * 4 + j
            others = np.delete(np.arange(D), c)
            # channel c of the pooled vector is exactly that token's kv; to
            # compare after RMSNorm, recover the pooled vector's scale from
            # the uniform channels (plain means)
            allk = np.concatenate([kv[(k - 1) * 4:k * 4, :D], kv[k * 4:(k + 1) * 4, D:]])
            pooled = allk.mean(0)
            pooled[c] = kv[tok, cset * D + c]
            y = pooled / math.sqrt(np.mean(pooled ** 2) + 1e-6)
            assert np.allclose(res.out[k], y, rtol=1e-9, atol=1e-12), (j, cset, k)
            del others


# --------------------------------------------------------------------------
# projection, normalisation, rotation, Hadamard
# --------------------------------------------------------------------------
def test_projection_brute_force_rows():
    rng = np.random.default_rng(6)
    x = O.bf16_to_f64(bf(rng.standard_normal((5, 33))))
    wk = O.bf16_to_f64(bf(rng.standard_normal((7, 33))))
    wg = O.bf16_to_f64(bf(rng.standard_normal((7, 33))))
    kv, z = O.project(x, wk, wg)
    for i in range(5):
        for c in range(7):
            assert abs(kv[i, c] - math.fsum(x[i, h] * wk[c, h] for h in range(33))) < 1e-12
            assert abs(z[i, c] - math.fsum(x[i, h] * wg[c, h] for h in range(33))) < 1e-12
    zz = O.add_ape(z, np.array([0, 1, 2, 3, 4]), np.arange(28.).reshape(4, 7), 4)
    assert np.allclose(zz[4] - z[4], np.arange(7.0))          # position 4 -> Ape row 0
    assert np.allclose(zz[3] - z[3], np.arange(21.0, 28.0))   # position 3 -> Ape row 3


def test_rms_norm_against_torch_and_identities():
    rng = np.random.default_rng(7)
    c = rng.standard_normal((6, 512)) * 3
    g = 1 + 0.2 * rng.standard_normal(512)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(c), (512,), torch.from_numpy(g), eps=1e-6)
    assert np.allclose(O.rms_norm(c, g), ref.numpy(), rtol=1e-13, atol=1e-13)
    y = O.rms_norm(c, np.ones(512))
    rc = np.sqrt(np.mean(c * c, -1))
    assert np.allclose(np.sqrt(np.mean(y * y, -1)), rc / np.sqrt(rc ** 2 + 1e-6), rtol=1e-13)
    # scale invariance up to the epsilon term (eps / mean(c^2) ~ 1e-7 here)
    assert np.allclose(O.rms_norm(1e3 * c, g), O.rms_norm(c, g), rtol=1e-6)


def test_rope_against_complex_rotation():
    """With half-duplicated tables, the interleaved layout rotates the complex
    number t[2i] + i t[2i+1] by angle theta_i (the usual rotary embedding)."""
    rng = np.random.default_rng(8)
    t = rng.standard_normal((3, 64))
    theta = rng.uniform(-4, 4, (3, 32))
    cos = np.concatenate([np.cos(theta)] * 2, -1)
    sin = np.concatenate([np.sin(theta)] * 2, -1)
    got = O.rope_interleaved(t, cos, sin)
    z = torch.view_as_complex(torch.from_numpy(t).reshape(3, 32, 2).contiguous())
    ref = torch.view_as_real(z * torch.polar(torch.ones(3, 32, dtype=torch.float64),
                                             torch.from_numpy(theta))).reshape(3, 64).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    # identity, pair norms, and theta then -theta
    assert np.array_equal(O.rope_interleaved(t, np.ones((3, 64)), np.zeros((3, 64))), t)
    n0 = t[:, 0::2] ** 2 + t[:, 1::2] ** 2
    n1 = got[:, 0::2] ** 2 + got[:, 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)
    assert np.allclose(O.rope_interleaved(got, cos, -sin), t, rtol=1e-12, atol=1e-13)


def test_rope_uses_column_i_for_even_and_half_plus_i_for_odd():
    t = np.zeros((1, 64))
    t[0, 2 * 5] = 1.0                      # even element of pair 5
    cos = np.zeros((1, 64))
    sin = np.zeros((1, 64))
    sin[0, 32 + 5] = 2.0                   # drives the odd element of pair 5
    cos[0, 5] = 3.0                        # drives the even element of pair 5
    out = O.rope_interleaved(t, cos, sin)
    expect = np.zeros((1, 64))
    expect[0, 10] = 3.0                    # t_even * cos[i]
    expect[0, 11] = 2.0                    # t_even * sin[32+i]
    assert np.array_equal(out, expect)


def _fwht(v):
    """Textbook in-place fast Walsh-Hadamard transform (natural order)."""
    v = np.array(v, np.float64)
    h = 1
    n = v.shape[-1]
    while h < n:
        for i in range(0, n, 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v


@pytest.mark.parametrize("d", [128, 512])
def test_hadamard_against_fwht(d):
    rng = np.random.default_rng(9)
    y = rng.standard_normal((4, d))
    had = O.bf16_to_f64(workloads.sylvester_hadamard_bf16(d))
    c = had[0, 0]
    assert np.allclose(O.hadamard_rotate(y, had), c * _fwht(y), rtol=1e-13, atol=1e-12)
    assert np.allclose(had @ had, c * c * d * np.eye(d), rtol=0, atol=1e-12)
    if d == 512:
        assert c == 0.044189453125 and abs(c * c * d - 0.99979) < 1e-5


# --------------------------------------------------------------------------
# the printed rules: trigger, shapes, coff
# --------------------------------------------------------------------------
def test_plan_matches_printed_trigger_rule_and_shapes():
    spec = json.load(open(os.path.join(GOLDEN, "p1_example_cases.json")))
    for case in spec["cases"]:
        r, B, s, S = case["ratio"], case["bsz"], case["start_pos"], case["seq"]
        plan = O.make_plan(r, B, B * S, None, None, np.full(B, s))
        fires = sum(1 for i in range(S) if (s + i + 1) % r == 0)
        assert np.all(plan.nwin == fires), case["name"]
        assert O.coff_of(r) == 1 + (r == 4)
        T = B * S
        assert plan.nrows.sum() <= min(T, T // r + B)


def test_plan_random_against_trigger_rule():
    rng = np.random.default_rng(10)
    for r in (2, 4, 8, 128):
        n = rng.integers(0, 600, 50)
        s = rng.integers(0, 5000, 50)
        cu = np.concatenate([[0], np.cumsum(n)])
        plan = O.make_plan(r, 50, int(cu[-1]), cu, None, s)
        for b in range(50):
            fires = sum(1 for i in range(n[b]) if (s[b] + i + 1) % r == 0)
            assert plan.nwin[b] == fires
            assert plan.nwin[b] <= plan.nrows[b]
        T = int(cu[-1])
        assert plan.nrows.sum() <= min(T, T // r + 50)


def test_live_positions_are_exactly_the_ones_future_windows_pool():
    """A call stores a position iff some window not yet complete pools it."""
    for r in (4, 128, 8):
        coff = O.coff_of(r)
        for s in range(0, 3 * r):
            for n in range(0, 3 * r):
                e = s + n
                need = set()
                for wi in range(e // r, e // r + 3):
                    need.update(p for p, _ in O.window_slot_positions(wi, r, coff))
                expect = [p for p in range(s, e) if p in need]
                assert list(O.live_positions(s, e, r, coff)) == expect, (r, s, n)


def test_ring_slots_of_live_positions_never_collide():
    for r in (4, 128):
        coff = O.coff_of(r)
        for e in range(0, 4 * r):
            live = list(O.live_positions(0, e, r, coff))
            # plus every position a window in progress still needs from earlier calls
            qs = [O.ring_slot(p, r, coff) for p in live]
            assert len(set(qs)) == len(qs)


# --------------------------------------------------------------------------
# r = 1: linear layer plus RMSNorm (a textbook composition)
# --------------------------------------------------------------------------
def test_ratio_one_reduces_to_linear_plus_rmsnorm():
    rng = np.random.default_rng(11)
    D, H, T = 64, 40, 9
    w = make_inputs(ratio=1, D=D, H=H, x=rng.standard_normal((T, H)),
                    wkv=rng.standard_normal((D, H)), wgate=rng.standard_normal((D, H)),
                    ape=rng.standard_normal((1, D)), gamma=1 + rng.standard_normal(D) * 0.1,
                    lengths=[T])
    res = O.compressor(w)
    lin = torch.nn.functional.linear(torch.from_numpy(O.bf16_to_f64(w["x"])),
                                     torch.from_numpy(O.bf16_to_f64(w["wkv"])))
    ref = torch.nn.functional.rms_norm(lin, (D,), torch.from_numpy(O.bf16_to_f64(w["weight"])),
                                       eps=1e-6).numpy()
    assert np.allclose(res.out[:T], ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# where RoPE and the Hadamard product act, through the whole call
# --------------------------------------------------------------------------
def _uniform_windows(ratio, D, H, T, seed, **kw):
    """Inputs with Wgate = 0, Ape = 0 and weight 1, so that window k's pooled
    vector is the plain mean of its slots' kv, and the RMS-normalised means
    y_k (projection by explicit sums, pooling by plain means, RMSNorm by its
    closed form): everything the output holds before RoPE and the Hadamard
    product."""
    rng = np.random.default_rng(seed)
    coff = O.coff_of(ratio)
    w = make_inputs(ratio=ratio, D=D, H=H, x=rng.standard_normal((T, H)),
                    wkv=rng.standard_normal((coff * D, H)), wgate=np.zeros((coff * D, H)),
                    ape=np.zeros((ratio, coff * D)), lengths=[T], **kw)
    xb, wb = O.bf16_to_f64(w["x"]), O.bf16_to_f64(w["wkv"])
    kv = np.array([[math.fsum(xb[p, h] * wb[c, h] for h in range(H)) for c in range(coff * D)]
                   for p in range(T)])
    ys = []
    for k in range(T // ratio):
        if coff == 1:
            c = kv[k * ratio:(k + 1) * ratio].mean(0)
        elif k == 0:
            c = kv[0:4, D:].mean(0)
        else:
            c = np.concatenate([kv[(k - 1) * 4:k * 4, :D], kv[k * 4:(k + 1) * 4, D:]]).mean(0)
        ys.append(c / math.sqrt(np.mean(c * c) + 1e-6))
    return w, ys


@pytest.mark.parametrize("ratio", [4, 128])
def test_rope_acts_on_the_trailing_slice_only(ratio):
    """Every pair of the rotary slice turned by a quarter turn (cos 0, sin 1,
    exact in bf16): channels [0, D-64) keep their values and the trailing
    pairs (D-64+2i, D-64+2i+1) become (-odd, even) ([PyPTO]
    数值精度与验证要点: RoPE on the last rope_head_dim channels)."""
    D, H = 128, 12
    T = 3 * ratio
    rows = T // ratio + 1
    w, ys = _uniform_windows(ratio, D, H, T, 12, cos=np.zeros((rows, 64)),
                             sin=np.ones((rows, 64)), out_rows=rows)
    res = O.compressor(w)
    for k, y in enumerate(ys):
        want = y.copy()
        want[D - 64::2] = -y[D - 63::2]
        want[D - 63::2] = y[D - 64::2]
        assert np.allclose(res.out[k], want, rtol=1e-12, atol=1e-12), k
        assert np.array_equal(res.out[k][:D - 64], y[:D - 64])


def test_rope_row_angles_against_complex_rotation_in_pipeline():
    """Row-dependent angles: output row k rotates pair i of the trailing
    slice by its own angle theta[k, i] (the complex product of
    (y[D-64+2i] + j y[D-64+2i+1]) with e^{j theta}, computed by torch), and
    channels below the slice are untouched."""
    D, H, r, T = 128, 10, 4, 20
    rows = T // r + 1
    rng = np.random.default_rng(13)
    theta = rng.uniform(-3, 3, (rows, 32))
    cos = O.bf16_to_f64(bf(np.concatenate([np.cos(theta)] * 2, -1)))
    sin = O.bf16_to_f64(bf(np.concatenate([np.sin(theta)] * 2, -1)))
    w, ys = _uniform_windows(r, D, H, T, 14, cos=cos, sin=sin, out_rows=rows)
    res = O.compressor(w)
    for k, y in enumerate(ys):
        c, s = torch.from_numpy(cos[k, :32]), torch.from_numpy(sin[k, :32])
        z = torch.view_as_complex(torch.from_numpy(y[D - 64:]).reshape(32, 2).contiguous())
        rot = torch.view_as_real(z * torch.complex(c, s)).reshape(64).numpy()
        want = np.concatenate([y[:D - 64], rot])
        assert np.allclose(res.out[k], want, rtol=1e-12, atol=1e-12), k


def test_hadamard_product_orientation():
    """out = y @ Had ([PyPTO] kernel 派发逻辑), checked with matrices that are
    not symmetric: the upper triangular all-ones matrix U (y @ U is the
    running sum of y, y @ U^T the running sum from the end) and a
    permutation matrix P with P[k, perm[k]] = 1 (y @ P moves channel k to
    perm[k])."""
    rng = np.random.default_rng(15)
    y = rng.standard_normal((3, 64))
    U = np.triu(np.ones((64, 64)))
    assert np.allclose(O.hadamard_rotate(y, U), np.cumsum(y, axis=-1), rtol=1e-13, atol=1e-13)
    perm = rng.permutation(64)
    P = np.zeros((64, 64))
    P[np.arange(64), perm] = 1.0
    got = O.hadamard_rotate(y, P)
    assert np.array_equal(got[:, perm], y)


@pytest.mark.parametrize("ratio", [4, 128])
def test_hadamard_orientation_in_pipeline(ratio):
    """rotate with the upper triangular all-ones matrix (exact in bf16):
    every output row is the running sum of its normalised vector."""
    D, H = 128, 9
    T = 2 * ratio + 3
    w, ys = _uniform_windows(ratio, D, H, T, 16, had=np.triu(np.ones((D, D))))
    res = O.compressor(w)
    for k, y in enumerate(ys):
        assert np.allclose(res.out[k], np.cumsum(y), rtol=1e-11, atol=1e-11), k


def test_f32_state_rounding():
    """States are rounded once from fp64 to fp32, nearest-even: against
    torch's own conversion, and at ties."""
    rng = np.random.default_rng(17)
    v = rng.standard_normal(100000) * np.exp(rng.uniform(-60, 60, 100000))
    ref = torch.from_numpy(v).to(torch.float32).numpy()
    assert np.array_equal(O.f64_to_f32(v).view(np.uint32), ref.view(np.uint32))
    e = 2.0 ** -24                         # half an fp32 ulp at 1
    assert O.f64_to_f32(1 + e) == np.float32(1.0)
    assert O.f64_to_f32(1 + 3 * e) == np.float32(1 + 4 * e)
    assert O.f64_to_f32(1 + e + 2.0 ** -50) == np.float32(1 + 2 * e)
