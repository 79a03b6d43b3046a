"""Pins of the NSA compression oracle against what the page and arithmetic
fix (no GPU): one-hot and uniform weights, the trigger rule, paged == packed
layouts, untouched slots, and the rounding of both output dtypes."""
import numpy as np
import pytest

from oracle import nsa_oracle as N
from oracle.compressor_oracle import f64_to_bf16


def _case(rng, B, heads, D, cbs, stride, page, dtype, lengths, paged=True):
    nblk_per = -(-max(lengths) // page)
    x = rng.standard_normal((B * nblk_per + 2, page, heads, D))
    enc = lambda v: N.encode_dtype(v, dtype)
    inp = enc(x)
    table = rng.permutation(B * nblk_per + 2)[: B * nblk_per].reshape(B, nblk_per)
    w = enc(rng.standard_normal((cbs, heads)) * 0.3)
    slots = rng.permutation(3 * B)[:B]
    out = enc(rng.standard_normal((3 * B, heads, D)))
    return inp, w, slots, np.asarray(lengths, np.int64), table, out


def test_trigger_rule_brute_force():
    for cbs in (16, 32, 48, 64):
        for stride in (16, 32, 48, 64):
            if stride > cbs:
                continue
            for s in range(0, 400):
                # windows [i*stride, i*stride + cbs) ending exactly at s
                ends = [i * stride + cbs for i in range(0, 400)]
                want = (s - cbs) // stride if s in ends else None
                assert N.compress_index(s, cbs, stride) == want


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_hot_weight_copies_a_token(dtype):
    rng = np.random.default_rng(1)
    cbs, stride, page = 32, 16, 64
    lengths = [48, 80, 33, 64]                  # 48, 80, 64 compress; 33 does not
    inp, w, slots, lens, table, out = _case(rng, 4, 4, 32, cbs, stride, page, dtype, lengths)
    # head h takes token j_h of the window: weight column h is one-hot at j_h
    js = [5, 0, 31, 17]
    onehot = np.zeros((cbs, 4))
    for h, j in enumerate(js):
        onehot[j, h] = 1.0
    w = N.encode_dtype(onehot, dtype)
    exact, new, written = N.nsa_compress(inp, w, slots, lens, table, out, cbs=cbs,
                                         stride=stride, page_block_size=page, dtype=dtype)
    assert [b for b, _ in written] == [0, 1, 3]
    for b, slot in written:
        for h, j in enumerate(js):
            t = int(lens[b]) - cbs + j          # the last cbs tokens, token j of them
            blk, row = table[b, t // page], t % page
            assert np.array_equal(new[slot][h], inp[blk, row][h])
    # the batch that does not compress leaves every slot alone
    untouched = set(range(out.shape[0])) - {s for _, s in written}
    for s in untouched:
        assert np.array_equal(new[s], out[s])


def test_uniform_weights_give_the_mean_of_the_last_tokens():
    rng = np.random.default_rng(2)
    cbs, stride, page = 16, 16, 128
    lengths = [16, 160]
    inp, w, slots, lens, table, out = _case(rng, 2, 2, 16, cbs, stride, page, "bf16", lengths)
    w = f64_to_bf16(np.full((cbs, 2), 1.0 / 16))    # exact in bf16
    exact, new, written = N.nsa_compress(inp, w, slots, lens, table, out, cbs=cbs,
                                         stride=stride, page_block_size=page, dtype="bf16")
    x = N.decode_dtype(inp, "bf16")
    for b, slot in written:
        toks = [x[table[b, t // page], t % page] for t in range(int(lens[b]) - cbs, int(lens[b]))]
        assert np.allclose(exact[slot], np.mean(toks, axis=0), rtol=1e-15, atol=1e-15)


def test_paged_and_packed_layouts_agree():
    rng = np.random.default_rng(3)
    cbs, stride, page, heads, D = 48, 32, 64, 3, 16
    lengths = [48, 112, 80, 144]
    inp, w, slots, lens, table, out = _case(rng, 4, heads, D, cbs, stride, page, "f16", lengths)
    # the same tokens packed batch after batch
    packed = np.concatenate([np.stack([inp[table[b, t // page], t % page] for t in range(lengths[b])])
                             for b in range(4)])
    a = N.nsa_compress(inp, w, slots, lens, table, out, cbs=cbs, stride=stride,
                       page_block_size=page, dtype="f16")
    b = N.nsa_compress(packed, w, slots, lens, None, out, cbs=cbs, stride=stride,
                       page_block_size=page, dtype="f16")
    assert np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_rounding_is_nearest_even_from_the_exact_sum():
    # fp16: 1 + 2^-11 is halfway between 1 and 1 + 2^-10 -> 1 (even);
    # 1 + 2^-11 + 2^-30 is above halfway -> 1 + 2^-10 (a float32 round trip
    # would lose the 2^-30 and round to even)
    v = N.f64_to_f16(np.array([1 + 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -30, 1 + 3 * 2.0 ** -11]))
    assert list(N.f16_to_f64(v)) == [1.0, 1 + 2.0 ** -10, 1 + 2 * 2.0 ** -10]
    b = f64_to_bf16(np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40]))
    assert list(N.decode_dtype(b, "bf16")) == [1.0, 1 + 2.0 ** -7]
