"""fp64 CPU oracle of NsaCompressWithCache (the NSA KV-compression operator).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests and the benchmark use it.  It shares no
code with the HIP library.

What it computes, and where the page states it
----------------------------------------------
Page cited (by title): [NSA] the aclnnNsaCompressWithCache article
(功能说明与压缩算法流程, 计算公式, 参数说明, 约束说明).

For every batch b with current length s = actSeqLen[b] ([NSA] 算法流程 step 1):
  the batch compresses in this call iff s >= compressBlockSize and
  (s - compressBlockSize) % stride == 0; then
  compressIdx = (s - compressBlockSize) / stride        ([NSA] 计算公式)
  out[slotMapping[b], n, d] = sum over j < compressBlockSize of
      input[token compressIdx*stride + j of batch b, n, d] * weight[j, n]
  i.e. the last compressBlockSize tokens of the batch, each head weighted by
  its own column of weight (weight [compressBlockSize, N] broadcast over D).
The page's kernel casts to fp32, multiplies, reduces and casts back with
round-to-nearest-even (CAST_RINT); the oracle takes the exact sum in fp64 and
rounds once to the input dtype (bf16 or fp16), nearest-even.
Token t of batch b lives, with a block table ([NSA] PageAttention 场景), at
input[blockTable[b, t // pageBlockSize], t % pageBlockSize]; without one (TND
layout, actSeqLenType 1 = per-batch lengths), at row cu[b] + t of input
[T, N, D] with cu the prefix sums of actSeqLen.  Batches that do not
compress leave outputCache unchanged.

Readings (listed in the design notes too): actSeqLen holds the batch lengths
after this step's token (the trigger counts the tokens present); slots that
no batch writes keep their contents; a slot or block index out of range is a
device error and the batch writes nothing.
"""
from __future__ import annotations

import numpy as np

from oracle.compressor_oracle import bf16_to_f64, f64_to_bf16


def f16_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16(x) -> np.ndarray:
    """Round float64 to fp16 codes, nearest-even, in one step: numpy's
    double -> half conversion is correctly rounded."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def decode_dtype(bits, dtype: str) -> np.ndarray:
    return bf16_to_f64(bits) if dtype == "bf16" else f16_to_f64(bits)


def encode_dtype(x, dtype: str) -> np.ndarray:
    return f64_to_bf16(x) if dtype == "bf16" else f64_to_f16(x)


def compress_index(s: int, cbs: int, stride: int):
    """compressIdx of a batch of length s, or None if it does not compress."""
    if s < cbs or (s - cbs) % stride:
        return None
    return (s - cbs) // stride


def token_rows(b, first, count, act_seq_len, block_table, page_block_size):
    """(block, row) of tokens first .. first+count-1 of batch b (paged), or
    the packed rows (TND)."""
    if block_table is not None:
        return [(int(block_table[b, t // page_block_size]), t % page_block_size)
                for t in range(first, first + count)]
    cu = int(np.sum(np.asarray(act_seq_len[:b], dtype=np.int64)))
    return [cu + t for t in range(first, first + count)]


def nsa_compress(inp, weight, slot_mapping, act_seq_len, block_table, out_cache, *, cbs, stride,
                 page_block_size, dtype, absolute=False):
    """Returns (exact fp64 out cache values of written slots, the new cache
    codes, the list of (b, slot) written).  inp / weight / out_cache are codes
    (uint16) of `dtype`.  absolute=True sums |token| * |weight| instead (the
    scale of a rounding-error bound)."""
    x = decode_dtype(inp, dtype)
    w = decode_dtype(weight, dtype)                     # [cbs, N]
    if absolute:
        x, w = np.abs(x), np.abs(w)
    new = np.array(out_cache, dtype=np.uint16, copy=True)
    exact = {}
    written = []
    for b in range(len(slot_mapping)):
        s = int(act_seq_len[b])
        ci = compress_index(s, cbs, stride)
        if ci is None:
            continue
        rows = token_rows(b, ci * stride, cbs, act_seq_len, block_table, page_block_size)
        acc = np.zeros(x.shape[-2:], dtype=np.float64)   # [N, D]
        for j, r in enumerate(rows):
            tok = x[r] if block_table is None else x[r[0], r[1]]
            acc += tok * w[j][:, None]
        slot = int(slot_mapping[b])
        exact[slot] = acc
        new[slot] = encode_dtype(acc, dtype)
        written.append((b, slot))
    return exact, new, written
