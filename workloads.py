"""Seeded synthetic inputs for the Compressor workloads.

This module only draws and lays out input tensors.  It holds no part of the
operator's arithmetic (no projection, pooling, normalisation, rotation or
state addressing), so both the fp64 oracle and the HIP path can take their
inputs from it without sharing any of the method.

Conventions
-----------
* bf16 tensors are returned as ``numpy.uint16`` arrays of raw bf16 bits,
  rounded to nearest-even from fp32 draws; fp32 tensors as ``float32``;
  indices as ``int32``.
* ``N(mu, v)`` below means a normal with mean ``mu`` and *variance* ``v``.
* Random generator: ``numpy.random.Generator(PCG64(seed))``; the draw order is
  fixed by :func:`build` and never depends on the sizes of earlier draws'
  consumers.

Shapes follow the operator's parameter table on the page "CANN PyPTO 算子实战：
Compressor 长序列 KV Cache 压缩算子的原理、参数与调用方法" (section 参数说明):
x [T, H] (packed), kv_state / score_state [block_num, block_size, coff*D] fp32,
block tables int32, sin / cos [out_rows, rope_head_dim] bf16, wkv / wgate
[coff*D, H] bf16, ape [ratio, coff*D] fp32, weight [D] bf16, hadamard [D, D]
bf16, start_pos [B] int32; cu_seqlens / seqused come from the torch_extension
reference page and the Triton-Ascend article (variable-length packing).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

ROPE_DIM = 64


# --------------------------------------------------------------------------
# dtype helpers (input preparation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even) and return the raw 16-bit codes."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float, mean: float = 0.0,
                chunk: int = 1 << 25) -> np.ndarray:
    """Draw N(mean, std^2) in fp32 in fixed-size chunks and round to bf16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = f32_to_bf16_bits(v)
    return out.reshape(shape)


# --------------------------------------------------------------------------
# fixed input tensors
# --------------------------------------------------------------------------
def sylvester_hadamard_bf16(d: int) -> np.ndarray:
    """D x D Sylvester Hadamard matrix times bf16(1/sqrt(D)), as bf16 bits.

    Every entry is +-c with c = bf16(1/sqrt(D)), so the matrix is exact in bf16.
    """
    assert d > 0 and d & (d - 1) == 0
    h = np.ones((1, 1), dtype=np.float32)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    c = bf16_bits_to_f32(f32_to_bf16_bits(np.array([1.0 / math.sqrt(d)], np.float32)))[0]
    return f32_to_bf16_bits(h * c)


def rope_tables(positions: Sequence[float], rope_dim: int = ROPE_DIM,
                base: float = 10000.0):
    """cos / sin tables [len(positions), rope_dim] in bf16 bits.

    Frequency i (0 <= i < rope_dim/2) is base^(-2i/rope_dim); the table stores
    the rope_dim/2 angles twice (columns i and i + rope_dim/2 hold the same
    angle), the usual half-duplicated layout.
    """
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    half = rope_dim // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / rope_dim)
    ang = pos * inv.reshape(1, -1)
    ang = np.concatenate([ang, ang], axis=1)
    return (f32_to_bf16_bits(np.cos(ang).astype(np.float32)),
            f32_to_bf16_bits(np.sin(ang).astype(np.float32)))


# --------------------------------------------------------------------------
# workload specification
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    ratio: int
    head_dim: int
    hidden: int
    rotate: bool
    block_size: int
    batch: int
    # token count per request: a fixed tuple, or ("uniform", lo, hi) inclusive
    lengths: object
    # start positions: None (all zero / argument omitted), a fixed tuple,
    # or ("uniform", lo, hi) inclusive
    start_pos: object = None
    # extra packed rows after each request's valid tokens (cu_seqlens slot
    # longer than seqused); 0 means seqused is omitted
    pad_rows: int = 0
    # "identity" or "perm" block tables; kv table may be omitted (shares the
    # state table) when separate_kv_table is False
    tables: str = "perm"
    separate_kv_table: bool = True
    spare_blocks: int = 3
    # number of output rows; None means the operator's bound min(T, T//ratio + B)
    out_rows: Optional[int] = None
    rope_dim: int = ROPE_DIM

    @property
    def coff(self) -> int:
        # a second, overlapping channel set exists only for ratio 4
        return 2 if self.ratio == 4 else 1


def _draw_ints(rng, spec_val, batch, default):
    if spec_val is None:
        return np.full(batch, default, dtype=np.int64)
    if isinstance(spec_val, tuple) and len(spec_val) == 3 and spec_val[0] == "uniform":
        _, lo, hi = spec_val
        return rng.integers(lo, hi + 1, size=batch, dtype=np.int64)
    vals = np.asarray(spec_val, dtype=np.int64).reshape(-1)
    if vals.size == 1:
        vals = np.full(batch, int(vals[0]), dtype=np.int64)
    assert vals.size == batch
    return vals


def build(spec: Spec, seed: int, with_x: bool = True) -> dict:
    """Draw every input of one operator call.

    Draw order: lengths, start_pos, x, wkv, wgate, ape, weight, block tables,
    kv_state, score_state.  (The Hadamard matrix and rope tables are fixed
    functions of the shapes.)
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    r, coff, D, H, B = spec.ratio, spec.coff, spec.head_dim, spec.hidden, spec.batch
    lengths = _draw_ints(rng, spec.lengths, B, 0)
    start = _draw_ints(rng, spec.start_pos, B, 0)
    slot_len = lengths + spec.pad_rows
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(slot_len)
    T = int(cu[-1])

    x = normal_bf16(rng, (T, H), 1.0) if with_x else None
    wstd = math.sqrt(1.0 / H)
    wkv = normal_bf16(rng, (coff * D, H), wstd)
    wgate = normal_bf16(rng, (coff * D, H), wstd)
    ape = (rng.standard_normal((r, coff * D), dtype=np.float32)
           * np.float32(math.sqrt(0.1)))
    weight = normal_bf16(rng, (D,), math.sqrt(0.05), mean=1.0)

    slots = coff * r
    stride = -(-slots // spec.block_size)
    nblocks = B * stride + spec.spare_blocks
    if spec.tables == "identity":
        st_tab = np.arange(B * stride, dtype=np.int64).reshape(B, stride)
        kv_tab = st_tab.copy()
    else:
        st_tab = rng.permutation(nblocks)[: B * stride].reshape(B, stride)
        kv_tab = rng.permutation(nblocks)[: B * stride].reshape(B, stride)
    if not spec.separate_kv_table:
        kv_tab = st_tab.copy()
    kv_state = rng.standard_normal((nblocks, spec.block_size, coff * D), dtype=np.float32)
    score_state = rng.standard_normal((nblocks, spec.block_size, coff * D), dtype=np.float32)

    out_rows = spec.out_rows if spec.out_rows is not None else min(T, T // r + B)
    # rotary angles of row rho are those of position rho
    cos, sin = rope_tables(np.arange(out_rows), spec.rope_dim)

    return dict(
        name=spec.name, ratio=r, coff=coff, head_dim=D, hidden=H, rotate=spec.rotate,
        rope_dim=spec.rope_dim, block_size=spec.block_size, batch=B, T=T,
        x=x, wkv=wkv, wgate=wgate, ape=ape, weight=weight,
        hadamard=sylvester_hadamard_bf16(D) if spec.rotate else None,
        start_pos=(start.astype(np.int32) if spec.start_pos is not None else None),
        cu_seqlens=cu.astype(np.int32),
        seqused=(lengths.astype(np.int32) if spec.pad_rows > 0 else None),
        kv_block_table=(kv_tab.astype(np.int32) if spec.separate_kv_table else None),
        state_block_table=st_tab.astype(np.int32),
        kv_state=kv_state, score_state=score_state,
        out_rows=int(out_rows), cos=cos, sin=sin,
        num_blocks=int(nblocks), table_stride=int(stride),
    )


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------
SEED_BASE = 20260

# C4Li smallest case: one 64-token prefill from position 0.
C4LI_SMALL = Spec("c4li_small", ratio=4, head_dim=128, hidden=1024, rotate=False,
                  block_size=16, batch=1, lengths=(64,), tables="identity",
                  separate_kv_table=False, spare_blocks=0, out_rows=16)
# C128A prefill, 8192 tokens, and 8192+77 so a partial window stays in state.
C128A_8192 = Spec("c128a_8192", ratio=128, head_dim=512, hidden=4096, rotate=False,
                  block_size=128, batch=1, lengths=(8192,), tables="identity",
                  separate_kv_table=False, spare_blocks=0, out_rows=64)
C128A_8269 = dataclasses.replace(C128A_8192, name="c128a_8269", lengths=(8269,), out_rows=65)
# C4A 128K-token prefill with the Hadamard rotation.
C4A_128K = Spec("c4a_128k", ratio=4, head_dim=512, hidden=7168, rotate=True,
                block_size=128, batch=1, lengths=(131072,), tables="identity",
                separate_kv_table=False, spare_blocks=0, out_rows=32768)
# 32-request decode, one token each, start positions uniform in [0, 65536).
DECODE_C4A = Spec("decode_c4a", ratio=4, head_dim=512, hidden=7168, rotate=False,
                  block_size=64, batch=32, lengths=(1,), start_pos=("uniform", 0, 65535),
                  tables="perm", separate_kv_table=False, spare_blocks=0, out_rows=32)
DECODE_C128A = dataclasses.replace(DECODE_C4A, name="decode_c128a", ratio=128)
# decode where every request completes a window (the step that emits output)
DECODE_C4A_ALL = dataclasses.replace(DECODE_C4A, name="decode_c4a_all")
DECODE_C128A_ALL = dataclasses.replace(DECODE_C128A, name="decode_c128a_all")
# multi-token decode (two tokens per request per call, packed with cu_seqlens)
DECODE_C4A_MTP2 = dataclasses.replace(DECODE_C4A, name="decode_c4a_mtp2", lengths=(2,),
                                      out_rows=64)
# variable-length packed prefill with continuation
VARLEN_C4A = Spec("varlen_c4a", ratio=4, head_dim=512, hidden=4096, rotate=True,
                  block_size=256, batch=8, lengths=("uniform", 1, 16384),
                  start_pos=("uniform", 1, 4095), tables="perm", separate_kv_table=True)
VARLEN_C4A_PADDED = dataclasses.replace(VARLEN_C4A, name="varlen_c4a_padded", pad_rows=5)

# The three test shapes of the PyPTO example script: batch 64, 2 tokens each.
P1_COMP_128 = Spec("p1_comp_128", ratio=128, head_dim=512, hidden=4096, rotate=False,
                   block_size=128, batch=64, lengths=(2,), start_pos=(8192,))
P1_COMP_4 = Spec("p1_comp_4", ratio=4, head_dim=512, hidden=4096, rotate=False,
                 block_size=128, batch=64, lengths=(2,), start_pos=(2,))
P1_COMP_INDEXER = Spec("p1_comp_indexer", ratio=4, head_dim=128, hidden=4096, rotate=True,
                       block_size=128, batch=64, lengths=(2,), start_pos=(1,))

ALL = {s.name: s for s in (C4LI_SMALL, C128A_8192, C128A_8269, C4A_128K, DECODE_C4A,
                            DECODE_C128A, DECODE_C4A_ALL, DECODE_C128A_ALL, DECODE_C4A_MTP2,
                            VARLEN_C4A,
                            VARLEN_C4A_PADDED, P1_COMP_128, P1_COMP_4, P1_COMP_INDEXER)}
CONFIG_INDEX = {"c4li_small": 0, "c128a_8192": 1, "c128a_8269": 1, "c4a_128k": 2,
                "decode_c4a": 3, "decode_c128a": 3, "decode_c4a_all": 3,
                "decode_c128a_all": 3, "varlen_c4a": 4, "varlen_c4a_padded": 4}


def seed_for(name: str) -> int:
    return SEED_BASE + CONFIG_INDEX.get(name, 10 + sorted(ALL).index(name))


def build_named(name: str, with_x: bool = True) -> dict:
    w = build(ALL[name], seed_for(name), with_x=with_x)
    if name.endswith("_all"):
        # every request sits on the last token of a window: start_pos = r-1 mod r
        r = w["ratio"]
        sp = w["start_pos"].astype(np.int64)
        w["start_pos"] = (sp - sp % r + (r - 1)).astype(np.int32)
    return w


# --------------------------------------------------------------------------
# NSA KV compression (NsaCompressWithCache) inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class NsaSpec:
    name: str
    head_num: int
    head_dim: int
    cbs: int                 # compress block size
    stride: int
    page: int                # page block size
    dtype: str               # "bf16" or "f16"
    layout: str              # "paged" or "tnd"
    batch: int
    max_len: int             # lengths are drawn in [1, max_len]
    fire_fraction: float     # share of batches whose length triggers a compression
    slot_factor: int = 3     # result_len = slot_factor * batch


def _codes(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float16).view(np.uint16)


def build_nsa(spec: NsaSpec, seed: int) -> dict:
    """Draw every input of one NSA compression call.  Draw order: lengths,
    firing choice, cache values, block table, weight, slots, output cache."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, N, D = spec.batch, spec.head_num, spec.head_dim
    lengths = rng.integers(1, spec.max_len + 1, size=B, dtype=np.int64)
    fire = rng.random(B) < spec.fire_fraction
    # a firing length is cbs + k * stride (<= max_len); the others are moved
    # off that lattice
    kmax = max((spec.max_len - spec.cbs) // spec.stride, 0)
    ks = rng.integers(0, kmax + 1, size=B, dtype=np.int64)
    lengths = np.where(fire, spec.cbs + ks * spec.stride, lengths)
    hits = (lengths >= spec.cbs) & ((lengths - spec.cbs) % spec.stride == 0)
    lengths = np.where(~fire & hits, lengths - 1, lengths)
    lengths = np.maximum(lengths, 1)
    if spec.layout == "paged":
        per = -(-int(lengths.max()) // spec.page)
        nblocks = B * per + 3
        cache = normal_bf16(rng, (nblocks, spec.page, N, D), 1.0) if spec.dtype == "bf16" else \
            _codes(rng.standard_normal((nblocks, spec.page, N, D), dtype=np.float32), "f16")
        table = rng.permutation(nblocks)[: B * per].reshape(B, per).astype(np.int32)
    else:
        T = int(lengths.sum())
        cache = normal_bf16(rng, (T, N, D), 1.0) if spec.dtype == "bf16" else \
            _codes(rng.standard_normal((T, N, D), dtype=np.float32), "f16")
        table = None
    weight = _codes(rng.standard_normal((spec.cbs, N), dtype=np.float32)
                    * np.float32(1.0 / math.sqrt(spec.cbs)), spec.dtype)
    result_len = spec.slot_factor * B
    slots = rng.permutation(result_len)[:B].astype(np.int32)
    out_cache = _codes(rng.standard_normal((result_len, N, D), dtype=np.float32), spec.dtype)
    return dict(name=spec.name, head_num=N, head_dim=D, cbs=spec.cbs, stride=spec.stride,
                page=spec.page, dtype=spec.dtype, layout=spec.layout, batch=B,
                act_seq_len=lengths.astype(np.int64), input=cache, block_table=table,
                weight=weight, slot_mapping=slots, output_cache=out_cache,
                result_len=result_len)


# NSA decode step: 128 sequences that all compress (32-token window, stride
# 16, 32 heads of 128), paged with 128-token pages
NSA_DECODE = NsaSpec("nsa_decode", head_num=32, head_dim=128, cbs=32, stride=16, page=128,
                     dtype="bf16", layout="paged", batch=128, max_len=256, fire_fraction=1.0)


# --------------------------------------------------------------------------
# Quantised cache write after the operator (compressor_epilog): compressed
# rows bf16 [rows, D] with blocks of 128 channels at mixed magnitudes (as
# normalised rows times weights of various sizes), a slot mapping that is a
# seeded permutation into a larger cache with every `skip`-th row at -1, and
# a cache pre-filled with random bytes and scales (rows nobody writes must
# keep them).
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class EpilogSpec:
    name: str
    rows: int
    head_dim: int
    num_slots: int
    skip: int = 0                 # every skip-th row has slot -1 (0: none)
    bad_slots: tuple = ()         # (row, slot) pairs set after the permutation


def build_epilog(spec: EpilogSpec, seed: int) -> dict:
    rng = np.random.default_rng(seed)
    nb = spec.head_dim // 128
    x = rng.standard_normal((spec.rows, spec.head_dim)).astype(np.float32)
    mag = rng.choice(np.float32([1e-3, 0.05, 1.0, 30.0]), (spec.rows, nb))
    x *= np.repeat(mag, 128, axis=1)
    slots = rng.permutation(spec.num_slots)[: spec.rows].astype(np.int32)
    if spec.skip:
        slots[:: spec.skip] = -1
    for r, s in spec.bad_slots:
        slots[r] = s
    return {"rows": f32_to_bf16_bits(x), "slot_mapping": slots,
            "cache": rng.integers(0, 256, (spec.num_slots, spec.head_dim), dtype=np.uint8),
            "cache_scale": rng.standard_normal((spec.num_slots, nb)).astype(np.float32),
            "head_dim": spec.head_dim}


# the 128K C4A output (32768 rows of D = 512), the indexer's D = 128 rows
# and a ragged case with rows that name no slot or a slot outside the cache
EPILOG_C4A = EpilogSpec("epilog_c4a_128k", rows=32768, head_dim=512, num_slots=40000, skip=7)
EPILOG_INDEXER = EpilogSpec("epilog_indexer", rows=64, head_dim=128, num_slots=64)
EPILOG_RAGGED = EpilogSpec("epilog_ragged", rows=37, head_dim=128, num_slots=50, skip=5,
                           bad_slots=((3, -2), (11, 50)))
