"""fp64 CPU oracle of the DeepSeek-V4 Compressor operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes, and where the pages state it
----------------------------------------------
Pages cited (by title):
  [PyPTO]   "CANN PyPTO 算子实战：Compressor 长序列 KV Cache 压缩算子的原理、参数与调用方法"
  [CANN]    "compressor-算子接口（torch_extension）-算子库-API参考-CANN9.2.0-beta.1开发文档"
  [AscendC] "NPU DeepSeek-V4 Ascend C 融合算子优化", section Compressor
  [Triton]  the 10100.com article on the Triton-Ascend Compressor built with
            CANNBot's triton-op-generator

1. Projection: kv = X Wkv^T, z = X Wgate^T, then z += Ape[p mod r]
   ([CANN] 计算公式 step 1 and the grouped addition of step 2; [AscendC]
   具体计算流程 矩阵乘法 / 分组加法; [PyPTO] 主要计算过程 投影与打分).
2. Windows: C128A pools the 128 rows of a window; C4A pools 8 slots: the first
   D channels ("a" set) of the previous window's 4 rows followed by the last D
   channels ("b" set) of the current window's 4 rows; the previous window of
   window 0 is padded with kv 0 and score -inf ([PyPTO] 压缩窗口与状态更新 and
   数值精度与验证要点; [AscendC] C4A 计算公式 and 数据重排 figure text).
3. Per-channel softmax over the slots, Hadamard (elementwise) product with kv,
   sum over slots ([CANN] 计算公式 steps 3-5; [AscendC] closed forms for C4A
   and C128A).
4. RMSNorm with epsilon 1e-6 times the weight ([PyPTO] 压缩窗口与状态更新,
   算子级辅助函数).
5. Interleaved RoPE on the trailing rope_head_dim channels ([PyPTO]
   压缩窗口与状态更新: rotate_half plus transpose/reshape).
6. If rotate: multiply by the D x D Hadamard matrix ([PyPTO] kernel 派发逻辑).
7. Output rows of entries that complete no window are zero; shape
   [min(T, T//ratio + B), D] ([PyPTO] 返回值说明).
8. State: projected rows of windows not yet complete are kept in the paged
   fp32 kv_state / score_state for the next call ([Triton] 流式调用 / 状态要跨调用保留;
   [PyPTO] 压缩窗口与状态更新); requests find their rows through the block
   table ([Triton] state_block_table example).

Readings taken where the pages are silent or garbled (each is listed, with
the reasoning, in the design notes of the repository):
  R1  state addressing: request b owns a ring of coff*r slots; position p uses
      slot q = p mod (coff*r), stored at [table[b, q // bs], q % bs].
  R2  C4A pairing: output of window w pools a-rows of window w-1 with b-rows
      of window w (the PyPTO golden semantics); Ape row j of the a set is
      ape[j, :D], of the b set ape[j, D:].
  R3  output row placement: request b owns rows [o_b, o_b + ceil(n_b/r)),
      o_b the prefix sum; its k-th completed window goes to row o_b + k,
      every other row is +0.
  R4  write set: after all reads, positions p in
      [max(s, r*floor(e/r) - (coff-1)*r), e) are stored; no other slot
      changes.
  R5  RoPE layout: de-interleave the 64 channels, rotate_half, re-interleave
      (pairs (2i, 2i+1) rotate together; column i of the tables drives the
      even element, column 32+i the odd one).
  R6  Ape is added to the scores only, and the stored score rows include it.
  R9  token rows of request b are x[cu[b] : cu[b] + seqused[b]].
  R11 arithmetic is exact fp64 from the bf16/fp32 input values; the output is
      rounded once to bf16 (nearest-even) and states once to fp32.

Pins: tests/test_oracle_pins.py checks every function below against closed
forms, hand-worked values, textbook routines and invariants.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

RMS_EPS = 1e-6


# --------------------------------------------------------------------------
# exact conversions
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 codes (uint16) -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 to bf16 codes, nearest-even, in one step (no double
    rounding through float32).

    A bf16 number carries 8 significant bits, so the rounding quantum of x is
    2^(e-8) for x = m 2^e with 0.5 <= |m| < 1, never below the subnormal
    spacing 2^-133.  Dividing by a power of two is exact, and numpy's rint
    rounds halves to even.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(x)
        q = np.ldexp(1.0, np.maximum(ex - 8, -133))
        v = np.rint(x / q) * q
        v = np.where(np.isfinite(x) & (np.abs(v) >= 2.0 ** 128), np.copysign(np.inf, x), v)
        v = np.where(np.isinf(x), x, v)
    code = (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), code).astype(np.uint16)


def f64_to_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# per-request bookkeeping
# --------------------------------------------------------------------------
def coff_of(ratio: int) -> int:
    """Number of channel sets: 2 (a and b, overlapping windows) for ratio 4,
    else 1 ([PyPTO] 参数说明: coff = 1 + (ratio == 4))."""
    return 2 if ratio == 4 else 1


@dataclasses.dataclass
class Plan:
    start: np.ndarray      # s_b, first position of this call's tokens
    ntok: np.ndarray       # n_b, valid tokens of request b in this call
    end: np.ndarray        # e_b = s_b + n_b
    row0: np.ndarray       # packed row of request b's first token
    nwin: np.ndarray       # c_b, windows completed in this call
    nrows: np.ndarray      # u_b = ceil(n_b / r), output rows owned by request b
    out0: np.ndarray       # o_b, first output row of request b


def make_plan(ratio, batch, T, cu_seqlens=None, seqused=None, start_pos=None) -> Plan:
    """Request layout of one call (reading R3, R9).

    cu_seqlens None means B equal-length requests of T/B tokens (x given as
    [B, S, H]); seqused None means every packed row of the slot is valid;
    start_pos None means every request starts at position 0.
    """
    B = int(batch)
    if cu_seqlens is None:
        assert T % B == 0
        cu = np.arange(B + 1, dtype=np.int64) * (T // B)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    slot = cu[1:] - cu[:-1]
    n = slot.copy() if seqused is None else np.asarray(seqused, dtype=np.int64)
    s = np.zeros(B, np.int64) if start_pos is None else np.asarray(start_pos, np.int64)
    e = s + n
    c = e // ratio - s // ratio
    u = -(-n // ratio)
    o = np.zeros(B, np.int64)
    o[1:] = np.cumsum(u)[:-1]
    return Plan(start=s, ntok=n, end=e, row0=cu[:-1].copy(), nwin=c, nrows=u, out0=o)


def ring_slot(p, ratio, coff):
    """Ring slot of position p in its request's state (reading R1)."""
    return p % (coff * ratio)


def state_location(table, b, q, block_size):
    """(block, offset) of ring slot q of request b (reading R1)."""
    return int(table[b, q // block_size]), int(q % block_size)


def live_positions(s, e, ratio, coff):
    """Positions whose rows a call stores into the state (reading R4):
    the incomplete window, plus for coff = 2 the last complete window whose
    a-set rows the next window still pools."""
    lo = max(s, ratio * (e // ratio) - (coff - 1) * ratio)
    return range(lo, e)


# --------------------------------------------------------------------------
# the arithmetic steps
# --------------------------------------------------------------------------
def project(x_rows, wkv, wgate):
    """kv = x Wkv^T, z = x Wgate^T (fp64, before Ape)."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    return x_rows @ np.asarray(wkv, np.float64).T, x_rows @ np.asarray(wgate, np.float64).T


def add_ape(z, positions, ape, ratio):
    """Grouped addition: score of position p gets ape[p mod r] (reading R6)."""
    return z + np.asarray(ape, np.float64)[np.asarray(positions) % ratio]


def window_slot_positions(w, ratio, coff):
    """Positions and channel sets pooled by window w (reading R2).

    Returns a list of (position, channel_set) for the window's slots in order:
    C128A: (w*r + j, 0) for j < r.  C4A: (w-1)*r + j with set a (0), then
    w*r + j with set b (1).
    """
    if coff == 1:
        return [(w * ratio + j, 0) for j in range(ratio)]
    return ([((w - 1) * ratio + j, 0) for j in range(ratio)]
            + [(w * ratio + j, 1) for j in range(ratio)])


def softmax_pool(kv_slots, z_slots):
    """Per-channel softmax over the slot axis, times kv, summed over slots.

    kv_slots, z_slots: [n_slots, D].  Scores may be -inf (padding) and get
    weight 0; the max is subtracted first ([PyPTO] 算子级辅助函数 softmax:
    amax, subtract, exp, sum, divide; [CANN] 计算公式 steps 3-5).
    """
    z = np.asarray(z_slots, np.float64)
    kv = np.asarray(kv_slots, np.float64)
    m = np.max(z, axis=0, keepdims=True)
    e = np.exp(z - m)
    return np.sum(e * kv, axis=0) / np.sum(e, axis=0)


def rms_norm(c, gamma, eps=RMS_EPS):
    """y = c / sqrt(mean(c^2) + eps) * gamma over the last axis."""
    c = np.asarray(c, np.float64)
    ms = np.mean(c * c, axis=-1, keepdims=True)
    return c / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def rope_interleaved(t, cos_row, sin_row):
    """Interleaved RoPE on a rope_head_dim-wide slice (reading R5).

    u = [t0, t2, ..., t1, t3, ...]          (de-interleave)
    u' = u * cos + rotate_half(u) * sin     (rotate_half(u) = [-u_hi, u_lo])
    t'[2i] = u'[i], t'[2i+1] = u'[half + i] (re-interleave)
    """
    t = np.asarray(t, np.float64)
    half = t.shape[-1] // 2
    u = np.concatenate([t[..., 0::2], t[..., 1::2]], axis=-1)
    rot = np.concatenate([-u[..., half:], u[..., :half]], axis=-1)
    up = u * np.asarray(cos_row, np.float64) + rot * np.asarray(sin_row, np.float64)
    out = np.empty_like(t)
    out[..., 0::2] = up[..., :half]
    out[..., 1::2] = up[..., half:]
    return out


def hadamard_rotate(y, had):
    """y <- y @ Had, with the given D x D matrix."""
    return np.asarray(y, np.float64) @ np.asarray(had, np.float64)


def postprocess(c, gamma, cos_row, sin_row, had, rope_dim):
    """RMSNorm, RoPE on the trailing rope_dim channels, optional Hadamard."""
    y = rms_norm(c, gamma)
    D = y.shape[-1]
    y = y.copy()
    y[..., D - rope_dim:] = rope_interleaved(y[..., D - rope_dim:], cos_row, sin_row)
    if had is not None:
        y = hadamard_rotate(y, had)
    return y


# --------------------------------------------------------------------------
# the whole call
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Result:
    out: np.ndarray          # float64 [out_rows, D] before the final rounding
    out_bf16: np.ndarray     # uint16 [out_rows, D]
    kv_state: np.ndarray     # float32, the pool after the call
    score_state: np.ndarray
    kv_written: np.ndarray   # bool [num_blocks, block_size], slots stored
    score_written: np.ndarray
    plan: Plan
    window_rows: list        # (b, w, out_row) of every emitted window


def _row_source(b, p, plan, proj, pool_kv, pool_sc, kv_tab, st_tab, ratio, coff, bs):
    """kv and score rows (full coff*D) of position p of request b (reading R1, R6).

    Positions of this call come from the projection; earlier ones from the
    pool as it was at call entry; negative positions are None (padding).
    """
    if p < 0:
        return None
    if p >= plan.start[b]:
        return proj[b][0][p - plan.start[b]], proj[b][1][p - plan.start[b]]
    q = ring_slot(p, ratio, coff)
    kb, ko = state_location(kv_tab, b, q, bs)
    sb, so = state_location(st_tab, b, q, bs)
    return (pool_kv[kb, ko].astype(np.float64), pool_sc[sb, so].astype(np.float64))


def compressor(w: dict, windows=None, project_all=True) -> Result:
    """Run one operator call on the input dict ``w`` (layout of workloads.build).

    windows: None computes every output row; otherwise an iterable of output
    row indices, and only those rows are computed (the others stay NaN).
    project_all=False projects only the rows the requested windows and the
    state write need (for sampled checks at large sizes).
    """
    r, coff, D, rope_dim = w["ratio"], w["coff"], w["head_dim"], w["rope_dim"]
    B, T, bs = w["batch"], w["T"], w["block_size"]
    plan = make_plan(r, B, T, w["cu_seqlens"], w["seqused"], w["start_pos"])
    st_tab = np.asarray(w["state_block_table"])
    kv_tab = st_tab if w["kv_block_table"] is None else np.asarray(w["kv_block_table"])
    pool_kv = np.asarray(w["kv_state"], np.float32)
    pool_sc = np.asarray(w["score_state"], np.float32)
    wkv = bf16_to_f64(w["wkv"])
    wgate = bf16_to_f64(w["wgate"])
    ape = np.asarray(w["ape"], np.float64)
    gamma = bf16_to_f64(w["weight"])
    had = None if w["hadamard"] is None else bf16_to_f64(w["hadamard"])
    cos = bf16_to_f64(w["cos"])
    sin = bf16_to_f64(w["sin"])
    out_rows = w["out_rows"]

    # output rows to compute: (row -> (b, k))
    emitted = []
    for b in range(B):
        for k in range(int(plan.nwin[b])):
            emitted.append((b, int(plan.start[b] // r) + k, int(plan.out0[b]) + k))
    assert sum(plan.nrows) <= out_rows, "output rows exceed out_rows"
    if windows is None:
        todo = emitted
    else:
        want = set(int(i) for i in windows)
        todo = [t for t in emitted if t[2] in want]

    # projected rows needed per request: positions of this call
    need = [set() for _ in range(B)]
    for b in range(B):
        s, e = int(plan.start[b]), int(plan.end[b])
        if project_all:
            need[b].update(range(s, e))
        else:
            need[b].update(live_positions(s, e, r, coff))
    if not project_all:
        for b, wi, _ in todo:
            for p, _set in window_slot_positions(wi, r, coff):
                if plan.start[b] <= p < plan.end[b]:
                    need[b].add(p)
    proj = []
    for b in range(B):
        s, n = int(plan.start[b]), int(plan.ntok[b])
        kv_b = np.full((n, coff * D), np.nan)
        z_b = np.full((n, coff * D), np.nan)
        pos = np.array(sorted(need[b]), dtype=np.int64)
        if pos.size:
            rows = plan.row0[b] + (pos - s)
            xr = bf16_to_f64(w["x"][rows])
            kv, z = project(xr, wkv, wgate)
            kv_b[pos - s] = kv
            z_b[pos - s] = add_ape(z, pos, ape, r)
        proj.append((kv_b, z_b))

    out = np.full((out_rows, D), np.nan)
    # rows that complete no window are zero
    done = np.zeros(out_rows, dtype=bool)
    for b, wi, row in emitted:
        done[row] = True
    out[~done] = 0.0
    if windows is not None:
        keep = np.zeros(out_rows, dtype=bool)
        keep[list(want)] = True
        out[~keep & done] = np.nan

    for b, wi, row in todo:
        slots = window_slot_positions(wi, r, coff)
        kv_s = np.empty((len(slots), D))
        z_s = np.empty((len(slots), D))
        for j, (p, cs) in enumerate(slots):
            src = _row_source(b, p, plan, proj, pool_kv, pool_sc, kv_tab, st_tab, r, coff, bs)
            if src is None:                       # before the sequence start
                kv_s[j] = 0.0
                z_s[j] = -np.inf
            else:
                kv_s[j] = src[0][cs * D:(cs + 1) * D]
                z_s[j] = src[1][cs * D:(cs + 1) * D]
        c = softmax_pool(kv_s, z_s)
        out[row] = postprocess(c, gamma, cos[row], sin[row], had, rope_dim)

    # state write-back, after every read above
    new_kv = pool_kv.copy()
    new_sc = pool_sc.copy()
    kv_written = np.zeros(pool_kv.shape[:2], dtype=bool)
    sc_written = np.zeros(pool_sc.shape[:2], dtype=bool)
    for b in range(B):
        s, e = int(plan.start[b]), int(plan.end[b])
        for p in live_positions(s, e, r, coff):
            q = ring_slot(p, r, coff)
            kb, ko = state_location(kv_tab, b, q, bs)
            sb, so = state_location(st_tab, b, q, bs)
            new_kv[kb, ko] = f64_to_f32(proj[b][0][p - s])
            new_sc[sb, so] = f64_to_f32(proj[b][1][p - s])
            kv_written[kb, ko] = True
            sc_written[sb, so] = True

    out_bf16 = f64_to_bf16(np.nan_to_num(out, nan=0.0))
    return Result(out=out, out_bf16=out_bf16, kv_state=new_kv, score_state=new_sc,
                  kv_written=kv_written, score_written=sc_written, plan=plan,
                  window_rows=emitted)
