"""Comparison of GPU results with the oracle.

Bars (written here, used by every parity test):
* out rows holding a window: per element |g - o| / max(|o|, rms(o_row)) <= 2e-2
  (the oracle is exact fp64 then one bf16 rounding; the kernel rounds its
  bf16 operands and output, 2^-9 relative each);
* out rows holding no window: bit-exact +0 (0x0000);
* state slots the oracle writes: |g - o| <= 1e-3 * max(|o|, 1) (fp32 sums over
  H terms vs fp64);
* state slots the oracle does not write: bit-identical to the input pool, and
  the set of changed slots equals the oracle's write set.
"""
import numpy as np

from oracle import compressor_oracle as O

OUT_RTOL = 2e-2
STATE_TOL = 1e-3


def out_errors(gpu_bits: np.ndarray, res, rows=None):
    """Returns (max scaled error, mean abs error) over the window rows checked;
    asserts the zero rows."""
    g = O.bf16_to_f64(gpu_bits)
    done = np.zeros(res.out.shape[0], dtype=bool)
    for _, _, row in res.window_rows:
        done[row] = True
    check = np.arange(res.out.shape[0]) if rows is None else np.asarray(sorted(rows))
    win = [r for r in check if done[r]]
    zero = [r for r in check if not done[r]]
    if zero:
        bad = np.nonzero(np.any(gpu_bits[zero] != 0, axis=1))[0]
        assert bad.size == 0, f"rows {[zero[i] for i in bad[:8]]} should be +0"
    if not win:
        return 0.0, 0.0
    o = res.out[win]
    gg = g[win]
    assert np.all(np.isfinite(o)), "oracle produced non-finite values"
    rms = np.sqrt(np.mean(o * o, axis=1, keepdims=True))
    scaled = np.abs(gg - o) / np.maximum(np.abs(o), rms)
    return float(np.max(scaled)), float(np.mean(np.abs(gg - o)))


def assert_out(gpu_bits, res, rows=None, rtol=OUT_RTOL):
    mx, mae = out_errors(gpu_bits, res, rows)
    assert mx <= rtol, f"max scaled error {mx:.3e} > {rtol} (MAE {mae:.3e})"
    return mx, mae


def assert_states(gpu_kv, gpu_sc, w, res):
    for name, g, inp, ref, wr in (("kv", gpu_kv, w["kv_state"], res.kv_state, res.kv_written),
                                  ("score", gpu_sc, w["score_state"], res.score_state,
                                   res.score_written)):
        changed = np.any(g.view(np.uint32) != np.asarray(inp, np.float32).view(np.uint32), axis=2)
        assert np.array_equal(changed, wr), (
            f"{name}: written-slot mask differs at {np.argwhere(changed != wr)[:8].tolist()}")
        if wr.any():
            gw, ow = g[wr].astype(np.float64), ref[wr].astype(np.float64)
            err = np.abs(gw - ow) / np.maximum(np.abs(ow), 1.0)
            assert err.max() <= STATE_TOL, f"{name}: state error {err.max():.3e}"
