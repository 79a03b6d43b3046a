"""A C99 program (tests/abi_c_gpu.c) makes prefill and decode calls through
include/compressor.h with the HIP runtime alone (no Python binding, no
torch): its output rows and both state pools equal those of the Python
binding on the same inputs bit for bit, and match the oracle."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest
import torch

import workloads
from compare import assert_out, assert_states
from oracle import compressor_oracle as O

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def c_caller(tmp_path_factory):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    import long_context_kv_wkv_amd as cmp
    cmp.library()                                # raises if the library is not built
    pkg = os.path.dirname(cmp.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path_factory.mktemp("c_caller") / "abi_c_gpu")
    build = subprocess.run(
        [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "tests", "abi_c_gpu.c"),
         "-L", pkg, "-l:" + os.path.basename(cmp.LIB_PATH), "-L", os.path.join(rocm, "lib"),
         "-lamdhip64", "-Wl,-rpath," + pkg, "-Wl,-rpath," + os.path.join(rocm, "lib"),
         "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    return exe


def _write_case(d, w, decode):
    has_cu = not decode
    fields = (int(decode), w["ratio"], w["head_dim"], w["hidden"], int(w["rotate"]),
              w["block_size"], w["num_blocks"], w["table_stride"], w["T"], w["batch"],
              w["out_rows"], int(has_cu), int(w["kv_block_table"] is not None))
    with open(os.path.join(d, "case.txt"), "w") as f:
        f.write(" ".join(str(int(v)) for v in fields) + "\n")
    arrays = {"x": (w["x"], np.uint16), "wkv": (w["wkv"], np.uint16),
              "wgate": (w["wgate"], np.uint16), "ape": (w["ape"], np.float32),
              "weight": (w["weight"], np.uint16), "cos": (w["cos"], np.uint16),
              "sin": (w["sin"], np.uint16), "hadamard": (w["hadamard"], np.uint16),
              "start_pos": (w["start_pos"], np.int32),
              "cu_seqlens": (w["cu_seqlens"] if has_cu else None, np.int32),
              "seqused": (w["seqused"], np.int32),
              "state_block_table": (w["state_block_table"], np.int32),
              "kv_block_table": (w["kv_block_table"], np.int32),
              "kv_state": (w["kv_state"], np.float32),
              "score_state": (w["score_state"], np.float32)}
    for name, (a, dt) in arrays.items():
        if a is None:
            continue
        a = np.ascontiguousarray(a)
        if dt == np.uint16:
            a = a.view(np.uint16)
        else:
            a = a.astype(dt, copy=False)
        a.tofile(os.path.join(d, name + ".bin"))


@pytest.mark.parametrize("name,mode", [("c4li_small", "prefill"),
                                       ("p1_comp_indexer", "prefill"),
                                       ("decode_c4a_all", "decode"),
                                       ("decode_c128a_all", "decode")])
def test_c_caller_matches_binding_and_oracle(c_caller, tmp_path, name, mode):
    print(f"[case] C caller {name} ({mode})", flush=True)
    sys.stdout.flush()
    import gpu_harness
    w = workloads.build_named(name)
    decode = mode == "decode"
    _write_case(str(tmp_path), w, decode)
    run = subprocess.run([c_caller, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi_c_gpu: ok" in run.stdout
    D = w["head_dim"]
    out = np.fromfile(os.path.join(tmp_path, "out.bin"), np.uint16).reshape(w["out_rows"], D)
    kv = np.fromfile(os.path.join(tmp_path, "kv_out.bin"), np.float32).reshape(
        w["kv_state"].shape)
    sc = np.fromfile(os.path.join(tmp_path, "score_out.bin"), np.float32).reshape(
        w["score_state"].shape)
    # the Python binding on the same inputs
    case = gpu_harness.DeviceCase(w)
    getattr(case, mode)()
    torch.cuda.synchronize()
    assert case.device_error() == 0
    assert np.array_equal(out, case.out_bits())
    kb, sb = case.states()
    assert np.array_equal(kv.view(np.uint32), kb.view(np.uint32))
    assert np.array_equal(sc.view(np.uint32), sb.view(np.uint32))
    # and the oracle
    res = O.compressor(w)
    mx, mae = assert_out(out, res)
    assert_states(kv, sc, w, res)
    print(f"C caller {name}: max scaled err {mx:.2e}, MAE {mae:.2e}")
