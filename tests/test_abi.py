"""The C-ABI library loads and exports every function include/*.h declares;
host-only entry points and argument checks work without a GPU."""
import ctypes
import glob
import os
import re

import pytest

import long_context_kv_wkv_amd as cmp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names.update(re.findall(r"^(?:int|const char\*)\s+((?:compressor|nsa)_\w+)\s*\(", src,
                                flags=re.M))
    return names


def test_header_declares_the_binding_exports():
    assert declared_functions() == set(cmp.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = cmp.library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_prefill_tile_rows_setting():
    lib = cmp.library()
    for bad in (-1, 1, 64, 192, 512):
        assert lib.compressor_set_prefill_tile_rows(bad) == 2          # CMP_ERR_INVALID
    for good in (128, 256, 0):
        assert lib.compressor_set_prefill_tile_rows(good) == 0
    with pytest.raises(cmp.CompressorError):
        cmp.compressor_set_prefill_tile_rows(100)


def test_status_strings():
    assert cmp.compressor_status_str(0) == "ok"
    assert "workspace" in cmp.compressor_status_str(4)
    assert cmp.compressor_status_str(99) == "unknown status"


def test_workspace_sizes_and_shape_checks():
    sh = cmp.make_shape(4, 512, 7168, True, 128, 1, 1)
    n = cmp.compressor_prefill_workspace_size(sh, 131072, 1, 32768)
    # pooled rows, staging and split-window statistics; no projection buffer
    assert 32768 * 512 * 4 <= n < 131072 * 2048 * 4
    assert cmp.compressor_decode_workspace_size(sh, 32, 32) > 0
    for bad, status in ((cmp.make_shape(3, 512, 7168, True, 128, 1, 1), 3),
                        (cmp.make_shape(4, 256, 7168, True, 128, 1, 1), 3),
                        (cmp.make_shape(4, 512, 7000, True, 128, 1, 1), 2),
                        (cmp.make_shape(4, 512, 7168, True, 2000, 1, 1), 2),
                        (cmp.make_shape(4, 512, 7168, True, 4, 1, 1), 2),      # stride < 2
                        (cmp.make_shape(4, 512, 7168, True, 128, 1, 1, 32), 3)):
        with pytest.raises(cmp.CompressorError) as ei:
            cmp.compressor_prefill_workspace_size(bad, 64, 1, 16)
        assert ei.value.status == status
    with pytest.raises(cmp.CompressorError) as ei:
        cmp.compressor_decode_workspace_size(sh, 65, 65)
    assert ei.value.status == 3
    # every listed ratio is accepted (table stride covers coff * ratio slots),
    # nothing else
    for r in (2, 8, 16, 32, 64, 128):
        ok = cmp.make_shape(r, 512, 4096, False, 16, 64, -(-r // 16))
        assert cmp.compressor_prefill_workspace_size(ok, 1000, 2, 600) > 0
        assert cmp.compressor_decode_workspace_size(ok, 32, 32) > 0
    for r in (1, 6, 12, 256):
        with pytest.raises(cmp.CompressorError) as ei:
            cmp.compressor_prefill_workspace_size(cmp.make_shape(r, 512, 4096, False, 256, 64, 1),
                                                  64, 1, 16)
        assert ei.value.status == 3


def test_null_arguments_rejected_before_any_launch():
    lib = cmp.library()
    sh = cmp.make_shape(4, 512, 4096, False, 256, 8, 1)
    assert lib.compressor_prefill(ctypes.byref(sh), None, None) == 1
    assert lib.compressor_decode(ctypes.byref(sh), None, None) == 1
    args = cmp.Args()                      # every pointer NULL
    args.batch, args.T = 1, 4
    assert lib.compressor_prefill(ctypes.byref(sh), ctypes.byref(args), None) == 1
    assert lib.compressor_pack_weights(ctypes.byref(sh), None, None, None, None) == 1
    assert lib.compressor_state_init(ctypes.byref(sh), None, None, None) == 1
    reset = lib.compressor_state_reset
    assert reset(ctypes.byref(sh), None, None, None, None, None, 0, 0, None, None) == 0   # n == 0
    assert reset(ctypes.byref(sh), None, None, None, None, None, -1, 4, None, None) == 2
    assert reset(ctypes.byref(sh), None, None, None, None, None, 2, 0, None, None) == 2  # no table rows
    assert reset(ctypes.byref(sh), None, None, None, None, None, 2, 4, None, None) == 1
    code = ctypes.c_int32()
    assert lib.compressor_last_device_error(None, None, ctypes.byref(code)) == 1
    n = ctypes.c_int32()
    ms = ctypes.c_double()
    assert lib.compressor_timing_query(b"gemm", ctypes.byref(n), ctypes.byref(ms)) == 0
    assert n.value == 0
    # timing modes: 0 off, 1 every launch, 2 the projection GEMM only
    for mode, status in ((2, 0), (1, 0), (0, 0), (3, 2), (-1, 2)):
        assert lib.compressor_timing_enable(mode) == status, mode


def test_nsa_shape_checks_before_any_launch():
    lib = cmp.library()
    args = cmp.NsaArgs()                         # every pointer NULL
    good = cmp.make_nsa_shape(32, 128, 32, 16, 128, cmp.NSA_BF16, cmp.NSA_LAYOUT_PAGED)
    assert lib.nsa_compress_with_cache(ctypes.byref(good), ctypes.byref(args), None) == 1
    for bad in (cmp.make_nsa_shape(65, 128, 32, 16, 128, 0, 0),    # too many heads
                cmp.make_nsa_shape(51, 128, 32, 16, 128, 0, 0),    # odd head count above 50
                cmp.make_nsa_shape(32, 136, 32, 16, 128, 0, 0),    # head_dim not a multiple of 16
                cmp.make_nsa_shape(32, 272, 32, 16, 128, 0, 0),    # head_dim above 256
                cmp.make_nsa_shape(32, 128, 80, 16, 128, 0, 0),    # window above 64
                cmp.make_nsa_shape(32, 128, 16, 32, 128, 0, 0),    # window below stride
                cmp.make_nsa_shape(32, 128, 32, 24, 128, 0, 0),    # stride not 16/32/48/64
                cmp.make_nsa_shape(32, 128, 32, 16, 256, 0, 0),    # page size
                cmp.make_nsa_shape(32, 128, 32, 16, 128, 2, 0),    # dtype
                cmp.make_nsa_shape(32, 128, 32, 16, 128, 0, 2)):   # layout
        assert lib.nsa_compress_with_cache(ctypes.byref(bad), ctypes.byref(args), None) == 3


def test_epilog_argument_checks_before_any_launch():
    lib = cmp.library()
    f = lib.compressor_epilog
    assert f(None, 0, 512, None, None, None, 0, None, None) == 0          # nothing to do
    assert f(None, 4, 512, None, None, None, 8, None, None) == 1          # NULL rows
    for n, d, slots in ((4, 100, 8), (4, 0, 8), (4, 8320, 8), (-1, 512, 8), (4, 512, -1)):
        assert f(None, n, d, None, None, None, slots, None, None) == 2, (n, d, slots)
    # the block count must stay below 2^31
    assert f(None, 2 ** 31 - 1, 8192, None, None, None, 8, None, None) == 2


def test_every_decode_layout_fits_the_noalloc_scratch():
    """compressor_decode_noalloc works in a fixed per-device scratch of
    CMP_DECODE_SCRATCH_BYTES: the decode workspace of every accepted shape
    at the largest batch fits it."""
    src = open(os.path.join(ROOT, "include", "compressor.h")).read()
    m = re.search(r"#define CMP_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    limit = int(m.group(1)) << int(m.group(2))
    worst = 0
    for r in (2, 4, 8, 16, 32, 64, 128):
        for d in (128, 512):
            for h in range(1024, 10241, 512):
                coff = 2 if r == 4 else 1
                sh = cmp.make_shape(r, d, h, False, 16, 64, -(-coff * r // 16))
                worst = max(worst, cmp.compressor_decode_workspace_size(sh, 64, 64))
    assert 0 < worst <= limit, (worst, limit)
    lib = cmp.library()
    sh = cmp.make_shape(4, 512, 4096, False, 256, 8, 1)
    assert lib.compressor_decode_noalloc(ctypes.byref(sh), None, None, None) == 1


def test_ceiling_probe_library_loads():
    """libpeak.so (the benchmark's measured MFMA and HBM ceilings) is built
    beside the operator library and rejects bad arguments before any launch."""
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_kv_wkv_amd", "libpeak.so"))
    lib.peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p]
    assert lib.peak_mfma_bf16(None, None, 1, 2, None) != 0
    assert lib.peak_mfma_bf16(1, 1, 1, 3, None) != 0            # odd iteration count
    assert lib.peak_stream_read(None, 16384, None, 1, None) != 0
    assert lib.peak_stream_read(1, 1000, 1, 1, None) != 0       # not a multiple of 16 KiB


def test_c99_caller_links_and_calls_host_paths(tmp_path):
    """tests/abi_c_check.c, compiled as C99 with warnings as errors against
    include/*.h and linked to the built library, passes its host-only checks
    (the prototypes and structs as a C caller sees them)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    cmp.library()                                # raises if the library is not built
    pkg = os.path.dirname(cmp.LIB_PATH)
    exe = str(tmp_path / "abi_c_check")
    build = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                            "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "abi_c_check.c"),
                            "-L", pkg, "-l:" + os.path.basename(cmp.LIB_PATH),
                            "-Wl,-rpath," + pkg, "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi_c_check: 0 failures" in run.stdout


def test_binding_checks_tensor_sizes_against_the_shape():
    """make_args(shape=...) refuses tensors whose sizes differ from what the
    C ABI reads or writes for the shape (the library sees plain pointers)."""
    import torch
    sh = cmp.make_shape(4, 128, 1024, True, 16, 6, 1)
    B, T, out_rows = 2, 40, 12
    bf, f, i = torch.bfloat16, torch.float32, torch.int32
    good = dict(x=torch.empty(T, 1024, dtype=bf), batch=B,
                kv_state=torch.empty(6, 16, 256), score_state=torch.empty(6, 16, 256),
                state_block_table=torch.zeros(B, 1, dtype=i),
                w_packed=torch.empty(512, 1024, dtype=bf), ape=torch.empty(4, 256),
                norm_weight=torch.empty(128, dtype=bf), sin=torch.empty(out_rows, 64, dtype=bf),
                cos=torch.empty(out_rows, 64, dtype=bf), out=torch.empty(out_rows, 128, dtype=bf),
                cu_seqlens=torch.zeros(B + 1, dtype=i), start_pos=torch.zeros(B, dtype=i),
                hadamard=torch.empty(128, 128, dtype=bf))
    cmp.check_sizes(sh, **good)
    bad_cases = {"x": torch.empty(T, 512, dtype=bf), "w_packed": torch.empty(256, 1024, dtype=bf),
                 "ape": torch.empty(128, 256), "norm_weight": torch.empty(64, dtype=bf),
                 "sin": torch.empty(out_rows - 1, 64, dtype=bf),
                 "out": torch.empty(out_rows, 64, dtype=bf),
                 "kv_state": torch.empty(5, 16, 256), "score_state": torch.empty(6, 16, 128),
                 "state_block_table": torch.zeros(B - 1, 1, dtype=i),
                 "kv_block_table": torch.zeros(B, 2, dtype=i),
                 "cu_seqlens": torch.zeros(B, dtype=i), "start_pos": torch.zeros(B + 1, dtype=i),
                 "hadamard": None}
    for name, t in bad_cases.items():
        with pytest.raises(ValueError):
            cmp.check_sizes(sh, **dict(good, **{name: t}))
    # no output rows: the rotary tables are not read
    cmp.check_sizes(sh, **dict(good, out=torch.empty(0, 128, dtype=bf),
                               sin=torch.empty(0, 64, dtype=bf), cos=torch.empty(0, 64, dtype=bf)))


def test_nsa_binding_checks_tensor_sizes():
    import torch
    sh = cmp.make_nsa_shape(4, 32, 32, 16, 64, cmp.NSA_BF16, cmp.NSA_LAYOUT_PAGED)
    bf, i = torch.bfloat16, torch.int32
    good = dict(input=torch.empty(10, 64, 4, 32, dtype=bf), weight=torch.empty(32, 4, dtype=bf),
                slot_mapping=torch.zeros(3, dtype=i), act_seq_len=torch.zeros(3, dtype=torch.int64),
                output_cache=torch.empty(6, 4, 32, dtype=bf), block_table=torch.zeros(3, 2, dtype=i))
    for name, t in (("input", torch.empty(10, 64, 4, 16, dtype=bf)),
                    ("weight", torch.empty(16, 4, dtype=bf)),
                    ("output_cache", torch.empty(6, 2, 32, dtype=bf)),
                    ("act_seq_len", torch.zeros(2, dtype=torch.int64)),
                    ("block_table", torch.zeros(2, 2, dtype=i))):
        with pytest.raises(ValueError):
            cmp.nsa_compress_with_cache(sh, **dict(good, **{name: t}))
    # consistent sizes pass the size checks and then need device tensors
    with pytest.raises(ValueError, match="device tensor"):
        cmp.nsa_compress_with_cache(sh, **good)
