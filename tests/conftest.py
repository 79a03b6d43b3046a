import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs; minutes of CPU time")


@pytest.fixture(params=[128, 256], ids=lambda r: f"bm{r}")
def tile_rows(request):
    """Runs a prefill test once per projection tile height (4-wave 128-row
    and 8-wave 256-row tiles), then restores the automatic choice."""
    import long_context_kv_wkv_amd as cmp
    cmp.compressor_set_prefill_tile_rows(request.param)
    try:
        yield request.param
    finally:
        cmp.compressor_set_prefill_tile_rows(0)
