"""Register use of the built kernels: no kernel may spill to scratch memory (a spill in the
attention or GEMM main loop turns every iteration into scratch traffic).  Reads the
per-kernel resource table the build writes from the compiler's resource-usage remarks."""
import glob
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "pixel_space_flow_amd")
TABLE = os.path.join(PKG, "_build", "kernel_resources.txt")


def table_rows():
    if not os.path.exists(TABLE):
        pytest.skip("no build yet (python pixel_space_flow_amd/build.py writes the table)")
    newest_src = max(os.path.getmtime(f) for f in glob.glob(os.path.join(PKG, "csrc", "*")))
    if os.path.getmtime(TABLE) < newest_src:
        pytest.skip("kernel sources changed after the last build")
    rows = []
    for line in open(TABLE):
        name, *kv = line.split()
        rows.append((name, {k: int(v) for k, v in (x.split("=") for x in kv)}))
    return rows


def test_no_kernel_spills_to_scratch():
    rows = table_rows()
    assert rows, "empty resource table"
    spills = [(n, r["scratch"]) for n, r in rows if r["scratch"] > 0]
    assert not spills, f"kernels with scratch (bytes/lane): {spills}"


def test_hot_kernels_are_in_the_table():
    names = " ".join(n for n, _ in table_rows())
    for k in ("attn_v2_kernel", "gemm_k32_kernel", "gemm_fast_kernel", "pack_kv_knorm_tile_kernel", "route_kernel"):
        assert k in names, k
