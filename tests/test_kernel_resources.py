"""Resource use of the hot kernels as the compiler reports it for gfx950 (no GPU
needed): no register spills to scratch memory (a spill costs HBM writes on every
launch and waits on the hot loops), and the selection kernel within the
registers and LDS that let two of its 8-wave workgroups share a CU."""
import concurrent.futures
import os
import re
import subprocess

import pytest

from long_context_prefill_attn_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")

HOT = {  # source -> mangled-name fragments of its hot kernels
    "attention.hip": ["attn_dense_kernel", "attn_blocksparse_kernel"],
    "pool_select.hip": ["select_kernel", "pool_kernel"],
}


def _resources(src):
    """{mangled kernel name: {field: int}} from the compiler's resource remarks."""
    cmd = [B.HIPCC, *B.FLAGS, "-x", "hip", "--cuda-device-only", "-c", os.path.join(B.CSRC, src),
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return out


@pytest.fixture(scope="module")
def resources():
    with concurrent.futures.ThreadPoolExecutor(max_workers=2) as ex:
        parts = dict(zip(HOT, ex.map(_resources, HOT)))
    return parts


def test_hot_kernels_do_not_spill(resources):
    seen = 0
    for src, frags in HOT.items():
        for name, r in resources[src].items():
            if not any(f in name for f in frags) or "merge" in name:
                continue
            seen += 1
            assert r["ScratchSize"] == 0, (name, r)
            assert r["VGPRs Spill"] == 0, (name, r)
    assert seen >= 6   # dense (two variants) and block-sparse, selection (d 64 and 128), pooling


def test_select_kernel_fits_two_workgroups_per_cu(resources):
    sel = {n: r for n, r in resources["pool_select.hip"].items() if "select_kernel" in n and "merge" not in n}
    assert len(sel) == 2
    for name, r in sel.items():
        assert r["VGPRs"] + r.get("AGPRs", 0) <= 128, (name, r)   # four waves per SIMD
        assert r["LDS Size"] <= 160 * 1024 // 2, (name, r)          # two workgroups per CU
