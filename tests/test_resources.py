"""Compile-time resource checks of every HIP kernel (no GPU needed).

Each source of libfa.so is compiled for gfx950 with the compiler's
per-kernel resource report. Every kernel instance must use no scratch
memory (a register spill would put per-lane scratch traffic into the hot
loops) and must fit the 160 KiB of LDS of one compute unit.
"""
import concurrent.futures as cf
import re

import pytest

from exact_attention_41_amd import build

LDS_BYTES = 160 * 1024


def kernel_resources(src: str) -> dict:
    """{kernel name: {"scratch": bytes per lane, "lds": bytes per block}}."""
    out, cur = {}, None
    for line in build.resource_report(src).splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        if cur is None:
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m:
            out[cur]["scratch"] = int(m.group(1))
        m = re.search(r"LDS Size \[bytes/block\]: (\d+)", line)
        if m:
            out[cur]["lds"] = int(m.group(1))
    return out


@pytest.fixture(scope="module")
def reports():
    with cf.ThreadPoolExecutor(max_workers=len(build.SOURCES)) as ex:
        return dict(zip(build.SOURCES, ex.map(kernel_resources, build.SOURCES)))


@pytest.mark.parametrize("src", build.SOURCES)
def test_no_scratch_and_lds_fits(reports, src):
    kernels = {k: v for k, v in reports[src].items() if "scratch" in v}
    if src != "fa_api.hip":
        assert kernels, f"{src}: no kernel found in the resource report"
    for name, r in kernels.items():
        assert r["scratch"] == 0, f"{src}: {name} spills {r['scratch']} bytes per lane"
        assert r.get("lds", 0) <= LDS_BYTES, f"{src}: {name} uses {r['lds']} bytes of LDS"
