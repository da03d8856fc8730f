"""The kernels' register budgets, from the compiler's resource report.

Every kernel must compile without spilling vector registers to scratch, and
the occupancy each launch is sized for (the waves per SIMD that its
`amdgpu_waves_per_eu` asks for, which the host's residency figures and the
merge kernel's LDS sizing assume) must be what the compiler delivers.  The
report is the one the last build wrote next to the library; when it is
missing or older than the sources, the device code is compiled again here
(hipcc cross-compiles for gfx950 without a GPU, in about a minute).
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from rejection_sampling_verifier_amd import build as BUILD

CSRC = os.path.join(BUILD.PKG, "csrc")
INCLUDE = os.path.join(BUILD.ROOT, "include")


def _sources():
    for d in (CSRC, INCLUDE):
        for f in os.listdir(d):
            yield os.path.join(d, f)


def _report_text() -> str:
    path = BUILD.RESOURCES
    if os.path.exists(path) and os.path.getmtime(path) >= max(os.path.getmtime(f) for f in _sources()):
        return open(path).read()
    if not os.path.exists(BUILD.HIPCC):
        pytest.skip("hipcc is not installed")
    flags = [f for f in BUILD.FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as tmp:
        res = subprocess.run([BUILD.HIPCC, "--cuda-device-only", "-c", *flags, "-o", os.path.join(tmp, "k.o"),
                              *BUILD.SOURCES], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return res.stderr


def _demangle(names):
    if shutil.which("c++filt") is None:
        return {n: n for n in names}
    out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout.splitlines()
    return dict(zip(names, out))


@pytest.fixture(scope="module")
def kernels():
    """{demangled kernel name: {field: value}} for every kernel in the report."""
    raw, cur = {}, None
    for line in _report_text().splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = raw.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    names = _demangle(sorted(raw))
    ks = {names[k]: v for k, v in raw.items() if "_kernel" in names[k]}
    assert len(ks) >= 40, sorted(ks)
    return ks


def _find(kernels, pattern):
    hits = {k: v for k, v in kernels.items() if re.search(pattern, k)}
    assert hits, pattern
    return hits


def test_no_kernel_spills_vector_registers(kernels):
    spilled = {k: v["VGPRs Spill"] for k, v in kernels.items() if int(v["VGPRs Spill"]) != 0}
    assert not spilled, spilled


@pytest.mark.parametrize("pattern, waves", [
    (r"stats_kernel<unsigned short, true, 4>", 4),       # dense drafts
    (r"stats_kernel<unsigned short, true, 5>", 5),       # truncated drafts
    (r"[^_]merge_kernel<", 8),                           # all of config 4's 2048 work-groups resident
    (r"ee_first_kernel<unsigned short, true, 6>", 6),    # early exit's first launch, truncated drafts
    (r"early_exit_kernel<unsigned short, true, ", 4),    # the walk
    (r"tree_stats_kernel<unsigned short, true>", 4),
])
def test_occupancy_of_the_measured_kernels(kernels, pattern, waves):
    for name, v in _find(kernels, pattern).items():
        assert int(v["Occupancy [waves/SIMD]"]) == waves, (name, v)


def test_merge_kernel_lds_lets_eight_work_groups_share_a_cu(kernels):
    # 160 KB of LDS per CU on gfx950, eight work-groups of the merge kernel.
    for name, v in _find(kernels, r"[^_]merge_kernel<").items():
        assert int(v["LDS Size [bytes/block]"]) * 8 <= 160 * 1024, (name, v)
