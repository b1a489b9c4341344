"""Register and occupancy budgets of the measured kernels (CPU: compiles the
sources for gfx950 and reads the compiler's resource-usage remarks).

Each kernel below was tuned for a number of resident waves per SIMD that its
LDS footprint allows; two more registers than the budget silently halve the
resident workgroups of the long-stream linear-attention launch (measured:
277 -> 338 us), and a spill puts scratch traffic on the loop.  These checks
make such a change fail at build time instead of showing up as a slower
benchmark."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_recurrent_memory_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (source, mangled-name prefix, minimum waves per SIMD)
BUDGETS = [
    # linear attention, bf16, dk = dv = 64: two four-wave workgroups per CU
    # (uniform batches with the two last-read policies, packed batches)
    ("la_prefill.hip", "_ZN2la12_GLOBAL__N_115la_fused_kernelItLi64ELi64ELb0ELi1E", 2),
    ("la_prefill.hip", "_ZN2la12_GLOBAL__N_115la_fused_kernelItLi64ELi64ELb0ELi2E", 2),
    ("la_prefill.hip", "_ZN2la12_GLOBAL__N_115la_fused_kernelItLi64ELi64ELb1ELi0E", 2),
    # delta rule, dk = dv = 128: T pass four eight-wave workgroups per CU,
    # map pass one sixteen-wave workgroup, output and state passes one
    # eight-wave workgroup
    ("delta_prefill.hip", "_ZN2la12_GLOBAL__N_117delta_tinv_kernelILi128ELb0ELb0E", 8),
    ("delta_prefill.hip", "_ZN2la12_GLOBAL__N_117delta_tinv_kernelILi128ELb1ELb0E", 8),
    ("delta_prefill.hip", "_ZN2la12_GLOBAL__N_118delta_chunk_kernelILi128ELi128ELi0ELb0ELb0ELi16E", 4),
    ("delta_prefill.hip", "_ZN2la12_GLOBAL__N_118delta_chunk_kernelILi128ELi128ELi0ELb1ELb0ELi16E", 4),
    ("delta_prefill.hip", "_ZN2la12_GLOBAL__N_118delta_chunk_kernelILi128ELi128ELi1ELb0ELb0ELi8E", 2),
    ("delta_prefill.hip", "_ZN2la12_GLOBAL__N_118delta_chunk_kernelILi128ELi128ELi1ELb1ELb0ELi8E", 2),
    ("delta_prefill.hip", "_ZN2la12_GLOBAL__N_118delta_chunk_kernelILi128ELi128ELi2ELb0ELb0ELi8E", 2),
    # delta-rule backward, dk = dv = 128: one eight-wave workgroup per CU
    ("delta_backward.hip", "_ZN2la12_GLOBAL__N_116dlb_chain_kernelILi128ELi128ELb0ELb0E", 2),
    ("delta_backward.hip", "_ZN2la12_GLOBAL__N_116dlb_chain_kernelILi128ELi128ELb1ELb0E", 2),
    ("delta_backward.hip", "_ZN2la12_GLOBAL__N_115dlb_grad_kernelILi128ELi128ELb0E", 2),
    ("delta_backward.hip", "_ZN2la12_GLOBAL__N_115dlb_grad_kernelILi128ELi128ELb1E", 2),
]


def _usage(src):
    """{mangled kernel name: {field: int}} from -Rpass-analysis=kernel-resource-usage."""
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    info, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            info[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?): (\d+)", line)
        if m and cur:
            info[cur][m.group(1).strip()] = int(m.group(2))
    return info


@pytest.fixture(scope="module")
def usage():
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    srcs = sorted({s for s, _, _ in BUDGETS})
    with cf.ThreadPoolExecutor(len(srcs)) as ex:
        return dict(zip(srcs, ex.map(_usage, srcs)))


@pytest.mark.parametrize("src,prefix,min_waves", BUDGETS, ids=[p[len("_ZN2la12_GLOBAL__N_1"):][:60] for _, p, _ in BUDGETS])
def test_kernel_keeps_its_occupancy_without_spills(usage, src, prefix, min_waves):
    hits = {k: v for k, v in usage[src].items() if k.startswith(prefix)}
    assert len(hits) == 1, f"{prefix}: {len(hits)} matching kernels"
    (name, u), = hits.items()
    occ = u.get("Occupancy [waves/SIMD]")
    assert occ is not None and occ >= min_waves, (
        f"{name}: {occ} waves per SIMD (VGPRs {u.get('VGPRs')}, AGPRs {u.get('AGPRs')}), needs {min_waves}")
    assert u.get("VGPRs Spill", 0) == 0, f"{name}: {u.get('VGPRs Spill')} VGPRs spilled"
    assert u.get("ScratchSize [bytes/lane]", 0) == 0, f"{name}: scratch {u.get('ScratchSize [bytes/lane]')} B/lane"
