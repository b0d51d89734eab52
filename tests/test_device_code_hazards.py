"""Every read of an MFMA result in the compiled attention kernels comes at
least 8 wait states after the MFMA on every control-flow path (the count the
compiler keeps behind the 4-pass MFMAs these kernels use).  A branch placed
straight after the score MFMAs was once compiled with one instruction on the
path that skipped it; the check below would have failed on that build."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

import pytest

from paged_kv_cache_464_amd import build
from tests import asm_hazards

REQUIRED = 8

SYNTHETIC = """\
_Zfake_kernel:
\tv_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], v[0:3]
\ts_cbranch_scc1 .LBB0_2
\ts_nop 7
\tv_max_f32_e32 v12, v0, v1
.LBB0_2:
\tv_max_f32_e32 v13, v2, v3
\tglobal_store_dwordx4 v[20:21], v[0:3], off
\ts_endpgm
.Lfunc_end0:
"""


def test_checker_flags_a_read_on_the_path_that_skips_the_wait():
    (name, body), = asm_hazards.functions(SYNTHETIC)
    found = asm_hazards.check_function(body, REQUIRED)
    # the branch path reaches both reads in .LBB0_2 after one instruction
    assert [(b, ins.split()[0]) for b, _, ins, _ in found] == [(".LBB0_2", "v_max_f32_e32"),
                                                               (".LBB0_2", "global_store_dwordx4")]
    fixed = SYNTHETIC.replace("\ts_cbranch_scc1", "\ts_nop 7\n\ts_cbranch_scc1")
    (name, body), = asm_hazards.functions(fixed)
    assert asm_hazards.check_function(body, REQUIRED) == []


# hipcc's code for an earlier form of the decode step that masked the tail
# scores behind a branch right after the score MFMA (fp16, B = 8, one column
# tile): the path that skips the masking reaches the maxima one instruction
# after the MFMA; the fall-through path has exactly 8 wait states.
BRANCH_MISCOMPILE = """\
_Zdecode_excerpt_kernel:
\tv_cmp_lt_i32_e64 s[6:7], 2, v143
\tv_cmp_lt_i32_e64 s[2:3], 3, v143
\ts_waitcnt vmcnt(10)
\tv_mfma_f32_16x16x32_f16 v[98:101], v[106:109], v[34:37], v[98:101]
\ts_cbranch_scc1 .LBB0_54
; %bb.53:
\ts_or_b64 s[6:7], s[2:3], s[6:7]
\ts_or_b64 s[4:5], s[6:7], s[4:5]
\tv_mov_b32_e32 v102, 0xff800000
\ts_or_b64 vcc, s[4:5], vcc
\ts_nop 2
\tv_cndmask_b32_e64 v100, v102, v100, s[6:7]
\tv_cndmask_b32_e64 v99, v102, v99, s[4:5]
\tv_cndmask_b32_e32 v98, v102, v98, vcc
\tv_cndmask_b32_e64 v101, v102, v101, s[2:3]
.LBB0_54:
\tv_max_f32_e32 v102, v100, v101
\tv_max3_f32 v102, v98, v99, v102
\tv_mov_b32_e32 v103, v102
\ts_endpgm
.Lfunc_end1:
"""


def test_checker_flags_the_branch_miscompile():
    (name, body), = asm_hazards.functions(BRANCH_MISCOMPILE)
    found = asm_hazards.check_function(body, REQUIRED)
    assert [(b, ins.split()[0], miss) for b, _, ins, miss in found] == [
        (".LBB0_54", "v_max_f32_e32", 7), (".LBB0_54", "v_max3_f32", 6)]


def _device_asm(src, defines, out):
    cmd = [build._hipcc(), *build.HIP_FLAGS, *build.COMMON, *build.FILE_FLAGS.get(src, []), *defines,
           "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    return out


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    jobs = [(build.INST_SOURCE, [f"-DPA_INST_KIND={k}", f"-DPA_INST_D={dd}"], str(d / f"inst_k{k}_d{dd}.s"))
            for k, dd in build.INSTANCES]
    jobs += [(src, [], str(d / f"{src}.s")) for src in build.HIP_SOURCES if src.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        return list(ex.map(lambda j: _device_asm(*j), jobs))


def test_mfma_results_are_read_only_after_enough_wait_states(device_asm):
    kernels = 0
    bad = []
    for path in device_asm:
        for name, body in asm_hazards.functions(open(path).read()):
            kernels += 1
            if any("mfma" in line for line in body):
                bad += [(name, b, ins, miss) for b, _, ins, miss in asm_hazards.check_function(body, REQUIRED)]
    assert kernels >= 100
    assert not bad, bad[:10]


def test_every_attention_kernel_uses_the_matrix_cores(device_asm):
    inst = [p for p in device_asm if "inst_" in os.path.basename(p)]
    for path in inst:
        for name, body in asm_hazards.functions(open(path).read()):
            if "decode_kernel" in name or "multi_token_kernel" in name or "shared_prefix_kernel" in name:
                assert any("v_mfma" in line for line in body), name
