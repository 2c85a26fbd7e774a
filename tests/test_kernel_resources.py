"""The compiled kernels keep the resource shape their speed depends on: a
build-level check, no GPU.

A device-only compile of the library, with the build's own flags, reports
each kernel's VGPRs, scratch and occupancy, and its assembly shows whether
any scratch access is left in a kernel's body.  (A callee's frame counts in
the reported scratch size without any access in the body: the statistics
variants call their finishing code out of line on purpose, and the logits
walk's rare wide acceptance test is out of line too.)  What these checks
catch has happened: one more call site of an inlined helper pushed two
helpers out of line, the kernel arguments went to scratch, every buffer
descriptor became a per-lane value, and the sampled pass took 405 instead of
215 us; an address hoisted out of the logits walk and spilled made every
step's reduction wait for its row loads.  The assembly must also hold no
packed fp32 instruction (the build turns them off).
"""
import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_verification_row_amd import build as sv_build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not on PATH")

# (kernel, template arguments) -> least occupancy; every listed kernel must
# have no scratch access in its body.  sv_sample_kernel<VEC, STATS, ROWS,
# EARLY>, sv_logits_kernel<VEC, ROWS, EARLY>, sv_greedy_kernel<VEC, STATS>.
KERNELS = {
    ("sv_sample_kernel", (1, 0, 0, 0)): 4,   # walks, the benchmark's pass
    ("sv_sample_kernel", (1, 0, 1, 0)): 4,   # one block per draft row
    ("sv_sample_kernel", (1, 0, 0, 1)): 4,   # early exit
    ("sv_sample_kernel", (1, 1, 0, 0)): 4,   # with row statistics
    ("sv_sample_kernel", (0, 0, 0, 0)): 4,   # unaligned rows (scalar loads)
    ("sv_logits_kernel", (1, 0, 0)): 4,
    ("sv_logits_kernel", (1, 0, 1)): 4,
    ("sv_greedy_kernel", (1, 0)): 4,
    ("sv_greedy_kernel", (1, 1)): 4,
}


def _mangled(name, args):
    return "_ZN12_GLOBAL__N_1%d%sI%sEEvNS_4ArgsE" % (len(name), name, "".join("Lb%dE" % a for a in args))


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("kres") / "sv_verify.s")
    cmd = [c for c in sv_build.command(out) if c not in ("-shared", "-Wall")]
    cmd += ["--offload-device-only", "-S", "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    remarks = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            remarks[name] = {}
            continue
        m = re.search(r"remark: .*?\s{2,}([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if name and m:
            remarks[name][m.group(1).strip()] = m.group(2)
    with open(out) as f:
        asm = f.read()
    os.remove(out)
    return remarks, asm


def _body(asm, sym):
    i = asm.index(sym + ":")
    return asm[i:asm.index(".Lfunc_end", i)]


@pytest.mark.parametrize("key", list(KERNELS), ids=lambda k: "%s<%s>" % (k[0], ",".join(map(str, k[1]))))
def test_kernel_occupancy_and_no_scratch_in_body(compiled, key):
    remarks, asm = compiled
    sym = _mangled(*key)
    assert sym in remarks, f"{sym} not reported"
    r = remarks[sym]
    assert int(r["Occupancy"]) >= KERNELS[key], r
    assert int(r["VGPRs Spill"]) == 0, r
    body = _body(asm, sym)
    n = len(re.findall(r"^\s*scratch_(?:load|store)", body, re.M))
    assert n == 0, f"{n} scratch accesses in the body of {sym}"


def test_no_packed_fp32_instructions(compiled):
    _, asm = compiled
    assert not re.search(r"\bv_pk_(?:add|mul|fma)_f32\b", asm)
