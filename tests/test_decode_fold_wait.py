"""The decode kernel's early-row wait, checked in its own gfx950 assembly (no GPU needed).

A split item whose workgroup has a next item issues that item's first rows after its partial
stores and then waits with a vmcnt that leaves exactly those row loads in flight; since vector
memory operations complete in issue order, the partial stores are then complete before the
arrival count.  That holds only if the compiler emits, between the two scheduling barriers
around the row loads, as many vector-memory instructions as the wait leaves outstanding.  This
test builds the kernel source to assembly and checks that count for every folding
instantiation (bf16 and E4M3, both head dims, soft cap, contiguous cache).
"""
import os
import re
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

SRC = os.path.join(ROOT, "block_sparse_paged_bsr_amd", "csrc", "kernels", "attn_decode_bf16.hip")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


@pytest.mark.skipif(not HIPCC, reason="hipcc not found")
def test_early_row_wait_matches_the_loads_issued(tmp_path):
    out = tmp_path / "dec.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip", "--cuda-device-only", "-S",
           SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = out.read_text().splitlines()
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN3bsr23attn_decode_bf16_kernel\w*:", l)]
    assert starts
    checked = 0
    for i in starts:
        name = lines[i].split(":")[0]
        # template arguments <D, CAP, KV8, FOLD, AFF> in the mangled name
        args = re.search(r"ILi(\d+)ELb([01])ELb([01])ELb([01])ELb([01])EE", name)
        assert args, name
        fold = args.group(4) == "1"
        end = next(k for k in range(i, len(lines)) if lines[k].startswith(".Lfunc_end"))
        body = lines[i:end]
        bars = [k for k, l in enumerate(body) if "sched_barrier" in l]
        if not fold:
            assert not bars, name
            continue
        assert len(bars) == 2, (name, len(bars))
        a, b = bars
        vmem = [l for l in body[a:b] if re.match(r"\s*(global_|buffer_|flat_)", l)]
        assert all(re.match(r"\s*global_load_dwordx4", l) for l in vmem), (name, vmem)
        wait = re.match(r"\s*s_waitcnt vmcnt\((\d+)\)\s*$", body[b + 1])
        assert wait, (name, body[b + 1])
        assert int(wait.group(1)) == len(vmem) > 0, (name, wait.group(0), len(vmem))
        checked += 1
    assert checked == 10  # bf16 x {cap, no cap} x {d 64, 128}, E4M3 x 2 x 2, contiguous x 2
