"""CPU: no kernel of the library spills VGPRs to scratch memory.

Every csrc/*.hip is compiled for gfx950 with the library's own flags to AMD
assembly (device code only) and the per-kernel metadata is read: each kernel
must report `.vgpr_spill_count: 0`.  A spill puts scratch loads and stores
inside the chunk loops, so this guards the register budgets the launch bounds
assume (SGPR spills go to VGPR lanes, not to memory, and are not counted)."""
import concurrent.futures as cf
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asm(src, out_dir):
    from gated_linear_attention_rodimus_amd import build as B
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    p = subprocess.run([B.HIPCC, *B.CFLAGS, "--cuda-device-only", "-S", src, "-o", out],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout
    return out


def _spills(path):
    """(kernel name, vgpr spill count) for every kernel in one assembly file."""
    found, name = [], None
    for line in open(path):
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.match(r"\s+\.vgpr_spill_count:\s+(\d+)", line)
        if m and name is not None:
            found.append((name, int(m.group(1))))
    return found


def test_no_vgpr_spills(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "gated_linear_attention_rodimus_amd", "csrc", "*.hip")))
    assert srcs
    workers = min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        outs = list(ex.map(lambda s: _asm(s, str(tmp_path)), srcs))
    kernels, bad = 0, []
    for o in outs:
        for name, n in _spills(o):
            kernels += 1
            if n:
                bad.append((os.path.basename(o), name, n))
    print(f"{kernels} kernels in {len(outs)} files")
    assert kernels > 100
    assert not bad, bad
