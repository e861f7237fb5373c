"""Compile the hardware checks under tests/hw (test infrastructure, not part
of librr) with the library's own compiler flags, in place:
tests/hw/<name>.hip -> tests/hw/lib<name>.so.  Called by
__graft_entry__.build(); needs hipcc, no GPU."""

import os
import subprocess

from collective_communication_reduction_way_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False):
    out = []
    for name in sorted(os.listdir(HERE)):
        if not name.endswith(".hip"):
            continue
        src = os.path.join(HERE, name)
        lib = os.path.join(HERE, "lib" + name[:-4] + ".so")
        cmd = [B.hipcc(), *B.COMMON, *B.DEVICE, "-shared", src, "-o", lib]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        if verbose:
            print(f"  built {os.path.relpath(lib, os.path.dirname(HERE))}", flush=True)
        out.append(lib)
    return out
