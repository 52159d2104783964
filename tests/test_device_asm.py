"""Every HIP translation unit's gfx950 device code passes the compiler's own instruction
verifier.  Building an object (-c) does not run it; printing assembly (-S) does, and it
rejects instructions whose operands the hardware cannot encode (for instance an inline
constant register where a VGPR is required), which an object build would encode silently.
CPU only: nothing runs on a GPU."""
import os
import subprocess

import pytest

from long_context_attention_sparse_amd import build as bld


@pytest.mark.parametrize("src,flags", bld.SOURCES, ids=[s for s, _ in bld.SOURCES])
def test_device_assembly_verifies(src, flags, tmp_path):
    try:
        hipcc = bld.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    res = subprocess.run([hipcc, *bld.HIP_FLAGS, *flags, "-I", os.path.join(bld.ROOT, "include"), "-I", bld.CSRC,
                          "--cuda-device-only", "-S", os.path.join(bld.CSRC, src), "-o", str(tmp_path / "out.s")],
                         capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "Illegal instruction" not in out, out[-3000:]
