"""The decode kernels that stream records through LDS with LDS-DMA loads wait
for them with fixed s_waitcnt vmcnt counts, which hold only while no other
vector-memory operation of the wave is in flight between the loads and the
wait.  A register spill would put scratch stores there.  This compiles the
two decode sources to gfx950 assembly (no GPU needed) and checks that no
kernel using LDS-DMA loads has a scratch access or a private segment."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "kv_cache_quantization_kvarn_amd"))

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def kernels(asm):
    """(name, body, metadata) of every kernel in an assembly listing."""
    out = []
    for m in re.finditer(r"^(_Z\S+):\s*;\s*@", asm, flags=re.M):
        name = m.group(1)
        end = asm.find("s_endpgm", m.end())
        # the function's own end label bounds the body (it may hold several s_endpgm)
        stop = asm.find(f".Lfunc_end", m.end())
        body = asm[m.end():stop if stop > 0 else end]
        meta = re.search(r"\.name:\s+" + re.escape(name) + r"\b(.*?)(?=\n\s+- \.|\n\.end_amdgpu_metadata)", asm,
                         flags=re.S)
        out.append((name, body, meta.group(1) if meta else ""))
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not installed")
@pytest.mark.parametrize("src", ["decode_gqa.hip", "decode_mla.hip"])
def test_lds_dma_kernels_never_spill(src, tmp_path):
    import build  # the package's build script: the same flags as the library

    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")] + build.EXTRA.get(src, [])
    out = tmp_path / (src + ".s")
    cmd = [HIPCC] + flags + ["-I", os.path.join(ROOT, "include"), "-I", build.CSRC, "--cuda-device-only", "-S",
                             os.path.join(build.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    checked = 0
    for name, body, meta in kernels(asm):
        if "offen lds" not in body:
            continue
        checked += 1
        assert "scratch_" not in body, f"{name}: scratch access in a kernel with LDS-DMA loads"
        m = re.search(r"\.private_segment_fixed_size:\s+(\d+)", meta)
        assert m is None or int(m.group(1)) == 0, f"{name}: private segment in a kernel with LDS-DMA loads"
    assert checked > 0, "no kernel with LDS-DMA loads found"
