"""Build libkvarn.so (HIP for gfx950) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvarn.so")
SOURCES = ["api.cpp", "quantize.hip", "quantize_d128.hip", "quantize_d256.hip", "quantize_d512.hip",
           "decode_gqa.hip", "decode_gqa_w128.hip", "decode_gqa_w256.hip", "decode_gqa_w512.hip", "decode_mla.hip",
           "noalloc.hip", "commit.hip"]
HEADERS = ["kvarn_device.hpp", "kvarn_internal.hpp", "quantize_impl.hpp", "decode_gqa_impl.hpp",
           "decode_gqa_wide.hpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU forms anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# min/max reductions in the quantizer need no NaN canonicalization: inputs are
# finite fp16 values
EXTRA = {"quantize_d128.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee",
                              # the rotation's MFMA accumulators stay in ordinary VGPRs
                              "-mllvm", "-amdgpu-mfma-vgpr-form=1",
                              # loop heads on 64-byte instruction-cache lines (1-2 % on
                              # the D = 128 layers under the default scheduler, neutral
                              # under the one below and for D = 256 and 512)
                              "-falign-loops=64",
                              # see the note on the scheduler below
                              "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
         # The quantizer is bound by VALU issue and by dependent chains between
         # its barriers; the iterative ILP scheduler interleaves independent
         # rows and channels further than the default occupancy-driven one,
         # at the same occupancy (A/B in one process: 2-6 % on all five layers)
         "quantize_d256.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form=1",
                               "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
         "quantize_d512.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
         "decode_gqa.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_gqa_w128.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_gqa_w256.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_gqa_w512.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "decode_mla.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee",
                            # keep MFMA accumulators in ordinary VGPRs: the loop-carried
                            # output tile is otherwise copied to and from AGPRs every chunk
                            "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build() -> str:
    """Compile every source to an object in parallel, then link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for s in sources():
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [hipcc] + [f for f in FLAGS if f != "-shared"] + EXTRA.get(os.path.basename(s), []) + inc + \
            ["-c", s, "-o", o]
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = False
    for s, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that note is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"compile failed: {s}\n")
    if failed:
        raise RuntimeError("hipcc compile failed")
    tmp = LIB + ".tmp"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
