"""Build the gfx950 HIP library ``libember.so`` in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libember.so")
SOURCES = ["ember_api.hip", "kernels_misc.hip", "kernels_gemv.hip", "kernels_gemm.hip",
           "kernels_attn.hip", "kernels_flash.hip", "kernels_sample.hip", "kernels_peak.hip"]
ARCH = os.environ.get("EMBER_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         # packed-fp32 VALU ops disabled for every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Wno-unknown-pragmas"]
# per-file device options: the attention kernels keep MFMA results in arch VGPRs (their
# scores and outputs feed VALU work every tile; accumulation registers would cost a move
# per element each way)
FILE_FLAGS = {"kernels_flash.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_build", src + ".o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [hipcc, *[f for f in FLAGS if f != "-shared"], *FILE_FLAGS.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, src))
        objs.append(obj)
    procs = [(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), src)
             for cmd, src in jobs]
    for p, src in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            raise RuntimeError(f"hipcc failed on {src}")
        if verbose and out.strip():
            sys.stderr.write(out)
    tmp = LIB + ".tmp"
    link = [hipcc, *FLAGS, *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
