"""Build libdsp.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m draft_sampling_lossless_markov_amd.build
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsp.so")
SOURCES = ["draft.hip", "confidence.hip", "schedule.hip", "verify.hip", "sts.hip", "api.cpp"]
ARCH = "gfx950"


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _flags(extra=()):
    # packed-fp32 instructions are disabled: the compiler must not form
    # v_pk_{add,mul,fma}_f32 from scalar fp32 code.  MFMA results go to VGPRs
    # rather than AGPRs: the softmax epilogues read every accumulator with VALU
    # instructions, and the accumulator moves cost more than the AGPR form saves.
    return [*extra, "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result"]


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, src + ".o")
    cmd = [_hipcc(), *_flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return obj, noise


def build(verbose: bool = False, lib: str = LIB, build_dir: str = BUILD, extra=()) -> str:
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, build_dir, extra), SOURCES))
    for _, noise in results:
        if verbose and noise.strip():
            print(noise)
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
           *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
