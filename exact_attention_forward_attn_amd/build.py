"""Builds libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

``python -m exact_attention_forward_attn_amd.build`` compiles every source in
``csrc/`` into ``exact_attention_forward_attn_amd/libattn.so``. The build
always recompiles; nothing is cached.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
ARCH = os.environ.get("ATTN_OFFLOAD_ARCH", "gfx950")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fp8.hip", "attn_bwd.hip", "attn_decode.hip"]

# The compiler the kernels were validated with (parity suite green on the
# MI355X). The FP8 kernel pads the read of its last MFMA results by hand
# (this compiler spaced that read one wait state short), which relies on
# this compiler's code generation, so a different hipcc gets a warning (the
# GPU parity tests are the gate).
VALIDATED_HIP = "7.2.26015"

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# packed fp32 VALU forms are kept out of the generated code
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]
# MFMA accumulators in VGPRs: the forward's softmax reads every score, and
# AGPR-resident scores would need a copy per element. The backward keeps its
# dK/dV accumulators in AGPRs instead (they are read once, at the end), which
# its one-wave-per-SIMD dK/dV kernel needs for its register budget.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"attn_bwd.hip"}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, cwd=None):
    try:
        p = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True, timeout=60)
        return p.stdout.strip() if p.returncode == 0 else ""
    except (OSError, subprocess.SubprocessError):
        return ""


def build_info(hipcc):
    """Provenance compiled into attn_version(): the source commit (with
    "+dirty" for uncommitted changes), the HIP compiler and the ROCm release."""
    commit = _run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT) or "unknown"
    if commit != "unknown" and _run(["git", "status", "--porcelain", "--untracked-files=no"], cwd=ROOT):
        commit += "+dirty"
    ver = _run([hipcc, "--version"])
    hip = next((l.split(":", 1)[1].strip() for l in ver.splitlines() if l.startswith("HIP version")), "unknown")
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        rocm = "unknown"
    return {"commit": commit, "hip": hip, "rocm": rocm, "arch": ARCH}


def _compile(args):
    cmd, src = args
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return src, p.returncode, out


def build(verbose: bool = False, out: str = LIB) -> str:
    hipcc = _hipcc()
    info = build_info(hipcc)
    if not info["hip"].startswith(VALIDATED_HIP):
        print(f"warning: hipcc {info['hip']} differs from the validated {VALIDATED_HIP}; "
              "run the GPU parity tests before trusting this build", file=sys.stderr)
    info_def = "-DATTN_BUILD_INFO=\"commit {commit}, hip {hip}, rocm {rocm}, {arch}\"".format(**info)
    tmp = tempfile.mkdtemp(prefix="attn_build_")
    try:
        jobs = []
        objs = []
        for src in SOURCES:
            path = os.path.join(CSRC, src)
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            if src.endswith(".hip"):
                extra = [] if src in NO_VGPR_FORM else VGPR_FORM
                cmd = [hipcc, *HIP_FLAGS, *extra, *COMMON, "-c", path, "-o", obj]
            else:
                cmd = [hipcc, *COMMON, info_def, "-x", "c++", "-c", path, "-o", obj]
            jobs.append((cmd, src))
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            results = list(ex.map(_compile, jobs))
        failed = [r for r in results if r[1] != 0]
        for src, rc, txt in results:
            if verbose or rc != 0:
                if txt.strip():
                    print(f"[{src}]\n{txt}", file=sys.stderr)
        if failed:
            raise RuntimeError("compilation failed: " + ", ".join(r[0] for r in failed))
        tmp_lib = out + ".tmp"
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        p = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if p.returncode != 0:
            raise RuntimeError("link failed:\n" + p.stdout)
        os.replace(tmp_lib, out)
        return out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
