"""Compile the HIP sources of the package into libq4gemv.so (gfx950, in-tree).

    python -m q4_dequant_gemv_block_amd.build

Every call compiles: a stale library never survives a source change.
"""
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4gemv.so")
# the read-bandwidth probe the benchmark quotes the GEMV against (not part of the GEMV library)
STREAM_SRC = "stream.hip"
STREAM_LIB = os.path.join(HERE, "libq4stream.so")
SOURCES = ["gemv.hip", "smallm.hip", "prefill.hip", "verify.hip", "q8.hip", "api.cpp"]
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-ffp-contract=fast",
    "-Wall",
    # packed fp32 forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a work-queue atomic is issued by one lane and its result read much later;
    # the wave-aggregating rewrite would wait for it (and every older load) at once
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    # keep per-case updates of named accumulators as branches: merging them
    # into one store through a computed address would move the accumulators
    # to scratch memory
    "-mllvm", "-simplifycfg-sink-common=false",
    # per-kernel register and scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
    "-I" + os.path.join(ROOT, "include"),
]

_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|VGPRs|AGPRs):\s+(\S+)")


def check_resources(stderr: str, src: str) -> list:
    """Per-kernel resource report from the compiler's remarks; raises if a
    kernel of `src` uses scratch memory (private arrays or register spills)."""
    kernels, cur = [], None
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = {"name": val}
            kernels.append(cur)
        elif cur is not None:
            cur[key] = val
    bad = [k for k in kernels if k.get("ScratchSize [bytes/lane]", "0") != "0" or k.get("VGPRs Spill", "0") != "0"]
    if bad:
        raise RuntimeError("%s: kernels using scratch memory: %s" % (
            src, ", ".join("%s (scratch %s, vgpr spill %s)" % (k["name"], k.get("ScratchSize [bytes/lane]"),
                                                                k.get("VGPRs Spill")) for k in bad)))
    return kernels


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False, defines=()) -> str:
    """Compile every source and link libq4gemv.so; `defines` are extra -D flags."""
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        cmd = [hipcc()] + FLAGS + ["-D" + d for d in defines] + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
        diag = "\n".join(l for l in r.stderr.splitlines()
                         if "kernel-resource-usage" not in l and "packed-fp32-ops" not in l
                         and not re.match(r"^\s*\d*\s*\|", l))
        if diag.strip():
            print(diag, file=sys.stderr, flush=True)
        if r.returncode != 0:
            raise subprocess.CalledProcessError(r.returncode, cmd)
        if src.endswith(".hip"):
            for k in check_resources(r.stderr, src):
                if verbose:
                    print("  %-100s vgpr %s agpr %s sgpr-spill %s" % (k["name"][:100], k.get("VGPRs"), k.get("AGPRs"),
                                                                     k.get("SGPRs Spill")), flush=True)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    tmp = STREAM_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + FLAGS + ["-shared", os.path.join(CSRC, STREAM_SRC), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    if r.returncode != 0:
        print(r.stderr, file=sys.stderr, flush=True)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    check_resources(r.stderr, STREAM_SRC)
    os.replace(tmp, STREAM_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
