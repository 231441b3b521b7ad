"""Build libattn_fwd.so and libattn_ceilings.so (gfx950) in-tree with hipcc.

Always recompiles.  The libraries are written next to this file so that they travel
with the source tree; nothing is installed elsewhere.  libattn_ceilings.so holds the
calibration kernels of the roofline (measured MFMA and HBM ceilings), not attention.
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# (source, extra flags): the head-dim-256 instances keep their MFMA accumulators in VGPRs
# (see attn_fwd_d256.hip)
SOURCES = [(os.path.join(HERE, "csrc", "attn_fwd.hip"), []),
           (os.path.join(HERE, "csrc", "attn_fwd_d256.hip"), ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
           (os.path.join(HERE, "csrc", "attn_api.cpp"), [])]
LIBRARY = os.path.join(HERE, "libattn_fwd.so")
CEILINGS_SOURCES = [(os.path.join(HERE, "csrc", "ceilings.hip"), [])]
CEILINGS_LIBRARY = os.path.join(HERE, "libattn_ceilings.so")
# C++ host program that checks the C ABI without Python (links libattn_fwd.so)
C_CHECK_SOURCE = os.path.join(HERE, "csrc", "c_abi_check.cpp")
C_CHECK_BINARY = os.path.join(HERE, "c_abi_check")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code never produces NaN (masked scores are -inf, weights exp2(-inf) = 0), so
    # max/min need no NaN-quieting canonicalisation
    "-Xarch_device", "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(sources, library, verbose, resource_report=None):
    """Compile each (source, flags) to an object (in parallel), then link LIBRARY.

    Returns the error text, or None.  The library is replaced only when everything succeeded.
    """
    stem = os.path.splitext(os.path.basename(library))[0]
    tmpdir = tempfile.mkdtemp(prefix=f".{stem}.", dir=HERE)
    try:
        procs = []
        for src, extra in sources:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc()] + HIPCC_FLAGS + extra + ["-c", "-o", obj, src]
            if resource_report:
                cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), obj))
        outs, objs, failed = [], [], False
        for proc, obj in procs:
            out, err = proc.communicate()
            outs.append(out + err)
            objs.append(obj)
            failed = failed or proc.returncode != 0
        if resource_report:
            with open(resource_report, "w") as f:
                f.write("".join(outs))
        if failed:
            return "".join(outs)
        tmp = os.path.join(tmpdir, os.path.basename(library))
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            return res.stdout + res.stderr
        os.replace(tmp, library)
        return None
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)


def build(verbose=False, resource_report=None):
    """Compile the HIP sources into LIBRARY and CEILINGS_LIBRARY; returns LIBRARY's path.

    resource_report: optional path; when given, the compiler's per-kernel register /
    LDS / occupancy remarks for LIBRARY are written there.
    """
    failed = []
    for sources, library, report in ((SOURCES, LIBRARY, resource_report),
                                     (CEILINGS_SOURCES, CEILINGS_LIBRARY, None)):
        err = _compile(sources, library, verbose, report)
        if err is not None:
            sys.stderr.write(err)
            failed.append(os.path.basename(library))
    if failed:
        raise RuntimeError("hipcc failed: " + ", ".join(failed))
    _build_c_check(verbose)
    return LIBRARY


def _build_c_check(verbose):
    """Compile C_CHECK_SOURCE against the freshly built LIBRARY (rpath: its own directory)."""
    fd, tmp = tempfile.mkstemp(prefix=".c_abi_check.", suffix=".tmp", dir=HERE)
    os.close(fd)
    cmd = [hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           C_CHECK_SOURCE, "-L", HERE, "-lattn_fwd", "-Wl,-rpath,$ORIGIN", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed for {os.path.basename(C_CHECK_BINARY)} "
                           f"(status {res.returncode})")
    os.replace(tmp, C_CHECK_BINARY)


if __name__ == "__main__":
    print(build(verbose=True))
