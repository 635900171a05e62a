"""Build libgemmtune.so (HIP kernels for gfx950 + the host library) in-tree.

    python -m gemm_autotuning_amd.build            # incremental
    python -m gemm_autotuning_amd.build --force    # rebuild everything

Objects go to _build/ at the repository root; the library lands next to this
file, where the Python binding loads it.
"""
import concurrent.futures
import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
KDIR = os.path.join(CSRC, "kernels")
BUILD = os.path.join(ROOT, "_build")
GEN = os.path.join(BUILD, "gen")
LIB = os.path.join(PKG, "libgemmtune.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wno-unused-result",
             # packed fp32 instructions stay off (hipcc emits them from plain
             # float code otherwise); the host pass ignores the feature
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", KDIR, "-I", CSRC, "-I", GEN]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(ROCM, "include"), "-I", CSRC, "-I", GEN]
HOST_SOURCES = ["key.cpp", "candidates.cpp", "tuner.cpp", "cache.cpp", "device.cpp", "heuristic.cpp", "offline.cpp", "api.cpp"]


def _headers(kernel=False):
    """Headers an object depends on: device code sees only the kernel
    headers, the argument structs and the generated lists; host code sees
    every header."""
    if kernel:
        return glob.glob(os.path.join(KDIR, "*.h")) + [os.path.join(CSRC, "gt_args.h")] + \
            glob.glob(os.path.join(GEN, "*.inc"))
    hs = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(KDIR, "*.h"))
    hs += glob.glob(os.path.join(ROOT, "include", "*.h")) + glob.glob(os.path.join(GEN, "*.inc"))
    return hs


def _stale(obj, src, headers):
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(x) > t for x in [src] + headers)


def _compile(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, "\n".join(lines), cmd


def _resources(out):
    """Per-kernel resource remarks of one HIP compile: name -> {field: int}."""
    res, cur = {}, None
    for ln in out.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", ln)
        if m:
            cur = res.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\d+)", ln)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return res


def kernel_objects():
    """The HIP objects the library links (the current generation's shards
    only; a shard left from a larger earlier family is not among them)."""
    srcs = [os.path.join(KDIR, "small_kernels.hip"), os.path.join(KDIR, "gemv.hip"), os.path.join(KDIR, "scratch.hip")]
    srcs += sorted(glob.glob(os.path.join(GEN, "tiles_*.hip")))
    return [os.path.join(BUILD, os.path.basename(x) + ".o") for x in srcs]


def build(force=False, jobs=None, verbose=False):
    sys.path.insert(0, CSRC)
    try:
        import gen_kernels
    finally:
        sys.path.pop(0)
    os.makedirs(BUILD, exist_ok=True)
    tile_files = gen_kernels.generate(GEN)
    headers, kheaders = _headers(), _headers(kernel=True)
    hip_sources = [os.path.join(KDIR, "small_kernels.hip"), os.path.join(KDIR, "gemv.hip"),
                   os.path.join(KDIR, "scratch.hip")] + tile_files
    jobs_list, objs = [], []
    for src in hip_sources:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        if force or _stale(obj, src, kheaders):
            jobs_list.append([HIPCC] + HIP_FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj])
    for name in HOST_SOURCES:
        src = os.path.join(CSRC, name)
        obj = os.path.join(BUILD, name + ".o")
        objs.append(obj)
        if force or _stale(obj, src, headers):
            jobs_list.append([os.path.join(ROCM, "llvm", "bin", "clang++")] + HOST_FLAGS + ["-c", src, "-o", obj])
    n = jobs or min(16, os.cpu_count() or 4)
    failed, spills = [], []
    with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
        for rc, out, cmd in ex.map(_compile, jobs_list):
            if rc != 0:
                failed.append((cmd, out))
                continue
            # every kernel must fit its registers: scratch means spills
            bad = ["%s: %d bytes/lane of scratch" % (fn, r["ScratchSize [bytes/lane]"])
                   for fn, r in _resources(out).items() if r.get("ScratchSize [bytes/lane]", 0) > 0]
            if bad:
                spills += bad
                os.remove(cmd[-1])  # so the next incremental build checks it again
            if verbose:
                print("\n".join(ln for ln in out.splitlines() if "remark" not in ln))
    if spills:
        raise RuntimeError("kernels spill registers to scratch:\n  " + "\n  ".join(spills))
    if failed:
        for cmd, out in failed[:3]:
            msg = "\n".join(ln for ln in out.splitlines() if "remark" not in ln)
            sys.stderr.write(" ".join(cmd) + "\n" + msg + "\n")
        raise RuntimeError("%d compile step(s) failed" % len(failed))
    lib_stale = force or not os.path.exists(LIB) or any(os.path.getmtime(o) > os.path.getmtime(LIB) for o in objs)
    if lib_stale:
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + [
            "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
        rc, out, _ = _compile(cmd)
        if rc != 0:
            sys.stderr.write(out + "\n")
            raise RuntimeError("link failed")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv, verbose="-v" in sys.argv))
