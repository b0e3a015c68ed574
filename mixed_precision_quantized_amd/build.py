"""Build libkvq.so in-tree for gfx950 with hipcc (cross-compiles without a GPU).

The write path (quantize / pack / reorder) is compiled with -ffp-contract=off and
fp32 denormals kept, so its fp32 arithmetic rounds exactly as IEEE specifies.
Every HIP translation unit is compiled without packed fp32 instructions.

`python build.py --timeline` builds libkvq_timeline.so: the same sources with the decode
kernel's per-wave timeline compiled in (KVQ_WAVE_TIMELINE; kvq_wave_timeline records
it), for `bench.py --timeline`.

`python build.py --sanitize` builds libkvq_san.so instead: the same sources with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (device code is
built as usual), for the CPU tests of the host entry points:

    KVQ_LIBRARY=mixed_precision_quantized_amd/libkvq_san.so \
    LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) ASAN_OPTIONS=detect_leaks=0 \
    python -m pytest -q tests/test_abi_host.py tests/test_tags_and_widths.py tests/test_head_groups.py"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvq.so")
LIB_SAN = os.path.join(HERE, "libkvq_san.so")
LIB_TIMELINE = os.path.join(HERE, "libkvq_timeline.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
HIP = ["--offload-arch=" + ARCH, "-fno-gpu-flush-denormals-to-zero",
       "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [
    ("kvq_host.cpp", ["-ffp-contract=off"]),
    ("kvq_tags.cpp", ["-ffp-contract=off"]),
    ("kvq_write.hip", HIP + ["-ffp-contract=off"]),
    # The decode kernels never rely on NaN semantics (the softmax runs from a finite
    # start, masked logits are -inf); without NaNs to honour, max needs no quieting and
    # DPP row reductions fold into v_max_f32_dpp.
    ("kvq_decode.hip", HIP + ["-fno-honor-nans"]),
    ("kvq_select.hip", HIP),
    ("kvq_prefill.hip", HIP + ["-fno-honor-nans"]),
]


# Host-side sanitizers (each -fsanitize= right after -Xarch_host: never on device code).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False, timeline: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    extra = SANITIZE if sanitize else []
    for src, flags in SOURCES:
        probe = timeline and src == "kvq_decode.hip"  # the other objects are shared
        obj = os.path.join(BUILD, src + (".san.o" if sanitize else ".timeline.o" if probe else ".o"))
        defs = ["-DKVQ_WAVE_TIMELINE"] if probe else []
        cmd = ["hipcc", *COMMON, *flags, *defs, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "packed-fp32-ops"  # host pass does not know the feature: harmless
        err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{err}")
        if err.strip() and verbose:
            print(err, flush=True)
        objs.append(obj)
    out = LIB_SAN if sanitize else LIB_TIMELINE if timeline else LIB
    tmp = out + ".tmp"
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    if sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:], timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
