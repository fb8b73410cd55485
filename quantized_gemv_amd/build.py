"""Build libmk (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

Three variants: libmk.so (headline build), libmk_xray.so (compiled with
MK_XRAY, the per-phase timestamp stamps) and libmk_stress.so (compiled with
MK_STRESS: pseudo-random pauses before every exchange store and hand-over,
for the race-detection tests).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["mk_decode.hip", "mk_pack.hip", "mk_prefill.hip", "mk_abi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


VARIANTS = {"": "libmk.so", "xray": "libmk_xray.so", "stress": "libmk_stress.so"}


def lib_path(xray=False) -> str:
    """Path of a library variant: False / "" the headline build, True / "xray"
    the X-ray build, "stress" the stress build."""
    kind = "xray" if xray is True else ("" if xray is False else xray)
    return os.path.join(HERE, VARIANTS[kind])


def build(xray=False, verbose: bool = False, out: str = "") -> str:
    kind = "xray" if xray is True else ("" if xray is False else xray)
    out = out or lib_path(kind)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-FP32 instructions anywhere in the device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # every loop starts on a 64-byte boundary: the exchange polls and
           # the layer loops ran 0.5-1 % faster per token than unaligned
           "-falign-loops=64",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if kind == "xray":
        cmd.append("-DMK_XRAY")
    if kind == "stress":
        cmd.append("-DMK_STRESS")
    cmd.append("-Rpass-analysis=kernel-resource-usage")
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if verbose:
        sys.stderr.write(r.stderr)
    bad = [f"{k}: {v}" for k, v in resource_usage(r.stderr).items()
           if "decode_kernel" in k and (v.get("scratch", 0) or v.get("vgpr_spill", 0))]
    if bad and kind == "":   # the X-ray stamps and stress pauses may spill; those builds are for tests
        os.remove(out + ".tmp")
        raise RuntimeError("decode kernel spills to scratch memory (slow in the layer loop):\n" + "\n".join(bad))
    os.replace(out + ".tmp", out)
    return out


def resource_usage(remarks: str) -> dict:
    """Per kernel: VGPRs, spills and scratch bytes from the compiler's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    keys = {"VGPRs": "vgpr", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
            "ScratchSize [bytes/lane]": "scratch"}
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        text = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        if text.startswith("Function Name:"):
            cur = text.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur and ":" in text:
            k, v = text.rsplit(":", 1)
            if k.strip() in keys:
                try:
                    out[cur][keys[k.strip()]] = int(v.strip())
                except ValueError:
                    pass
    return out


def build_all(verbose: bool = False):
    """Every variant, compiled side by side."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(VARIANTS)) as ex:
        return list(ex.map(lambda k: build(k, verbose), list(VARIANTS)))


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print(p)
