"""Register, LDS and spill figures of every kernel instantiation the library
builds, read from the gfx950 code objects' AMDGPU metadata notes.

Each HIP source is compiled for the device only (same flags as build.py,
unbundled), and ``llvm-readelf --notes`` gives, per kernel: VGPRs, AGPRs,
SGPRs, VGPR and SGPR spills, the private (scratch) segment size and the
static LDS (group segment) size.  Waves per SIMD follow from the unified
512-entry register file of a CDNA3/CDNA4 SIMD (VGPRs and AGPRs each
allocated in granules of 8) and the 8-wave cap.  Dynamic LDS (the down
kernel's mid codes, the 1-bit nibble tables) is sized at launch and is not
part of the static figure.

    python -m bit_moe_decode_amd.kernel_resources [out.md]

writes a markdown table (default: profiles/kernel_resources_gfx950.md).
"""
import os
import re
import subprocess
import sys

from . import build as B

LLVM = "/opt/rocm/llvm/bin"
FIELDS = ("vgpr_count", "agpr_count", "sgpr_count", "vgpr_spill_count", "sgpr_spill_count",
          "private_segment_fixed_size", "group_segment_fixed_size", "max_flat_workgroup_size")


def _device_object(src: str) -> str:
    out = os.path.join(B.BUILD, os.path.splitext(src)[0] + f".{B.ARCH}.co")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    cmd = ["hipcc", *flags, "--cuda-device-only", "--no-gpu-bundle-output", "-c",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device-only compile of {src} failed:\n{r.stderr}")
    return out


def _kernels(co: str):
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co],
                           capture_output=True, text=True, check=True).stdout
    # the kernel list: entries start with "  - .agpr_count:" (keys sorted)
    blocks = re.split(r"\n  - (?=\.agpr_count:)", notes)
    out = []
    for b in blocks[1:]:
        name = re.search(r"^\s+\.name:\s+(\S+)", b, re.M)
        if not name:
            continue
        rec = {"mangled": name.group(1)}
        for f in FIELDS:
            m = re.search(rf"^\s+\.{f}:\s+(\d+)", b, re.M)
            rec[f] = int(m.group(1)) if m else 0
        out.append(rec)
    return out


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names),
                       capture_output=True, text=True, check=True)
    return r.stdout.strip().splitlines()


def _waves_per_simd(vgpr, agpr):
    g = lambda n: -(-max(n, 1) // 8) * 8
    return min(8, 512 // (g(vgpr) + (g(agpr) if agpr else 0)))


def collect():
    os.makedirs(B.BUILD, exist_ok=True)
    rows = []
    for src in B.SOURCES:
        ks = _kernels(_device_object(src))
        for k, d in zip(ks, _demangle([k["mangled"] for k in ks])):
            k["name"] = d
            k["source"] = src
            rows.append(k)
    return rows


def write(path: str) -> None:
    rows = collect()
    lines = [
        "# Kernel resources (gfx950 code objects of this library)",
        "",
        "Command: `python -m bit_moe_decode_amd.kernel_resources` (device-only hipcc compile of "
        "each source with the library's flags, then `llvm-readelf --notes`).",
        "Waves/SIMD = min(8, 512 / (VGPRs + AGPRs, each rounded up to 8)); LDS is the static "
        "group segment in bytes (dynamic LDS is sized at launch).",
        "",
        "| source | kernel | VGPR | AGPR | SGPR | VGPR spill | SGPR spill | scratch B | LDS B | "
        "waves/SIMD |",
        "|---|---|---|---|---|---|---|---|---|---|",
    ]
    for k in rows:
        name = k["name"].replace("moe::", "").replace("|", "\\|")
        name = re.sub(r"\(.*\)$", "", name)
        lines.append(
            f"| {k['source']} | `{name}` | {k['vgpr_count']} | {k['agpr_count']} | "
            f"{k['sgpr_count']} | {k['vgpr_spill_count']} | {k['sgpr_spill_count']} | "
            f"{k['private_segment_fixed_size']} | {k['group_segment_fixed_size']} | "
            f"{_waves_per_simd(k['vgpr_count'], k['agpr_count'])} |")
    spills = [k for k in rows if k["vgpr_spill_count"] or k["sgpr_spill_count"]
              or k["private_segment_fixed_size"]]
    lines += ["", f"{len(rows)} kernel instantiations; "
              f"{len(spills)} with spills or scratch."]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    root = os.path.dirname(B.HERE)
    write(sys.argv[1] if len(sys.argv) > 1 else
          os.path.join(root, "profiles", "kernel_resources_gfx950.md"))
