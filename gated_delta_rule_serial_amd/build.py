"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_delta_rule_serial_amd.build [--resources-md PATH]

Every source is compiled for gfx950 only, with packed-FP32 instruction
selection switched off (``-packed-fp32-ops``), then linked into
``gated_delta_rule_serial_amd/libgdn.so``.  Objects go to ``_build/``.

After linking, the gfx950 code object of each object file is taken out of its
offload bundle and read back: its kernel descriptors' metadata (VGPRs, AGPRs,
SGPRs, spills, private segment, static LDS) and a digest of each kernel's
machine code go to ``gated_delta_rule_serial_amd/kernel_manifest.json``.  The
test suite checks that no kernel uses scratch; the benchmark keys its stored
counter records on the digests of the kernels they measured.
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
MANIFEST = os.path.join(PKG, "kernel_manifest.json")
LLVM = "/opt/rocm/llvm/bin"

SOURCES = ["gdn_api.cpp", "gdn_runtime.cpp", "prefill_scan.hip", "prefill_chunked.hip", "prefill_split.hip", "prefill_wide.hip", "decode_step.hip",
           "gate_prologue.hip", "causal_conv.hip", "gated_rmsnorm.hip", "static_workspace.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # CDNA packed FP32 (v_pk_fma_f32 and friends) stays off in all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _code_object(obj: str):
    """The gfx950 code object inside obj's offload bundle, written next to it
    (None for an object without device code)."""
    secs = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-S", "--wide", obj], check=True,
                          capture_output=True, text=True).stdout
    if ".hip_fatbin" not in secs:
        return None
    fatbin = obj + ".fatbin"
    co = obj + f".{ARCH}.co"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}", obj,
                    obj + ".strip.o"], check=True, capture_output=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fatbin}",
                    f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"], check=True,
                   capture_output=True)
    for f in (fatbin, obj + ".strip.o"):
        os.remove(f)
    return co


_FIELDS = {".vgpr_count": "vgprs", ".agpr_count": "agprs", ".sgpr_count": "sgprs",
           ".vgpr_spill_count": "vgpr_spills", ".sgpr_spill_count": "sgpr_spills",
           ".private_segment_fixed_size": "private_segment_bytes",
           ".group_segment_fixed_size": "static_lds_bytes", ".max_flat_workgroup_size": "max_workgroup_size"}


def _kernels_of(co: str) -> dict:
    """Per kernel symbol: resource fields from the code object's metadata note
    and the sha256 (16 hex digits) of its machine code."""
    import yaml
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True, capture_output=True,
                           text=True).stdout
    lines = notes.splitlines()
    first = next(i for i, l in enumerate(lines) if l.startswith("amdhsa.kernels:"))
    doc = []
    for l in lines[first:]:
        if l.strip() == "...":
            break
        doc.append(l)
    kernels = {}
    for k in yaml.safe_load("\n".join(doc))["amdhsa.kernels"]:
        kernels[k[".name"]] = {_FIELDS[f]: int(k[f]) for f in _FIELDS if f in k}
    # machine code digests from the symbol table and the section headers
    secs = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-S", "--wide", co], check=True, capture_output=True,
                          text=True).stdout
    text_addr = text_off = None
    for line in secs.splitlines():
        m = re.search(r"\]\s+\.text\s+PROGBITS\s+([0-9a-f]+)\s+([0-9a-f]+)", line)
        if m:
            text_addr, text_off = int(m.group(1), 16), int(m.group(2), 16)
    syms = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-s", "--wide", co], check=True, capture_output=True,
                          text=True).stdout
    with open(co, "rb") as fh:
        blob = fh.read()
    for line in syms.splitlines():
        parts = line.split()
        if len(parts) >= 8 and parts[3] == "FUNC" and parts[7] in kernels and text_addr is not None:
            addr, size = int(parts[1], 16), int(parts[2])
            code = blob[text_off + addr - text_addr: text_off + addr - text_addr + size]
            kernels[parts[7]]["code_bytes"] = size
            kernels[parts[7]]["code_sha256_16"] = hashlib.sha256(code).hexdigest()[:16]
    for k in kernels.values():
        k.pop("name", None)
        # waves per SIMD that the register file allows (512 registers per lane,
        # granule 8); on gfx950 the vgpr count is already the unified total,
        # the architectural registers (aligned to 4) plus the accumulation ones
        total = k.get("vgprs", 0)
        k["waves_per_simd_by_registers"] = min(8, 512 // max(8, (total + 7) // 8 * 8))
    return kernels


def write_manifest(objs) -> dict:
    """kernel_manifest.json: {mangled kernel name: resources, digest, source}."""
    manifest = {}
    for obj in objs:
        src = os.path.basename(obj)[:-2]
        co = _code_object(obj)
        if co is None:
            continue
        for name, rec in _kernels_of(co).items():
            rec["object"] = src
            manifest[name] = rec
    tmp = MANIFEST + ".tmp%d" % os.getpid()
    with open(tmp, "w") as fh:
        json.dump(manifest, fh, indent=1, sort_keys=True)
    os.replace(tmp, MANIFEST)
    return manifest


def load_manifest() -> dict:
    with open(MANIFEST) as fh:
        return json.load(fh)


def kernel_base_name(mangled: str) -> str:
    """The unqualified template name of a kernel symbol in namespace gdn (or
    gdn's anonymous namespace): _ZN3gdn[12_GLOBAL__N_1]<len><name>..."""
    m = re.match(r"_ZN3gdn(?:12_GLOBAL__N_1)?(\d+)", mangled)
    if not m:
        return mangled
    n = int(m.group(1))
    return mangled[m.end():m.end() + n]


def resources_markdown(manifest: dict) -> str:
    """One row per kernel template: its instantiations' largest register and
    LDS figures, total spills and scratch, and the lowest register occupancy."""
    fam = {}
    for n in sorted(manifest):
        fam.setdefault((kernel_base_name(n), manifest[n]["object"]), []).append(manifest[n])
    rows = ["| kernel | source | instantiations | max VGPR | max AGPR | max SGPR | spills (V+S) | max scratch B | "
            "static LDS B | min waves/SIMD by regs |", "|---|---|---|---|---|---|---|---|---|---|"]
    for (base, obj), ks in sorted(fam.items()):
        lds = sorted({k.get("static_lds_bytes", 0) for k in ks})
        rows.append(f"| `{base}` | {obj} | {len(ks)} | {max(k.get('vgprs', 0) for k in ks)} | "
                    f"{max(k.get('agprs', 0) for k in ks)} | {max(k.get('sgprs', 0) for k in ks)} | "
                    f"{sum(k.get('vgpr_spills', 0) + k.get('sgpr_spills', 0) for k in ks)} | "
                    f"{max(k.get('private_segment_bytes', 0) for k in ks)} | "
                    f"{lds[0] if len(lds) == 1 else f'{lds[0]}-{lds[-1]}'} | "
                    f"{min(k.get('waves_per_simd_by_registers', 8) for k in ks)} |")
    return "\n".join(rows) + "\n"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    write_manifest(objs)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    if len(sys.argv) == 3 and sys.argv[1] == "--resources-md":
        head = ("# Kernel resources (gfx950 code objects of libgdn.so)\n\n"
                "Made by `python -m gated_delta_rule_serial_amd.build --resources-md profiles/kernel_resources.md`: "
                "the metadata of every kernel descriptor in the built code objects.  Dynamic LDS (the chunked "
                "kernels' `extern __shared__` buffers) is not in the static figure.  Waves per SIMD count the "
                "register file alone (512 per lane, granule 8).\n\n")
        with open(sys.argv[2], "w") as fh:
            fh.write(head + resources_markdown(load_manifest()))
    sys.exit(0)
