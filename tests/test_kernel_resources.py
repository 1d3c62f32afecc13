"""Kernel resource usage read from the gfx950 code objects (CPU only).

Every kernel of the library must run without scratch memory: private segment
0 bytes and no VGPR spills (a spill to scratch was the pages' own profiler
finding: the one-thread-per-column CUDA kernel's per-thread array lived in
local memory, [P4] onnx-runtime-ep-cuda, src/kernels/linear_attention.rs,
the cooperative kernel's doc).  SGPR spills go to VGPR lanes, not memory, and
are only reported.  The figures come from the code objects' kernel-descriptor
metadata (kernel_manifest.json, written by the build); when the manifest is
older than a source, the sources are compiled afresh into a temporary folder.
"""
import json
import os

import pytest

from gated_delta_rule_serial_amd import build as libbuild


def _manifest(tmp_path_factory):
    srcs = [os.path.join(libbuild.CSRC, f) for f in os.listdir(libbuild.CSRC)]
    if os.path.exists(libbuild.MANIFEST) and \
            os.path.getmtime(libbuild.MANIFEST) >= max(os.path.getmtime(f) for f in srcs):
        return libbuild.load_manifest()
    tmp = str(tmp_path_factory.mktemp("co"))
    old = libbuild.BUILD
    try:
        libbuild.BUILD = tmp
        objs = [libbuild._compile(s) for s in libbuild.SOURCES]
    finally:
        libbuild.BUILD = old
    out = {}
    for obj in objs:
        co = libbuild._code_object(obj)
        if co is not None:
            for name, rec in libbuild._kernels_of(co).items():
                rec["object"] = os.path.basename(obj)[:-2]
                out[name] = rec
    return out


@pytest.fixture(scope="module")
def manifest(tmp_path_factory):
    return _manifest(tmp_path_factory)


def test_every_kernel_is_described(manifest):
    families = {libbuild.kernel_base_name(n) for n in manifest}
    for k in ("decode_kernel", "scan_kernel", "scan_plain_kernel", "chunk_kernel", "chunk_prep_kernel", "chunk_trec_kernel",
              "chunk_state_kernel", "chunk_rows_kernel", "chunk_table_kernel", "wide_prep_kernel",
              "wide_state_kernel", "gate_kernel", "conv_window_kernel", "conv_generic_kernel",
              "conv_state_kernel", "conv_step_kernel", "rmsnorm_kernel"):
        assert k in families, k
    for name, k in manifest.items():
        for field in ("vgprs", "sgprs", "private_segment_bytes", "vgpr_spills", "code_sha256_16"):
            assert field in k, (name, field)


def test_no_kernel_uses_scratch(manifest):
    bad = {n: (k["private_segment_bytes"], k["vgpr_spills"]) for n, k in manifest.items()
           if k["private_segment_bytes"] != 0 or k["vgpr_spills"] != 0}
    assert not bad, f"kernels with scratch (private segment bytes, VGPR spills): {bad}"


def test_hot_path_occupancy(manifest):
    """The decode kernel's register budget (the headline, HBM-bound: it needs
    waves in flight) and the state passes' budgets as designed."""
    fam = {}
    for n, k in manifest.items():
        fam.setdefault(libbuild.kernel_base_name(n), []).append(k)
    assert min(k["waves_per_simd_by_registers"] for k in fam["decode_kernel"]) >= 2
    print(json.dumps({f: {"max_vgprs": max(k["vgprs"] for k in ks), "max_agprs": max(k.get("agprs", 0) for k in ks),
                          "min_waves_per_simd": min(k["waves_per_simd_by_registers"] for k in ks)}
                      for f, ks in sorted(fam.items())}, indent=1))
