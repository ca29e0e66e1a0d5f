"""Resource report of the built library's gfx950 code objects (CPU only).

The kernels are tuned to run without register spills: a spill puts per-lane scratch
traffic in the weight stream's way. The library's `.hip_fatbin` section holds one
clang offload bundle per HIP source; the gfx950 code object of each carries the
compiler's AMDGPU metadata (one record per kernel), which llvm-readelf prints. Every
kernel must report no private segment and no vector-register spills (scalar spills,
which go to vector-register lanes, stay few outside the element-wise fallback), and
every kernel family the launchers name must be present.
"""

from __future__ import annotations

import os
import re
import shutil
import struct
import subprocess

import pytest

import block_quantized_weight_amd as bqw

READELF = next((p for p in (shutil.which("llvm-readelf"), "/opt/rocm/llvm/bin/llvm-readelf")
                if p and os.path.exists(p)), None)
LIB = os.path.join(os.path.dirname(os.path.abspath(bqw.__file__)), "libqgemv.so")
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

pytestmark = pytest.mark.skipif(READELF is None or not os.path.exists(LIB),
                                reason="needs llvm-readelf and the built libqgemv.so")


def _section(path, name):
    out = subprocess.run([READELF, "-S", "-W", path], capture_output=True, text=True, check=True).stdout
    for line in out.splitlines():
        f = line.split()
        if name in f:
            i = f.index(name)
            off, size = int(f[i + 3], 16), int(f[i + 4], 16)
            with open(path, "rb") as fh:
                fh.seek(off)
                return fh.read(size)
    raise AssertionError(f"{name} not found in {path}")


def _gfx950_objects(blob):
    """Code objects for gfx950 from every offload bundle in blob (bundle layout: the
    magic, an entry count, then per entry offset, size, triple length and triple)."""
    objs, pos = [], 0
    while True:
        p = blob.find(BUNDLE_MAGIC, pos)
        if p < 0:
            return objs
        (count,) = struct.unpack_from("<Q", blob, p + 24)
        q = p + 32
        for _ in range(count):
            eoff, esize, tlen = struct.unpack_from("<QQQ", blob, q)
            q += 24
            triple = blob[q:q + tlen].decode()
            q += tlen
            if triple.endswith("gfx950"):
                objs.append(blob[p + eoff:p + eoff + esize])
        pos = p + len(BUNDLE_MAGIC)


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    objs = _gfx950_objects(_section(LIB, ".hip_fatbin"))
    assert len(objs) == 4, ("one gfx950 code object per HIP source expected (two kernel files, the scratch array, "
                            "the tuner's cache sweep)")
    recs = {}
    for i, obj in enumerate(objs):
        path = tmp_path_factory.mktemp("co") / f"co{i}.o"
        path.write_bytes(obj)
        notes = subprocess.run([READELF, "--notes", str(path)], capture_output=True, text=True, check=True).stdout
        # one metadata record per kernel: fields up to and including .wavefront_size
        cur = {}
        for line in notes.splitlines():
            m = re.match(r"\s*-?\s*\.(\w+):\s+(\S+)\s*$", line)
            if not m:
                continue
            key, val = m.groups()
            cur[key] = val
            if key == "wavefront_size":
                if "name" in cur:
                    recs[cur["name"]] = cur
                cur = {}
    return recs


def test_every_kernel_family_is_built(kernels):
    names = " ".join(kernels)
    for fam in ("k_stream1", "k_stream", "k_generic", "k_mfma", "k_mfma_dma"):
        assert re.search(rf"\d{fam}I", names), fam
    assert re.search(r"\d+k_sweep", names), "k_sweep"
    assert len(kernels) > 100


def test_no_kernel_spills_or_uses_scratch(kernels):
    """No kernel has a private (scratch) segment or spills vector registers. Scalar
    registers may spill into vector-register lanes (no memory traffic: the private
    segment stays empty): a handful in the fast kernels, more only in the
    element-wise fallback."""
    bad = {}
    for name, r in kernels.items():
        sgpr = int(r.get("sgpr_spill_count", 0))
        vals = (int(r.get("private_segment_fixed_size", 0)), int(r.get("vgpr_spill_count", 0)),
                0 if ("k_generic" in name or sgpr <= 4) else sgpr)
        if any(vals):
            bad[name] = vals
    assert not bad, f"{len(bad)} kernels spill: {sorted(bad.items())[:5]}"


def test_wave64_and_register_budgets(kernels):
    """wave64 everywhere, and no kernel beyond the 512 registers of one wave per SIMD."""
    for name, r in kernels.items():
        assert r.get("wavefront_size") == "64", name
        assert int(r["vgpr_count"]) + int(r.get("agpr_count", 0)) <= 512, name
