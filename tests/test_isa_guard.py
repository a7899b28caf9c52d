"""CPU guard on the gfx950 assembly of the library's kernels (built here from source).

* Every matrix product uses the one MFMA shape, v_mfma_f32_16x16x32_bf16.  A chain
  that accumulated a 16x16x16 product onto the result of a 16x16x32 one read part
  of its accumulator before that was written (caught by the GPU parity tests); the
  most likely cause is a missing wait between MFMAs of different pass counts, which
  one shape throughout cannot meet.  This test fails as soon as a second shape
  appears, before any GPU run.
* No packed fp32 VALU instruction is emitted (the build disables the feature).
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from gated_delta_rule_62_amd import _build

ALLOWED_MFMA = {"v_mfma_f32_16x16x32_bf16"}


@pytest.fixture(scope="module")
def device_asm():
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        for src in _build.SOURCES:
            asm = os.path.join(tmp, src + ".s")
            cmd = ([_build.hipcc()] + _build.HIP_FLAGS +
                   ["--cuda-device-only", "-S", "-x", "hip", os.path.join(_build.CSRC, src),
                    "-o", asm])
            subprocess.run(cmd, check=True, capture_output=True)
            out[src] = open(asm).read()
    return out


def _mnemonics(text):
    ops = set()
    for line in text.splitlines():
        line = line.split(";")[0].strip()
        if line and not line.startswith((".", "_")) and not line.endswith(":"):
            ops.add(line.split()[0])
    return ops


def test_one_mfma_shape(device_asm):
    kernel_ops = _mnemonics(device_asm["kda_kernel.hip"])
    mfma = {op for op in kernel_ops if op.startswith("v_mfma")}
    assert mfma == ALLOWED_MFMA, mfma
    for src, text in device_asm.items():
        other = {op for op in _mnemonics(text) if op.startswith(("v_mfma", "v_smfmac"))}
        assert other <= ALLOWED_MFMA, (src, other)


def test_no_packed_fp32(device_asm):
    for src, text in device_asm.items():
        packed = {op for op in _mnemonics(text) if re.match(r"v_pk_\w+_f32", op)}
        assert not packed, (src, packed)
