"""The committed rocprofv3 summaries under profiles/ were taken on the current kernel sources: each
records the sha256 of the source files it covers, and a kernel change that was not profiled again
leaves a stale figure behind. The forward's summaries that name no files cover flashgau.hip,
kernels.h and common.h (the files bench.py hashes before it quotes their HBM bytes)."""

import hashlib
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "efficient_transformer_attention_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
FORWARD = ("flashgau.hip", "kernels.h", "common.h")


def _sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _summaries():
    return sorted(f for f in os.listdir(PROFILES) if f.endswith(".txt"))


def test_there_are_summaries_for_the_forward_backward_and_decoding():
    names = _summaries()
    for part in ("flash_layer_c3_", "flash_layer_backward_c3_", "flash_decode_c3_"):
        assert any(n.startswith(part) for n in names), part


@pytest.mark.parametrize("name", _summaries())
def test_summary_matches_the_current_sources(name):
    with open(os.path.join(PROFILES, name)) as fh:
        text = fh.read()
    m = re.search(r"sha256(?: \(([^)]*)\))?: ([0-9a-f]{64})", text)
    assert m, f"{name} records no source sha256"
    files = tuple(x.strip() for x in m.group(1).split(",")) if m.group(1) else FORWARD
    assert m.group(2) == _sha(files), f"{name} was taken on other sources than {files}"
    assert "command" in text, f"{name} does not give the command that made it"
