"""Test configuration.

Markers: ``gpu`` tests need an MI355X (gfx950) and call the HIP library
through its C ABI; everything else runs on the CPU.  Native libraries are
built in-tree by ``__graft_entry__.build()``; if one is missing the session
builds it once before collecting.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_LIBS = [
    "oracle/libzsoracle.so",
    "seeded_inputs/libzsgen_host.so",
    "seeded_inputs/libzsgen_dev.so",
    "sharded_mixed_precision_zero_amd/libzeroshard.so",
]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU (runs the HIP path)")
    if not all(os.path.exists(os.path.join(ROOT, p)) for p in _LIBS):
        import __graft_entry__

        __graft_entry__.build()
