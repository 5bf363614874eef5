"""pytest configuration: the ``gpu`` marker and import paths.

CPU tests (``-m "not gpu"``) cover the oracle against its pins, the seeded
generator, the host-side stream logic of the library (error paths and empty
batches launch nothing), and that the library exports every declared symbol.
GPU tests (``-m gpu``) compare the HIP path with the oracle.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")
