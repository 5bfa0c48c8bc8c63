"""Shared pytest configuration.

Tests marked ``gpu`` need a real MI355X and call the HIP library through its
C ABI; everything else runs on the CPU (oracle pins, host-side validation and
the library's export table).  If the oracle or libcvx has not been built yet,
it is built once here, before collection.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    if not os.path.exists(os.path.join(ROOT, "conv2d_batchnorm_activation_amd", "libcvx.so")):
        from conv2d_batchnorm_activation_amd import build as cvx_build
        cvx_build.build()
