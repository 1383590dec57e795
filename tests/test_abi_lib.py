"""Which build of the library the binding loaded (run by the sanitized ABI
test, which points QGEMV_LIBRARY at the host-sanitized build)."""
import os

import pytest

qg = pytest.importorskip("block_quant_gemv_amd", reason="libqgemv.so not built")


def test_binding_loads_the_requested_build():
    want = os.environ.get("QGEMV_LIBRARY")
    if want:
        assert qg.lib_path() == want
    else:
        assert qg.lib_path().endswith(os.path.join("block_quant_gemv_amd", "libqgemv.so"))
