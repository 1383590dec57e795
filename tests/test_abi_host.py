"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every function include/qgemv.h and include/qattn.h declare, the descriptor layout matches the
binding, and every validation error is reported before anything touches the
device."""
import ctypes
import os
import re
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "qattn.h")]

qg = pytest.importorskip("block_quant_gemv_amd", reason="libqgemv.so not built")
lib = qg._lib

OK, EINVAL, EFORMAT, ESHAPE, EALIGN, EWORKSPACE, EVERSION, EHIP = 0, -1, -2, -3, -4, -5, -6, -7


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(q\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 14 and "qattn_decode" in names and "qattn_workspace_size" in names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", qg.lib_path()], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_descriptor_layout_matches_c(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text(textwrap.dedent(f"""
        #include <stdio.h>
        #include <stddef.h>
        #include "{HEADER}"
        int main(void) {{
          printf("%zu %zu %zu %zu %zu\\n", sizeof(qgemv_desc), offsetof(qgemv_desc, n),
                 offsetof(qgemv_desc, hidden), offsetof(qgemv_desc, n_experts),
                 offsetof(qgemv_desc, codebook16));
          return 0;
        }}"""))
    exe = tmp_path / "sz"
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    D = qg._Desc
    assert got == [ctypes.sizeof(D), D.n.offset, D.hidden.offset, D.n_experts.offset, D.codebook16.offset]


def _desc(**kw):
    d = qg._Desc()
    d.kind, d.layout_version, d.fmt, d.max_m, d.n, d.k = 0, 1, 1, 1, 64, 256
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _create(d):
    h = ctypes.c_void_p()
    rc = lib.qgemv_create(ctypes.byref(h), ctypes.byref(d))
    return rc, h


def test_create_validation():
    assert _create(_desc(layout_version=2))[0] == EVERSION
    assert _create(_desc(fmt=0))[0] == EFORMAT
    assert _create(_desc(fmt=9))[0] == EFORMAT
    assert _create(_desc(fmt=8))[0] == EFORMAT
    assert _create(_desc(fmt=6, k=128))[0] == ESHAPE          # Q5_K needs K % 256 == 0
    assert _create(_desc(fmt=7))[0] == EINVAL                 # IQ4_XS without codebook
    assert _create(_desc(k=48))[0] == ESHAPE
    assert _create(_desc(fmt=3, k=128))[0] == ESHAPE          # Q4_K needs K % 256 == 0
    assert _create(_desc(n=0))[0] == ESHAPE
    assert _create(_desc(max_m=0))[0] == ESHAPE
    assert _create(_desc(max_m=33))[0] == ESHAPE
    assert _create(_desc(kind=7))[0] == EINVAL
    assert _create(_desc(fmt=5))[0] == EINVAL                 # IQ4_NL without codebook
    bad = (ctypes.c_int8 * 16)(*([5] * 16))
    assert _create(_desc(fmt=5, codebook16=ctypes.cast(bad, ctypes.POINTER(ctypes.c_int8))))[0] == EINVAL
    assert b"ascending" in lib.qgemv_last_error()
    good = (ctypes.c_int8 * 16)(*range(-8, 8))
    for fmt in (5, 7):
        rc, h = _create(_desc(fmt=fmt, k=512, codebook16=ctypes.cast(good, ctypes.POINTER(ctypes.c_int8))))
        assert rc == OK and h.value
        lib.qgemv_destroy(h)
    rc, h = _create(_desc(fmt=6, k=512))
    assert rc == OK and h.value
    lib.qgemv_destroy(h)
    assert lib.qgemv_create(None, None) == EINVAL


def test_ffn_and_moe_validation():
    d = _desc(kind=1, fmt=0, fmt_gateup=3, fmt_down=4, hidden=4096, inter=12288)
    rc, h = _create(d)
    assert rc == OK
    lib.qgemv_destroy(h)
    assert _create(_desc(kind=1, fmt_gateup=3, fmt_down=4, hidden=4096, inter=12300))[0] == ESHAPE
    assert _create(_desc(kind=1, fmt_gateup=3, fmt_down=4, hidden=4096, inter=12288, max_m=17))[0] == ESHAPE
    m = dict(kind=2, hidden=2048, inter=512, n_experts=256, top_k=8, fmt_expert=1)
    rc, h = _create(_desc(**m))
    assert rc == OK
    lib.qgemv_destroy(h)
    assert _create(_desc(**{**m, "top_k": 0}))[0] == ESHAPE
    assert _create(_desc(**{**m, "top_k": 17}))[0] == ESHAPE
    assert _create(_desc(**{**m, "n_experts": 4, "top_k": 8}))[0] == ESHAPE


def test_workspace_and_weight_sizes():
    rc, h = _create(_desc(fmt=3, n=12288, k=4096, max_m=4))
    assert rc == OK
    b = ctypes.c_size_t()
    assert lib.qgemv_workspace_size(h, 1, ctypes.byref(b)) == OK and b.value >= 4096 + 2 * 512
    assert lib.qgemv_workspace_size(h, 5, ctypes.byref(b)) == ESHAPE
    assert lib.qgemv_weight_bytes(h, 0, ctypes.byref(b)) == OK and b.value == 12288 * 2304
    assert lib.qgemv_weight_bytes(h, 1, ctypes.byref(b)) == EINVAL
    off = ctypes.c_size_t()
    assert lib.qgemv_workspace_offset(h, 2, b"dx", ctypes.byref(off)) == OK and off.value % 256 == 0
    assert lib.qgemv_workspace_offset(h, 2, b"nope", ctypes.byref(off)) == EINVAL
    lib.qgemv_destroy(h)


def test_run_validation_before_any_device_work(monkeypatch):
    rc, h = _create(_desc(fmt=1, n=64, k=256, max_m=2))
    assert rc == OK
    ws = ctypes.c_size_t()
    lib.qgemv_workspace_size(h, 1, ctypes.byref(ws))
    A = 0x10000  # aligned fake addresses: validation never dereferences them
    run = lambda w, x, y, m, p, n: lib.qgemv_run(h, w, x, y, m, p, n, None)
    assert run(None, A, A, 1, A, ws.value) == EINVAL
    assert run(A + 8, A, A, 1, A, ws.value) == EALIGN
    assert run(A, A + 4, A, 1, A, ws.value) == EALIGN
    assert run(A, A, A, 1, A + 16, ws.value) == EALIGN
    assert run(A, A, A, 3, A, ws.value) == ESHAPE
    assert run(A, A, A, 0, A, ws.value) == ESHAPE
    assert run(A, A, A, 1, A, ws.value - 1) == EWORKSPACE
    monkeypatch.setenv("QGEMV_FAULT", "launch")
    assert run(A, A, A, 1, A, ws.value) == EHIP
    assert b"injected" in lib.qgemv_last_error()
    assert lib.qffn_run(h, A, A, A, A, 1, A, ws.value, None) == EINVAL   # wrong kind
    lib.qgemv_destroy(h)
    assert lib.qgemv_status_string(EWORKSPACE) == b"workspace too small"
    assert lib.qgemv_status_string(-99) == b"unknown status"


def test_binding_refuses_cpu_tensors():
    import torch
    g = qg.GEMV("q4_0", 64, 256)
    w = torch.zeros(g.weight_bytes(), dtype=torch.uint8)
    with pytest.raises(ValueError):
        g.run(w, torch.zeros(1, 256))


def test_attention_validation_before_launch():
    sz = ctypes.c_size_t()
    # supported shapes: head_dim 128/256, heads/kv_heads in {1, 2, 4, 8}
    assert lib.qattn_workspace_size(16, 2, 256, 32768, ctypes.byref(sz)) == OK and sz.value > 0
    assert lib.qattn_workspace_size(16, 2, 256, 8, ctypes.byref(sz)) == OK and sz.value == 0  # one chunk
    assert lib.qattn_workspace_size(16, 2, 64, 100, ctypes.byref(sz)) == ESHAPE
    assert lib.qattn_workspace_size(12, 8, 128, 100, ctypes.byref(sz)) == ESHAPE
    assert lib.qattn_workspace_size(48, 3, 128, 100, ctypes.byref(sz)) == ESHAPE  # group of 16
    assert lib.qattn_workspace_size(16, 2, 256, 0, ctypes.byref(sz)) == ESHAPE
    assert lib.qattn_workspace_size(16, 2, 256, 1 << 22, ctypes.byref(sz)) == ESHAPE  # 32-bit offsets
    assert lib.qattn_workspace_size(16, 2, 256, 100, None) == EINVAL
    a = 1 << 20  # fake, never dereferenced: every call below fails validation
    assert lib.qattn_decode(None, a, a, a, 16, 2, 256, 100, a, 1 << 30, None) == EINVAL
    assert lib.qattn_decode(a, a, a, a, 16, 2, 200, 100, a, 1 << 30, None) == ESHAPE
    assert lib.qattn_decode(a + 4, a, a, a, 16, 2, 256, 100, a, 1 << 30, None) == EALIGN
    assert lib.qattn_decode(a, a, a + 8, a, 16, 2, 256, 100, a, 1 << 30, None) == EALIGN
    assert lib.qattn_workspace_size(16, 2, 256, 4096, ctypes.byref(sz)) == OK
    assert lib.qattn_decode(a, a, a, a, 16, 2, 256, 4096, a, sz.value - 1, None) == EWORKSPACE
    assert lib.qattn_decode(a, a, a, a, 16, 2, 256, 4096, None, sz.value, None) == EINVAL
    assert lib.qattn_decode(a, a, a, a, 16, 2, 256, 4096, a + 16, sz.value, None) == EALIGN
    assert b"workspace" in lib.qgemv_last_error() or b"ws" in lib.qgemv_last_error()


def test_s16_validation_before_launch():
    def plan(fmt, n, k):
        d = _desc(fmt=fmt, n=n, k=k)
        h = ctypes.c_void_p()
        assert lib.qgemv_create(ctypes.byref(h), ctypes.byref(d)) == OK
        return h

    sz = ctypes.c_size_t()
    h = plan(3, 64, 4096)  # Q4_K
    assert lib.qgemv_workspace_size_s16(h, ctypes.byref(sz)) == OK
    assert sz.value == 8192 + 512 + 512
    a = 1 << 20  # fake device addresses: every call below fails validation first
    assert lib.qgemv_run_s16(h, a, a, a, a, sz.value - 1, None) == EWORKSPACE
    assert lib.qgemv_run_s16(h, a + 8, a, a, a, sz.value, None) == EALIGN
    assert lib.qgemv_run_s16(h, None, a, a, a, sz.value, None) == EINVAL
    assert lib.qgemv_debug_block_dots_s16(h, a, a + 2, a, None) == EALIGN
    lib.qgemv_destroy(h)
    h8 = plan(2, 64, 4096)  # Q8_0: no 16-bit path
    assert lib.qgemv_workspace_size_s16(h8, ctypes.byref(sz)) == EFORMAT
    assert lib.qgemv_run_s16(h8, a, a, a, a, 1 << 30, None) == EFORMAT
    lib.qgemv_destroy(h8)
    hk = plan(3, 64, 1024)  # K not a multiple of 2048
    assert lib.qgemv_run_s16(hk, a, a, a, a, 1 << 30, None) == ESHAPE
    lib.qgemv_destroy(hk)
    assert lib.qgemv_debug_quantize_s16(a, a, a, a, 1, 100, None) == ESHAPE
    assert lib.qgemv_debug_quantize_s16(a + 4, a, a, a, 1, 128, None) == EALIGN


def test_new_entry_points_report_injected_launch_failure(monkeypatch):
    # With QGEMV_FAULT=launch a call that passes validation returns EHIP
    # instead of launching (no device needed).
    monkeypatch.setenv("QGEMV_FAULT", "launch")
    a = 1 << 20
    sz = ctypes.c_size_t()
    assert lib.qattn_workspace_size(16, 2, 256, 4096, ctypes.byref(sz)) == OK
    assert lib.qattn_decode(a, a, a, a, 16, 2, 256, 4096, a, sz.value, None) == EHIP
    assert b"injected" in lib.qgemv_last_error()
    d = _desc(fmt=3, n=64, k=4096)
    h = ctypes.c_void_p()
    assert lib.qgemv_create(ctypes.byref(h), ctypes.byref(d)) == OK
    assert lib.qgemv_workspace_size_s16(h, ctypes.byref(sz)) == OK
    assert lib.qgemv_run_s16(h, a, a, a, a, sz.value, None) == EHIP
    assert lib.qgemv_debug_block_dots_s16(h, a, a, a, None) == EHIP
    assert lib.qgemv_debug_quantize_s16(a, a, a, a, 1, 4096, None) == EHIP
    lib.qgemv_destroy(h)


def test_moe_s16_validation_before_launch():
    a = 1 << 20
    d = qg._Desc()
    d.kind, d.layout_version, d.max_m = 2, 1, 1
    d.hidden, d.inter, d.n_experts, d.top_k, d.fmt_expert = 2048, 512, 16, 4, 2  # Q8_0 experts
    h = ctypes.c_void_p()
    assert lib.qgemv_create(ctypes.byref(h), ctypes.byref(d)) == OK
    sz = ctypes.c_size_t()
    assert lib.qgemv_workspace_size(h, 1, ctypes.byref(sz)) == OK
    assert lib.qmoe_run_s16(h, a, a, a, a, a, a, a, 1, a, sz.value, None) == EFORMAT
    lib.qgemv_destroy(h)
    d.fmt_expert, d.inter = 1, 768  # Q4_0, but inter not in {512, 1024, 2048, 4096}
    assert lib.qgemv_create(ctypes.byref(h), ctypes.byref(d)) == OK
    assert lib.qgemv_workspace_size(h, 1, ctypes.byref(sz)) == OK
    assert lib.qmoe_run_s16(h, a, a, a, a, a, a, a, 1, a, sz.value, None) == ESHAPE
    assert lib.qmoe_run_s16(h, a, a, a, a, a, None, a, 1, a, sz.value, None) == EINVAL
    lib.qgemv_destroy(h)


def test_f32act_validation_before_launch():
    def plan(fmt, n, k):
        d = _desc(fmt=fmt, n=n, k=k)
        h = ctypes.c_void_p()
        assert lib.qgemv_create(ctypes.byref(h), ctypes.byref(d)) == OK
        return h

    a = 1 << 20  # fake device addresses: every call below fails validation first
    h = plan(2, 64, 4096)  # Q8_0
    assert lib.qgemv_run_f32act(h, a, a, a, 0, None) == ESHAPE
    assert lib.qgemv_run_f32act(h, a, a, a, 33, None) == ESHAPE
    assert lib.qgemv_run_f32act(h, None, a, a, 1, None) == EINVAL
    assert lib.qgemv_run_f32act(h, a, a + 4, a, 1, None) == EALIGN
    assert lib.qgemv_run_f32act(h, a + 8, a, a, 1, None) == EALIGN
    assert lib.qgemv_run_f32act(None, a, a, a, 1, None) == EINVAL
    lib.qgemv_destroy(h)
    hk = plan(3, 64, 4096)  # Q4_K: no float-activation kernel
    assert lib.qgemv_run_f32act(hk, a, a, a, 1, None) == EFORMAT
    lib.qgemv_destroy(hk)



def test_stream_read_validation_before_launch():
    A = 0x10000  # aligned fake addresses: validation never dereferences them
    f = lib.qgemv_debug_stream_read
    assert f(None, 1024, A, None) == EINVAL
    assert f(A, 1024, None, None) == EINVAL
    assert f(A + 8, 1024, A, None) == EALIGN       # buffer not 16-byte aligned
    assert f(A, 1000, A, None) == EALIGN           # size not a multiple of 16
    assert f(A, 1024, A + 2, None) == EALIGN       # out not 4-byte aligned
    assert b"stream_read" in lib.qgemv_last_error()
