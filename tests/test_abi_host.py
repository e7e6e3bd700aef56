"""Host-side checks of the C ABI: no GPU needed, nothing is launched.

Every call here carries exactly one argument error, so the library must
return that error's code before touching the HIP runtime.  Fake device
addresses are never dereferenced.
"""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "e2f.h")

e2f = pytest.importorskip("interatomic_potentials_amd")
lib = e2f.lib
C = e2f.STATUS_CODES

BASE = 0x7F0000000000           # fake, 256-byte aligned device addresses
MB = 1 << 20


def fake(k):
    return ctypes.c_void_p(BASE + k * 64 * MB)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(e2f_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert set(syms) == set(e2f.SIGNATURES), syms
    for name in syms:
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", e2f.LIB_PATH], capture_output=True,
                             text=True).stdout
        exported = set(re.findall(r"\bT (e2f_\w+)", out))
        assert set(syms) <= exported


def test_header_is_plain_c(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    src = tmp_path / "use.c"
    src.write_text('#include "e2f.h"\nint main(void){ return e2f_path_count(2) == 15 ? 0 : 1; }\n')
    res = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                          "-I/opt/rocm/include", f"-I{os.path.dirname(HEADER)}", "-c", str(src),
                          "-o", str(tmp_path / "use.o")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_status_strings_and_path_counts():
    for code, name in e2f._STATUS.items():
        assert e2f.status_string(code) == name
    assert e2f.status_string(12345) == "E2F_ERR_UNKNOWN"
    assert [e2f.path_count(l) for l in (0, 1, 2)] == [1, 5, 15]
    assert e2f.path_count(3) == C["E2F_ERR_SHAPE"]
    assert e2f.path_count(-1) == C["E2F_ERR_SHAPE"]


def _r256(b):
    return (b + 255) // 256 * 256


def _expected_ws(N, lmax, C, esize):
    """Documented layout: rows | query rows | 256 B flag | order + cells (4N each) | cell counts |
    bbox partials."""
    sched = 2 * _r256(4 * N) + _r256(4 * 2 ** 15) + _r256(256 * 6 * 4)
    return _r256(N * ((lmax + 1) ** 2 + 1) * C * esize) + _r256(N * C * esize) + 256 + sched


def test_workspace_bytes():
    wb = lib.e2f_attn_workspace_bytes
    assert wb(32768, 2, 128, 0) == _expected_ws(32768, 2, 128, 4)
    assert wb(32768, 2, 128, 0) - 32768 * 11 * 128 * 4 - 256 < 2 ** 20   # scratch is small
    assert wb(100000, 2, 128, 1) == _expected_ws(100000, 2, 128, 2)
    assert wb(3, 1, 5, 0) == _expected_ws(3, 1, 5, 4)          # 300 B of rows round up to 512
    assert wb(0, 2, 128, 0) == _expected_ws(0, 2, 128, 4)
    assert wb(10, 3, 128, 0) == 0
    assert wb(10, 2, 128, 5) == 0
    assert wb(-1, 2, 128, 0) == 0


def _agg(**kw):
    a = dict(stream=None, N=1000, K=64, lmax=2, C=128, H=16, dt=0, pos=fake(1), idx=fake(2),
             mask=fake(3), scale=0.0, env=0.0, pw=None, ws=fake(4), ws_bytes=1 << 30,
             out=fake(8), msg=None, lse=None, flags=0)
    a.update(kw)
    return lib.e2f_attn_aggregate(a["stream"], a["N"], a["K"], a["lmax"], a["C"], a["H"], a["dt"],
                                  a["pos"], a["idx"], a["mask"], a["scale"], a["env"], a["pw"],
                                  a["ws"], a["ws_bytes"], a["out"], a["msg"], a["lse"], a["flags"])


def _fwd(**kw):
    a = dict(stream=None, N=1000, K=64, lmax=2, C=128, H=16, dt=0, pos=fake(1), h=fake(9),
             idx=fake(2), mask=fake(3), scale=0.0, env=0.0, pw=None, ws=fake(4),
             ws_bytes=1 << 30, out=fake(8), msg=None, lse=None, flags=0)
    a.update(kw)
    return lib.e2f_attn_forward(a["stream"], a["N"], a["K"], a["lmax"], a["C"], a["H"], a["dt"],
                                a["pos"], a["h"], a["idx"], a["mask"], a["scale"], a["env"],
                                a["pw"], a["ws"], a["ws_bytes"], a["out"], a["msg"], a["lse"],
                                a["flags"])


def _eaas(fn=None, **kw):
    a = dict(stream=None, n=1000, lmax=2, C=128, dt=0, r=fake(1), h=fake(2), pw=None, out=fake(3))
    a.update(kw)
    fn = fn or lib.e2f_eaas_couple
    return fn(a["stream"], a["n"], a["lmax"], a["C"], a["dt"], a["r"], a["h"], a["pw"], a["out"])


def _pre(**kw):
    a = dict(stream=None, N=1000, lmax=2, C=128, dt=0, pos=fake(1), h=fake(2), pw=None, ws=fake(4),
             ws_bytes=1 << 30)
    a.update(kw)
    return lib.e2f_attn_precouple(a["stream"], a["N"], a["lmax"], a["C"], a["dt"], a["pos"], a["h"],
                                  a["pw"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("fn", [_agg, _fwd])
def test_attention_argument_errors(fn):
    assert fn(dt=2) == C["E2F_ERR_DTYPE"]
    assert fn(N=-1) == C["E2F_ERR_SHAPE"]
    assert fn(K=0) == C["E2F_ERR_SHAPE"]
    assert fn(lmax=3) == C["E2F_ERR_SHAPE"]
    assert fn(lmax=-1) == C["E2F_ERR_SHAPE"]
    assert fn(C=0) == C["E2F_ERR_SHAPE"]
    assert fn(H=0) == C["E2F_ERR_SHAPE"]
    assert fn(C=128, H=3) == C["E2F_ERR_SHAPE"]
    # any C % H == 0 layout up to 512 channels is served (the general kernel where no
    # lane-vector width fits): the call gets as far as the pointer checks
    assert fn(C=12, H=4, out=None) == C["E2F_ERR_NULL"]          # d = 3
    assert fn(C=96, H=16, out=None) == C["E2F_ERR_NULL"]         # d = 6
    assert fn(C=512, H=4, out=None) == C["E2F_ERR_NULL"]         # fp32, 512 channels
    assert fn(C=1024, H=8) == C["E2F_ERR_UNSUPPORTED"]           # wider rows
    assert fn(C=1024, H=8, dt=1) == C["E2F_ERR_UNSUPPORTED"]
    assert fn(flags=32) == C["E2F_ERR_SHAPE"]                 # unknown flag bit
    assert fn(flags=4, out=None) == C["E2F_ERR_NULL"]         # E2F_MSG_F32 is known
    assert fn(flags=8, out=None) == C["E2F_ERR_NULL"]         # E2F_SHARED_ROWS too
    assert fn(flags=16, out=None) == C["E2F_ERR_NULL"]        # E2F_MATRIX_TILES too
    assert fn(N=0, pos=None, idx=None, mask=None, ws=None, out=None) == C["E2F_OK"]
    assert fn(pos=None) == C["E2F_ERR_NULL"]
    assert fn(idx=None) == C["E2F_ERR_NULL"]
    assert fn(mask=None) == C["E2F_ERR_NULL"]
    assert fn(ws=None) == C["E2F_ERR_NULL"]
    assert fn(out=None) == C["E2F_ERR_NULL"]
    assert fn(out=ctypes.c_void_p(BASE + 8 * 64 * MB + 8)) == C["E2F_ERR_ALIGN"]
    assert fn(ws=ctypes.c_void_p(BASE + 4 * 64 * MB + 4)) == C["E2F_ERR_ALIGN"]
    assert fn(msg=ctypes.c_void_p(BASE + 12 * 64 * MB + 2)) == C["E2F_ERR_ALIGN"]
    assert fn(idx=ctypes.c_void_p(BASE + 2 * 64 * MB + 2)) == C["E2F_ERR_ALIGN"]
    need = lib.e2f_attn_workspace_bytes(1000, 2, 128, 0)
    assert fn(ws_bytes=need - 1) == C["E2F_ERR_WORKSPACE"]
    assert fn(out=fake(4)) == C["E2F_ERR_ALIAS"]             # out inside the workspace
    assert fn(out=fake(1)) == C["E2F_ERR_ALIAS"]             # out over the positions
    assert fn(msg=fake(8)) == C["E2F_ERR_ALIAS"]             # message over the output
    assert fn(msg=fake(2)) == C["E2F_ERR_ALIAS"]             # message over the indices
    assert fn(lse=fake(8)) == C["E2F_ERR_ALIAS"]             # lse over the output
    assert fn(lse=ctypes.c_void_p(BASE + 13 * 64 * MB + 2)) == C["E2F_ERR_ALIGN"]


def test_forward_specific_errors():
    assert _fwd(h=None) == C["E2F_ERR_NULL"]
    assert _fwd(h=ctypes.c_void_p(BASE + 9 * 64 * MB + 4)) == C["E2F_ERR_ALIGN"]
    assert _fwd(out=fake(9)) == C["E2F_ERR_ALIAS"]           # out over h
    assert _fwd(ws=fake(9)) == C["E2F_ERR_ALIAS"]            # workspace over h


@pytest.mark.parametrize("fn", ["e2f_eaas_couple", "e2f_dense_couple"])
def test_coupling_errors(fn):
    f = getattr(lib, fn)
    assert _eaas(f, dt=9) == C["E2F_ERR_DTYPE"]
    assert _eaas(f, n=-2) == C["E2F_ERR_SHAPE"]
    assert _eaas(f, lmax=3) == C["E2F_ERR_SHAPE"]
    assert _eaas(f, C=0) == C["E2F_ERR_SHAPE"]
    assert _eaas(f, n=0, r=None, h=None, out=None) == C["E2F_OK"]
    assert _eaas(f, r=None) == C["E2F_ERR_NULL"]
    assert _eaas(f, out=None) == C["E2F_ERR_NULL"]
    assert _eaas(f, h=ctypes.c_void_p(BASE + 2 * 64 * MB + 8)) == C["E2F_ERR_ALIGN"]
    assert _eaas(f, out=ctypes.c_void_p(BASE + 2 * 64 * MB + 4096)) == C["E2F_ERR_ALIAS"]
    assert _eaas(f, out=fake(1)) == C["E2F_ERR_ALIAS"]


def test_eaas_and_precouple_errors():
    assert _eaas(dt=9) == C["E2F_ERR_DTYPE"]
    assert _eaas(n=-2) == C["E2F_ERR_SHAPE"]
    assert _eaas(lmax=4) == C["E2F_ERR_SHAPE"]
    assert _eaas(C=0) == C["E2F_ERR_SHAPE"]
    assert _eaas(n=0, r=None, h=None, out=None) == C["E2F_OK"]
    assert _eaas(r=None) == C["E2F_ERR_NULL"]
    assert _eaas(h=None) == C["E2F_ERR_NULL"]
    assert _eaas(out=None) == C["E2F_ERR_NULL"]
    assert _eaas(h=ctypes.c_void_p(BASE + 2 * 64 * MB + 8)) == C["E2F_ERR_ALIGN"]
    assert _eaas(r=ctypes.c_void_p(BASE + 64 * MB + 2)) == C["E2F_ERR_ALIGN"]
    assert _eaas(out=ctypes.c_void_p(BASE + 2 * 64 * MB + 4096)) == C["E2F_ERR_ALIAS"]  # partial
    assert _eaas(out=fake(1)) == C["E2F_ERR_ALIAS"]
    assert _pre(dt=3) == C["E2F_ERR_DTYPE"]
    assert _pre(lmax=5) == C["E2F_ERR_SHAPE"]
    assert _pre(N=0, pos=None, h=None, ws=None) == C["E2F_OK"]
    assert _pre(ws=None) == C["E2F_ERR_NULL"]
    assert _pre(ws_bytes=100) == C["E2F_ERR_WORKSPACE"]
    assert _pre(ws=fake(2)) == C["E2F_ERR_ALIAS"]
    assert _pre(h=ctypes.c_void_p(BASE + 2 * 64 * MB + 2)) == C["E2F_ERR_ALIGN"]


def test_frames_errors():
    f = lib.e2f_frames
    assert f(None, -1, 2, fake(1), fake(2), fake(3)) == C["E2F_ERR_SHAPE"]
    assert f(None, 10, 3, fake(1), fake(2), fake(3)) == C["E2F_ERR_SHAPE"]
    assert f(None, 0, 2, None, None, None) == C["E2F_OK"]
    assert f(None, 10, 2, None, fake(2), fake(3)) == C["E2F_ERR_NULL"]
    assert f(None, 10, 2, fake(1), fake(1), fake(3)) == C["E2F_ERR_ALIAS"]


def _bwd(**kw):
    a = dict(stream=None, N=1000, K=64, lmax=2, C=128, H=16, dt=0, pos=fake(1), h=fake(9),
             idx=fake(2), mask=fake(3), scale=0.0, env=0.0, pw=None, ws=fake(4),
             ws_bytes=1 << 30, msg=fake(10), lse=fake(11), gout=fake(12), gh=fake(13),
             gp=fake(14), bws=fake(16), bws_bytes=1 << 30, flags=0)
    a.update(kw)
    return lib.e2f_attn_backward(a["stream"], a["N"], a["K"], a["lmax"], a["C"], a["H"], a["dt"],
                                 a["pos"], a["h"], a["idx"], a["mask"], a["scale"], a["env"],
                                 a["pw"],
                                 a["ws"], a["ws_bytes"], a["msg"], a["lse"], a["gout"], a["gh"],
                                 a["gp"], a["bws"], a["bws_bytes"], a["flags"])


def test_backward_argument_errors():
    wb = lib.e2f_attn_backward_workspace_bytes
    assert wb(1000, 64, 2, 128, 16, 0) > 1000 * 11 * 128 * 4 + 1000 * 64 * 4
    assert wb(1000, 64, 3, 128, 16, 0) == 0
    assert _bwd(dt=1, gh=None) == C["E2F_ERR_NULL"]           # bf16 storage is served
    assert wb(1000, 64, 2, 128, 16, 1) > wb(1000, 64, 2, 128, 16, 0)   # + fp32 copies
    assert _bwd(dt=5) == C["E2F_ERR_DTYPE"]
    assert _bwd(K=0) == C["E2F_ERR_SHAPE"]
    assert _bwd(flags=1) == C["E2F_ERR_SHAPE"]               # no index validation here
    assert _bwd(flags=4) == C["E2F_ERR_SHAPE"]               # nor a message dtype flag
    assert _bwd(flags=32) == C["E2F_ERR_SHAPE"]              # nor an unknown bit
    assert _bwd(flags=8, gh=None) == C["E2F_ERR_NULL"]       # E2F_SHARED_ROWS is known
    assert _bwd(flags=16, gh=None) == C["E2F_ERR_NULL"]      # so is E2F_MATRIX_TILES
    assert _bwd(N=0, pos=None, h=None) == C["E2F_OK"]
    for name in ("pos", "h", "idx", "mask", "ws", "msg", "lse", "gout", "gh", "gp", "bws"):
        assert _bwd(**{name: None}) == C["E2F_ERR_NULL"], name
    assert _bwd(gh=ctypes.c_void_p(BASE + 13 * 64 * MB + 4)) == C["E2F_ERR_ALIGN"]
    assert _bwd(bws_bytes=wb(1000, 64, 2, 128, 16, 0) - 1) == C["E2F_ERR_WORKSPACE"]
    assert _bwd(ws_bytes=100) == C["E2F_ERR_WORKSPACE"]
    assert _bwd(gh=fake(9)) == C["E2F_ERR_ALIAS"]             # grad_h over h
    assert _bwd(gp=fake(12)) == C["E2F_ERR_ALIAS"]            # grad_pos over grad_out
    assert _bwd(bws=fake(13)) == C["E2F_ERR_ALIAS"]           # scratch over grad_h


def _pproj(**kw):
    a = dict(stream=None, N=1000, lmax=2, C=128, dt=0, pos=fake(1), h=fake(2), wq=fake(20),
             wk=fake(21), wv=fake(22), pw=None, ws=fake(4), ws_bytes=1 << 30)
    a.update(kw)
    return lib.e2f_attn_precouple_proj(a["stream"], a["N"], a["lmax"], a["C"], a["dt"], a["pos"],
                                       a["h"], a["wq"], a["wk"], a["wv"], a["pw"], a["ws"],
                                       a["ws_bytes"])


def _fproj(**kw):
    a = dict(stream=None, N=1000, K=64, lmax=2, C=128, H=16, dt=0, pos=fake(1), h=fake(9),
             wq=fake(20), wk=fake(21), wv=fake(22), idx=fake(2), mask=fake(3), scale=0.0, env=0.0,
             pw=None, ws=fake(4), ws_bytes=1 << 30, out=fake(8), msg=None, lse=None, flags=0)
    a.update(kw)
    return lib.e2f_attn_forward_proj(a["stream"], a["N"], a["K"], a["lmax"], a["C"], a["H"],
                                     a["dt"], a["pos"], a["h"], a["wq"], a["wk"], a["wv"],
                                     a["idx"], a["mask"], a["scale"], a["env"], a["pw"], a["ws"],
                                     a["ws_bytes"], a["out"], a["msg"], a["lse"], a["flags"])


@pytest.mark.parametrize("fn", [_agg, _fwd, _bwd, _fproj])
def test_envelope_cutoff_errors(fn):
    for bad in (-1.0, float("inf"), float("-inf"), float("nan")):
        assert fn(env=bad) == C["E2F_ERR_SHAPE"], bad
    assert fn(env=3.0, N=0, pos=None, h=None) == C["E2F_OK"]
    assert fn(env=3.0, out=None, gh=None) == C["E2F_ERR_NULL"]   # a valid radius passes the check


@pytest.mark.parametrize("fn", [_pproj, _fproj])
def test_projection_argument_errors(fn):
    assert fn(N=0, pos=None, h=None) == C["E2F_OK"]
    assert fn(wq=None) == C["E2F_ERR_NULL"]
    assert fn(wk=None) == C["E2F_ERR_NULL"]
    assert fn(wv=None) == C["E2F_ERR_NULL"]
    assert fn(wv=ctypes.c_void_p(BASE + 22 * 64 * MB + 4)) == C["E2F_ERR_ALIGN"]
    assert fn(ws_bytes=100) == C["E2F_ERR_WORKSPACE"]
    assert fn(wk=fake(4)) == C["E2F_ERR_ALIAS"]                  # weights inside the workspace
    assert fn(dt=7) == C["E2F_ERR_DTYPE"]
    assert fn(lmax=3) == C["E2F_ERR_SHAPE"]
    # any C up to 1024 (the matrix cores for C in {16, 32, 64, 128} fp32, {32, 64, 128} bf16,
    # the vector ALUs otherwise): other widths get as far as the pointer checks
    assert fn(C=96, wq=None, **({"H": 12} if fn is _fproj else {})) == C["E2F_ERR_NULL"]
    assert fn(C=16, dt=1, wq=None, **({"H": 2} if fn is _fproj else {})) == C["E2F_ERR_NULL"]
    assert fn(C=2048, **({"H": 16} if fn is _fproj else {})) == C["E2F_ERR_UNSUPPORTED"]


def _nl(**kw):
    a = dict(stream=None, N=1000, K=64, rc=5.0, pos=fake(1), idx=fake(2), mask=fake(3), nw=None,
             order=None, ws=fake(4), ws_bytes=1 << 30)
    a.update(kw)
    return lib.e2f_neighbour_list(a["stream"], a["N"], a["K"], a["rc"], a["pos"], a["idx"],
                                  a["mask"], a["nw"], a["order"], a["ws"], a["ws_bytes"])


def _expected_nl_ws(N):
    """Documented layout: bbox partials | grid | cell per atom | cell starts | cursors |
    scan tile sums | grouped atoms | their positions (float4); 2^(3 b) >= N cells, 1 <= b <= 7."""
    b = 1
    while b < 7 and 2 ** (3 * b) < N:
        b += 1
    cells = 2 ** (3 * b)
    return (_r256(256 * 6 * 4) + 256 + _r256(4 * N) + _r256(4 * (cells + 1)) + _r256(4 * cells)
            + _r256(4 * 4096) + _r256(4 * N) + _r256(16 * N))


def test_neighbour_workspace_bytes():
    wb = lib.e2f_neighbour_workspace_bytes
    for N in (0, 1, 9, 64, 648, 32768, 100000, 3_000_000):
        assert wb(N) == _expected_nl_ws(N), N
    assert wb(-1) == 0
    assert wb(2 ** 30 + 1) == 0


def test_neighbour_list_argument_errors():
    assert _nl(N=-1) == C["E2F_ERR_SHAPE"]
    assert _nl(K=0) == C["E2F_ERR_SHAPE"]
    assert _nl(rc=0.0) == C["E2F_ERR_SHAPE"]
    assert _nl(rc=-1.0) == C["E2F_ERR_SHAPE"]
    assert _nl(rc=float("inf")) == C["E2F_ERR_SHAPE"]
    assert _nl(rc=float("nan")) == C["E2F_ERR_SHAPE"]
    assert _nl(K=1985) == C["E2F_ERR_UNSUPPORTED"]
    assert _nl(N=2 ** 30 + 1) == C["E2F_ERR_UNSUPPORTED"]
    assert _nl(N=0, pos=None, idx=None, mask=None, ws=None) == C["E2F_OK"]
    assert _nl(pos=None) == C["E2F_ERR_NULL"]
    assert _nl(idx=None) == C["E2F_ERR_NULL"]
    assert _nl(mask=None) == C["E2F_ERR_NULL"]
    assert _nl(ws=None) == C["E2F_ERR_NULL"]
    assert _nl(pos=ctypes.c_void_p(BASE + 64 * MB + 2)) == C["E2F_ERR_ALIGN"]
    assert _nl(ws=ctypes.c_void_p(BASE + 4 * 64 * MB + 4)) == C["E2F_ERR_ALIGN"]
    assert _nl(nw=ctypes.c_void_p(BASE + 5 * 64 * MB + 2)) == C["E2F_ERR_ALIGN"]
    assert _nl(ws_bytes=lib.e2f_neighbour_workspace_bytes(1000) - 1) == C["E2F_ERR_WORKSPACE"]
    assert _nl(idx=fake(1)) == C["E2F_ERR_ALIAS"]
    assert _nl(mask=ctypes.c_void_p(BASE + 2 * 64 * MB + 1000)) == C["E2F_ERR_ALIAS"]
    assert _nl(nw=fake(4)) == C["E2F_ERR_ALIAS"]
    assert _nl(order=fake(3)) == C["E2F_ERR_ALIAS"]


# ------------------------------------------------ two HIP runtimes in one process

def test_runtime_scan_of_maps_text():
    maps = "\n".join([
        "7f00-7f01 r-xp 00000000 00:00 1 /opt/rocm-7.2.0/lib/libamdhip64.so.7.2.70200",
        "7f01-7f02 r--p 00001000 00:00 1 /opt/rocm-7.2.0/lib/libamdhip64.so.7.2.70200",
        "7f02-7f03 r-xp 00000000 00:00 2 /site/torch/lib/libamdhip64.so",
        "7f03-7f04 rw-p 00000000 00:00 0 ",
        "7f04-7f05 r-xp 00000000 00:00 3 /usr/lib/libc.so.6",
    ])
    assert len(e2f.hip_runtimes_mapped(maps)) == 2
    with pytest.raises(ImportError, match="two HIP runtimes"):
        e2f._check_one_runtime(maps)
    one = "\n".join(maps.splitlines()[:2])
    assert len(e2f.hip_runtimes_mapped(one)) == 1
    e2f._check_one_runtime(one)
    # this test process loaded torch first, so only one runtime is mapped
    assert len(e2f.hip_runtimes_mapped()) <= 1


def test_library_loaded_before_torch_refuses_to_run():
    """libe2f.so loaded by hand before torch maps two HIP runtimes: every launching entry point
    returns E2F_ERR_RUNTIME before touching HIP, and importing the binding raises ImportError.
    CPU only: no HIP call is made in the child process."""
    import sys
    code = f"""
import ctypes, sys
sys.path.insert(0, {ROOT!r})
so = ctypes.CDLL({e2f.LIB_PATH!r})
import torch
f = so.e2f_eaas_couple
f.restype = ctypes.c_int
f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
print("rc", f(None, 1, 2, 128, 0, None, None, None, None))
g = so.e2f_frames
g.restype = ctypes.c_int
g.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
              ctypes.c_void_p]
print("rc", g(None, 1, 2, None, None, None))
try:
    import interatomic_potentials_amd
    print("imported")
except ImportError as e:
    print("ImportError", "two HIP runtimes" in str(e))
"""
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    lines = res.stdout.split("\n")
    assert f"rc {C['E2F_ERR_RUNTIME']}" in lines, res.stdout + res.stderr
    assert lines.count(f"rc {C['E2F_ERR_RUNTIME']}") == 2, res.stdout + res.stderr
    assert "ImportError True" in lines, res.stdout + res.stderr


# ------------------------------------------------ shape checks of the binding

def _cpu_inputs(N=6, K=4, lmax=1, C=16, H=2):
    import torch
    S = (lmax + 1) ** 2
    return dict(pos=torch.zeros(N, 3), h=torch.zeros(N, S, C),
                idx=torch.zeros(N, K, dtype=torch.int32), mask=torch.zeros(N, K, dtype=torch.uint8),
                ws=torch.zeros(1024, dtype=torch.uint8), N=N, K=K, lmax=lmax, C=C, H=H, S=S)


def test_binding_rejects_mismatched_shapes_before_any_launch():
    """Every size the library trusts is checked in Python first (ValueError), so a buffer too
    small for the sizes passed beside it never reaches a kernel.  CPU tensors: a shape error is
    reported before the device check, so nothing here touches the library."""
    import torch
    a = _cpu_inputs()
    N, K, S, C, H = a["N"], a["K"], a["S"], a["C"], a["H"]
    pos, h, idx, mask, ws = a["pos"], a["h"], a["idx"], a["mask"], a["ws"]
    bad = [
        (lambda: e2f.attn_forward(pos[:-1], h, idx, mask, H), "pos"),
        (lambda: e2f.attn_forward(pos, h, idx[:-1], mask[:-1], H), "nbr_idx"),
        (lambda: e2f.attn_forward(pos, h, idx, mask[:, :-1], H), "nbr_mask"),
        (lambda: e2f.attn_forward(pos, h, idx, mask, H, out=torch.zeros(N, S, C + 1)), "out"),
        (lambda: e2f.attn_forward(pos, h[:, :3], idx, mask, H), "square"),
        (lambda: e2f.attn_aggregate(pos[:-1], idx, mask, ws, H, 1, C, torch.float32), "pos"),
        (lambda: e2f.attn_aggregate(pos, idx, mask[:-1], ws, H, 1, C, torch.float32), "nbr_mask"),
        (lambda: e2f.attn_aggregate(pos, idx, mask, ws, H, 1, C, torch.float32,
                                    out=torch.zeros(N, S + 1, C)), "out"),
        (lambda: e2f.attn_precouple(pos[:, :2], h), "pos"),
        (lambda: e2f.eaas_couple(pos[:-1], h), "r"),
        (lambda: e2f.eaas_couple(pos, h, out=torch.zeros(N, S, C // 2)), "out"),
        (lambda: e2f.attn_precouple(pos, h, proj=(torch.zeros(C, C), torch.zeros(C, C + 1),
                                                  torch.zeros(2, C, C))), "w_k"),
        (lambda: e2f.frames(pos[:, :2]), "r"),
        (lambda: e2f.neighbour_list(pos[:, :2], 1.0, 4), "pos"),
    ]
    g = torch.zeros(N, S, C)
    lse = torch.zeros(N, H)
    bwd = dict(msg=g, lse=lse, grad_out=g)
    bad += [
        (lambda: e2f.attn_backward(pos, h, idx, mask, H, ws, g[:-1], lse, g), "msg"),
        (lambda: e2f.attn_backward(pos, h, idx, mask, H, ws, g, lse[:, :-1], g), "lse"),
        (lambda: e2f.attn_backward(pos, h, idx, mask, H, ws, g, lse, g[:, :, :-1]), "grad_out"),
        (lambda: e2f.attn_backward(pos, h, idx, mask, H, ws, **bwd,
                                   grad_h=torch.zeros(N, S, C + 4)), "grad_h"),
        (lambda: e2f.attn_backward(pos, h, idx, mask, H, ws, **bwd,
                                   grad_pos=torch.zeros(N + 1, 3)), "grad_pos"),
        (lambda: e2f.attn_backward(pos[:-1], h, idx, mask, H, ws, **bwd), "pos"),
        (lambda: e2f.attn_backward(pos, h, idx[:, :-1], mask, H, ws, **bwd), "nbr_mask"),
    ]
    for fn, what in bad:
        with pytest.raises(ValueError, match=what):
            fn()
    # matching shapes on the CPU stop at the device check instead
    with pytest.raises(ValueError, match="GPU"):
        e2f.attn_forward(pos, h, idx, mask, H)


def _bproj(**kw):
    a = dict(stream=None, N=1000, K=64, lmax=2, C=128, H=16, dt=0, pos=fake(1), h=fake(9),
             wq=fake(20), wk=fake(21), wv=fake(22), idx=fake(2), mask=fake(3), scale=0.0, env=0.0,
             pw=None, ws=fake(4), ws_bytes=1 << 30, msg=fake(10), lse=fake(11), gout=fake(12),
             gh=fake(13), gp=fake(14), gwq=fake(23), gwk=fake(24), gwv=fake(25), bws=fake(16),
             bws_bytes=1 << 30, flags=0)
    a.update(kw)
    return lib.e2f_attn_backward_proj(
        a["stream"], a["N"], a["K"], a["lmax"], a["C"], a["H"], a["dt"], a["pos"], a["h"], a["wq"],
        a["wk"], a["wv"], a["idx"], a["mask"], a["scale"], a["env"], a["pw"], a["ws"],
        a["ws_bytes"], a["msg"], a["lse"], a["gout"], a["gh"], a["gp"], a["gwq"], a["gwk"],
        a["gwv"], a["bws"], a["bws_bytes"], a["flags"])


def test_backward_proj_argument_errors():
    wb = lib.e2f_attn_backward_proj_workspace_bytes
    plain = lib.e2f_attn_backward_workspace_bytes(1000, 64, 2, 128, 16, 0)
    # + v, dv (2 N S C floats), dk (N C) and the weight gradients' partial sums
    assert wb(1000, 64, 2, 128, 16, 0) >= plain + (2 * 9 + 1) * 1000 * 128 * 4 + 5 * 128 * 128 * 4
    assert wb(1000, 64, 2, 128, 16, 1) > wb(1000, 64, 2, 128, 16, 0)   # + fp32 copies
    assert wb(1000, 64, 3, 128, 16, 0) == 0
    assert wb(1000, 64, 2, 2048, 16, 0) == 0
    assert _bproj(N=0, pos=None, h=None) == C["E2F_OK"]
    for name in ("pos", "h", "wq", "wk", "wv", "idx", "mask", "ws", "msg", "lse", "gout", "gh",
                 "gp", "gwq", "gwk", "gwv", "bws"):
        assert _bproj(**{name: None}) == C["E2F_ERR_NULL"], name
    assert _bproj(dt=1, msg=None, lse=None, gh=None) == C["E2F_ERR_NULL"]   # bf16: msg, lse optional
    assert _bproj(wv=ctypes.c_void_p(BASE + 22 * 64 * MB + 4)) == C["E2F_ERR_ALIGN"]
    assert _bproj(gwk=ctypes.c_void_p(BASE + 24 * 64 * MB + 2)) == C["E2F_ERR_ALIGN"]
    assert _bproj(bws_bytes=wb(1000, 64, 2, 128, 16, 0) - 1) == C["E2F_ERR_WORKSPACE"]
    assert _bproj(gwq=fake(20)) == C["E2F_ERR_ALIAS"]          # dW_Q over W_Q
    assert _bproj(gwv=fake(16)) == C["E2F_ERR_ALIAS"]          # dW_V inside the scratch
    assert _bproj(gwk=fake(23)) == C["E2F_ERR_ALIAS"]          # dW_K over dW_Q
    assert _bproj(flags=4) == C["E2F_ERR_SHAPE"]
    assert _bproj(C=2048) == C["E2F_ERR_UNSUPPORTED"]
    assert _bproj(C=96, H=6, wq=None) == C["E2F_ERR_NULL"]    # vector-ALU widths are served


@pytest.mark.parametrize("N,C,H", [(1000, 128, 16), (100000, 128, 16), (50000, 256, 16),
                                   (7, 16, 2)])
def test_backward_proj_workspace_bounds(N, C, H):
    """The projected backward's extra scratch: v and dv ([N, S, C] fp32), dk ([N, C]), and the
    weight gradients' partial sums, at least one [C, C] matrix per weight and at most 2^25 floats
    in all (plus one matrix per weight when the cap leaves a job a single chunk)."""
    wb = lib.e2f_attn_backward_proj_workspace_bytes
    plain = lib.e2f_attn_backward_workspace_bytes(N, 64, 2, C, H, 0)
    extra = wb(N, 64, 2, C, H, 0) - plain
    rows = (2 * 9 + 1) * N * C * 4
    parts = extra - rows
    jobs = 5
    assert parts >= jobs * C * C * 4 - 5 * 256
    assert parts <= max(4 << 25, jobs * C * C * 4) + 8 * 256


def test_backward_proj_needs_an_fp32_lane_width():
    # C = 1024 projects, but the backward's passes have no fp32 lane layout for it
    assert lib.e2f_attn_backward_proj_workspace_bytes(1000, 64, 2, 1024, 16, 0) == 0
    assert _bproj(C=1024, H=16) == C["E2F_ERR_UNSUPPORTED"]
