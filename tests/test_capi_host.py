"""The C-ABI library loads, exports every entry point include/smcsd.h declares, and rejects
bad arguments on the host before any launch (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

import smc_verification_resampling_amd as sm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smcsd.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smcsd_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sm.LIB_PATH):
        import __graft_entry__  # noqa: F401
        from smc_verification_resampling_amd import build
        build.build()
    return sm.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(sm.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", sm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (smcsd_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_gfx950_code_object_present(lib):
    data = open(sm.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_version_and_status_strings(lib):
    assert lib.smcsd_version() == 7
    assert sm.status_string(0) == "ok"
    assert "workspace" in sm.status_string(-4)
    assert "pool" in sm.status_string(sm.ST_NOSPACE)
    assert "free stack" in sm.status_string(sm.ST_KV_INCONSISTENT)


def test_workspace_sizes(lib):
    v = sm.workspace_bytes(sm.OP_VERIFY_SMC, 32, 16, 4, 128256)
    assert v >= 32 * 16 * 9 * 16 * 8           # (max, sum) pair per row and 8192-element chunk
    assert sm.workspace_bytes(sm.OP_VERIFY_SPS, 16, 1, 8, 128256) > 0
    assert sm.workspace_bytes(sm.OP_KV, 32, 16, 0, 0, 145920) >= 145920 // 8
    assert sm.workspace_bytes(sm.OP_VERIFY_SMC, 1, 1, 33, 10) == 0   # K above the limit
    assert sm.workspace_bytes(sm.OP_KV, 1, 1, 0, 0, 0) == 0
    assert sm.workspace_bytes(sm.OP_DRAFT, 512, 1, 0, 128256) >= 512 * 16 * 8
    assert sm.workspace_bytes(sm.OP_KV_CHECK, 0, 0, 0, 0, 1000) >= 2 * 4 * 1000
    assert sm.workspace_bytes(sm.OP_KV_CHECK, 0, 0, 0, 0, 0) == 0


def _verify_rc(lib, **kw):
    a = dict(tgt=ctypes.c_void_p(0x1000), drf=ctypes.c_void_p(0x1000), dtype=1, rs=64, step=1,
             tok=ctypes.c_void_p(0x1000), B=1, N=1, K=1, V=64, T=1.0, alpha=1.0, mode=0, lse=None,
             lw=ctypes.c_void_p(0x1000), out=ctypes.c_void_p(0x1000), st=ctypes.c_void_p(0x1000),
             ws=ctypes.c_void_p(0x1000), wsb=1 << 20, logq=None)
    a.update(kw)
    return lib.smcsd_verify(a["tgt"], a["drf"], a["dtype"], a["rs"], a["step"], a["tok"], a["B"],
                            a["N"], a["K"], a["V"], a["T"], a["alpha"], a["mode"], 0, 0, a["lse"],
                            a["logq"], a["lw"], a["out"], None, None, None, None, a["st"], a["ws"],
                            a["wsb"], None)


def test_verify_host_validation(lib):
    assert _verify_rc(lib, dtype=7) == -2
    assert _verify_rc(lib, K=33) == -1
    assert _verify_rc(lib, V=0) == -1
    assert _verify_rc(lib, rs=10) == -1                       # row stride below V
    assert _verify_rc(lib, T=0.0) == -1
    assert _verify_rc(lib, T=float("nan")) == -1
    assert _verify_rc(lib, tgt=None) == -1
    assert _verify_rc(lib, tgt=ctypes.c_void_p(0x1001)) == -1  # not element-aligned
    assert _verify_rc(lib, lw=None) == -1                      # SMC mode needs log-weights
    assert _verify_rc(lib, wsb=16) == -4
    assert _verify_rc(lib, ws=None) == -4
    assert _verify_rc(lib, ws=ctypes.c_void_p(0x1010)) == -4    # workspace not 256-byte aligned
    assert _verify_rc(lib, mode=3) == -1
    assert _verify_rc(lib, mode=2, lw=None) == -1              # the race mode is an SMC mode
    assert _verify_rc(lib, mode=2, lse=ctypes.c_void_p(0x1000)) == -1
    assert _verify_rc(lib, mode=2, wsb=16) == -4
    assert _verify_rc(lib, B=0) == 0                            # empty batch: nothing enqueued
    p = ctypes.c_void_p(0x1000)
    assert _verify_rc(lib, mode=1, logq=p) == -1                # the draft's log q: SMC mode only
    assert _verify_rc(lib, drf=None, logq=p, B=0) == 0          # draft rows not needed with it
    assert _verify_rc(lib, drf=None, logq=p, B=0, mode=2) == 0


def test_resample_kv_reassign_host_validation(lib):
    p = ctypes.c_void_p(0x1000)

    def rc(**kw):
        a = dict(lw=p, B=2, N=4, tau=0.5, anc=p, ess=p, res=p, T=p, M=8, bs=4, L=0, R=1, rc=p,
                 fl=p, top=p, P=64, cow=p, ncow=p, st=p, ws=p, wsb=1 << 20)
        a.update(kw)
        return lib.smcsd_resample_kv_reassign(a["lw"], a["B"], a["N"], a["tau"], 0, 0, a["anc"],
                                              a["ess"], a["res"], a["T"], a["M"], a["bs"], a["L"],
                                              a["R"], a["rc"], a["fl"], a["top"], a["P"], a["cow"],
                                              a["ncow"], a["st"], a["ws"], a["wsb"], None)
    assert rc(tau=float("nan")) == -1
    assert rc(N=0) == -1 and rc(N=1025) == -1
    assert rc(L=30, R=8) == -1                                   # beyond M_cap slots
    assert rc(lw=None) == -1 and rc(anc=None) == -1 and rc(ess=None) == -1 and rc(res=None) == -1
    assert rc(T=None) == -1 and rc(top=None) == -1
    assert rc(wsb=16) == -4 and rc(ws=ctypes.c_void_p(0x1010)) == -4
    assert rc(B=0) == 0                                          # empty batch: nothing enqueued


def test_draft_sample_host_validation(lib):
    p = ctypes.c_void_p(0x1000)

    def rc(**kw):
        a = dict(d=p, dtype=1, rs=64, n=4, V=64, T=1.0, pos=0, out=p, lq=p, st=p, ws=p,
                 wsb=1 << 20)
        a.update(kw)
        return lib.smcsd_draft_sample(a["d"], a["dtype"], a["rs"], a["n"], a["V"], a["T"], 0, 0,
                                      a["pos"], a["out"], a["lq"], a["st"], a["ws"], a["wsb"],
                                      None)
    assert rc(dtype=5) == -2
    assert rc(V=0) == -1
    assert rc(rs=10) == -1
    assert rc(T=0.0) == -1
    assert rc(pos=-1) == -1 and rc(pos=1 << 24) == -1
    assert rc(d=None) == -1
    assert rc(out=None) == -1
    assert rc(wsb=8) == -4
    assert rc(ws=ctypes.c_void_p(0x1010)) == -4
    assert rc(n=0) == 0


def test_resample_and_kv_host_validation(lib):
    p = ctypes.c_void_p(0x1000)
    assert lib.smcsd_resample(p, 1, 0, 0.5, 0, 0, p, p, p, p, None) == -1
    assert lib.smcsd_resample(p, 1, 1025, 0.5, 0, 0, p, p, p, p, None) == -1
    assert lib.smcsd_resample(p, 1, 4, float("inf"), 0, 0, p, p, p, p, None) == -1
    assert lib.smcsd_resample(p, 0, 4, 0.5, 0, 0, p, p, p, p, None) == 0
    # capacity: ceil((L + R) / bs) must fit M_cap
    assert lib.smcsd_kv_reassign(p, p, 1, 4, p, 3, 4, 10, 3, p, p, p, 100, p, p, p, p, 1 << 20,
                                 None) == -1
    assert lib.smcsd_kv_reassign(p, p, 1, 4, p, 4, 4, 10, 3, p, p, p, 100, p, p, p, None, 1 << 20,
                                 None) == -4
    assert lib.smcsd_kv_reassign(p, p, 1, 4, p, 4, 4, 10, 3, p, p, p, 100, p, p, p,
                                 ctypes.c_void_p(0x1010), 1 << 20, None) == -4
    assert lib.smcsd_kv_reassign(p, p, 0, 4, p, 4, 4, 10, 3, p, p, p, 100, p, p, p, p, 1 << 20,
                                 None) == 0
    assert lib.smcsd_philox4x32_10(p, p, -1, p, None) == -1
    assert lib.smcsd_philox4x32_10(p, p, 0, p, None) == 0


def test_binding_refuses_host_tensors(lib):
    import torch
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(sm.SmcsdError):
        sm.philox4x32_10(t.view(1, 4), torch.zeros(2, dtype=torch.int32).view(1, 2), t.view(1, 4))


def test_verify_static_host_validation(lib):
    p = ctypes.c_void_p(0x1000)

    def rc(**kw):
        a = dict(dtype=1, B=1, N=1, K=1, V=64, T=1.0, mode=0, lw=p)
        a.update(kw)
        return lib.smcsd_verify_static(p, p, a["dtype"], a["V"], 1, p, a["B"], a["N"], a["K"],
                                       a["V"], a["T"], 1.0, a["mode"], 0, 0, None, None, a["lw"],
                                       p, None, None, None, None, p, None)
    assert rc(dtype=7) == -2
    assert rc(K=33) == -1
    assert rc(T=0.0) == -1
    assert rc(lw=None) == -1
    assert rc(B=0) == 0
    # beyond the library's scratch array: refused before anything is enqueued
    assert sm.workspace_bytes(sm.OP_VERIFY_SMC, 64, 64, 8, 128256) > sm.STATIC_SCRATCH_BYTES
    assert rc(B=64, N=64, K=8, V=128256) == -5
    assert sm.status_string(-5) == "call needs more scratch than the static array holds"


def test_step_host_validation(lib):
    p = ctypes.c_void_p(0x1000)

    def rc(**kw):
        a = dict(dtype=1, B=2, N=4, K=1, V=64, T=1.0, mode=0, tau=0.5, lw=p, M=8, bs=4, L=4, R=2,
                 P=64, vws=p, vwsb=1 << 20, kws=p, kwsb=1 << 20)
        a.update(kw)
        return lib.smcsd_step(p, p, a["dtype"], a["V"], p, a["B"], a["N"], a["K"], a["V"], a["T"],
                              1.0, a["mode"], a["tau"], 0, 0, None, a["lw"], p, None, None, None, None,
                              p, p, p, p, a["M"], a["bs"], a["L"], a["R"], p, p, p, a["P"], p, p, p,
                              a["vws"], a["vwsb"], a["kws"], a["kwsb"], None)
    assert rc(dtype=7) == -2
    assert rc(mode=1) == -1                     # SpS is not a round of SMC-SD
    assert rc(tau=float("nan")) == -1
    assert rc(T=0.0) == -1
    assert rc(N=0) == -1 and rc(K=33) == -1
    assert rc(L=30, R=8) == -1                  # beyond M_cap slots
    assert rc(lw=None) == -1
    assert rc(vwsb=16) == -4 and rc(kwsb=16) == -4
    assert rc(vws=ctypes.c_void_p(0x1010)) == -4
    assert rc(B=0) == 0


def test_kv_check_host_validation(lib):
    p = ctypes.c_void_p(0x1000)

    def rc(**kw):
        a = dict(T=p, S=4, M=8, slots=3, P=100, viol=p, st=p, ws=p, wsb=1 << 20)
        a.update(kw)
        return lib.smcsd_kv_check(a["T"], a["S"], a["M"], a["slots"], p, p, p, a["P"], a["viol"],
                                  a["st"], a["ws"], a["wsb"], None)
    assert rc(S=-1) == -1 and rc(M=0) == -1
    assert rc(slots=9) == -1 and rc(slots=-1) == -1   # beyond M_cap
    assert rc(P=0) == -1 and rc(P=1 << 31) == -1
    assert rc(T=None) == -1 and rc(viol=None) == -1 and rc(st=None) == -1
    assert rc(wsb=799) == -4                          # two counters of 4 bytes per block
    assert rc(ws=ctypes.c_void_p(0x1010)) == -4       # not 256-byte aligned
    assert rc(ws=None) == -4


def test_stream_read_host_validation(lib):
    p, out = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)
    f = lib.smcsd_stream_read
    assert f(p, -16, out, None) == -1                             # negative size
    assert f(p, 24, out, None) == -1                              # not a multiple of 16
    assert f(ctypes.c_void_p(0x1008), 32, out, None) == -1        # not 16-byte aligned
    assert f(None, 32, out, None) == -1 and f(p, 32, None, None) == -1
    assert f(p, (1 << 40) + 16, out, None) == -1                  # beyond the limit
    assert f(None, 0, None, None) == 0                            # empty: nothing to do


def test_header_is_c99_and_a_c_client_links(lib, tmp_path):
    """include/smcsd.h compiles as strict C99 and a C program linked against libsmcsd.so
    gets the documented host-side answers (tests/helpers/abi_c_client.c)."""
    exe = tmp_path / "abi_c_client"
    libdir = os.path.dirname(sm.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "helpers", "abi_c_client.c"), "-L", libdir, "-lsmcsd",
           "-Wl,-rpath," + libdir, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
