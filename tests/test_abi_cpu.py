"""CPU tests of the C ABI: the library loads, exports exactly what
include/kda.h declares, and rejects bad arguments with status codes before
anything reaches the GPU (no compute call is made here)."""
import ctypes
import subprocess

import pytest

from gated_delta_rule_95_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_match_header(lib):
    declared = _lib.header_functions()
    assert declared == ["kda_bwd_chunked", "kda_bwd_workspace_bytes", "kda_decode_commit",
                        "kda_decode_spec", "kda_decode_step", "kda_decode_verify",
                        "kda_fwd_chunked", "kda_fwd_chunked_gated", "kda_fwd_chunked_noalloc",
                        "kda_fwd_workspace_bytes", "kda_last_error", "kda_status_string",
                        "kda_version"]
    for name in declared:
        assert hasattr(lib, name)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines()
                       if " T " in ln and ln.split()[-1].startswith("kda_")})
    assert exported == declared


def test_status_strings(lib):
    assert _lib.status_string(0) == "KDA_OK"
    assert _lib.status_string(1) == "KDA_ERR_INVALID_ARG"
    assert _lib.status_string(2) == "KDA_ERR_UNSUPPORTED"
    assert _lib.status_string(3) == "KDA_ERR_HIP"
    assert "gfx950" in _lib.version()


P = 0x10000   # a fake, suitably aligned address: never dereferenced, every
              # call below fails validation before any launch


def fwd(lib, **kw):
    a = dict(q=P, k=P * 2, v=P * 3, g=P * 4, beta=P * 5, S0=None, cu=None, n_seqs=1,
             n_tokens=16, H=1, dk=16, dv=16, ind=1, outd=1, o=P * 6, ST=None, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_fwd_chunked(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"],
                               a["n_seqs"], a["n_tokens"], a["H"], a["dk"], a["dv"], a["ind"],
                               a["outd"], a["o"], a["ST"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), 1, "q is NULL"),
    (dict(beta=None), 1, "beta is NULL"),
    (dict(o=None), 1, "o is NULL"),
    (dict(dk=48), 2, "d_k"),
    (dict(dv=256), 2, "d_k"),
    (dict(H=0), 1, "H must be"),
    (dict(n_seqs=-1), 1, "n_seqs"),
    (dict(n_tokens=-5), 1, "n_tokens"),
    (dict(n_seqs=3, n_tokens=16), 1, "multiple"),
    (dict(ind=7), 1, "in_dtype"),
    (dict(ind=0, outd=1), 2, "fp32 inputs"),
    (dict(q=P + 2), 1, "aligned"),
    (dict(v=P * 3 + 4), 1, "aligned"),
    (dict(g=P * 4 + 4), 1, "aligned"),
    (dict(cu=P + 2), 1, "cu_seqlens"),
    (dict(n_seqs=0, n_tokens=5), 1, "n_seqs == 0"),
    (dict(o=P * 2), 1, "overlaps"),
    (dict(n_tokens=1 << 31, n_seqs=1), 1, "int32"),
    (dict(n_tokens=(1 << 31) - 32, n_seqs=1), 1, "int32"),
    (dict(H=1 << 18, dk=128, dv=128, n_tokens=0, n_seqs=1), 1, "2^25"),
    (dict(ws=None, wsb=4096), 1, "workspace is NULL"),
    (dict(ws=P * 8 + 64, wsb=4096), 1, "workspace is not 256-byte aligned"),
])
def test_fwd_validation(lib, kw, status, msg):
    assert fwd(lib, **kw) == status
    assert msg in _lib.last_error()


def test_fwd_nothing_to_do_is_ok(lib):
    assert fwd(lib, n_seqs=0, n_tokens=0) == 0
    assert _lib.last_error() == ""


def dec(lib, **kw):
    a = dict(q=P, k=P * 2, v=P * 3, g=P * 4, beta=P * 5, S=P * 64, N=2, H=2, dk=16, dv=16,
             ind=1, outd=1, o=P * 7)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["N"],
                               a["H"], a["dk"], a["dv"], a["ind"], a["outd"], a["o"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(S=None), 1, "S is NULL"),
    (dict(N=-1), 1, "N must be"),
    (dict(dk=8), 2, "d_k"),
    (dict(S=P), 1, "S overlaps"),
    (dict(o=P), 1, "overlaps"),
    (dict(g=P * 4 + 2), 1, "aligned"),
    (dict(S=P * 64 + 8), 1, "aligned"),
])
def test_decode_validation(lib, kw, status, msg):
    assert dec(lib, **kw) == status
    assert msg in _lib.last_error()


def test_decode_nothing_to_do_is_ok(lib):
    assert dec(lib, N=0) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libkda.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_workspace_size_query(lib):
    """kda_fwd_workspace_bytes: 0 where the chains fill the device (the bench
    workload) or the batch is empty or invalid; nonzero for one long
    sequence with few heads."""
    ws = lib.kda_fwd_workspace_bytes
    assert ws(4, 4 * 4096, 32, 128, 128, 1) == 0
    assert ws(0, 0, 8, 128, 128, 1) == 0
    assert ws(1, 65536, 8, 48, 128, 1) == 0          # unsupported d_k
    assert ws(1, 65536, 8, 128, 128, 7) == 0         # not a dtype
    assert ws(1, 65536, 8, 128, 128, 1) > 0
    assert ws(1, 65536, 8, 128, 128, 1) % 256 == 0


def test_workspace_grows_with_chunks_not_state(lib):
    """Pin p4 on the library: the scratch holds per-token operands and
    per-segment summaries, so bytes per 16-token chunk stay below a bound
    that does not depend on T (state size never scales with T)."""
    H, dk, dv = 8, 128, 128
    per_chunk_bound = H * (16 * (dk + dv) * 4 + dk * (2 * dv + dk) * 4 // 8) + 4 * 256
    for T in (1024, 4096, 16384, 65536, 262144, 1 << 20):
        b = lib.kda_fwd_workspace_bytes(1, T, H, dk, dv, 1)
        chunks = (T + 15) // 16
        assert b <= chunks * per_chunk_bound, (T, b)


def test_too_small_workspace_rejected(lib):
    need = lib.kda_fwd_workspace_bytes(1, 65536, 8, 128, 128, 1)
    assert need > 0
    st = fwd(lib, n_tokens=65536, H=8, dk=128, dv=128, ws=P * 8, wsb=need - 256)
    assert st == 1 and "below" in _lib.last_error()


def test_noalloc_rejects_scratch_beyond_its_maximum(lib):
    """kda_fwd_chunked_noalloc refuses sizes whose split workspace exceeds
    its fixed array, before touching the device."""
    need = lib.kda_fwd_workspace_bytes(1, 65536, 64, 128, 128, 1)
    assert need > 64 << 20
    st = lib.kda_fwd_chunked_noalloc(P, P * 2, P * 3, P * 4, P * 5, None, None, 1, 65536, 64,
                                     128, 128, 1, 1, P * 6, None, None)
    assert st == 1 and "scratch" in _lib.last_error()


def test_spec_validation(lib):
    ver, com, spec = lib.kda_decode_verify, lib.kda_decode_commit, lib.kda_decode_spec
    # verify: K out of range, S misaligned, o overlapping an input
    assert ver(P, P * 2, P * 3, P * 4, P * 5, P * 64, 2, 0, 1, 16, 16, 1, 1, P * 7, None) == 1
    assert "K must be in [1, 16]" in _lib.last_error()
    assert ver(P, P * 2, P * 3, P * 4, P * 5, P * 64, 2, 17, 1, 16, 16, 1, 1, P * 7, None) == 1
    assert ver(P, P * 2, P * 3, P * 4, P * 5, P * 64 + 8, 2, 4, 1, 16, 16, 1, 1, P * 7,
               None) == 1 and "aligned" in _lib.last_error()
    assert ver(P, P * 2, P * 3, P * 4, P * 5, P * 64, 2, 4, 1, 16, 16, 1, 1, P, None) == 1
    assert "overlaps" in _lib.last_error()
    assert ver(P, P * 2, P * 3, P * 4, P * 5, P * 64, 0, 4, 1, 16, 16, 1, 1, P * 7, None) == 0
    # commit: n_accept required, K = 0 is a no-op, S overlapping
    assert com(P, P * 3, P * 4, P * 5, None, P * 64, 2, 3, 1, 16, 16, 1, None) == 1
    assert "n_accept is NULL" in _lib.last_error()
    assert com(P, P * 3, P * 4, P * 5, None, P * 64, 2, 0, 1, 16, 16, 1, None) == 0
    assert com(P, P * 3, P * 4, P * 5, P * 6, P, 2, 3, 1, 16, 16, 1, None) == 1
    assert "S overlaps" in _lib.last_error()
    # spec: K_prev out of range; previous drafts required when K_prev > 0
    assert spec(None, None, None, None, None, 17, P, P * 2, P * 3, P * 4, P * 5, 2, P * 64,
                1, 1, 16, 16, 1, 1, P * 7, None) == 1
    assert "K_prev" in _lib.last_error()
    assert spec(None, None, None, None, None, 2, P, P * 2, P * 3, P * 4, P * 5, 2, P * 64,
                1, 1, 16, 16, 1, 1, P * 7, None) == 1
    assert "k_prev is NULL" in _lib.last_error()


def test_gated_validation(lib):
    f = lib.kda_fwd_chunked_gated
    base = [P, P * 2, P * 3, P * 4, P * 8, P * 5, None, None, 1, 16, 1, 16, 16, 1, 1, P * 6,
            None, None, 0, None]
    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)
    assert call(a4=None) == 1 and "A_log is NULL" in _lib.last_error()
    assert call(a3=None) == 1 and "z is NULL" in _lib.last_error()
    assert call(a5=None) == 1 and "b is NULL" in _lib.last_error()
    assert call(a3=P * 4 + 2) == 1 and "aligned" in _lib.last_error()
    assert call(a15=P * 4) == 1 and "overlaps" in _lib.last_error()
    assert call(a8=0, a9=0) == 0


def test_bwd_validation(lib):
    f = lib.kda_bwd_chunked
    need = lib.kda_bwd_workspace_bytes(1, 32, 1, 16, 16)
    assert need > 0 and need % 256 == 0
    # every slot (32 / 16 + 1 + 1 = 4) holds a 16 x 16 checkpoint
    assert need >= 4 * 16 * 16 * 4
    base = [P, P * 2, P * 3, P * 4, P * 5, None, None, 1, 32, 1, 16, 16, 1, P * 6, None,
            P * 7, P * 8, P * 9, P * 10, P * 11, None, P * 16, need, None]
    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)
    assert call(a21=None) == 1 and "workspace is NULL" in _lib.last_error()
    assert call(a22=need - 256) == 1 and "below" in _lib.last_error()
    assert call(a21=P * 16 + 64) == 1 and "aligned" in _lib.last_error()
    assert call(a13=None) == 1 and "dO is NULL" in _lib.last_error()
    assert call(a15=P) == 1 and "overlaps" in _lib.last_error()
    assert call(a7=0, a8=0) == 0


def test_binding_exports_every_name():
    """Every name the Python binding lists exists (bench.py and the tests
    call them by these names)."""
    import gated_delta_rule_95_amd as m
    for name in m.__all__:
        assert callable(getattr(m, name)), name
