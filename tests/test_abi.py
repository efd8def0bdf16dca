"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects invalid arguments on the host before anything is launched.

Only calls that fail host-side validation are made here (plus the workspace
size queries), so no kernel is ever enqueued.
"""
import ctypes
import os
import re

import pytest

import visual_token_sparsity_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sv.lib_path()), reason="libsv.so not built")

FAKE = 0x10000  # 16-byte aligned non-NULL address; never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = sv.load()
    names = declared_functions()
    assert {"sv_retrieve", "sv_sparse_decode_attn", "sv_salience_prune",
            "sv_retrieve_attend"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_empty_error():
    lib = sv.load()
    assert lib.sv_version() >= 100
    assert isinstance(lib.sv_last_error(), bytes)


def test_wait_limit_and_status_query_host_side():
    """The wait bound is a host-side setting (no launch)."""
    lib = sv.load()
    default = sv.set_wait_limit(5)
    assert default == 1 << 24
    assert sv.set_wait_limit(0) == 5          # 0 restores the default
    assert sv.set_wait_limit(0) == 1 << 24


def test_waiting_workspaces_begin_with_a_status_line():
    # sv_retrieve and sv_retrieve_attend reserve 256 bytes ahead of their
    # scores; the smallest request still holds the status line
    assert sv.retrieve_workspace_bytes(0, 0, 0) == 256
    assert sv.retrieve_workspace_bytes(1, 1, 1) >= 256 + 256
    assert sv.retrieve_attend_workspace_bytes(0, 1, 1, 64, 1, 1, 0) == 256


def test_workspace_sizes():
    assert sv.retrieve_workspace_bytes(8, 1440, 360) >= 8 * 1440 * 4
    assert sv.retrieve_workspace_bytes(8, 1440, 360) % 256 == 0
    w = sv.sparse_decode_attn_workspace_bytes(8, 32, 32, 128, 360, 256)
    assert w >= 8 * 32 * 130 * 4 and w % 256 == 0
    assert sv.salience_prune_workspace_bytes(256, 16, 729) >= 256 * 16 * 729 * 4
    f = sv.retrieve_attend_workspace_bytes(8, 32, 32, 128, 1440, 360, 256)
    assert f % 256 == 0
    assert f >= sv.retrieve_workspace_bytes(8, 1440, 360) + w
    # rows over 2048 tokens: retrieval also holds the parallel select's
    # histograms and candidate lists (at least 16384 candidates of 8 bytes each)
    short = sv.retrieve_workspace_bytes(1, 2048, 100)
    long_ = sv.retrieve_workspace_bytes(1, 2049, 100)
    assert long_ % 256 == 0 and long_ - short >= 16384 * 8
    # the salience workspace ends with one 32-bit flag per (frame, head)
    assert (sv.salience_prune_workspace_bytes(256, 16, 729)
            >= 256 * 16 * 729 * 4 + 256 * 729 * 4 + 256 * 16 * 4)


def test_retrieve_rejects_slices_of_2gib():
    # 131072 rows of 8192 bf16 elements = 2 GiB per sequence: past 32-bit offsets.
    assert _retrieve(N=131072, k=4096, Hkv=64, Hq=64, ts=8192, bs=131072 * 8192,
                     wsb=1 << 30) == 2
    assert b"2 GiB" in sv.load().sv_last_error()


def _retrieve(**kw):
    a = dict(q=FAKE, B=1, Tq=1, Hq=32, kv=FAKE, bs=576 * 4096, ts=4096, N=576, Hkv=32, D=128,
             dt=sv.SV_BF16, k=144, idx=FAKE, sc=None, ws=FAKE, wsb=1 << 20, st=None)
    a.update(kw)
    lib = sv.load()
    return lib.sv_retrieve(a["q"], a["B"], a["Tq"], a["Hq"], a["kv"], a["bs"], a["ts"], a["N"],
                           a["Hkv"], a["D"], a["dt"], a["k"], a["idx"], a["sc"], a["ws"], a["wsb"],
                           a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=577), 1), (dict(k=-1), 1), (dict(N=0), 1), (dict(B=0), 1), (dict(Tq=0), 1),
    (dict(Hq=30, Hkv=4), 1), (dict(q=None), 1), (dict(idx=None), 1), (dict(ws=None), 1),
    (dict(ts=100), 1), (dict(ts=4100), 1), (dict(q=FAKE + 2), 1),
    (dict(D=96), 2), (dict(dt=7), 2), (dict(Hkv=128, Hq=128), 2),
    (dict(wsb=100), 3),
])
def test_retrieve_rejects(kw, status):
    assert _retrieve(**kw) == status
    assert sv.load().sv_last_error()


def _attn(**kw):
    a = dict(q=FAKE, B=1, Hq=28, kv=FAKE, vv=FAKE, vbs=0, vts=512, N=100, Hkv=4, D=128, idx=FAKE,
             k=10, kt=FAKE, vt=FAKE, tbs=0, tts=512, tl=FAKE, Tmax=8, dt=sv.SV_BF16, scale=0.0,
             out=FAKE, ws=FAKE, wsb=1 << 22, st=None)
    a.update(kw)
    lib = sv.load()
    return lib.sv_sparse_decode_attn(a["q"], a["B"], a["Hq"], a["kv"], a["vv"], a["vbs"], a["vts"],
                                     a["N"], a["Hkv"], a["D"], a["idx"], a["k"], a["kt"], a["vt"],
                                     a["tbs"], a["tts"], a["tl"], a["Tmax"], a["dt"], a["scale"],
                                     a["out"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=101), 1), (dict(k=-1), 1), (dict(k=0, Tmax=0), 1), (dict(Hq=30), 1),
    (dict(kv=None), 1), (dict(kt=None), 1), (dict(tl=None), 1), (dict(out=None), 1),
    (dict(vts=500), 1), (dict(B=0), 1),
    (dict(Hq=36, Hkv=4), 2), (dict(D=80), 2), (dict(dt=3), 2),
    (dict(wsb=16), 3),
])
def test_attn_rejects(kw, status):
    assert _attn(**kw) == status


def _sal(**kw):
    a = dict(q=FAKE, k=FAKE, F=2, H=16, N=729, D=72, dt=sv.SV_BF16, scale=0.0, keep=364,
             sal=None, idx=FAKE, ws=FAKE, wsb=1 << 24, st=None)
    a.update(kw)
    lib = sv.load()
    return lib.sv_salience_prune(a["q"], a["k"], a["F"], a["H"], a["N"], a["D"], a["dt"],
                                 a["scale"], a["keep"], a["sal"], a["idx"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(keep=730), 1), (dict(keep=-1), 1), (dict(F=0), 1), (dict(idx=None), 1),
    (dict(q=None), 1), (dict(q=FAKE + 8), 1),
    (dict(dt=sv.SV_F32), 2), (dict(D=136), 2), (dict(D=100), 2), (dict(D=70), 2),
    (dict(wsb=1024), 3), (dict(N=16384, keep=100, wsb=1 << 20), 3),
    (dict(F=1 << 20, H=1 << 10, N=16384, keep=100), 2),
])
def test_salience_rejects(kw, status):
    assert _sal(**kw) == status


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sv.retrieve(q, kv, 2)


def _fused(**kw):
    a = dict(q=FAKE, B=2, Hq=28, kv=FAKE, vv=FAKE, vbs=100 * 512, vts=512, N=100, Hkv=4, D=128,
             k=10, kt=FAKE, vt=FAKE, tbs=8 * 512, tts=512, tl=FAKE, Tmax=8, dt=sv.SV_BF16,
             scale=0.0, idx=FAKE, sc=None, out=FAKE, ws=FAKE, wsb=1 << 22, st=None)
    a.update(kw)
    lib = sv.load()
    return lib.sv_retrieve_attend(a["q"], a["B"], a["Hq"], a["kv"], a["vv"], a["vbs"], a["vts"],
                                  a["N"], a["Hkv"], a["D"], a["k"], a["kt"], a["vt"], a["tbs"],
                                  a["tts"], a["tl"], a["Tmax"], a["dt"], a["scale"], a["idx"],
                                  a["sc"], a["out"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), 1), (dict(k=101), 1), (dict(N=0), 1), (dict(B=0), 1), (dict(Hq=30), 1),
    (dict(q=None), 1), (dict(vv=None), 1), (dict(idx=None), 1), (dict(out=None), 1),
    (dict(ws=None), 1), (dict(kt=None), 1), (dict(tl=None), 1), (dict(vts=500), 1),
    (dict(tts=100), 1), (dict(q=FAKE + 4), 1), (dict(Tmax=-1), 1),
    (dict(Hq=36, Hkv=4), 2), (dict(D=96), 2), (dict(dt=5), 2), (dict(Hkv=128, Hq=128), 2),
    (dict(wsb=64), 3),
])
def test_retrieve_attend_rejects(kw, status):
    assert _fused(**kw) == status
    assert sv.load().sv_last_error()


def _pack(**kw):
    a = dict(kv=FAKE, vv=FAKE, bs=1440 * 4096, ts=4096, N=1440, Hkv=32, D=128, dt=sv.SV_BF16,
             idx=FAKE, B=8, k=360, kp=FAKE, vp=FAKE, st=None)
    a.update(kw)
    lib = sv.load()
    return lib.sv_pack_selected(a["kv"], a["vv"], a["bs"], a["ts"], a["N"], a["Hkv"], a["D"],
                                a["dt"], a["idx"], a["B"], a["k"], a["kp"], a["vp"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(N=0), 1), (dict(k=-1), 1), (dict(Hkv=0), 1),
    (dict(idx=None), 1), (dict(kv=None), 1), (dict(vp=None), 1),
    (dict(ts=4000), 1), (dict(ts=4100), 1), (dict(bs=-8), 1), (dict(Hkv=1, D=4), 1),
    (dict(kp=FAKE + 8), 1), (dict(vv=FAKE + 4), 1),
    (dict(dt=3), 2), (dict(Hkv=1 << 13, D=1 << 12, ts=1 << 25, bs=1 << 35), 2),
])
def test_pack_rejects(kw, status):
    assert _pack(**kw) == status


def test_pack_k0_enqueues_nothing():
    # k == 0 is a valid empty request: OK without touching any pointer.
    assert _pack(k=0, kv=None, vv=None, idx=None, kp=None, vp=None) == 0


def _summ(**kw):
    a = dict(q=FAKE, k=FAKE, F=2, H=16, N=577, D=64, dt=sv.SV_BF16, scale=0.0, S=1, keep=288,
             sal=None, idx=FAKE, ws=FAKE, wsb=1 << 24, st=None)
    a.update(kw)
    lib = sv.load()
    return lib.sv_summary_salience_prune(a["q"], a["k"], a["F"], a["H"], a["N"], a["D"], a["dt"],
                                         a["scale"], a["S"], a["keep"], a["sal"], a["idx"],
                                         a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(S=0), 1), (dict(S=578), 1), (dict(keep=578), 1), (dict(keep=-1), 1), (dict(F=0), 1),
    (dict(idx=None), 1), (dict(q=None), 1), (dict(ws=None), 1), (dict(k=FAKE + 8), 1),
    (dict(dt=sv.SV_F32), 2), (dict(D=136), 2), (dict(D=60), 2), (dict(S=17, N=600), 2),
    (dict(N=4097, keep=10), 2), (dict(S=16, N=800), 2), (dict(F=65536), 2),
    (dict(wsb=1024), 3),
])
def test_summary_salience_rejects(kw, status):
    assert _summ(**kw) == status


def test_summary_salience_workspace_size():
    lib = sv.load()
    assert lib.sv_summary_salience_prune_workspace(2, 16, 577) >= (2 * 16 * 577 + 2 * 577) * 4


def test_noalloc_rejects_sizes_beyond_the_static_scratch():
    """Eight sequences of 131072 tokens at 32 x 128 heads fit the 16 MiB scratch;
    sixteen do not: SV_EWORKSPACE before anything is launched."""
    lib = sv.load()
    lib.sv_retrieve_attend_noalloc.restype = ctypes.c_int
    assert sv.retrieve_attend_workspace_bytes(8, 32, 32, 128, 131072, 4096, 256) <= 16 << 20
    assert sv.retrieve_attend_workspace_bytes(16, 32, 32, 128, 131072, 4096, 256) > 16 << 20
    p = ctypes.c_void_p(FAKE)
    st = lib.sv_retrieve_attend_noalloc(p, 16, 32, p, p, ctypes.c_int64(131072 * 4096),
                                        ctypes.c_int64(4096), 131072, 32, 128, 4096, p, p,
                                        ctypes.c_int64(256 * 4096), ctypes.c_int64(4096), p, 256,
                                        sv.SV_BF16, ctypes.c_float(0.0), p, None, p, None)
    assert st == 3, lib.sv_last_error()
    assert b"static scratch" in lib.sv_last_error()


def _pf(**kw):
    a = dict(q=FAKE, B=2, Tq=8, Hq=8, kv=FAKE, vv=FAKE, vbs=1000 * 1024, vts=1024, N=1000, Hkv=8,
             D=128, kt=FAKE, vt=FAKE, tbs=64 * 1024, tts=1024, tl=FAKE, Tmax=64, dt=sv.SV_BF16,
             scale=0.0, k=100, out=FAKE, idx=FAKE, sc=None, ws=FAKE, wsb=16, st=None)
    a.update(kw)
    lib = sv.load()
    return lib.sv_prefill_attend_retrieve(
        a["q"], a["B"], a["Tq"], a["Hq"], a["kv"], a["vv"], a["vbs"], a["vts"], a["N"], a["Hkv"],
        a["D"], a["kt"], a["vt"], a["tbs"], a["tts"], a["tl"], a["Tmax"], a["dt"], a["scale"],
        a["k"], a["out"], a["idx"], a["sc"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(ws=None), 1), (dict(B=0), 1), (dict(Tq=0), 1),
    (dict(k=1001), 1), (dict(k=-1), 1), (dict(idx=None), 1), (dict(tl=None), 1),
    (dict(Hq=12), 1), (dict(vts=1000), 1), (dict(tts=1020), 1), (dict(kv=FAKE + 8), 1),
    (dict(dt=sv.SV_F32), 2), (dict(D=96), 2), (dict(Tq=1 << 18, Hq=64, Hkv=8), 2),
    (dict(wsb=16), 3),
])
def test_prefill_rejects(kw, status):
    assert _pf(**kw) == status


def test_prefill_workspace_grows_with_the_question():
    small = sv.prefill_attend_retrieve_workspace_bytes(8, 8, 32, 32, 128, 1440, 256)
    big = sv.prefill_attend_retrieve_workspace_bytes(8, 64, 32, 32, 128, 1440, 256)
    assert small % 256 == 0 and big > small >= 8 * 1440 * 4
