"""C ABI checks that need no GPU: the library loads, exports every function
include/ulysses.h declares, and rejects bad arguments on the host with a
status code and a message before any HIP call."""
import ctypes
import os
import re

import pytest

import sequence_parallelism_ulysses_amd as uly

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")

pytestmark = pytest.mark.skipif(not os.path.exists(uly.lib_path()), reason="libulysses.so not built")

# A fake, 16-byte-aligned device address. Only invalid-argument paths are
# exercised, which return before anything dereferences or launches.
FAKE = 0x7F0000001000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "attn_bwd", "attn_bwd_accumulate", "attn_bwd_ex", "attn_bwd_noalloc", "attn_bwd_workspace_size", "attn_fwd", "attn_fwd_from_shards", "attn_merge", "uly_check_cu_seqlens", "uly_last_error",
        "ulysses_pack", "ulysses_pack_heads", "ulysses_pack_multi", "ulysses_pack_qkv", "ulysses_unpack",
        "ulysses_unpack_heads", "ulysses_unpack_multi", "ulysses_unpack_qkv"])


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(uly.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(uly.SIGNATURES)


def _ptrs(n, base=FAKE):
    return (ctypes.c_void_p * n)(*[base + 4096 * i for i in range(n)])


def _pack(**kw):
    a = dict(shards=_ptrs(4), P=4, T=256, H=8, D=64, dt=uly.ULY_F32, group=0, out=FAKE, stream=None)
    a.update(kw)
    return uly.lib().ulysses_pack(a["shards"], a["P"], a["T"], a["H"], a["D"], a["dt"], a["group"], a["out"], a["stream"])


def _unpack(**kw):
    a = dict(inp=FAKE, P=4, T=256, H=8, D=64, dt=uly.ULY_BF16, group=0, shards=_ptrs(4), stream=None)
    a.update(kw)
    return uly.lib().ulysses_unpack(a["inp"], a["P"], a["T"], a["H"], a["D"], a["dt"], a["group"], a["shards"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(P=0, shards=_ptrs(1)), uly.ULY_ERR_INVALID_ARG, "P=0"),
    (dict(P=65, shards=_ptrs(65)), uly.ULY_ERR_INVALID_ARG, "P=65"),
    (dict(T=0), uly.ULY_ERR_INVALID_ARG, "T=0"),
    (dict(H=6), uly.ULY_ERR_INVALID_ARG, "H=6"),
    (dict(D=96), uly.ULY_ERR_INVALID_ARG, "D=96"),
    (dict(dt=7), uly.ULY_ERR_INVALID_ARG, "dtype"),
    (dict(group=4), uly.ULY_ERR_INVALID_ARG, "group=4"),
    (dict(group=-1), uly.ULY_ERR_INVALID_ARG, "group=-1"),
    (dict(out=None), uly.ULY_ERR_INVALID_ARG, "out"),
    (dict(out=FAKE + 8), uly.ULY_ERR_INVALID_ARG, "aligned"),
    (dict(shards=(ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)), uly.ULY_ERR_INVALID_ARG, "shards[2]"),
    (dict(shards=(ctypes.c_void_p * 4)(FAKE, FAKE + 4, FAKE, FAKE)), uly.ULY_ERR_INVALID_ARG, "shards[1]"),
    (dict(T=1 << 26, H=64, D=128, P=1, shards=_ptrs(1)), uly.ULY_ERR_UNSUPPORTED, "32 GiB"),
])
def test_pack_rejects(kw, status, needle):
    assert _pack(**kw) == status
    assert needle in uly.last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(inp=None), "in is NULL"), (dict(H=9), "H=9"), (dict(group=5), "group=5"),
    (dict(shards=(ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, None)), "shards[3]"),
])
def test_unpack_rejects(kw, needle):
    assert _unpack(**kw) == uly.ULY_ERR_INVALID_ARG
    assert needle in uly.last_error()


def _pack_qkv(**kw):
    a = dict(shards=_ptrs(8), P=8, T=4096, Hq=32, Hkv=8, D=128, dt=uly.ULY_BF16, group=0,
             q=FAKE, k=FAKE + 4096, v=FAKE + 8192, stream=None)
    a.update(kw)
    return uly.lib().ulysses_pack_qkv(a["shards"], a["P"], a["T"], a["Hq"], a["Hkv"], a["D"], a["dt"], a["group"],
                                      a["q"], a["k"], a["v"], a["stream"])


def _unpack_qkv(**kw):
    a = dict(dq=FAKE, dk=FAKE + 4096, dv=FAKE + 8192, P=8, T=4096, Hq=32, Hkv=8, D=128, dt=uly.ULY_BF16,
             group=0, shards=_ptrs(8), stream=None)
    a.update(kw)
    return uly.lib().ulysses_unpack_qkv(a["dq"], a["dk"], a["dv"], a["P"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                        a["dt"], a["group"], a["shards"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(P=0, shards=_ptrs(1)), uly.ULY_ERR_INVALID_ARG, "P=0"),
    (dict(T=0), uly.ULY_ERR_INVALID_ARG, "T=0"),
    (dict(Hq=30), uly.ULY_ERR_INVALID_ARG, "Hq=30"),
    (dict(Hkv=4), uly.ULY_ERR_INVALID_ARG, "Hkv=4"),
    (dict(Hkv=0), uly.ULY_ERR_INVALID_ARG, "Hkv=0"),
    (dict(D=32), uly.ULY_ERR_INVALID_ARG, "D=32"),
    (dict(dt=5), uly.ULY_ERR_INVALID_ARG, "dtype"),
    (dict(group=8), uly.ULY_ERR_INVALID_ARG, "group=8"),
    (dict(k=None), uly.ULY_ERR_INVALID_ARG, "k_out"),
    (dict(v=FAKE + 8), uly.ULY_ERR_INVALID_ARG, "v_out"),
    (dict(shards=(ctypes.c_void_p * 8)(*([FAKE] * 7 + [None]))), uly.ULY_ERR_INVALID_ARG, "shards[7]"),
    (dict(T=1 << 26, Hq=64, Hkv=8, P=1, shards=_ptrs(1)), uly.ULY_ERR_UNSUPPORTED, "32 GiB"),
    (dict(T=1 << 26, Hq=8, Hkv=64, P=1, shards=_ptrs(1)), uly.ULY_ERR_UNSUPPORTED, "32 GiB"),
])
def test_pack_qkv_rejects(kw, status, needle):
    assert _pack_qkv(**kw) == status
    assert needle in uly.last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(dq=None), "dq is NULL"), (dict(dv=FAKE + 4), "dv is NULL"), (dict(Hkv=12), "Hkv=12"),
    (dict(shards=None), "shards is NULL"),
])
def test_unpack_qkv_rejects(kw, needle):
    assert _unpack_qkv(**kw) == uly.ULY_ERR_INVALID_ARG
    assert needle in uly.last_error()


def _merge(**kw):
    a = dict(op=_ptrs(3), lp=_ptrs(3, base=FAKE + (1 << 20)), n=3, N=1024, hq=4, D=128, dt=uly.ULY_BF16,
             o=FAKE + (2 << 20), lse=FAKE + (3 << 20), stream=None)
    a.update(kw)
    return uly.lib().attn_merge(a["op"], a["lp"], a["n"], a["N"], a["hq"], a["D"], a["dt"], a["o"], a["lse"],
                                a["stream"])


@pytest.mark.parametrize("kw,needle", [
    (dict(n=0), "nparts=0"), (dict(n=65), "nparts=65"), (dict(N=0), "N=0"), (dict(hq=0), "hq=0"),
    (dict(D=96), "D=96"), (dict(dt=9), "dtype"), (dict(op=None), "NULL"), (dict(o=None), "o is NULL"),
    (dict(lse=FAKE + 4), "lse is NULL"), (dict(op=(ctypes.c_void_p * 3)(FAKE, None, FAKE)), "o_parts[1]"),
    (dict(lp=(ctypes.c_void_p * 3)(FAKE, FAKE, FAKE + 8)), "lse_parts[2]"),
    (dict(o=FAKE + 4096), "aliases"),
])
def test_merge_rejects(kw, needle):
    assert _merge(**kw) == uly.ULY_ERR_INVALID_ARG
    assert needle in uly.last_error()


def test_merge_rejects_grids_beyond_2_31_threads():
    assert _merge(N=1 << 30, hq=1024) == uly.ULY_ERR_UNSUPPORTED
    assert "2^34" in uly.last_error()


def _multi(fn="ulysses_pack_multi", **kw):
    a = dict(n=3, shards=_ptrs(24), H=(ctypes.c_int * 3)(32, 8, 8), P=8, T=4096, D=128, dt=uly.ULY_BF16, group=0,
             packed=_ptrs(3, base=FAKE + (1 << 24)), stream=None)
    a.update(kw)
    return getattr(uly.lib(), fn)(a["n"], a["shards"] if fn == "ulysses_pack_multi" else a["packed"], a["H"], a["P"],
                                  a["T"], a["D"], a["dt"], a["group"],
                                  a["packed"] if fn == "ulysses_pack_multi" else a["shards"], a["stream"])


@pytest.mark.parametrize("fn", ["ulysses_pack_multi", "ulysses_unpack_multi"])
@pytest.mark.parametrize("kw,status,needle", [
    (dict(n=0), uly.ULY_ERR_INVALID_ARG, "ntensors=0"),
    (dict(n=4), uly.ULY_ERR_INVALID_ARG, "ntensors=4"),
    (dict(H=None), uly.ULY_ERR_INVALID_ARG, "H is NULL"),
    (dict(H=(ctypes.c_int * 3)(32, 12, 8)), uly.ULY_ERR_INVALID_ARG, "tensor 1"),
    (dict(D=96), uly.ULY_ERR_INVALID_ARG, "D=96"),
    (dict(group=8), uly.ULY_ERR_INVALID_ARG, "group=8"),
    (dict(shards=(ctypes.c_void_p * 24)(*([FAKE] * 20 + [None] + [FAKE] * 3))), uly.ULY_ERR_INVALID_ARG, "shards[20]"),
    (dict(packed=(ctypes.c_void_p * 3)(FAKE, FAKE + 8, FAKE)), uly.ULY_ERR_INVALID_ARG, "[1] is NULL or not"),
    (dict(T=1 << 26, H=(ctypes.c_int * 3)(64, 8, 8), P=1, shards=_ptrs(3)), uly.ULY_ERR_UNSUPPORTED, "32 GiB"),
])
def test_multi_rejects(fn, kw, status, needle):
    assert _multi(fn, **kw) == status
    assert needle in uly.last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(h0=-1), uly.ULY_ERR_INVALID_ARG, "heads [-1"),
    (dict(h0=7, nh=2), uly.ULY_ERR_INVALID_ARG, "heads [7"),
    (dict(nh=0), uly.ULY_ERR_INVALID_ARG, "heads [0"),
    (dict(D=32), uly.ULY_ERR_INVALID_ARG, "D=32"),
    (dict(P=0), uly.ULY_ERR_INVALID_ARG, "P=0"),
    (dict(out=FAKE + 4), uly.ULY_ERR_INVALID_ARG, "not 16-byte"),
])
def test_heads_rejects(kw, status, needle):
    a = dict(P=4, T=256, H=8, D=64, dt=uly.ULY_BF16, h0=0, nh=1, out=FAKE)
    a.update(kw)
    sh = _ptrs(max(a["P"], 1))
    assert uly.lib().ulysses_pack_heads(sh, a["P"], a["T"], a["H"], a["D"], a["dt"], a["h0"], a["nh"], a["out"],
                                        None) == status
    assert needle in uly.last_error()
    assert uly.lib().ulysses_unpack_heads(a["out"], a["P"], a["T"], a["H"], a["D"], a["dt"], a["h0"], a["nh"], sh,
                                          None) == status
    assert needle in uly.last_error()


def _fwd_sh(**kw):
    a = dict(q=_ptrs(8), k=_ptrs(8, base=FAKE + (1 << 24)), v=_ptrs(8, base=FAKE + (2 << 24)), P=8, T=4096, Hq=32,
             Hkv=8, D=128, dt=uly.ULY_BF16, group=0, o=FAKE + (3 << 24), lse=FAKE + (4 << 24), cu=None, nd=0,
             scale=0.088, causal=1, stream=None)
    a.update(kw)
    return uly.lib().attn_fwd_from_shards(a["q"], a["k"], a["v"], a["P"], a["T"], a["Hq"], a["Hkv"], a["D"], a["dt"],
                                          a["group"], a["o"], a["lse"], a["cu"], a["nd"], a["scale"], a["causal"],
                                          a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dt=uly.ULY_F32), uly.ULY_ERR_UNSUPPORTED, "bf16"),
    (dict(T=4000), uly.ULY_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(Hq=30), uly.ULY_ERR_INVALID_ARG, "Hq=30"),
    (dict(Hkv=4), uly.ULY_ERR_INVALID_ARG, "Hkv=4"),
    (dict(group=8), uly.ULY_ERR_INVALID_ARG, "group=8"),
    (dict(P=0), uly.ULY_ERR_INVALID_ARG, "P=0"),
    (dict(D=96), uly.ULY_ERR_INVALID_ARG, "D=96"),
    (dict(causal=3), uly.ULY_ERR_INVALID_ARG, "causal=3"),
    (dict(k=None), uly.ULY_ERR_INVALID_ARG, "NULL"),
    (dict(v=(ctypes.c_void_p * 8)(*([FAKE] * 5 + [FAKE + 2] + [FAKE] * 2))), uly.ULY_ERR_INVALID_ARG, "shard 5"),
    (dict(lse=FAKE + 4), uly.ULY_ERR_INVALID_ARG, "o or lse"),
])
def test_fwd_from_shards_rejects(kw, status, needle):
    assert _fwd_sh(**kw) == status
    assert needle in uly.last_error()


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, N=1024, hq=4, hk=1, D=128, dt=uly.ULY_BF16,
             cu=None, nd=0, scale=0.088, causal=1, stream=None)
    a.update(kw)
    return uly.lib().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["N"], a["hq"], a["hk"], a["D"], a["dt"],
                              a["cu"], a["nd"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(N=0), uly.ULY_ERR_INVALID_ARG, "N=0"),
    (dict(hq=3, hk=2), uly.ULY_ERR_INVALID_ARG, "multiple"),
    (dict(hk=0), uly.ULY_ERR_INVALID_ARG, "hk=0"),
    (dict(D=32), uly.ULY_ERR_INVALID_ARG, "D=32"),
    (dict(dt=2), uly.ULY_ERR_INVALID_ARG, "dtype"),
    (dict(scale=0.0), uly.ULY_ERR_INVALID_ARG, "softmax_scale"),
    (dict(scale=float("nan")), uly.ULY_ERR_INVALID_ARG, "softmax_scale"),
    (dict(scale=float("inf")), uly.ULY_ERR_INVALID_ARG, "softmax_scale"),
    (dict(causal=2), uly.ULY_ERR_INVALID_ARG, "causal=2"),
    (dict(cu=FAKE, nd=0), uly.ULY_ERR_INVALID_ARG, "ndocs=0"),
    (dict(cu=FAKE + 2, nd=3), uly.ULY_ERR_INVALID_ARG, "4-byte"),
    (dict(q=None), uly.ULY_ERR_INVALID_ARG, "q is NULL"),
    (dict(lse=FAKE + 4), uly.ULY_ERR_INVALID_ARG, "lse"),
    (dict(v=FAKE + 1), uly.ULY_ERR_INVALID_ARG, "v is NULL or not"),
])
def test_attn_fwd_rejects(kw, status, needle):
    assert _fwd(**kw) == status
    assert needle in uly.last_error()


def _bwd(fn="attn_bwd", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, N=1024, hq=4, hk=1,
             D=128, dt=uly.ULY_BF16, cu=None, nd=0, scale=0.088, causal=1, ws=FAKE, wsb=1 << 30, stream=None)
    gdt = kw.pop("gdt", None)
    a.update(kw)
    args = [a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["N"], a["hq"], a["hk"],
            a["D"], a["dt"], a["cu"], a["nd"], a["scale"], a["causal"], a["ws"], a["wsb"], a["stream"]]
    if fn == "attn_bwd_ex":
        args.append(a["dt"] if gdt is None else gdt)
    return getattr(uly.lib(), fn)(*args)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dk=None), uly.ULY_ERR_INVALID_ARG, "dk is NULL"),
    (dict(do=FAKE + 2), uly.ULY_ERR_INVALID_ARG, "dout"),
    (dict(wsb=16), uly.ULY_ERR_INVALID_ARG, "workspace_bytes"),
    (dict(ws=None), uly.ULY_ERR_INVALID_ARG, "workspace"),
    (dict(D=256), uly.ULY_ERR_INVALID_ARG, "D=256"),
    (dict(N=-5), uly.ULY_ERR_INVALID_ARG, "N=-5"),
    (dict(causal=2), uly.ULY_ERR_INVALID_ARG, "causal=2"),
])
@pytest.mark.parametrize("fn", ["attn_bwd", "attn_bwd_ex", "attn_bwd_accumulate"])
def test_attn_bwd_rejects(fn, kw, status, needle):
    assert _bwd(fn, **kw) == status
    assert needle in uly.last_error()
    assert fn in uly.last_error()


@pytest.mark.parametrize("dt,gdt,status", [
    (uly.ULY_BF16, 5, uly.ULY_ERR_INVALID_ARG),
    (uly.ULY_F32, uly.ULY_BF16, uly.ULY_ERR_UNSUPPORTED),
])
def test_attn_bwd_ex_rejects_grad_dt(dt, gdt, status):
    assert _bwd("attn_bwd_ex", dt=dt, gdt=gdt) == status
    assert "grad_dt" in uly.last_error()


def test_workspace_size():
    n = ctypes.c_size_t(0)
    assert uly.lib().attn_bwd_workspace_size(32768, 4, 1, 128, uly.ULY_BF16, ctypes.byref(n)) == uly.ULY_OK
    assert n.value >= 4 * 4 * 32768
    assert uly.lib().attn_bwd_workspace_size(32768, 4, 3, 128, uly.ULY_BF16, ctypes.byref(n)) == uly.ULY_ERR_INVALID_ARG
    assert uly.lib().attn_bwd_workspace_size(32768, 4, 1, 128, uly.ULY_BF16, None) == uly.ULY_ERR_INVALID_ARG


@pytest.mark.parametrize("cu,N,ok", [
    ([0, 5], 5, True), ([0, 3, 3, 5], 5, True), ([0, 0, 5, 5], 5, True),
    ([1, 5], 5, False), ([0, 4, 3, 5], 5, False), ([0, 3], 5, False), ([0], 0, False),
    # offsets beyond N or negative: rejected on the host (the kernels clamp
    # them to [0, N] so that such offsets cannot index outside the tensors)
    ([0, 9, 5], 5, False), ([0, 3, 9], 5, False), ([0, -1, 5], 5, False), ([0, 2, 6, 6], 5, False),
])
def test_check_cu_seqlens(cu, N, ok):
    if ok:
        uly.uly_check_cu_seqlens(cu, N)
        assert uly.lib().uly_check_cu_seqlens((ctypes.c_int32 * len(cu))(*cu), len(cu) - 1, N) == uly.ULY_OK
    else:
        with pytest.raises(uly.UlyssesError) as e:
            uly.uly_check_cu_seqlens(cu, N)
        assert e.value.status == uly.ULY_ERR_INVALID_ARG and "uly_check_cu_seqlens" in e.value.message


def test_null_cu_pointer_rejected():
    assert uly.lib().uly_check_cu_seqlens(None, 1, 5) == uly.ULY_ERR_INVALID_ARG


def test_last_error_is_thread_local():
    import threading
    _fwd(N=0)
    msgs = {}

    def other():
        msgs["t"] = uly.last_error()
    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert msgs["t"] == ""
    assert "N=0" in uly.last_error()


# ---------------------------------------------------------------------------
# Prototypes: the header's declarations of the boundary calls, parameter by
# parameter, and the binding's ctypes signatures derived from them.
# ---------------------------------------------------------------------------
def declared_prototypes():
    """name -> (return type, [(parameter type, parameter name), ...]) from the header."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*((?:const\s+)?[a-z_]+\s*\*?)\s*([a-z_]+)\s*\(([^;]*?)\)\s*;", text, flags=re.M | re.S):
        ret, name, params = m.group(1), m.group(2), m.group(3)
        plist = []
        for p in params.split(","):
            p = " ".join(p.split())
            if p == "void":
                continue
            pm = re.match(r"^(.*?[\s*])([A-Za-z_][A-Za-z_0-9]*)$", p)
            assert pm, (name, p)
            plist.append((re.sub(r"\s*\*\s*", "* ", pm.group(1)).strip().replace("* *", "**"), pm.group(2)))
        out[name] = (" ".join(ret.split()), plist)
    return out


# The calls of the boundary as the blueprint of this library states them:
# argument order, types and names (device pointers, sizes, a stream).
BOUNDARY = {
    "ulysses_pack": "const void* const* shards, int P, int64_t T, int H, int D, uly_dtype dt, int group, "
                    "void* out, hipStream_t stream",
    "ulysses_unpack": "const void* in, int P, int64_t T, int H, int D, uly_dtype dt, int group, "
                      "void* const* shards, hipStream_t stream",
    "attn_fwd": "const void* q, const void* k, const void* v, void* o, float* lse, int64_t N, int hq, int hk, "
                "int D, uly_dtype dt, const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal, "
                "hipStream_t stream",
    "attn_bwd_workspace_size": "int64_t N, int hq, int hk, int D, uly_dtype dt, size_t* bytes",
    "attn_bwd": "const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, "
                "void* dq, void* dk, void* dv, int64_t N, int hq, int hk, int D, uly_dtype dt, "
                "const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal, void* workspace, "
                "size_t workspace_bytes, hipStream_t stream",
    "uly_last_error": "",
    "uly_check_cu_seqlens": "const int32_t* host_cu, int ndocs, int64_t N",
}


def _norm_params(text):
    return [" ".join(p.split()).replace(" *", "*") for p in text.split(",")] if text else []


@pytest.mark.parametrize("name", sorted(BOUNDARY))
def test_boundary_prototype_matches(name):
    decl = declared_prototypes()[name][1]
    got = [f"{t} {n}".replace(" *", "*") for t, n in decl]
    assert got == _norm_params(BOUNDARY[name])


def test_extended_backward_calls_extend_the_boundary_list():
    """attn_bwd_ex is attn_bwd's list plus grad_dt at the end;
    attn_bwd_accumulate has exactly attn_bwd's list; attn_bwd_noalloc has it
    without the workspace."""
    protos = declared_prototypes()
    base = protos["attn_bwd"][1]
    assert protos["attn_bwd_ex"][1] == base + [("uly_dtype", "grad_dt")]
    assert protos["attn_bwd_accumulate"][1] == base
    assert protos["attn_bwd_noalloc"][1] == [p for p in base if p[1] not in ("workspace", "workspace_bytes")]


def _noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, N=1024, hq=4, hk=1,
             D=128, dt=uly.ULY_BF16, cu=None, nd=0, scale=0.088, causal=1, stream=None)
    a.update(kw)
    return uly.lib().attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                      a["N"], a["hq"], a["hk"], a["D"], a["dt"], a["cu"], a["nd"], a["scale"],
                                      a["causal"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dq=None), uly.ULY_ERR_INVALID_ARG, "dq is NULL"),
    (dict(o=FAKE + 4), uly.ULY_ERR_INVALID_ARG, "o is NULL or not"),
    (dict(hk=3), uly.ULY_ERR_INVALID_ARG, "multiple"),
    (dict(causal=3), uly.ULY_ERR_INVALID_ARG, "causal=3"),
    # the static buffer holds the workspace of up to 51780 tokens at 4 q heads
    # on 1 kv head, D = 128, bf16
    (dict(N=51781), uly.ULY_ERR_UNSUPPORTED, "static buffer"),
    (dict(N=1 << 20), uly.ULY_ERR_UNSUPPORTED, "static buffer"),
])
def test_attn_bwd_noalloc_rejects(kw, status, needle):
    assert _noalloc(**kw) == status
    assert needle in uly.last_error() and "attn_bwd_noalloc" in uly.last_error()


def test_noalloc_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define ULY_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == uly.ULY_NOALLOC_SCRATCH_BYTES
    assert "up to 51780" in text


_SCALAR = {"int": ctypes.c_int, "uly_dtype": ctypes.c_int, "int64_t": ctypes.c_int64, "size_t": ctypes.c_size_t,
           "float": ctypes.c_float, "uly_status": ctypes.c_int}


def _ctypes_ok(ctype, t):
    t = t.replace("const ", "").strip()
    if t in _SCALAR:
        return ctype is _SCALAR[t]
    if t == "hipStream_t":
        return ctype is ctypes.c_void_p
    if t.endswith("**") or t.endswith("* const*") or t.count("*") == 2:
        return ctype is ctypes.POINTER(ctypes.c_void_p)
    base = t.rstrip("*").strip()
    if base in ("void", "float", "char"):
        return ctype in (ctypes.c_void_p, ctypes.c_char_p)
    if base in ("int32_t", "int"):
        return ctype in (ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32))
    if base == "size_t":
        return ctype is ctypes.POINTER(ctypes.c_size_t)
    return False


@pytest.mark.parametrize("name", sorted(uly.SIGNATURES))
def test_binding_signature_follows_the_header(name):
    ret, params = declared_prototypes()[name]
    res, args = uly.SIGNATURES[name]
    assert len(args) == len(params), (name, len(args), len(params))
    for (t, pname), a in zip(params, args):
        assert _ctypes_ok(a, t), (name, pname, t, a)
    assert (res is ctypes.c_char_p) if ret == "const char*" else (res is ctypes.c_int), (name, ret, res)
