"""The C-ABI library loads, exports every symbol ``include/fa.h`` declares, and
rejects invalid calls with the documented status before anything is launched.
These calls never reach a kernel, so they run without a GPU."""
import ctypes
import os
import re

import pytest

from tiled_attention_14_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from tiled_attention_14_amd import build
        build.build()
    return fa.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert names == ["fa_build_hash", "fa_bwd", "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_dropout", "fa_bwd_noalloc",
                     "fa_bwd_preprocess",
                     "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_dropout", "fa_fwd_fp8", "fa_fwd_splitkv",
                     "fa_fwd_splitkv_workspace_size", "fa_merge", "fa_status_string"]
    raw = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(lib):
    for st in range(6):
        s = fa.fa_status_string(st)
        assert s.startswith("FA_OK" if st == 0 else "FA_ERR")
    assert fa.fa_status_string(99) == "FA_ERR_UNKNOWN"


GOOD = dict(B=1, H=4, Hkv=2, N=100, d=64, scale=0.125, causal=1, dtype=fa.FA_BF16)
P = 0x10000  # a fake, 256-byte aligned address: these calls must never dereference it


def _fwd(**kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 5)
    return fa.fa_fwd(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], 0)


def _bwd(**kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 9)
    ws = a.pop("ws", P)
    wsb = a.pop("wsb", 1 << 40)
    return fa.fa_bwd(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                     ws, wsb, 0)


def _pre(**kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 3)
    return fa.fa_bwd_preprocess(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["dtype"],
                                a.pop("ws", P), a.pop("wsb", 1 << 40), 0)


def _dkdv(**kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 6)
    return fa.fa_bwd_dkdv(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                          a.pop("ws", P), a.pop("wsb", 1 << 40), 0)


def _dq(**kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 7)
    return fa.fa_bwd_dq(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"],
                        a.pop("ws", P), a.pop("wsb", 1 << 40), 0)


@pytest.mark.parametrize("call", [_fwd, _bwd, _dkdv, _dq])
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(N=-5), fa.FA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=2), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 20, H=1 << 10, N=1 << 20), fa.FA_ERR_INVALID_ARG),
])
def test_invalid_arguments(lib, call, kw, status):
    assert call(**kw) == status


@pytest.mark.parametrize("i", range(5))
def test_fwd_null_and_misaligned_pointers(lib, i):
    ptrs = [P] * 5
    ptrs[i] = None
    assert _fwd(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG
    ptrs[i] = P + 8
    assert _fwd(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("i", range(9))
def test_bwd_null_and_misaligned_pointers(lib, i):
    ptrs = [P] * 9
    ptrs[i] = None
    assert _bwd(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG
    ptrs[i] = P + 4
    assert _bwd(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("call", [_pre, _dkdv, _dq])
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), fa.FA_ERR_INVALID_ARG), (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), fa.FA_ERR_INVALID_ARG), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED), (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws=P + 64), fa.FA_ERR_WORKSPACE), (dict(wsb=16), fa.FA_ERR_WORKSPACE),
])
def test_phase_invalid_arguments(lib, call, kw, status):
    assert call(**kw) == status


@pytest.mark.parametrize("call,n", [(_pre, 3), (_dkdv, 6), (_dq, 7)])
def test_phase_null_and_misaligned_pointers(lib, call, n):
    for i in range(n):
        ptrs = [P] * n
        ptrs[i] = None
        assert call(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG
        ptrs[i] = P + 2
        assert call(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG


def test_workspace_errors(lib):
    need = fa.fa_bwd_workspace_size(1, 4, 2, 100, 64, fa.FA_BF16)
    assert _bwd(ws=None) == fa.FA_ERR_WORKSPACE
    assert _bwd(ws=P + 16) == fa.FA_ERR_WORKSPACE          # not 256-byte aligned
    assert _bwd(wsb=need - 1) == fa.FA_ERR_WORKSPACE


def test_workspace_size_is_linear_in_n(lib):
    """Two floats per query row, plus (GQA only) float32 partial dK/dV of at most
    8 B H N d bytes: O(N) extra memory, never O(N^2)."""
    for dt in (fa.FA_BF16, fa.FA_F32):
        for (B, H, Hkv, N, d) in [(1, 1, 1, 1, 64), (2, 32, 32, 4096, 128), (1, 64, 8, 8192, 128),
                                  (1, 8, 8, 65536, 128), (3, 4, 2, 129, 64), (1, 64, 1, 4096, 128)]:
            n = fa.fa_bwd_workspace_size(B, H, Hkv, N, d, dt)
            rows = B * H * N
            assert 8 * rows <= n <= 8 * rows * (1 + d) + 512, (dt, B, H, N, d, n)
            if H == Hkv:
                assert n <= 8 * rows + 512, (dt, B, H, N, d, n)
    # The named multi-head shapes need nothing beyond the two row statistics.
    assert fa.fa_bwd_workspace_size(2, 32, 32, 4096, 128, fa.FA_BF16) == 2 * 4 * 2 * 32 * 4096
    # O(N): doubling N at most doubles the workspace (up to alignment padding).
    for (H, Hkv) in ((8, 8), (64, 8), (16, 1)):
        a = fa.fa_bwd_workspace_size(1, H, Hkv, 32768, 128, fa.FA_BF16)
        b = fa.fa_bwd_workspace_size(1, H, Hkv, 65536, 128, fa.FA_BF16)
        assert b <= 2 * a + 512, (H, Hkv, a, b)
    assert fa.fa_bwd_workspace_size(0, 1, 1, 1, 64, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 1, 1, 80, fa.FA_BF16) == 0


# ------------------------------------------------------------------ key/value-cache forward and merge
KV = dict(B=2, H=8, Hkv=2, Nq=3, Nk=500, d=128, scale=0.09, causal=1, dtype=fa.FA_BF16, nsplit=0)


def _splitkv(**kw):
    a = dict(KV); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 5)
    ws = a.pop("ws", P)
    wsb = a.pop("wsb", 1 << 40)
    return fa.fa_fwd_splitkv(*ptrs, a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                             a["dtype"], a["nsplit"], ws, wsb, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=501), fa.FA_ERR_INVALID_ARG),            # causal needs Nq <= Nk
    (dict(nsplit=-1), fa.FA_ERR_INVALID_ARG),
    (dict(H=7), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(ws=P + 16), fa.FA_ERR_WORKSPACE),
    (dict(wsb=1024), fa.FA_ERR_WORKSPACE),
    (dict(ptrs=[P, P, None, P, P]), fa.FA_ERR_INVALID_ARG),
    (dict(ptrs=[P, P, P, P + 4, P]), fa.FA_ERR_INVALID_ARG),
])
def test_splitkv_invalid_arguments(lib, kw, status):
    assert _splitkv(**kw) == status


def test_splitkv_workspace_size(lib):
    a = KV
    # Two float32 per row and range plus the outputs: one range per 64-key tile at most.
    n1 = fa.fa_fwd_splitkv_workspace_size(a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["dtype"], 1)
    assert n1 >= a["B"] * a["H"] * a["Nq"] * (a["d"] + 1) * 4
    n4 = fa.fa_fwd_splitkv_workspace_size(a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["dtype"], 4)
    assert n4 >= 4 * a["B"] * a["H"] * a["Nq"] * (a["d"] + 1) * 4
    big = fa.fa_fwd_splitkv_workspace_size(a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["dtype"], 10 ** 6)
    assert big == fa.fa_fwd_splitkv_workspace_size(a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["dtype"], 8)
    assert fa.fa_fwd_splitkv_workspace_size(a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], 96, a["dtype"], 0) == 0
    # A workspace one byte short is rejected before anything is launched.
    assert _splitkv(nsplit=4, wsb=n4 - 1) == fa.FA_ERR_WORKSPACE


@pytest.mark.parametrize("args,status", [
    (dict(nsplit=0), fa.FA_ERR_INVALID_ARG),
    (dict(rows=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(ptrs=[P, None, P, P]), fa.FA_ERR_INVALID_ARG),
    (dict(ptrs=[P, P, P + 2, P]), fa.FA_ERR_INVALID_ARG),
])
def test_merge_invalid_arguments(lib, args, status):
    a = dict(nsplit=3, rows=10, d=64, dtype=fa.FA_F32, ptrs=[P] * 4)
    a.update(args)
    assert fa.fa_merge(*a["ptrs"], a["nsplit"], a["rows"], a["d"], a["dtype"], 0) == status


# ------------------------------------------------------------------ fp8 forward
F8 = dict(B=1, H=4, Hkv=2, N=100, d=128, scale=0.09, qs=0.01, ks=0.01, vs=0.01, causal=1)


def _fp8(**kw):
    a = dict(F8); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 5)
    return fa.fa_fwd_fp8(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["qs"], a["ks"], a["vs"],
                         a["causal"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(qs=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(ks=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(vs=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(ptrs=[P, None, P, P, P]), fa.FA_ERR_INVALID_ARG),
    (dict(ptrs=[P, P, P, P, P + 4]), fa.FA_ERR_INVALID_ARG),
])
def test_fp8_invalid_arguments(lib, kw, status):
    assert _fp8(**kw) == status


def _fwd_drop(p_drop, **kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 5)
    return fa.fa_fwd_dropout(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], p_drop,
                             0x1234, 7, a["dtype"], 0)


def _bwd_drop(p_drop, **kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 9)
    ws = a.pop("ws", P)
    return fa.fa_bwd_dropout(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], p_drop,
                             0x1234, 7, a["dtype"], ws, 1 << 40, 0)


@pytest.mark.parametrize("p_drop", [-0.01, float("nan"), float("inf"), 0.999, 1.0, 2.0])
def test_dropout_rate_rejected(lib, p_drop):
    assert _fwd_drop(p_drop) == fa.FA_ERR_INVALID_ARG
    assert _bwd_drop(p_drop) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("p_drop", [0.0, 0.1, 255 / 256])
@pytest.mark.parametrize("kw,status", [(dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(H=3), fa.FA_ERR_INVALID_ARG),
                                       (dict(N=0), fa.FA_ERR_INVALID_ARG), (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
                                       (dict(dtype=5), fa.FA_ERR_UNSUPPORTED)])
def test_dropout_shape_errors(lib, p_drop, kw, status):
    # Valid rates (0 included, which takes the plain entry points) with a bad shape.
    assert _fwd_drop(p_drop, **kw) == status
    assert _bwd_drop(p_drop, **kw) == status


@pytest.mark.parametrize("i", range(5))
def test_dropout_null_and_misaligned_pointers(lib, i):
    for bad in (0, P + 4):
        ptrs = [P] * 5; ptrs[i] = bad
        assert _fwd_drop(0.2, ptrs=ptrs) == fa.FA_ERR_INVALID_ARG
        ptrs = [P] * 9; ptrs[i] = bad
        assert _bwd_drop(0.2, ptrs=ptrs) == fa.FA_ERR_INVALID_ARG
    assert _bwd_drop(0.2, ws=0) == fa.FA_ERR_WORKSPACE


def test_build_hash_matches_the_sources(lib):
    """The loaded library was built from the sources in this tree (fa.lib()
    refuses it otherwise), and a changed source changes the hash."""
    from tiled_attention_14_amd import build
    assert lib.fa_build_hash().decode() == build.source_hash()
    assert len(build.source_hash()) == 16


def _noalloc(**kw):
    a = dict(GOOD); a.update(kw)
    ptrs = a.pop("ptrs", [P] * 9)
    return fa.fa_bwd_noalloc(*ptrs, a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), fa.FA_ERR_INVALID_ARG), (dict(H=3, Hkv=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    # 64 x 32 x 4096 query rows need 64 MiB of workspace: more than the fixed scratch
    (dict(B=64, H=32, Hkv=32, N=4096, d=128), fa.FA_ERR_TOO_LARGE),
])
def test_noalloc_rejects_before_any_device_call(lib, kw, status):
    assert _noalloc(**kw) == status


@pytest.mark.parametrize("i", range(9))
def test_noalloc_null_and_misaligned_pointers(lib, i):
    ptrs = [P] * 9
    ptrs[i] = None
    assert _noalloc(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG
    ptrs[i] = P + 8
    assert _noalloc(ptrs=ptrs) == fa.FA_ERR_INVALID_ARG


def test_noalloc_limit_matches_the_workspace_rule(lib):
    """The 32 MiB limit is the workspace fa_bwd would need for the same sizes."""
    limit = 32 << 20
    big = dict(B=64, H=32, Hkv=32, N=4096, d=128)
    assert fa.fa_bwd_workspace_size(64, 32, 32, 4096, 128, fa.FA_BF16) > limit
    assert fa.fa_bwd_workspace_size(2, 32, 32, 4096, 128, fa.FA_BF16) <= limit
    assert "32 MiB" in fa.fa_status_string(fa.FA_ERR_TOO_LARGE)
    assert _noalloc(**big) == fa.FA_ERR_TOO_LARGE
