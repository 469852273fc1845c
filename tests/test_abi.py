"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol declared in include/libgdn.h, and rejects invalid calls before any
launch."""
import ctypes
import os
import re

import pytest

from gated_deltanet_layer_causal_amd import capi as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "libgdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_names():
    assert sorted(L.EXPORTS) == _declared()


def test_library_exports_every_declared_symbol():
    lib = L.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = L.load()
    for s in range(6):
        assert lib.gdn_status_string(s)


def _shape(**kw):
    base = dict(n_seq=1, total_tokens=128, hk=2, hv=4, d=128, dtype=L.GDN_BF16)
    base.update(kw)
    return L.make_shape(base["n_seq"], base["total_tokens"], base["hk"], base["hv"], base["d"],
                        base["dtype"])


def test_workspace_queries_are_host_only_and_sane():
    sh = _shape()
    assert L.gdn_chunk_bwd_workspace(sh) > L.gdn_chunk_fwd_workspace(sh) > 0
    assert L.gdn_conv_bwd_workspace(sh) > 0
    assert L.gdn_gate_bwd_workspace(sh) > 0
    assert L.gdn_gated_norm_bwd_workspace(128 * 4, 128) > 0
    bad = _shape(hv=3)
    assert L.gdn_chunk_fwd_workspace(bad) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(hv=3), 1),            # hv % hk != 0 -> invalid
    (dict(d=64), 2),            # head dim not supported
    (dict(n_seq=0), 1),
    (dict(total_tokens=-1), 1),
])
def test_invalid_shapes_rejected_before_launch(kw, status):
    lib = L.load()
    sh = _shape(**kw)
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    st = lib.gdn_conv_fwd(ctypes.byref(sh), fake, 1024, fake, fake, 1, 1e-6, fake, 1024, None)
    assert st == status


def test_null_and_misaligned_pointers_rejected():
    lib = L.load()
    sh = _shape()
    C = 2 * 2 * 128 + 4 * 128
    a16 = ctypes.c_void_p(256)
    assert lib.gdn_conv_fwd(ctypes.byref(sh), None, C, a16, a16, 1, 1e-6, a16, C, None) == 1
    assert lib.gdn_conv_fwd(ctypes.byref(sh), ctypes.c_void_p(258), C, a16, a16, 1, 1e-6, a16, C,
                            None) == 3
    assert lib.gdn_conv_fwd(ctypes.byref(sh), a16, C - 8, a16, a16, 1, 1e-6, a16, C, None) == 1
    # the cu_seqlens check: null or misaligned result pointers, bad shapes
    assert lib.gdn_check_cu_seqlens(ctypes.byref(sh), a16, None, None) == 1
    assert lib.gdn_check_cu_seqlens(ctypes.byref(sh), None, a16, None) == 1
    assert lib.gdn_check_cu_seqlens(ctypes.byref(sh), a16, ctypes.c_void_p(258), None) == 3
    assert lib.gdn_check_cu_seqlens(ctypes.byref(_shape(n_seq=0)), a16, a16, None) == 1
    # chunk op with a workspace that is too small
    st = lib.gdn_chunk_fwd(ctypes.byref(sh), a16, a16, a16, 1024, 1024, 1024, a16, a16,
                           ctypes.c_float(0.1), None, None, a16, a16, a16, 16, None)
    assert st == 4
    # norm: unsupported row length
    assert lib.gdn_gated_norm_fwd(10, 64, 0, a16, a16, a16, ctypes.c_float(1e-6), 0, a16, None) == 2


def test_stale_library_is_refused(tmp_path):
    """load() checks that the library was built from the sources in the tree."""
    import shutil
    from gated_deltanet_layer_causal_amd import build as B
    so = tmp_path / "libgdn.so"
    shutil.copy(L.LIB_PATH, so)
    with pytest.raises(RuntimeError, match="not built from"):
        L._check_built(str(so))          # no digest beside it
    (tmp_path / "libgdn.so.sources").write_text("0" * 64 + "\n")
    with pytest.raises(RuntimeError, match="not built from"):
        L._check_built(str(so))          # digest of other sources
    (tmp_path / "libgdn.so.sources").write_text(B.source_digest() + "\n")
    L._check_built(str(so))
    with pytest.raises(RuntimeError, match="missing"):
        L._check_built(str(tmp_path / "nothing.so"))


def test_wrappers_check_tensors_before_the_call():
    """Wrong dtype, size or layout is a Python error, raised before the
    library sees a pointer; a correct host tensor is refused as not on the
    device.  (Each case breaks the first tensor the wrapper checks.)"""
    import torch
    sh = _shape(total_tokens=100, hk=1, hv=2, d=32, dtype=L.GDN_FP32)
    T, hv, d = 100, 2, 32
    g = torch.zeros(T * hv)
    Al = torch.zeros(hv)
    a = torch.zeros(T, hv)
    with pytest.raises(TypeError):
        L.gdn_gate_fwd(sh, a.double(), a, Al, Al, g, g)
    with pytest.raises(ValueError, match="elements"):
        L.gdn_gate_fwd(sh, a[:-1], a, Al, Al, g, g)
    with pytest.raises(ValueError, match="must be contiguous"):
        L.gdn_gate_fwd(sh, a.t(), a, Al, Al, g, g)
    with pytest.raises(ValueError, match="device"):
        L.gdn_gate_fwd(sh, a, a, Al, Al, g, g)
    y = torch.zeros(T, 4 * 32)
    ws = torch.zeros(16, dtype=torch.uint8)
    cu = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="contiguous rows"):
        L.gdn_chunk_prepare(sh, y[:, ::4], y[:, 32:64], g, g, 0.1, cu, ws)
    with pytest.raises(ValueError, match="matrix"):
        L.gdn_chunk_fwd(sh, y[:-1, :32], y[:, 32:64], y[:, 64:], g, g, 0.1, None, None, cu,
                        torch.zeros(T, hv, d), ws)
    with pytest.raises(TypeError):
        L.gdn_chunk_fwd(sh, y[:, :32].double(), y[:, 32:64], y[:, 64:], g, g, 0.1, None, None, cu,
                        torch.zeros(T, hv, d), ws)
    o = torch.zeros(10, 32)
    with pytest.raises(ValueError, match="elements"):
        L.gdn_gated_norm_fwd(o, o[:-1], torch.zeros(32), o)
    with pytest.raises(ValueError, match="elements"):
        L.gdn_gated_norm_fwd(o, o, torch.zeros(31), o)
    with pytest.raises(ValueError, match="device"):
        L.gdn_gated_norm_fwd(o, o, torch.zeros(32), o)


def test_conv_bwd_noalloc_refuses_shapes_beyond_its_scratch():
    """The workspace-free conv backward checks its fixed scratch size on the
    host, before any device call (fake pointers are never dereferenced)."""
    import re as _re
    hdr = open(os.path.join(ROOT, "include", "libgdn.h")).read()
    assert int(eval(_re.search(r"#define GDN_CONV_BWD_NOALLOC_MAX_BYTES \((.*?)\)", hdr).group(1)
                    .replace("u", ""))) == L.CONV_BWD_NOALLOC_MAX_BYTES
    lib = L.load()
    a16 = ctypes.c_void_p(256)
    ok = _shape(total_tokens=131072, hk=16, hv=48)
    assert L.gdn_conv_bwd_workspace(ok) <= L.CONV_BWD_NOALLOC_MAX_BYTES
    big = _shape(total_tokens=262144, hk=16, hv=48)
    assert L.gdn_conv_bwd_workspace(big) > L.CONV_BWD_NOALLOC_MAX_BYTES
    C = 2 * 16 * 128 + 48 * 128
    st = lib.gdn_conv_bwd_noalloc(ctypes.byref(big), a16, C, a16, a16, 1, ctypes.c_float(1e-6), a16,
                                  C, a16, C, a16, None)
    assert st == 4          # GDN_ERR_WORKSPACE
    st = lib.gdn_conv_bwd_noalloc(ctypes.byref(ok), None, C, a16, a16, 1, ctypes.c_float(1e-6), a16,
                                  C, a16, C, a16, None)
    assert st == 1          # null pointer: invalid argument


def test_segmented_scan_workspace():
    """The segment-parallel state scan's summaries live in the chunk
    workspace: forcing segments grows it, forbidding them does not change
    the unsplit size, and the library splits the 4 / 8-head 65536-token
    shape (32 chains) but not the 16 / 48-head one (192 chains)."""
    def ws(tokens, hk, hv, seg):
        return L.gdn_chunk_fwd_workspace(L.make_shape(1, tokens, hk, hv, 128, L.GDN_BF16, seg))
    assert ws(4096, 2, 4, 2) > ws(4096, 2, 4, -1)
    assert ws(4096, 16, 48, 0) == ws(4096, 16, 48, -1)
    assert ws(65536, 16, 48, 0) == ws(65536, 16, 48, -1)
    assert ws(65536, 4, 8, 0) > ws(65536, 4, 8, -1)
    assert L.gdn_chunk_bwd_workspace(L.make_shape(1, 65536, 4, 8, 128, L.GDN_BF16)) > \
        L.gdn_chunk_fwd_workspace(L.make_shape(1, 65536, 4, 8, 128, L.GDN_BF16))
