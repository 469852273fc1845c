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
    # chunk op with a workspace that is too small
    st = lib.gdn_chunk_fwd(ctypes.byref(sh), a16, a16, a16, 1024, 1024, 1024, a16, a16,
                           ctypes.c_float(0.1), None, None, a16, a16, a16, 16, None)
    assert st == 4
    # norm: unsupported row length
    assert lib.gdn_gated_norm_fwd(10, 64, 0, a16, a16, a16, ctypes.c_float(1e-6), 0, a16, None) == 2
