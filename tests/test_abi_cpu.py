"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, the ctypes structs match the C layout, and host validation returns
the documented status before anything would be launched (fake device pointers
are never dereferenced on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_sparse_moe_amd as qm
from quantized_sparse_moe_amd import _lib
from quantized_sparse_moe_amd._lib import ExpertsC, LayerC, QTensorC, RouterC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsmoe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libqsmoe.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = qm.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_lib.EXPORTED) == names
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", nm))
    assert exported == set(names)


def test_struct_layout_matches_c(tmp_path):
    probe = tmp_path / "layout.cpp"
    probe.write_text(r'''
#include <cstdio>
#include <cstddef>
#include "qsmoe.h"
int main() {
  printf("%zu %zu %zu %zu\n", sizeof(moe_qtensor), sizeof(moe_experts), sizeof(moe_router), sizeof(moe_layer));
  printf("%zu %zu %zu\n", offsetof(moe_qtensor, codes), offsetof(moe_router, weight), offsetof(moe_router, routed_scale));
  printf("%zu %zu\n", offsetof(moe_layer, routed), offsetof(moe_layer, shared));
}
''')
    exe = tmp_path / "layout"
    r = subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
                        "-I/opt/rocm/include", str(probe), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()
    got = [int(v) for v in out]
    want = [ctypes.sizeof(QTensorC), ctypes.sizeof(ExpertsC), ctypes.sizeof(RouterC), ctypes.sizeof(LayerC),
            QTensorC.codes.offset, RouterC.weight.offset, RouterC.routed_scale.offset,
            LayerC.routed.offset, LayerC.shared.offset]
    assert got == want


# ---------------------------------------------------------------------------- host validation
FAKE = 0x10000  # 64 KiB-aligned fake device address; never dereferenced on these paths


def qt(fmt=0, bits=4, group=64, rows=128, cols=256, E=4, codes=FAKE, scales=FAKE, biases=FAKE):
    return QTensorC(fmt, bits, group, rows, cols, E, codes, scales, biases)


def make_layer(E=4, k=2, d=256, I=128, bits=4, group=64, mode=0, shared=False, **kw):
    routed = ExpertsC(qt(bits=bits, group=group, rows=I, cols=d, E=E, **kw), qt(bits=bits, group=group, rows=I, cols=d, E=E),
                      qt(bits=bits, group=group, rows=d, cols=I, E=E))
    router = RouterC(mode, E, k, d, 100 if mode == 1 else 0, FAKE, FAKE, FAKE if mode == 1 else None, 1.0)
    sh = ctypes.pointer(ExpertsC(qt(bits=8, rows=I, cols=d, E=1), qt(bits=8, rows=I, cols=d, E=1),
                                 qt(bits=8, rows=d, cols=I, E=1))) if shared else ctypes.POINTER(ExpertsC)()
    return LayerC(router, routed, sh)


def fwd(layer, T=3, x=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40, tok=None, out_dtype=0):
    return qm.load().moe_forward(ctypes.byref(layer), x, tok, T, out_dtype, out, ws, ws_bytes, None)


def test_workspace_size_accounts_for_buffers():
    lib = qm.load()
    L = make_layer()
    n1 = lib.moe_workspace_size(ctypes.byref(L), 1)
    n64 = lib.moe_workspace_size(ctypes.byref(L), 64)
    assert 0 < n1 < n64
    # y_slot fp32 [T*k][d] alone is 64*2*256*4 bytes
    assert n64 >= 64 * 2 * 256 * 4 + 64 * 2 * 128 * 2
    Ls = make_layer(shared=True)
    assert lib.moe_workspace_size(ctypes.byref(Ls), 64) > n64
    bad = make_layer(bits=5)
    assert lib.moe_workspace_size(ctypes.byref(bad), 64) == 0


def _layout(L, T):
    out = _lib.WsLayoutC()
    st = qm.load().moe_workspace_layout(ctypes.byref(L), T, ctypes.byref(out))
    return st, out


@pytest.mark.parametrize("mode,E,k,shared", [(1, 1024, 2, False), (0, 1024, 2, False), (1, 16, 6, True),
                                             (0, 256, 6, True)])
def test_workspace_size_serves_every_smaller_token_count(mode, E, k, shared):
    """moe_workspace_size never falls as max_tokens grows, and a workspace of
    that size holds moe_forward's layout for every T <= max_tokens (hash
    layers keep logits, keys and scores on the small-batch path only)."""
    lib = qm.load()
    L = make_layer(E=E, k=k, mode=mode, shared=shared)
    sizes = [lib.moe_workspace_size(ctypes.byref(L), n) for n in range(1, 41)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:])), sizes
    for n in (1, 3, 4, 5, 8, 40):
        for T in range(1, n + 1):
            st, lay = _layout(L, T)
            assert st == _lib.MOE_OK and 0 < lay.total <= sizes[n - 1], (n, T, lay.total, sizes[n - 1])


def test_workspace_layout_regions():
    """Regions are 256-byte aligned, inside the workspace and disjoint; the
    small-batch path keeps no buckets or y_slot, the general path does."""
    lib = qm.load()
    for mode, shared, T in [(0, True, 1), (0, True, 3), (0, True, 40), (1, False, 2), (1, False, 9)]:
        L = make_layer(E=16, k=2, mode=mode, shared=shared)
        st, lay = _layout(L, T)
        assert st == _lib.MOE_OK
        E, k, d, I = 16, 2, 256, 128
        sizes = {"ids": T * k * 4, "weights": T * k * 4, "logits": T * E * 4, "keys": T * E * 8,
                 "scores": T * E * 4, "offsets": (E + 1) * 4, "perm": T * k * 4, "h": T * k * I * 2,
                 "h_shared": T * I * 2, "y_slot": T * k * d * 4, "y_shared": T * d * 4}
        spans = []
        for name, size in sizes.items():
            off = getattr(lay, name)
            if off:
                assert off % 256 == 0 and off + size <= lay.total, name
                spans.append((off, off + size, name))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:])), spans
        assert lay.fused == (1 if T <= 4 else 0)
        present = {n for _, _, n in spans}
        assert {"ids", "weights", "h"} <= present
        assert ("y_slot" in present) == (not lay.fused) and ("perm" in present) == (not lay.fused)
        assert ("keys" in present) == (mode == 0 or T <= 4)
        assert ("h_shared" in present) == shared
    assert _layout(make_layer(), 0)[0] == _lib.MOE_ERR_INVALID_ARG
    assert _layout(make_layer(bits=5), 2)[0] == _lib.MOE_ERR_UNSUPPORTED


def test_zero_tokens_is_ok_without_launch():
    assert fwd(make_layer(), T=0) == _lib.MOE_OK


@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), _lib.MOE_ERR_UNSUPPORTED),
    (dict(group=16), _lib.MOE_ERR_UNSUPPORTED),
    (dict(k=5), _lib.MOE_ERR_INVALID_ARG),
    (dict(k=0), _lib.MOE_ERR_INVALID_ARG),
    (dict(E=2000, k=2), _lib.MOE_ERR_UNSUPPORTED),
    (dict(d=260), _lib.MOE_ERR_UNSUPPORTED),
    (dict(codes=FAKE + 4), _lib.MOE_ERR_ALIGNMENT),
])
def test_layer_validation(kw, status):
    assert fwd(make_layer(**kw)) == status


def test_pointer_and_workspace_checks():
    L = make_layer()
    assert fwd(L, x=None) == _lib.MOE_ERR_INVALID_ARG
    assert fwd(L, x=FAKE + 2) == _lib.MOE_ERR_ALIGNMENT
    assert fwd(L, ws=None) == _lib.MOE_ERR_WORKSPACE
    assert fwd(L, ws_bytes=1024) == _lib.MOE_ERR_WORKSPACE
    assert fwd(L, ws=FAKE + 16) == _lib.MOE_ERR_ALIGNMENT
    assert fwd(L, out_dtype=7) == _lib.MOE_ERR_INVALID_ARG
    Lh = make_layer(mode=1)
    assert fwd(Lh, tok=None) == _lib.MOE_ERR_INVALID_ARG
    Lm = make_layer()
    Lm.routed.gate.num_experts = 3
    assert fwd(Lm) == _lib.MOE_ERR_INVALID_ARG
    Lb = make_layer()
    Lb.routed.up.bits = 8
    assert fwd(Lb) == _lib.MOE_ERR_UNSUPPORTED


def test_mxfp4_requires_group_32():
    L = make_layer()
    for q in (L.routed.gate, L.routed.up, L.routed.down):
        q.format, q.group_size, q.biases = 1, 64, None
    assert fwd(L) == _lib.MOE_ERR_UNSUPPORTED


def test_stage_entry_points_validate():
    lib = qm.load()
    L = make_layer()
    assert lib.moe_permute(FAKE, 3, 9, 4, FAKE, FAKE, FAKE, 4096, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(FAKE, 3, 2, 4, FAKE, FAKE, None, 4096, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_permute(FAKE, 0, 2, 4, FAKE, FAKE, FAKE, 4096, None) == _lib.MOE_OK
    assert lib.moe_combine(FAKE, FAKE, None, 2, 2, 6, 0, FAKE, None) == _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(FAKE, FAKE, None, 0, 2, 8, 0, FAKE, None) == _lib.MOE_OK
    assert lib.moe_route(ctypes.byref(L.router), FAKE, None, 4, FAKE, FAKE, FAKE, 16, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_expert_ffn(ctypes.byref(L.routed), None, FAKE, 4, 2, FAKE, FAKE, FAKE, None, FAKE, 16,
                              None) == _lib.MOE_ERR_WORKSPACE
    Ls = make_layer(shared=True)
    assert lib.moe_expert_ffn(ctypes.byref(Ls.routed), Ls.shared, FAKE, 4, 2, FAKE, FAKE, FAKE, None, FAKE,
                              1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_init(None, 0, None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_status_string(-3) == b"misaligned pointer"


def test_quantize_affine_validates_before_launch():
    lib = _lib.load()
    F = 4096  # fake, aligned device addresses: every call below returns before any launch
    q = lib.moe_quantize_affine
    assert q(F, 2, 128, 5, 64, F, F, F, None, None) == _lib.MOE_ERR_UNSUPPORTED        # bits
    assert q(F, 2, 128, 4, 16, F, F, F, None, None) == _lib.MOE_ERR_UNSUPPORTED        # group
    assert q(F, 2, 96, 4, 64, F, F, F, None, None) == _lib.MOE_ERR_UNSUPPORTED         # cols % group
    assert q(F, -1, 128, 4, 64, F, F, F, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert q(None, 0, 128, 4, 64, None, None, None, None, None) == _lib.MOE_OK          # nothing to do
    assert q(None, 2, 128, 4, 64, F, F, F, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert q(F + 2, 2, 128, 4, 64, F, F, F, None, None) == _lib.MOE_ERR_ALIGNMENT
    assert q(F, 2, 128, 4, 64, F + 4, F, F, None, None) == _lib.MOE_ERR_ALIGNMENT


def test_mhc_sinkhorn_validates_before_launch():
    lib = _lib.load()
    F = 4096
    s = lib.moe_mhc_sinkhorn
    assert s(F, 8, 3, 10, 0.0, F, None) == _lib.MOE_ERR_UNSUPPORTED          # n
    assert s(F, -1, 4, 10, 0.0, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert s(F, 8, 4, -1, 0.0, F, None) == _lib.MOE_ERR_INVALID_ARG          # iters
    assert s(F, 8, 4, 10, -1.0, F, None) == _lib.MOE_ERR_INVALID_ARG         # eps
    assert s(F, 8, 4, 10, float("nan"), F, None) == _lib.MOE_ERR_INVALID_ARG
    assert s(None, 0, 4, 10, 0.0, None, None) == _lib.MOE_OK                 # nothing to do
    assert s(None, 8, 4, 10, 0.0, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert s(F + 2, 8, 4, 10, 0.0, F, None) == _lib.MOE_ERR_ALIGNMENT


def test_probe_entry_points_validate():
    lib = _lib.load()
    F = 4096
    assert lib.moe_probe_stream(None, 1024, 0, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_probe_stream(F, 1000, 0, F, None) == _lib.MOE_ERR_INVALID_ARG     # not a multiple of 128
    assert lib.moe_probe_stream(F, 1024, 3, F, None) == _lib.MOE_ERR_INVALID_ARG     # mode
    assert lib.moe_probe_stream(F, 1024, 0, None, None) == _lib.MOE_ERR_INVALID_ARG  # read needs a sink
    assert lib.moe_probe_stream(F + 8, 1024, 2, None, None) == _lib.MOE_ERR_ALIGNMENT
    assert lib.moe_probe_mfma(0, 10, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_probe_mfma(4, 10, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_probe_mfma(4, 10, F + 4, None) == _lib.MOE_ERR_ALIGNMENT
