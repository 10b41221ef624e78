"""Host-side checks of the C ABI (no GPU needed: no compute call is made).

The library must load and export every symbol ``include/dcn.h`` declares;
``dcn_create`` must validate descriptors and refuse what this build cannot
run (page 2, "patch_deform.py", refuses what it cannot prove in range rather
than guessing); pointer checks must fire before any launch.
"""
import ctypes
import os
import re

import pytest

from modulated_deformable_convolution_dcn_amd import _lib, Desc, Plan, DcnError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "dcn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _header_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.dcn_version() == 10100


def test_status_strings():
    lib = _lib.load()
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.dcn_status_string(code).decode().startswith(name)


def _desc(**kw):
    base = dict(batch=1, in_ch=64, height=16, width=16, out_ch=64, kernel_h=3, kernel_w=3,
                pad_h=1, pad_w=1, in_dtype=_lib.DCN_F32, out_dtype=_lib.DCN_F32,
                out_layout=_lib.DCN_OUT_NCHW)
    base.update(kw)
    return _lib.DcnDesc(**base)


def _create(**kw):
    lib = _lib.load()
    h = ctypes.c_void_p(1234)
    st = lib.dcn_create(ctypes.byref(_desc(**kw)), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(), _lib.DCN_OK),
    (dict(batch=0), _lib.DCN_OK),
    (dict(kernel_h=7, kernel_w=7, pad_h=3, pad_w=3), _lib.DCN_OK),
    (dict(in_dtype=_lib.DCN_BF16, in_ch=8), _lib.DCN_OK),
    (dict(out_layout=_lib.DCN_OUT_NHWC), _lib.DCN_OK),
    (dict(out_ch=300), _lib.DCN_OK),
    (dict(batch=-1), 2),
    (dict(in_ch=0), 2),
    (dict(height=0), 2),
    (dict(kernel_w=0), 2),
    (dict(pad_h=-1), 2),
    (dict(height=2, kernel_h=5, pad_h=1), 2),        # Ho = 2 + 2 - 5 + 1 = 0
    (dict(in_dtype=7), 3),
    (dict(out_layout=5), 3),
    (dict(out_dtype=9), 3),
    (dict(out_dtype=_lib.DCN_BF16), 4),
    (dict(in_ch=6), 4),                                 # not a multiple of 4 (fp32)
    (dict(in_dtype=_lib.DCN_BF16, in_ch=12), 4),        # not a multiple of 8 (bf16)
    (dict(batch=1024, height=1024, width=1024, in_ch=4), 4),  # x >= 2^31 bytes
])
def test_create_validates(kw, status):
    lib = _lib.load()
    st, h = _create(**kw)
    assert st == status, lib.dcn_last_error()
    if st == 0:
        assert h.value
        assert lib.dcn_destroy(h) == 0
    else:
        assert not h.value  # *plan set to NULL on failure
        assert lib.dcn_last_error().decode()


def test_null_arguments():
    lib = _lib.load()
    h = ctypes.c_void_p()
    assert lib.dcn_create(None, ctypes.byref(h)) == 1
    assert lib.dcn_create(ctypes.byref(_desc()), None) == 1
    assert lib.dcn_destroy(None) == 0
    sz = ctypes.c_size_t()
    assert lib.dcn_workspace_bytes(None, ctypes.byref(sz)) == 1


def test_output_size_and_workspace():
    p = Plan(Desc(2, 128, 200, 176, 128, 5, 5, 2, 2))
    assert (p.Ho, p.Wo) == (200, 176)
    # packed weight: 25 taps x 2 chunks of 64 channels x 128 outputs, fp32
    assert p.workspace_bytes == 25 * 128 * 128 * 4
    p2 = Plan(Desc(1, 64, 33, 40, 256, 7, 7, 3, 3))
    assert (p2.Ho, p2.Wo) == (33, 40)
    p3 = Plan(Desc(1, 4, 8, 8, 4, 3, 3, 1, 1))
    assert p3.workspace_bytes == 9 * 16 * 16 * 4  # padded to a 16-channel block, 16 outputs
    for p in (p, p2, p3):
        assert p.packed_weight_bytes == p.workspace_bytes  # grids that fill the GPU: no split


@pytest.mark.parametrize("shape,nsplit,kper,groups", [
    ((1, 64, 256, 256, 64, 7, 7, 3, 3), 1, 49, 1),  # 1024 workgroups: no split
    ((1, 64, 128, 128, 64, 7, 7, 3, 3), 1, 49, 2),  # 256 tiles: 8-wave workgroups, 25 + 24 taps
    ((1, 64, 64, 64, 64, 7, 7, 3, 3), 4, 13, 2),    # 64 tiles: four runs (13, 13, 13, 10)
    ((1, 64, 40, 40, 64, 1, 5, 0, 2), 2, 3, 2),     # K = 5, 25 tiles: runs of 3 and 2 taps
    ((1, 64, 20, 20, 64, 1, 3, 0, 1), 1, 3, 2),     # K = 3: no run could keep a tap per group
    ((1, 64, 20, 20, 64, 1, 1, 0, 0), 1, 1, 1),     # K = 1: nothing to split
    ((2, 96, 90, 90, 48, 3, 3, 1, 1), 1, 9, 2),     # 2 images x 127 tiles = 254 workgroups
    ((1, 64, 64, 64, 128, 7, 7, 3, 3), 1, 49, 1),   # 128 outputs: another kernel, no split
])
def test_tap_split_workspace(shape, nsplit, kper, groups):
    """fp32 plans of 17..64 output channels whose grid would fill at most half
    of the 512 resident 4-wave workgroups run 8-wave workgroups of two tap
    groups; if those fill at most half of the 256 resident 8-wave workgroups,
    the taps are also split into runs (at least one tap per group each), and
    the scratch holds one fp32 partial output per run (element count rounded
    up to 64)."""
    B, C, H, W_, O, kh, kw, ph, pw = shape
    p = Plan(Desc(B, C, H, W_, O, kh, kw, ph, pw))
    K = kh * kw
    assert (p.tap_runs, p.taps_per_run, p.tap_groups) == (nsplit, kper, groups)
    if O <= 64:
        assert p.packed_weight_bytes == ((K * -(-C // 64) * 64 * 64 * 4 + 255) // 256) * 256
    n = B * O * p.Ho * p.Wo
    scratch = 0 if nsplit == 1 else nsplit * (-(-n // 64) * 64) * 4
    assert p.workspace_bytes == p.packed_weight_bytes + scratch


def test_pointer_checks_fire_before_any_launch():
    """Null / misaligned / short-workspace errors are reported without touching the GPU."""
    lib = _lib.load()
    p = Plan(Desc(1, 64, 16, 16, 64, 3, 3, 1, 1))
    h = p._h
    fake = ctypes.c_void_p(0x10000)
    ws = p.workspace_bytes
    assert lib.dcn_forward_packed(h, None, fake, None, fake, ws, None, fake, None) == 1
    assert lib.dcn_forward_packed(h, fake, None, None, fake, ws, None, fake, None) == 1
    assert lib.dcn_forward_packed(h, fake, fake, None, fake, ws, None, None, None) == 1
    assert lib.dcn_forward_packed(h, fake, fake, None, None, ws, None, fake, None) == 8
    pw = p.packed_weight_bytes  # the least a forward accepts (no tap split)
    assert pw < ws
    assert lib.dcn_forward_packed(h, fake, fake, None, fake, pw - 1, None, fake, None) == 8
    odd = ctypes.c_void_p(0x10004)
    assert lib.dcn_forward_packed(h, odd, fake, None, fake, ws, None, fake, None) == 5
    assert lib.dcn_forward_packed(h, fake, ctypes.c_void_p(0x10002), None, fake, ws, None, fake,
                                  None) == 5
    assert lib.dcn_pack_weight(h, None, fake, ws, None) == 1
    assert lib.dcn_pack_weight(h, fake, fake, pw - 256, None) == 8
    assert lib.dcn_forward(None, fake, fake, None, fake, None, fake, fake, ws, None) == 1
    assert lib.dcn_debug_coords(h, None, fake, fake, None) == 1
    assert "required" in lib.dcn_last_error().decode()


def test_empty_batch_is_a_no_op():
    lib = _lib.load()
    p = Plan(Desc(0, 64, 16, 16, 64, 3, 3, 1, 1))
    # nothing to read or write: succeeds even with NULL buffers, no launch
    assert lib.dcn_forward(p._h, None, None, None, None, None, None, None, 0, None) == 0
    assert lib.dcn_forward_packed(p._h, None, None, None, None, 0, None, None, None) == 0


def test_python_binding_rejects_bad_tensors():
    import torch
    p = Plan(Desc(1, 4, 8, 8, 4, 3, 3, 1, 1))
    with pytest.raises(ValueError):
        p.forward(torch.zeros(1, 8, 8, 4), torch.zeros(1, 18, 8, 8), None,
                  torch.zeros(4, 4, 3, 3))  # CPU tensors are refused
    with pytest.raises(DcnError):
        Plan(Desc(1, 3, 8, 8, 4, 3, 3, 1, 1))


def test_row_band_checks_fire_before_any_launch():
    """dcn_forward_rows: row range, NULL and workspace errors without touching the GPU."""
    lib = _lib.load()
    p = Plan(Desc(1, 64, 16, 16, 64, 3, 3, 1, 1))  # Ho = 16
    h = p._h
    fake = ctypes.c_void_p(0x10000)
    ws = p.workspace_bytes
    call = lambda r0, n, x=fake, pk=fake, w=ws: lib.dcn_forward_rows(  # noqa: E731
        h, r0, n, x, fake, None, pk, w, None, fake, None)
    assert call(-1, 4) == 2
    assert call(0, -1) == 2
    assert call(13, 4) == 2          # 13 + 4 > 16
    assert call(16, 1) == 2
    assert "outside the output" in lib.dcn_last_error().decode()
    assert call(16, 0) == 0          # empty band at the end: no-op
    assert call(3, 0, x=None) == 0   # empty band: nothing is read
    assert call(3, 4, x=None) == 1
    assert call(3, 4, pk=None) == 8
    assert call(3, 4, w=p.packed_weight_bytes - 1) == 8
    assert lib.dcn_forward_rows(None, 0, 1, fake, fake, None, fake, ws, None, fake, None) == 1


def test_transpose_checks_fire_before_any_launch():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x10000)
    assert lib.dcn_nchw_to_nhwc(fake, fake, 1, 4, 4, 4, 7, None) == 3      # dtype
    assert lib.dcn_nchw_to_nhwc(fake, fake, 1, -4, 4, 4, 0, None) == 2     # negative size
    assert lib.dcn_nchw_to_nhwc(fake, fake, 1 << 16, 1 << 16, 1, 1, 0, None) == 2  # > 2^31 - 1
    assert lib.dcn_nchw_to_nhwc(None, None, 0, 4, 4, 4, 0, None) == 0      # empty: no-op
    assert lib.dcn_nchw_to_nhwc(None, fake, 1, 4, 4, 4, 0, None) == 1
    assert lib.dcn_nchw_to_nhwc(ctypes.c_void_p(0x10004), fake, 1, 4, 4, 4, 1, None) == 5


def test_multi_branch_checks_fire_before_any_launch():
    lib = _lib.load()
    a = Plan(Desc(1, 64, 16, 16, 64, 3, 3, 1, 1))
    b = Plan(Desc(1, 64, 16, 16, 32, 1, 1, 0, 0))
    c = Plan(Desc(1, 64, 16, 15, 64, 3, 3, 1, 1))   # different input width
    fake = 0x10000
    V = ctypes.c_void_p
    arr = lambda *xs: (V * len(xs))(*xs)  # noqa: E731
    sizes = lambda *ps: (ctypes.c_size_t * len(ps))(*[p.workspace_bytes for p in ps])  # noqa: E731

    def call(plans, n=None, x=fake, offs=None, outs=None, packs=None, ws=None):
        n = len(plans) if n is None else n
        offs = offs if offs is not None else arr(*[fake] * len(plans))
        outs = outs if outs is not None else arr(*[fake] * len(plans))
        packs = packs if packs is not None else arr(*[fake] * len(plans))
        ws = ws if ws is not None else sizes(*plans)
        return lib.dcn_forward_multi(n, arr(*[p._h.value for p in plans]), V(x), offs, None,
                                     packs, ws, None, outs, None)

    assert call([a, b], n=0) == 0
    assert call([a, b], n=-1) == 2
    assert call([a] * 9) == 4
    assert call([a, c]) == 2                             # branches read different inputs
    assert "different input" in lib.dcn_last_error().decode()
    assert call([a, b], outs=arr(fake, None)) == 1       # branch 1 has no output
    assert call([a, b], packs=arr(fake, None)) == 8
    short = (ctypes.c_size_t * 2)(a.workspace_bytes, b.workspace_bytes - 1)
    assert call([a, b], ws=short) == 8                   # branch 1's workspace too small
    assert call([a, b], x=0) == 1                        # shared input missing
    assert lib.dcn_forward_multi(1, None, V(fake), None, None, None, None, None, None, None) == 1


def test_backward_checks_fire_before_any_launch():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x10000)
    V = ctypes.c_void_p
    p = Plan(Desc(1, 64, 16, 16, 64, 3, 3, 1, 1))
    n = ctypes.c_size_t()
    assert lib.dcn_backward_workspace_bytes(p._h, ctypes.byref(n)) == 0
    assert n.value == 9 * 1 * 64 * 64 * 4       # taps x chunks x 64 outputs x 64 channels
    ws = n.value
    args = lambda **kw: [kw.get(k, fake) for k in (  # noqa: E731
        "x", "off", "mask", "w", "g", "gx", "goff", "gmask", "gw", "gb")]
    call = lambda plan=p, wsp=fake, wsn=ws, **kw: lib.dcn_backward(  # noqa: E731
        plan._h, *args(**kw), wsp, wsn, None)
    assert call(x=None) == 1
    assert call(g=None) == 1
    assert call(wsp=None) == 8
    assert call(wsn=ws - 1) == 8
    assert call(x=V(0x10004)) == 5
    assert call(gw=V(0x10002)) == 5
    bf = Plan(Desc(1, 64, 16, 16, 64, 3, 3, 1, 1, "bf16"))
    nb = ctypes.c_size_t()
    assert lib.dcn_backward_workspace_bytes(bf._h, ctypes.byref(nb)) == 0
    # the re-packed weight, then fp32 copies of x, offset, mask and weight
    r = lambda v: -(-v // 256) * 256  # noqa: E731
    assert nb.value == ws + r(16 * 16 * 64 * 4) + r(18 * 256 * 4) + r(9 * 256 * 4) + r(
        64 * 64 * 9 * 4)
    assert call(plan=bf) == 8                        # the fp32 plan's workspace is too small
    assert call(plan=bf, off=V(0x10001), wsn=nb.value) == 5
    wide = Plan(Desc(1, 64, 16, 16, 300, 3, 3, 1, 1))
    assert call(plan=wide) == 4
    assert "256" in lib.dcn_last_error().decode()
    empty = Plan(Desc(0, 64, 16, 16, 64, 3, 3, 1, 1))
    assert lib.dcn_backward(empty._h, *[None] * 10, None, 0, None) == 0


def test_msda_create_validates_and_checks_pointers():
    from modulated_deformable_convolution_dcn_amd import MsdaPlan
    lib = _lib.load()
    p = MsdaPlan(2, 10, 8, 32, [(8, 8), (4, 4)], 4, softmax=True)
    assert p.S == 80
    bad = [dict(shapes=[(8, 8)] * 9), dict(K=9), dict(D=30), dict(D=2048), dict(shapes=[(0, 4)])]
    want = [4, 4, 4, 4, 2]
    for kw, st in zip(bad, want):
        args = dict(B=1, Q=4, G=2, D=8, shapes=[(4, 4)], K=2)
        args.update(kw)
        with pytest.raises(_lib.DcnError) as e:
            MsdaPlan(args["B"], args["Q"], args["G"], args["D"], args["shapes"], args["K"])
        assert e.value.status == st, (kw, e.value.status)
    fake = ctypes.c_void_p(0x10000)
    h = p._h
    assert lib.dcn_msda_forward(h, None, fake, fake, fake, None) == 1
    assert lib.dcn_msda_forward(h, ctypes.c_void_p(0x10008), fake, fake, fake, None) == 5
    assert lib.dcn_msda_forward(h, fake, ctypes.c_void_p(0x10002), fake, fake, None) == 5
    assert lib.dcn_msda_forward(h, fake, fake, ctypes.c_void_p(0x10001), fake, None) == 5
    empty = MsdaPlan(0, 10, 8, 32, [(8, 8)], 4)
    assert lib.dcn_msda_forward(empty._h, None, None, None, None, None) == 0
