"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import moe_layer_forward_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols(header):
    with open(os.path.join(ROOT, "include", header)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["moe.h", "moe_measure.h"]


@pytest.mark.parametrize("header,binding", [("moe.h", moe), ("moe_measure.h", moe.measure)])
def test_library_exports_every_declared_symbol(header, binding):
    L = binding.lib()
    names = declared_symbols(header)
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_measure_helpers_not_in_layer_library():
    L = moe.lib()
    for n in moe.measure.EXPORTS:
        assert not hasattr(L, n), n


def test_strerror():
    assert moe.moe_strerror(0) == "ok"
    assert moe.moe_strerror(-2) == "workspace too small"
    assert moe.moe_strerror(-99) == "unknown status"


def test_workspace_bytes():
    s = moe.make_shape(8, 4096, 8, 2, 14336)
    n = moe.moe_workspace_bytes(s)
    # at least H (bf16) and y_perm (fp32) for the 16 assignments
    assert n >= 16 * 14336 * 2 + 16 * 4096 * 4
    assert n % 256 == 0
    s1 = moe.make_shape(64, 7168, 256, 8, 2048, "bf16", "int4", n_shared=1)
    n1 = moe.moe_workspace_bytes(s1)
    assert n1 >= 512 * 2048 * 2 + 512 * 7168 * 4 + 64 * 2048 * 2 + 64 * 7168 * 4
    assert moe.moe_workspace_bytes(moe.make_shape(8, 4096, 8, 9, 14336)) == 0


BAD_SHAPES = [
    (dict(T=-1), moe.MOE_EINVAL),
    (dict(E=0), moe.MOE_EINVAL),
    (dict(E=257), moe.MOE_EINVAL),
    (dict(k=0), moe.MOE_EINVAL),
    (dict(k=9), moe.MOE_EINVAL),
    (dict(E=32, k=17), moe.MOE_EINVAL),
    (dict(d=100), moe.MOE_EINVAL),
    (dict(F=0), moe.MOE_EINVAL),
    (dict(n_shared=2), moe.MOE_EINVAL),
    (dict(act=7), moe.MOE_EINVAL),
    (dict(wt=9), moe.MOE_EINVAL),
    (dict(wt="int4", d=4104), moe.MOE_EINVAL),
    (dict(act="f32", wt="bf16"), moe.MOE_EUNSUPPORTED),
    (dict(act="bf16", wt="f32"), moe.MOE_EUNSUPPORTED),
    (dict(d=20480), moe.MOE_EUNSUPPORTED),
    (dict(wt="int4", d=16384 + 128), moe.MOE_EUNSUPPORTED),          # int4 K above 16384
    (dict(wt="int4_tiled", d=4096 + 128), moe.MOE_EUNSUPPORTED),   # K not a multiple of 1024
    (dict(wt="int4_tiled", F=9216), moe.MOE_EUNSUPPORTED),         # K above 8192 (down)
    (dict(wt="int4_tiled", d=4104), moe.MOE_EINVAL),
    (dict(act="f32", wt="int4_tiled", F=4096), moe.MOE_EUNSUPPORTED),
    (dict(wt="mxfp4_tiled", d=4096 + 64), moe.MOE_EUNSUPPORTED),    # K not a multiple of 1024
    (dict(wt="mxfp4_tiled", d=4104), moe.MOE_EINVAL),               # not a multiple of 64
    (dict(wt="mxfp8_tiled", d=4096 + 64), moe.MOE_EUNSUPPORTED),    # K not a multiple of 1024
    (dict(wt="mxfp8_tiled", F=14336 + 512), moe.MOE_EUNSUPPORTED),  # down K not a multiple of 1024
    (dict(wt="mxfp8_tiled", d=4104), moe.MOE_EINVAL),               # not a multiple of 64
    (dict(act="f32", wt="mxfp8_tiled"), moe.MOE_EUNSUPPORTED),
]


@pytest.mark.parametrize("bad,code", BAD_SHAPES)
def test_bad_shape_rejected_before_any_launch(bad, code):
    args = dict(T=8, d=4096, E=8, k=2, F=14336, act="bf16", wt="bf16")
    args.update(bad)
    s = moe.make_shape(**args)
    fake = 1 << 20   # never dereferenced: validation fails first
    for call in (
        lambda: moe.moe_route(s, fake, fake, None, fake, fake, fake, stream=0),
        lambda: moe.moe_dispatch(s, fake, fake, fake, fake, fake, stream=0),
        lambda: moe.moe_combine(s, fake, fake, fake, None, None, fake, stream=0),
    ):
        with pytest.raises(moe.MoEError) as ei:
            call()
        assert ei.value.status == code


def test_null_and_misaligned_pointers():
    s = moe.make_shape(8, 64, 8, 2, 128, "f32", "f32")
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_route(s, None, 1 << 20, None, 1 << 20, 1 << 20, 1 << 20, stream=0)
    assert ei.value.status == moe.MOE_EINVAL and "x is NULL" in str(ei.value)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_route(s, (1 << 20) + 4, 1 << 20, None, 1 << 20, 1 << 20, 1 << 20, stream=0)
    assert "aligned" in str(ei.value)


def test_workspace_too_small_is_enomem():
    s = moe.make_shape(8, 64, 8, 2, 128, "f32", "f32")
    w = moe.make_weights(1 << 20, 1 << 20, 1 << 20)
    p = 1 << 20
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward(s, p, p, None, w, None, p, None, None, p, ws_bytes=256, stream=0)
    assert ei.value.status == moe.MOE_ENOMEM
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_expert_ffn(s, p, w, p, p, p, p, None, p, ws_bytes=0, stream=0)
    assert ei.value.status == moe.MOE_ENOMEM


def test_int4_needs_scales():
    s = moe.make_shape(8, 128, 8, 2, 128, "bf16", "int4")
    w = moe.make_weights(1 << 20, 1 << 20, 1 << 20)
    p = 1 << 20
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward(s, p, p, None, w, None, p, None, None, p, ws_bytes=1 << 30, stream=0)
    assert ei.value.status == moe.MOE_EINVAL and "s_gate" in str(ei.value)


def test_error_message_truncated_to_buffer():
    L = moe.lib()
    s = moe.make_shape(8, 4096, 8, 9, 14336)
    buf = ctypes.create_string_buffer(8)
    rc = L.moe_route(ctypes.byref(s), None, None, None, None, None, None, None, buf, 8)
    assert rc == moe.MOE_EINVAL
    assert len(buf.value) == 7   # NUL-terminated inside the 8 bytes
    rc = L.moe_route(ctypes.byref(s), None, None, None, None, None, None, None, None, 0)
    assert rc == moe.MOE_EINVAL


def test_rmsnorm_validation():
    s = moe.make_shape(4, 12, 8, 2, 128, "f32", "f32")
    with pytest.raises(moe.MoEError):
        moe.moe_rmsnorm(s, 1 << 20, None, 1e-6, 1 << 20, stream=0)
    s = moe.make_shape(4, 16, 8, 2, 128, "f32", "f32")
    with pytest.raises(moe.MoEError):
        moe.moe_rmsnorm(s, 1 << 20, None, -1.0, 1 << 20, stream=0)


def test_read_ceiling_validation():
    # rejected before any HIP call
    with pytest.raises(moe.MoEError) as e:
        moe.measure.moe_read_ceiling(4096, 100, 8192)
    assert e.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoEError):
        moe.measure.moe_read_ceiling(None, 1024, 8192)
    with pytest.raises(moe.MoEError):
        moe.measure.moe_read_ceiling(4096, 1024, None)
    with pytest.raises(moe.MoEError):
        moe.measure.moe_read_ceiling(4104, 1024, 8192)     # misaligned buffer
    assert moe.measure.moe_read_ceiling(None, 0, 8192) == 0


def test_pack_int4_tiled_validation():
    p, q = 1 << 20, 1 << 30
    for args in ((p, q, -1, 16, 128), (p, q, 1, 8, 128), (p, q, 1, 24, 128), (p, q, 1, 16, 100),
                 (p, q, 1, 16, 0), (None, q, 1, 16, 128), (p, None, 1, 16, 128),
                 (p + 8, q, 1, 16, 128),                 # misaligned
                 (p, p + 512, 1, 16, 128)):              # overlapping (1 KB each)
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_pack_int4_tiled(*args, stream=0)
        assert ei.value.status == moe.MOE_EINVAL, args
    assert moe.moe_pack_int4_tiled(None, None, 0, 16, 128, stream=0) == 0


def test_pack_mxfp8_tiled_validation():
    p, q = 1 << 20, 1 << 30
    for args in ((p, q, -1, 16, 128), (p, q, 1, 8, 128), (p, q, 1, 24, 128), (p, q, 1, 16, 100),
                 (p, q, 1, 16, 0), (None, q, 1, 16, 128), (p, None, 1, 16, 128),
                 (p + 8, q, 1, 16, 128),                 # misaligned
                 (p, p + 1024, 1, 16, 128)):             # overlapping (2 KB each)
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_pack_mxfp8_tiled(*args, stream=0)
        assert ei.value.status == moe.MOE_EINVAL, args
    assert moe.moe_pack_mxfp8_tiled(None, None, 0, 16, 128, stream=0) == 0


def test_mfma_ceiling_validation():
    p = 1 << 20
    for args in ((0, p, 1 << 20), ((1 << 24) + 1, p, 1 << 20), (10, None, 1 << 20), (10, p + 4, 1 << 20),
                 (10, p, 16)):
        with pytest.raises(moe.MoEError) as ei:
            moe.measure.moe_mfma_ceiling(*args, stream=0)
        assert ei.value.status == moe.MOE_EINVAL, args
    with pytest.raises(moe.MoEError):
        moe.measure.moe_mfma_ceiling(10, p, 1 << 20, clock=p + 4, stream=0)   # misaligned clock


def test_noalloc_rejects_shapes_beyond_its_array():
    """The allocation-free entry point refuses a workspace above its fixed
    128 MiB device array before any HIP call, with a clear message."""
    s = moe.make_shape(4096, 4096, 8, 2, 14336)
    assert moe.moe_workspace_bytes(s) > 128 << 20
    p = 1 << 20
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward_noalloc(s, p, p, None, moe.make_weights(p, p, p), None, p, None, None, stream=0)
    assert ei.value.status == moe.MOE_ENOMEM and "fixed device array" in str(ei.value)
    # an invalid shape reports the shape error, not the size
    bad = moe.make_shape(8, 4096, 8, 9, 14336)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward_noalloc(bad, p, p, None, moe.make_weights(p, p, p), None, p, None, None, stream=0)
    assert ei.value.status == moe.MOE_EINVAL
