"""The C ABI on the host: exports, descriptor validation, argument errors (no GPU needed).

The encoder's rules come from "2 · Le Tensor Memory Accelerator" §2.2–§2.3 (rank up to 5,
16-byte base and stride alignment, swizzle width) and "H100 · cuTensorMap" §8–§9, §14
(dimension ranges, element strides 1..8, box, NaN fill for floating types)."""
import ctypes
import subprocess

import numpy as np

import pytest

import tiled_bf16_gemm_amd as tbg

BASE = 0x7F00_0000_0000  # any 16-byte-aligned address: encoding never touches memory


def test_library_exports_every_declared_function():
    names = tbg.declared_functions()
    assert set(names) >= {"tbg_encode_tiled", "tbg_box_bytes", "tbg_tiled_copy", "tbg_tiled_copy_many",
                          "tbg_tiled_store", "tbg_tiled_store_many", "tbg_gemm_workspace_bytes", "tbg_gemm",
                          "tbg_gemm_ex", "tbg_status_string", "tbg_last_error"}
    lib = ctypes.CDLL(tbg.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", tbg.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, f"{n} not exported with C linkage"


def test_status_strings():
    assert tbg.status_string(tbg.OK) == "TBG_OK"
    assert tbg.status_string(tbg.ERR_MISALIGNED) == "TBG_ERR_MISALIGNED"
    assert tbg.status_string(99) == "TBG_ERR_UNKNOWN"


def _c1_args(**over):
    a = dict(dtype="bf16", rank=2, global_address=BASE, global_dim=[256, 256], global_strides=[512],
             box_dim=[64, 128], element_strides=[1, 1], swizzle="128B", l2="128B", oob="zero")
    a.update(over)
    return a


def _c3_args(**over):
    a = dict(dtype="bf16", rank=5, global_address=BASE, global_dim=[200, 129, 7, 5, 3],
             global_strides=[400, 51600, 361200, 1806000], box_dim=[64, 16, 4, 2, 2],
             element_strides=[1, 2, 1, 1, 1], swizzle="none", l2="none", oob="nan")
    a.update(over)
    return a


def test_workload_descriptors_encode():
    d = tbg.encode_tiled(**_c1_args())
    assert tbg.box_bytes(d) == 64 * 128 * 2 == 16384
    d = tbg.encode_tiled(**_c3_args())
    assert tbg.box_bytes(d) == 2 * (64 * 8 * 4 * 2 * 2) == 16384
    # GEMM operand boxes: A {64 k, 256 m} with the 2-row swizzle, B (K×N) {64 n, 64 k} 128B
    d = tbg.encode_tiled("bf16", 2, BASE, [8192, 8192], [16384], [64, 256], [1, 1], "128B_2ROW")
    assert tbg.box_bytes(d) == 32768
    d = tbg.encode_tiled("bf16", 2, BASE, [8192, 8192], [16384], [64, 64], [1, 1], "128B")
    assert tbg.box_bytes(d) == 8192


@pytest.mark.parametrize("over,status", [
    (dict(rank=0), tbg.ERR_UNSUPPORTED),
    (dict(rank=6, global_dim=[1] * 6, box_dim=[1] * 6, element_strides=[1] * 6, global_strides=[16] * 5),
     tbg.ERR_UNSUPPORTED),
    (dict(global_address=BASE + 8), tbg.ERR_MISALIGNED),
    (dict(global_address=0), tbg.ERR_INVALID_VALUE),
    (dict(global_strides=[520]), tbg.ERR_MISALIGNED),
    (dict(global_dim=[0, 256]), tbg.ERR_OUT_OF_RANGE),
    (dict(global_dim=[(1 << 32) + 1, 256]), tbg.ERR_OUT_OF_RANGE),
    (dict(box_dim=[0, 128]), tbg.ERR_OUT_OF_RANGE),
    (dict(box_dim=[64, 257]), tbg.ERR_OUT_OF_RANGE),
    (dict(element_strides=[0, 1]), tbg.ERR_OUT_OF_RANGE),
    (dict(element_strides=[1, 9]), tbg.ERR_OUT_OF_RANGE),
    (dict(box_dim=[128, 8]), tbg.ERR_INVALID_VALUE),             # 256-byte rows exceed the 128B span
    (dict(swizzle="64B"), tbg.ERR_INVALID_VALUE),                # 128-byte rows exceed the 64B span
    (dict(swizzle="32B", box_dim=[16, 8]), tbg.OK),
    (dict(swizzle="128B", box_dim=[8, 3], element_strides=[1, 1]), tbg.ERR_INVALID_VALUE),
    (dict(dtype="u16", oob="nan"), tbg.ERR_INVALID_VALUE),       # NaN fill needs a floating type
    (dict(dtype="f32", box_dim=[32, 128], oob="nan"), tbg.OK),
    (dict(swizzle=7), tbg.ERR_INVALID_VALUE),
    (dict(oob=3), tbg.ERR_INVALID_VALUE),
    (dict(l2=9), tbg.ERR_INVALID_VALUE),
    (dict(dtype=42), tbg.ERR_INVALID_VALUE),
    (dict(box_dim=[64, 256], element_strides=[1, 1], swizzle="none", global_strides=[512]), tbg.OK),
])
def test_encode_rejections(over, status):
    assert tbg.encode_tiled_status(**_c1_args(**over)) == status, tbg.last_error()


def test_encode_image_limit_and_estride_rounding():
    # 5 dims of box 8 with element stride 3: n = 3 per dim -> 3^5 = 243 elements
    d = tbg.encode_tiled("u8", 5, BASE, [9] * 5, [16, 160, 1600, 16000], [8] * 5, [3] * 5)
    assert tbg.box_bytes(d) == 243
    # 256 x 256 bf16 = 128 KiB image: over the 64 KiB limit
    assert tbg.encode_tiled_status("bf16", 2, BASE, [256, 256], [512], [256, 256], [1, 1]) == tbg.ERR_OUT_OF_RANGE
    assert "64 KiB" in tbg.last_error()


def test_box_bytes_of_garbage_is_zero():
    assert tbg.box_bytes(tbg.TensorDesc()) == 0


def test_gemm_argument_errors():
    g = dict(M=64, N=64, K=64, A=BASE, lda=64, B=BASE, ldb=64, b_layout="kn", C=BASE, ldc=64, c_dtype="f32")
    assert tbg.gemm_status(**{**g, "M": -1}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "lda": 63}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "ldb": 32}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "b_layout": "nk", "ldb": 63}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "ldc": 10}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "c_dtype": "u8"}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "b_layout": 5}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "lda": 1 << 22}) == tbg.ERR_UNSUPPORTED
    assert tbg.gemm_status(**{**g, "C": 0}) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_status(**{**g, "A": 0}) == tbg.ERR_INVALID_VALUE
    # empty output: nothing to do, no device needed
    assert tbg.gemm_status(**{**g, "M": 0, "A": 0, "B": 0, "C": 0}) == tbg.OK
    assert tbg.gemm_status(**{**g, "N": 0}) == tbg.OK


def test_workspace_bytes():
    assert tbg.gemm_workspace_bytes(8192, 8192, 8192, 8192, 8192, "kn") == 0
    assert tbg.gemm_workspace_bytes(16384, 14336, 4096, 4096, 4096, "nk") == 0
    # the ragged workload: lda = 777 and ldb = 2049 are not 16-byte pitches
    a = (3001 * 784 * 2 + 255) // 256 * 256
    b = (777 * 2056 * 2 + 255) // 256 * 256
    assert tbg.gemm_workspace_bytes(3001, 2049, 777, 777, 2049, "kn") == a + b
    # padded pitches but K = 777 still needs A repacked (a partial 16-byte chunk along K)
    assert tbg.gemm_workspace_bytes(3001, 2049, 777, 784, 2056, "kn") == a
    assert tbg.gemm_workspace_bytes(64, 64, 64, 64, 72, "nk") == 0
    assert tbg.gemm_workspace_bytes(64, 64, 60, 64, 64, "nk") == 2 * ((64 * 64 * 2 + 255) // 256 * 256)


def test_calls_without_a_device_fail_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = tbg.gemm_status(64, 64, 64, BASE, 64, BASE, 64, "kn", BASE, 64, "f32")
    assert st == tbg.ERR_NO_DEVICE, tbg.last_error()
    d = tbg.encode_tiled(**_c1_args())
    with pytest.raises(tbg.Error) as e:
        tbg.tiled_copy(d, [0, 0], BASE)
    assert e.value.status == tbg.ERR_NO_DEVICE
    with pytest.raises(tbg.Error) as e:
        tbg.tiled_copy(d, [0, 0], BASE + 8)
    assert e.value.status == tbg.ERR_MISALIGNED
    assert tbg.gemm_status(64, 64, 64, BASE, 64, BASE, 64, "kn", BASE, 64, "f32") == tbg.ERR_NO_DEVICE


def _gemm_ex_status(**kw):
    try:
        tbg.gemm_ex(**kw)
        return tbg.OK
    except tbg.Error as e:
        return e.status


def test_gemm_ex_argument_errors():
    """tbg_gemm_ex checks what tbg_gemm checks; alpha = 0 takes no operand (the product is skipped)."""
    g = dict(M=64, N=64, K=64, alpha=2.0, A=BASE, lda=64, B=BASE, ldb=64, b_layout="kn", beta=0.5, C=BASE, ldc=64,
             c_dtype="f32")
    assert _gemm_ex_status(**{**g, "M": -1}) == tbg.ERR_INVALID_VALUE
    assert _gemm_ex_status(**{**g, "lda": 63}) == tbg.ERR_INVALID_VALUE
    assert _gemm_ex_status(**{**g, "ldc": 10}) == tbg.ERR_INVALID_VALUE
    assert _gemm_ex_status(**{**g, "c_dtype": "u16"}) == tbg.ERR_INVALID_VALUE
    assert _gemm_ex_status(**{**g, "b_layout": 7}) == tbg.ERR_INVALID_VALUE
    assert _gemm_ex_status(**{**g, "A": 0}) == tbg.ERR_INVALID_VALUE
    assert _gemm_ex_status(**{**g, "C": 0}) == tbg.ERR_INVALID_VALUE
    assert _gemm_ex_status(**{**g, "N": 0, "C": 0}) == tbg.OK
    import torch
    if not torch.cuda.is_available():
        # alpha = 0: null operands and any leading dimensions pass the host checks
        st = _gemm_ex_status(**{**g, "alpha": 0.0, "A": 0, "B": 0, "lda": 0, "ldb": 0})
        assert st == tbg.ERR_NO_DEVICE, tbg.last_error()


def test_tiled_store_argument_errors():
    d = tbg.encode_tiled(**_c1_args())
    with pytest.raises(tbg.Error) as e:
        tbg.tiled_store(tbg.TensorDesc(), [0, 0], BASE)
    assert e.value.status == tbg.ERR_INVALID_VALUE
    with pytest.raises(tbg.Error) as e:
        tbg.tiled_store(d, [0, 0], 0)
    assert e.value.status == tbg.ERR_INVALID_VALUE
    with pytest.raises(tbg.Error) as e:
        tbg.tiled_store(d, [0, 0], BASE + 4)
    assert e.value.status == tbg.ERR_MISALIGNED
    tbg.tiled_store_many(d, 0, 0, 0)  # n == 0: nothing to do
    with pytest.raises(tbg.Error) as e:
        tbg.tiled_store_many(d, 0, 3, BASE)
    assert e.value.status == tbg.ERR_INVALID_VALUE
    import torch
    if not torch.cuda.is_available():
        with pytest.raises(tbg.Error) as e:
            tbg.tiled_store(d, [0, 0], BASE)
        assert e.value.status == tbg.ERR_NO_DEVICE


# Every configuration tbg.h lists as built, and some it does not.
BUILT_CONFIGS = ([("ring", "256x256", 2)] + [("ring", t, s) for t in ("256x128", "128x256") for s in (2, 3)]
                 + [("ring", "128x128", s) for s in (2, 3, 4, 5)] + [("ring", "64x64", s) for s in range(2, 7)]
                 + [("producer", t, s) for t in ("256x128", "128x256") for s in (2, 3)]
                 + [("producer", "128x128", s) for s in (2, 3, 4)] + [("producer", "64x64", s) for s in range(2, 7)])
NOT_BUILT = [("ring", "256x256", 3), ("producer", "256x256", 2), ("ring", "128x128", 6), ("producer", "128x128", 5),
             ("ring", "64x64", 7), ("ring", "96x96", 2), ("ring", "128x64", 2), ("producer", "64x64", 9)]


def test_gemm_configured_checks():
    """tbg_gemm_configured: malformed configurations are INVALID_VALUE, configurations that are not
    built are UNSUPPORTED, both before any device check; built ones pass the host checks."""
    import torch
    g = dict(M=64, N=64, K=64, alpha=1.0, A=BASE, lda=64, B=BASE, ldb=64, b_layout="kn", beta=0.0, C=BASE, ldc=64,
             c_dtype="f32")
    assert tbg.gemm_configured_status(**g, config=None) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_configured_status(**g, config=tbg.GemmConfig(0, 0, 0, 7)) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_configured_status(**g, config=tbg.GemmConfig(128, 0, 0, 1)) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_configured_status(**g, config=tbg.GemmConfig(128, 128, 1, 1)) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_configured_status(**g, config=tbg.GemmConfig(128, 128, -2, 1)) == tbg.ERR_INVALID_VALUE
    for pipe, tile, st in NOT_BUILT:
        s = tbg.gemm_configured_status(**g, config=tbg.gemm_config(tile, st, pipe))
        assert s == tbg.ERR_UNSUPPORTED, (pipe, tile, st, tbg.status_string(s))
        assert "built:" in tbg.last_error()
    # the usual argument checks still apply
    cfg = tbg.gemm_config("128x128", 2, "ring")
    assert tbg.gemm_configured_status(**{**g, "lda": 63}, config=cfg) == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_configured_status(**{**g, "M": 0}, config=cfg) == tbg.OK
    if not torch.cuda.is_available():
        for pipe, tile, st in BUILT_CONFIGS + [("auto", None, 0), ("producer", None, 0), ("ring", None, 4)]:
            s = tbg.gemm_configured_status(**g, config=tbg.gemm_config(tile, st, pipe))
            if pipe == "ring" and tile is None and st == 4:
                # the tile chosen for 64×64 is 64×64, built with 4 stages
                assert s == tbg.ERR_NO_DEVICE, tbg.last_error()
                continue
            assert s == tbg.ERR_NO_DEVICE, (pipe, tile, st, tbg.last_error())


def test_header_lists_the_built_configurations():
    """The configurations tbg.h documents are the ones the library accepts (and no more)."""
    import re
    text = open(tbg.HEADER_PATH).read()
    block = text[text.index("Built configurations"):text.index("typedef struct {\n    int32_t tile_m")]
    ring = block[block.index("ring:"):block.index("producer:")]
    prod = block[block.index("producer:"):]

    def expand(line):
        out = set()
        for part in line.split(";"):
            m = re.search(r"((?:\d+x\d+(?: and )?)+)/(\d)(?:-(\d))?", part)
            if not m:
                continue
            tiles = re.findall(r"\d+x\d+", m.group(1))
            lo, hi = int(m.group(2)), int(m.group(3) or m.group(2))
            out |= {(t, s) for t in tiles for s in range(lo, hi + 1)}
        return out

    assert expand(ring) == {(t, s) for p, t, s in BUILT_CONFIGS if p == "ring"}
    assert expand(prod) == {(t, s) for p, t, s in BUILT_CONFIGS if p == "producer"}


def _im2col_args(**over):
    a = dict(dtype="bf16", global_address=BASE, global_dim=[64, 56, 56, 32], global_strides=[128, 128 * 56, 128 * 56 * 56],
             pad_lo=[1, 1], pad_hi=[1, 1], conv_stride=[1, 1], dilation=[1, 1], filter=[3, 3], channels=64,
             pixels=128, swizzle="128B", l2="none", oob="zero")
    a.update(over)
    return a


def test_im2col_descriptor():
    """tbg_encode_im2col ("2 · Le Tensor Memory Accelerator", section "im2col"): image size and the
    checks the tiled encoder makes, plus the convolution geometry."""
    d = tbg.encode_im2col(**_im2col_args())
    assert tbg.box_bytes(d) == 64 * 128 * 2
    d = tbg.encode_im2col(**_im2col_args(channels=3, pixels=5, swizzle="none", dtype="f32", oob="nan"))
    assert tbg.box_bytes(d) == 3 * 5 * 4
    bad = [
        (dict(global_address=BASE + 8), tbg.ERR_MISALIGNED),
        (dict(global_strides=[128, 128 * 56 + 8, 128 * 56 * 56]), tbg.ERR_MISALIGNED),
        (dict(global_dim=[0, 56, 56, 32]), tbg.ERR_OUT_OF_RANGE),
        (dict(filter=[0, 3]), tbg.ERR_OUT_OF_RANGE),
        (dict(conv_stride=[1, 0]), tbg.ERR_OUT_OF_RANGE),
        (dict(dilation=[300, 1]), tbg.ERR_OUT_OF_RANGE),
        (dict(pad_lo=[-1, 0]), tbg.ERR_OUT_OF_RANGE),
        (dict(filter=[59, 3]), tbg.ERR_INVALID_VALUE),          # the window does not fit 56 + 2
        (dict(channels=0), tbg.ERR_OUT_OF_RANGE),
        (dict(pixels=257), tbg.ERR_OUT_OF_RANGE),
        (dict(channels=128, pixels=256, swizzle="none", dtype="f32"), tbg.ERR_OUT_OF_RANGE),  # 128 KiB image
        (dict(channels=128), tbg.ERR_INVALID_VALUE),            # 256-byte rows under a 128B swizzle
        (dict(oob="nan", dtype="u16"), tbg.ERR_INVALID_VALUE),
        (dict(swizzle=9), tbg.ERR_INVALID_VALUE),
        (dict(global_address=0), tbg.ERR_INVALID_VALUE),
    ]
    for over, status in bad:
        assert tbg.encode_im2col_status(**_im2col_args(**over)) == status, (over, tbg.last_error())
    # a descriptor of the other kind is refused by each copy call
    dt = tbg.encode_tiled(**_c1_args())
    with pytest.raises(tbg.Error) as e:
        tbg.im2col_copy(dt, [0, 0, 0, 0], BASE)
    assert e.value.status == tbg.ERR_INVALID_VALUE
    with pytest.raises(tbg.Error) as e:
        tbg.tiled_copy(d, [0, 0], BASE)
    assert e.value.status == tbg.ERR_INVALID_VALUE
    with pytest.raises(tbg.Error) as e:
        tbg.im2col_copy(d, [0, 0, 0, 0], BASE + 4)
    assert e.value.status == tbg.ERR_MISALIGNED
    tbg.im2col_copy_many(d, 0, 0, 0)


def test_conv2d_shapes_and_errors(orc):
    """Output extents agree with the oracle's; workspace only when c is not a multiple of 8;
    malformed shapes are INVALID_VALUE and limits UNSUPPORTED, before any device check."""
    import torch
    rng = np.random.default_rng(3)
    for _ in range(50):
        h, w = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        r, s = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        pad = tuple(int(x) for x in rng.integers(0, 4, 4))
        st, dl = tuple(int(x) for x in rng.integers(1, 4, 2)), tuple(int(x) for x in rng.integers(1, 3, 2))
        shp = tbg.conv2d_shape(2, h, w, 8, 4, r, s, pad, st, dl)
        oh = orc.conv_out_dim(h, pad[0], pad[2], st[0], dl[0], r)
        ow = orc.conv_out_dim(w, pad[1], pad[3], st[1], dl[1], s)
        if oh < 1 or ow < 1:
            with pytest.raises(tbg.Error) as e:
                tbg.conv2d_out_dims(shp)
            assert e.value.status == tbg.ERR_INVALID_VALUE
        else:
            assert tbg.conv2d_out_dims(shp) == (oh, ow)
    assert tbg.conv2d_workspace_bytes(tbg.conv2d_shape(2, 9, 9, 64, 4, 3, 3)) == 0
    c8 = 8
    want = ((2 * 9 * 9 * c8 * 2 + 255) // 256 * 256) + ((4 * 3 * 3 * c8 * 2 + 255) // 256 * 256)
    assert tbg.conv2d_workspace_bytes(tbg.conv2d_shape(2, 9, 9, 3, 4, 3, 3)) == want
    good = tbg.conv2d_shape(2, 9, 9, 16, 4, 3, 3, (1, 1, 1, 1))
    args = dict(alpha=1.0, x=BASE, w=BASE, beta=0.0, y=BASE, ldy=4, y_dtype="f32")
    assert tbg.conv2d_fwd_status(tbg.conv2d_shape(0, 9, 9, 16, 4, 3, 3), **args) == tbg.ERR_INVALID_VALUE
    assert tbg.conv2d_fwd_status(tbg.conv2d_shape(2, 9, 9, 16, 4, 3, 3, stride=(0, 1)), **args) == tbg.ERR_INVALID_VALUE
    assert tbg.conv2d_fwd_status(tbg.conv2d_shape(2, 9, 9, 16, 4, 3, 3, pad=(-1, 0, 0, 0)), **args) == tbg.ERR_INVALID_VALUE
    assert tbg.conv2d_fwd_status(tbg.conv2d_shape(2, 2, 9, 16, 4, 3, 3), **args) == tbg.ERR_INVALID_VALUE
    assert tbg.conv2d_fwd_status(tbg.conv2d_shape(2, 70000, 9, 16, 4, 3, 3), **args) == tbg.ERR_UNSUPPORTED
    assert tbg.conv2d_fwd_status(tbg.conv2d_shape(2, 9, 9, 16, 4, 300, 3), **args) == tbg.ERR_UNSUPPORTED
    assert tbg.conv2d_fwd_status(good, **{**args, "ldy": 3}) == tbg.ERR_INVALID_VALUE
    assert tbg.conv2d_fwd_status(good, **{**args, "y_dtype": "u8"}) == tbg.ERR_INVALID_VALUE
    assert tbg.conv2d_fwd_status(good, **{**args, "y": 0}) == tbg.ERR_INVALID_VALUE
    assert tbg.conv2d_fwd_status(good, **{**args, "x": 0}) == tbg.ERR_INVALID_VALUE
    # c % 8 != 0 needs the repack workspace
    assert tbg.conv2d_fwd_status(tbg.conv2d_shape(2, 9, 9, 3, 4, 3, 3), **args) == tbg.ERR_OUT_OF_RANGE
    if not torch.cuda.is_available():
        assert tbg.conv2d_fwd_status(good, **args) == tbg.ERR_NO_DEVICE
        # alpha == 0 needs neither operand
        assert tbg.conv2d_fwd_status(good, **{**args, "alpha": 0.0, "beta": 1.0, "x": 0, "w": 0}) == tbg.ERR_NO_DEVICE


def test_conv2d_config_checks():
    import torch
    good = tbg.conv2d_shape(2, 9, 9, 16, 4, 3, 3, (1, 1, 1, 1))
    args = dict(alpha=1.0, x=BASE, w=BASE, beta=0.0, y=BASE, ldy=4, y_dtype="f32")
    assert tbg.conv2d_fwd_status(good, **args, config=tbg.gemm_config("128x256")) == tbg.ERR_UNSUPPORTED
    assert tbg.conv2d_fwd_status(good, **args, config=tbg.gemm_config("128x128", 3)) == tbg.ERR_UNSUPPORTED
    assert tbg.conv2d_fwd_status(good, **args, config=tbg.gemm_config("128x128", 0, "producer")) == tbg.ERR_UNSUPPORTED
    assert tbg.conv2d_fwd_status(good, **args, config=tbg.GemmConfig(64, 0, 0, 0)) == tbg.ERR_INVALID_VALUE
    if not torch.cuda.is_available():
        for t in ("256x256", "256x128", "128x128", "64x64", None):
            assert tbg.conv2d_fwd_status(good, **args, config=tbg.gemm_config(t, 2, "ring")) == tbg.ERR_NO_DEVICE


def test_gemm_typed_checks():
    import torch
    g = dict(M=64, N=64, K=64, alpha=1.0, A=BASE, lda=64, B=BASE, ldb=64, b_layout="kn", beta=0.0, C=BASE, ldc=64,
             c_dtype="f32")
    assert tbg.gemm_typed_status(**g, ab_dtype="f32") == tbg.ERR_INVALID_VALUE
    assert tbg.gemm_typed_status(**g, ab_dtype="u16") == tbg.ERR_INVALID_VALUE
    # fp16 exists for the automatic choice's configurations only
    assert tbg.gemm_typed_status(**g, ab_dtype="f16", config=tbg.gemm_config("128x128", 4, "ring")) == tbg.ERR_UNSUPPORTED
    assert tbg.gemm_typed_status(**g, ab_dtype="f16", config=tbg.gemm_config("64x64", 2, "producer")) == tbg.ERR_UNSUPPORTED
    assert "fp16" in tbg.last_error()
    if not torch.cuda.is_available():
        for ab in ("bf16", "f16"):
            assert tbg.gemm_typed_status(**g, ab_dtype=ab) == tbg.ERR_NO_DEVICE
        assert tbg.gemm_typed_status(**g, ab_dtype="f16", config=tbg.gemm_config("64x64", 3, "producer")) == \
            tbg.ERR_NO_DEVICE


def test_interleaved_descriptor_rules():
    """The interleave rules of "H100 · cuTensorMap" §12.3-§12.4 (rank >= 3, base and strides
    aligned to the slice, 32B slices with the 32B swizzle), plus this library's reading that
    dimension 0 is one channel slice taken whole."""
    # NC/8HW8 bf16: a slice is 8 channels = 16 bytes; dims {8, W, H, C/8, N}
    dims16 = [8, 20, 12, 3, 2]
    st16 = [16, 16 * 20, 16 * 20 * 12, 16 * 20 * 12 * 3]
    d = tbg.encode_tiled_interleaved("bf16", 5, BASE, dims16, st16, [8, 16, 4, 3, 1], [1, 1, 1, 1, 1], "16B")
    assert tbg.box_bytes(d) == 16 * 16 * 4 * 3
    # NC/16HW16 bf16: 32-byte slices, with the 32B swizzle
    dims32 = [16, 20, 12, 2, 2]
    st32 = [32, 32 * 20, 32 * 20 * 12, 32 * 20 * 12 * 2]
    d = tbg.encode_tiled_interleaved("bf16", 5, BASE, dims32, st32, [16, 16, 4, 2, 1], [1] * 5, "32B", swizzle="32B")
    assert tbg.box_bytes(d) == 32 * 16 * 4 * 2
    bad = [
        (dict(rank=2, global_dim=[8, 20], global_strides=[16], box_dim=[8, 16], element_strides=[1, 1]),
         tbg.ERR_UNSUPPORTED),
        (dict(global_dim=[4] + dims16[1:]), tbg.ERR_INVALID_VALUE),                       # 8-byte "slice"
        (dict(box_dim=[4, 16, 4, 3, 1]), tbg.ERR_INVALID_VALUE),                          # box splits a slice
        (dict(element_strides=[2, 1, 1, 1, 1]), tbg.ERR_INVALID_VALUE),
        (dict(interleave="32B", global_dim=dims32, global_strides=st32, box_dim=[16, 16, 4, 2, 1]),
         tbg.ERR_INVALID_VALUE),                                                          # 32B needs the 32B swizzle
        (dict(interleave="32B", global_dim=dims32, global_strides=st32, box_dim=[16, 16, 4, 2, 1], swizzle="32B",
              global_address=BASE + 16), tbg.ERR_MISALIGNED),
        (dict(interleave="32B", global_dim=dims32, global_strides=[32, 32 * 20, 32 * 20 * 12 + 16, 99 * 32],
              box_dim=[16, 16, 4, 2, 1], swizzle="32B"), tbg.ERR_MISALIGNED),
        (dict(interleave=7), tbg.ERR_INVALID_VALUE),
    ]
    base = dict(dtype="bf16", rank=5, global_address=BASE, global_dim=dims16, global_strides=st16,
                box_dim=[8, 16, 4, 3, 1], element_strides=[1] * 5, interleave="16B")
    for over, status in bad:
        assert tbg.encode_tiled_interleaved_status(**{**base, **over}) == status, (over, tbg.last_error())
    # no interleave: the plain encoder's rules
    assert tbg.encode_tiled_interleaved_status(**{**base, "interleave": "none", "rank": 2, "global_dim": [64, 8],
                                                  "global_strides": [128], "box_dim": [64, 8],
                                                  "element_strides": [1, 1]}) == tbg.OK


def test_gemm_fp8_checks():
    import torch
    g = dict(M=64, N=64, K=128, alpha=1.0, A=BASE, lda=128, B=BASE, ldb=128, b_layout="nk", beta=0.0, C=BASE, ldc=64,
             c_dtype="f32")
    for ab in ("f8e4m3", "f8e5m2"):
        assert tbg.gemm_typed_status(**{**g, "b_layout": "kn"}, ab_dtype=ab) == tbg.ERR_UNSUPPORTED
        assert tbg.gemm_typed_status(**g, ab_dtype=ab, config=tbg.gemm_config("256x128", 2, "ring")) == tbg.ERR_UNSUPPORTED
        assert tbg.gemm_typed_status(**g, ab_dtype=ab, config=tbg.gemm_config("128x128", 2, "producer")) == \
            tbg.ERR_UNSUPPORTED
        assert tbg.gemm_typed_status(**g, ab_dtype=ab, config=tbg.gemm_config("128x128", 3, "ring")) == tbg.ERR_UNSUPPORTED
        assert tbg.gemm_typed_status(**{**g, "lda": 100}, ab_dtype=ab) == tbg.ERR_INVALID_VALUE
        # K = 100 is not a whole number of 16-byte chunks: the operands need the repack workspace
        assert tbg.gemm_typed_status(**{**g, "K": 100}, ab_dtype=ab) == tbg.ERR_OUT_OF_RANGE
        if not torch.cuda.is_available():
            assert tbg.gemm_typed_status(**g, ab_dtype=ab) == tbg.ERR_NO_DEVICE
            for t in ("256x256", "128x128", "64x64"):
                assert tbg.gemm_typed_status(**g, ab_dtype=ab, config=tbg.gemm_config(t, 2, "ring")) == tbg.ERR_NO_DEVICE
    # the 8-bit types as copy element types, NaN fill included
    d = tbg.encode_tiled("f8e4m3", 2, BASE, [256, 64], [256], [128, 8], [1, 1], "128B", "none", "nan")
    assert tbg.box_bytes(d) == 128 * 8


def test_benchmark_ceiling_library():
    """The benchmark's products-alone measurement lives in its own library, outside include/tbg.h;
    it exports one C function and rejects empty launches without touching a device."""
    import os
    path = os.path.join(os.path.dirname(tbg.library_path()), "diag", "libtbg_diag.so")
    lib = ctypes.CDLL(path)
    lib.tbg_diag_mfma_rate.restype = ctypes.c_int
    lib.tbg_diag_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
    assert lib.tbg_diag_mfma_rate(0, None, None, 0, 1, None, None) != 0
    assert lib.tbg_diag_mfma_rate(0, BASE, BASE, 4, 0, BASE, None) != 0
    assert lib.tbg_diag_mfma_rate(2, BASE, BASE, 4, 1, BASE, None) != 0
    main = subprocess.run(["nm", "-D", "--defined-only", tbg.library_path()], capture_output=True, text=True,
                          check=True).stdout
    assert "tbg_diag_mfma_rate" not in main, "the measurement aid must stay out of the library's ABI"


def test_transposing_read_swizzle_encodes():
    """TBG_SWIZZLE_128B_TR is a 128-byte-row mode: the GEMM's {64 n, 64 k} K×N bf16 box encodes with
    it; a wider inner extent or an image that is not whole 128-byte rows is refused."""
    d = tbg.encode_tiled("bf16", 2, BASE, [8192, 8192], [16384], [64, 64], [1, 1], "128B_TR")
    assert tbg.box_bytes(d) == 8192
    assert tbg.encode_tiled_status(**_c1_args(swizzle="128B_TR")) == tbg.OK
    assert tbg.encode_tiled_status(**_c1_args(swizzle="128B_TR", box_dim=[72, 128])) == tbg.ERR_INVALID_VALUE
    assert tbg.encode_tiled_status(**_c1_args(swizzle="128B_TR", box_dim=[8, 3])) == tbg.ERR_INVALID_VALUE
    assert tbg.encode_tiled_status(**_c1_args(swizzle=6)) == tbg.ERR_INVALID_VALUE


def _gemm_detail(**kw):
    """Status and the OUT_OF_RANGE detail's byte count of a tbg_gemm_typed call that stops at the
    workspace check (no device is reached)."""
    import re
    try:
        tbg.gemm_typed(**kw)
        return tbg.OK, None
    except tbg.Error as e:
        m = re.search(r"workspace of (\d+) bytes needed", e.message)
        return e.status, int(m.group(1)) if m else None


@pytest.mark.parametrize("ab", ["bf16", "f16", "f8e4m3", "f8e5m2"])
def test_workspace_query_matches_the_call(ab):
    """tbg_gemm_workspace_query gives exactly the bytes the product asks for in its OUT_OF_RANGE
    detail, for every repack case: misaligned bases, ragged leading dimensions, ragged K, both B
    layouts (8-bit types: B stored N×K only), and 0 when nothing is repacked."""
    layouts = ("kn", "nk") if ab in ("bf16", "f16") else ("nk",)
    cases = []
    for bl in layouts:
        for (M, N, K, lda, ldb) in [(300, 257, 136, 136, 264 if bl == "kn" else 136), (300, 257, 136, 137, 259),
                                    (300, 257, 100, 100, 257 if bl == "kn" else 100), (3001, 2049, 777, 777, 2049),
                                    (64, 64, 128, 128, 128)]:
            for a_off, b_off in ((0, 0), (2, 0), (0, 6), (8, 8)):
                if bl == "kn" and ldb < N:
                    continue
                cases.append((bl, M, N, K, lda, ldb, a_off, b_off))
    for bl, M, N, K, lda, ldb, a_off, b_off in cases:
        A, B = BASE + 0x100000 + a_off, BASE + 0x200000 + b_off
        q = tbg.gemm_workspace_query(M, N, K, ab, A, lda, B, ldb, bl)
        st, need = _gemm_detail(M=M, N=N, K=K, alpha=1.0, A=A, lda=lda, B=B, ldb=ldb, b_layout=bl, ab_dtype=ab,
                                beta=0.0, C=BASE, ldc=N, c_dtype="f32")
        what = f"{ab} {bl} M={M} N={N} K={K} lda={lda} ldb={ldb} offsets {a_off},{b_off}"
        if q == 0:
            assert st != tbg.ERR_OUT_OF_RANGE, what
        else:
            assert st == tbg.ERR_OUT_OF_RANGE and need == q, (what, q, need)
            # with exactly that much workspace the call gets past the check
            st2, _ = _gemm_detail(M=M, N=N, K=K, alpha=1.0, A=A, lda=lda, B=B, ldb=ldb, b_layout=bl, ab_dtype=ab,
                                  beta=0.0, C=BASE, ldc=N, c_dtype="f32", workspace=BASE + 0x4000000,
                                  workspace_bytes=q)
            assert st2 != tbg.ERR_OUT_OF_RANGE, what
    # aligned bf16 operands: the query agrees with the older size-only function
    assert tbg.gemm_workspace_query(3001, 2049, 777, "bf16", BASE, 777, BASE, 2049, "kn") == \
        tbg.gemm_workspace_bytes(3001, 2049, 777, 777, 2049, "kn")
    assert tbg.gemm_workspace_query(0, 64, 64, ab, BASE, 64, BASE, 64, "nk") == 0


def test_conv_workspace_query():
    shp = tbg.conv2d_shape(2, 17, 17, 24, 36, 3, 3, (1, 1, 1, 1))
    assert tbg.conv2d_workspace_query(shp, BASE, BASE) == tbg.conv2d_workspace_bytes(shp) == 0
    c8 = 24
    want = (2 * 17 * 17 * c8 * 2 + 255) // 256 * 256 + (36 * 3 * 3 * c8 * 2 + 255) // 256 * 256
    assert tbg.conv2d_workspace_query(shp, BASE + 2, BASE) == want
    assert tbg.conv2d_workspace_query(shp, BASE, BASE + 8) == want
    shp = tbg.conv2d_shape(2, 15, 13, 20, 40, 3, 3, (1, 1, 1, 1))
    assert tbg.conv2d_workspace_query(shp, BASE, BASE) == tbg.conv2d_workspace_bytes(shp) > 0


class _FakeDeviceTensor:
    """Stands in for a device tensor in the binding's host-side checks: every check it trips must
    raise before anything reaches the C ABI (no device is used)."""

    def __init__(self, shape, dtype, device="cuda:0", stride=None, ptr=BASE):
        import torch
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._stride = stride or tuple(int(np.prod(shape[i + 1:])) for i in range(len(shape)))
        self._ptr = ptr

    def dim(self):
        return len(self.shape)

    def stride(self, i=None):
        return self._stride if i is None else self._stride[i]

    def data_ptr(self):
        return self._ptr

    def numel(self):
        return int(np.prod(self.shape))

    def element_size(self):
        import torch
        return torch.empty(0, dtype=self.dtype).element_size()

    def is_contiguous(self):
        return True


def test_torch_ops_rejects_mismatched_outputs():
    """torch_ops.gemm refuses an `out` whose shape, element type or device does not match what the
    kernel writes (M rows of N elements of out_dtype), operands on different devices and a
    workspace on another device, before calling the library."""
    import torch
    from tiled_bf16_gemm_amd import torch_ops
    A = _FakeDeviceTensor((64, 32), torch.bfloat16)
    B = _FakeDeviceTensor((32, 48), torch.bfloat16)
    good = dict(out_dtype="bf16")
    for out, why in [(_FakeDeviceTensor((32, 48), torch.bfloat16), "too few rows"),
                     (_FakeDeviceTensor((64, 40), torch.bfloat16), "too few columns"),
                     (_FakeDeviceTensor((64, 48), torch.float32), "fp32 out for bf16"),
                     (_FakeDeviceTensor((64, 48), torch.bfloat16, device="cuda:1"), "another device"),
                     (_FakeDeviceTensor((64, 48), torch.bfloat16, stride=(48, 2)), "strided columns")]:
        with pytest.raises(ValueError):
            torch_ops.gemm(A, B, "kn", out=out, **good)
        print("refused:", why)
    with pytest.raises(ValueError):
        torch_ops.gemm(A, B, "kn", out=_FakeDeviceTensor((64, 48), torch.bfloat16), out_dtype="f32")
    with pytest.raises(ValueError):
        torch_ops.gemm(A, B, "kn", out_dtype="u8")
    with pytest.raises(ValueError):
        torch_ops.gemm(A, _FakeDeviceTensor((32, 48), torch.bfloat16, device="cuda:1"), "kn")
    with pytest.raises(ValueError):
        torch_ops.gemm(A, B, "kn", out=_FakeDeviceTensor((64, 48), torch.bfloat16),
                       workspace=_FakeDeviceTensor((4096,), torch.uint8, device="cuda:1"))
    with pytest.raises(ValueError):
        torch_ops.gemm(A, _FakeDeviceTensor((33, 48), torch.bfloat16), "kn")
