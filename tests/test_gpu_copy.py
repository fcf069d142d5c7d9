"""Tiled copies on the GPU against the oracle, byte for byte ("2 · Le Tensor Memory Accelerator"
§2.2–§2.5; "H100 · cuTensorMap" §8, §9, §11, §14).

Destinations are pre-filled with a 0xA5 sentinel with guard bytes past the last image, so a
missed or stray write shows up.  Cases cover both device paths: the direct-to-LDS atom loader
(2-D boxes of 128-byte rows, 128B and 2-row swizzles, zero fill; the GEMM's own loader) and the
register-staged path (any rank, element strides, NaN fill, every swizzle, ragged and negative
coordinates)."""
import sys

import numpy as np
import pytest
import torch

import workloads

gpu = pytest.mark.gpu
SENTINEL = 0xA5
GUARD = 4096


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tiled_bf16_gemm_amd import torch_ops
    return torch_ops


def _device_copy(ops, src_cpu: torch.Tensor, dtype, dims, strides, box, estr, swizzle, oob, coords_list, many):
    import tiled_bf16_gemm_amd as tbg
    src = src_cpu.cuda()
    desc = ops.encode(src, dtype, dims, strides, box, estr, swizzle, oob)
    nbytes = tbg.box_bytes(desc)
    n = len(coords_list)
    out = torch.full((n * nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
    if many:
        coords = torch.tensor(coords_list, dtype=torch.int32, device="cuda").contiguous()
        ops.tiled_copy_many(desc, coords, out=out)
        torch.cuda.synchronize()
        host = out.cpu().numpy()
        assert np.all(host[n * nbytes:] == SENTINEL), "write past the last image"
        return host[:n * nbytes].reshape(n, nbytes)
    images = []
    for c in coords_list:
        # one 16-byte-aligned destination per box, with its own guard
        buf = torch.full((nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        ops.tiled_copy(desc, c, out=buf[:nbytes])
        images.append(buf)
    torch.cuda.synchronize()
    rows = []
    for buf in images:
        host = buf.cpu().numpy()
        assert np.all(host[nbytes:] == SENTINEL), "write past the image"
        rows.append(host[:nbytes])
    return np.stack(rows)


def _src_bytes(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).numpy()


def _check_case(ops, orc, src_cpu, dtype, dims, strides, box, estr, swizzle, oob, coords_list, many=True):
    got = _device_copy(ops, src_cpu, dtype, dims, strides, box, estr, swizzle, oob, coords_list, many)
    srcb = _src_bytes(src_cpu)
    for i, c in enumerate(coords_list):
        want = orc.tiled_copy(srcb, dtype, dims, strides, box, estr, swizzle, oob == "nan", c)
        if not np.array_equal(got[i], want):
            bad = np.nonzero(got[i] != want)[0]
            raise AssertionError(f"image {i} coords {c}: {bad.size} bytes differ, first at {bad[:8]}")


@gpu
def test_c1_copy_worked_box(ops, orc):
    """The 128×64 bf16 box with 128B swizzle of the first workload, at its 11 coordinates."""
    w = workloads.COPIES["c1_copy"]
    src = workloads.copy_source(w)
    _say("c1 copy: DMA path, single and many")
    for many in (False, True):
        _check_case(ops, orc, src, "bf16", list(w.dims), [w.dims[0] * 2], list(w.box), list(w.estr), w.swizzle,
                    w.oob, [list(c) for c in w.coords], many=many)


@gpu
def test_c3_copy_5d_nan_fill(ops, orc):
    """432 boxes {64,16,4,2,2} with element strides {1,2,1,1,1} and NaN fill over the 5-D tensor,
    plus boxes with negative coordinates and the other reading of the element strides."""
    w = workloads.COPIES["c3_copy"]
    src = workloads.copy_source(w)
    d = list(w.dims)
    strides = [d[0] * 2, d[0] * d[1] * 2, d[0] * d[1] * d[2] * 2, d[0] * d[1] * d[2] * d[3] * 2]
    assert all(s % 16 == 0 for s in strides)
    _say("c3 copy: 432 boxes")
    coords = [list(c) for c in w.coords]
    assert len(coords) == 432
    _check_case(ops, orc, src, "bf16", d, strides, list(w.box), list(w.estr), w.swizzle, w.oob, coords)
    _say("c3 copy: negative and overhanging coordinates")
    extra = [[-8, -3, 0, 0, 0], [-64, 0, 0, 0, 0], [150, 120, 5, 4, 2], [192, 128, 6, 4, 2], [-100, -40, -9, -9, -9],
             [0, 0, 0, 0, 3], [16, 8, 3, 3, 1]]
    _check_case(ops, orc, src, "bf16", d, strides, list(w.box), list(w.estr), w.swizzle, w.oob, extra)
    _say("c3 copy: element stride 2 on the size-5 dimension")
    _check_case(ops, orc, src, "bf16", d, strides, list(w.box), [1, 1, 1, 2, 1], w.swizzle, w.oob,
                coords[:48] + extra)


@gpu
def test_c4_a_boxes_full_size(ops, orc):
    """All 8192 boxes of 64 columns x 128 rows (128B swizzle) of the 8192x8192 GEMM operand A, the
    launch the bench times.  Sampled boxes against the oracle byte for byte; at full size, undoing
    the 128-byte swizzle ("2 · Le Tensor Memory Accelerator" §2.4: the 16-byte unit index XORed
    with the row index within 8 rows of 128 bytes) on every image and putting the boxes back in
    their places gives A again, bit for bit."""
    w = workloads.COPIES["c4_a_boxes"]
    src = workloads.copy_source(w)
    rows, cols = w.shape_outer_first
    coords = [list(c) for c in w.coords]
    assert len(coords) == 8192
    _say("c4 A boxes: 8192 boxes, one launch")
    got = _device_copy(ops, src, "bf16", list(w.dims), [cols * 2], list(w.box), list(w.estr), w.swizzle, w.oob,
                       coords, True)
    srcb = _src_bytes(src)
    rng = np.random.default_rng(4)
    picks = sorted(set([0, 127, 8064, 8191] + rng.integers(0, 8192, 20).tolist()))
    for i in picks:
        want = orc.tiled_copy(srcb, "bf16", list(w.dims), [cols * 2], list(w.box), list(w.estr), w.swizzle, False,
                              coords[i])
        assert np.array_equal(got[i], want), f"box {i} at {coords[i]} differs from the oracle"
    _say("c4 A boxes: reassembling A from the unswizzled images")
    unit = np.arange(1024)                    # 16-byte units of a 16 KiB image
    logical = unit ^ ((unit >> 3) & 7)        # unit u of the image holds logical unit u ^ row8(u)
    imgs = got.reshape(8192, 1024, 16)
    plain = np.empty_like(imgs)
    plain[:, logical, :] = imgs[:, unit, :]
    # box (bx, by) -> A[128 by : 128 by + 128, 64 bx : 64 bx + 64]; 128 boxes per box row
    a = plain.reshape(rows // 128, cols // 64, 128, 128).transpose(0, 2, 1, 3).reshape(rows, cols * 2)
    assert np.array_equal(a, srcb.reshape(rows, cols * 2)), "images do not reassemble A"


@gpu
def test_dma_path_edges(ops, orc):
    """2-D boxes of 128-byte rows through the direct-to-LDS loader: ragged rows and columns,
    both swizzles, pitches wider than the rows, every chunk-aligned origin class."""
    rng = np.random.default_rng(21)
    for (rows, cols, pitch, brows, swz) in [(100, 72, 80, 64, "128B"), (256, 256, 256, 128, "128B_2ROW"),
                                            (37, 200, 256, 16, "128B"), (513, 64, 64, 256, "128B_2ROW"),
                                            (8, 8, 8, 8, "128B")]:
        src = torch.from_numpy(rng.integers(0, 1 << 16, (rows, pitch), dtype=np.int64).astype(np.int16)
                               ).view(torch.bfloat16)
        coords = [[x, y] for x in range(0, cols + 8, 8 * max(1, cols // 64)) for y in (0, 1, rows // 2, rows - 1)]
        coords += [[-8, 0], [0, -1], [cols, 0], [0, rows], [cols - 8, rows - 8]]
        _say(f"dma edges rows={rows} cols={cols} pitch={pitch} box=64x{brows} {swz}")
        _check_case(ops, orc, src, "bf16", [cols, rows], [pitch * 2], [64, brows], [1, 1], swz, "zero", coords)


@gpu
def test_transposing_read_layout(ops, orc):
    """The 128B_TR swizzle (the GEMM's layout of B tiles stored K×N) byte for byte against the
    oracle: {64, rows} bf16 boxes of K×N operands through the direct-to-LDS atom loader the GEMM
    uses (ragged rows and columns, negative and overhanging origins, pitches wider than the rows),
    the register-staged path (NaN fill, element strides, 8-bit and 32-bit elements, rank 3), and
    the store direction."""
    rng = np.random.default_rng(55)
    for (rows, cols, pitch, brows) in [(200, 136, 136, 64), (64, 64, 64, 64), (1000, 520, 528, 64),
                                       (37, 72, 80, 16), (513, 64, 64, 256)]:
        src = torch.from_numpy(rng.integers(0, 1 << 16, (rows, pitch), dtype=np.int64).astype(np.int16)
                               ).view(torch.bfloat16)
        coords = [[x, y] for x in range(0, cols + 8, 8 * max(1, cols // 64)) for y in (0, 1, rows // 2, rows - 1)]
        coords += [[-8, 0], [0, -1], [cols, 0], [0, rows], [cols - 8, rows - 8], [64, 64]]
        _say(f"128B_TR atom path rows={rows} cols={cols} pitch={pitch} box=64x{brows}")
        _check_case(ops, orc, src, "bf16", [cols, rows], [pitch * 2], [64, brows], [1, 1], "128B_TR", "zero", coords)
        _check_case(ops, orc, src, "bf16", [cols, rows], [pitch * 2], [64, brows], [1, 1], "128B_TR", "zero",
                    coords[:4], many=False)
    src = torch.from_numpy(rng.standard_normal((96, 72)).astype(np.float32)).to(torch.bfloat16)
    _say("128B_TR register-staged: NaN fill, element strides")
    _check_case(ops, orc, src, "bf16", [72, 96], [144], [64, 32], [1, 1], "128B_TR", "nan",
                [[0, 0], [16, 80], [-8, -3], [64, 90]])
    _check_case(ops, orc, src, "bf16", [72, 96], [144], [64, 48], [1, 3], "128B_TR", "zero", [[0, 0], [8, 50]])
    raw = rng.integers(0, 256, 40 * 12 * 144, dtype=np.int64).astype(np.uint8)
    _check_case(ops, orc, torch.from_numpy(raw), "u8", [144, 12, 40], [144, 144 * 12], [128, 4, 8], [1, 2, 1],
                "128B_TR", "zero", [[0, 0, 0], [16, 5, 33], [-16, -1, 2]])
    raw32 = rng.integers(0, 1 << 32, 50 * 40, dtype=np.uint64).astype(np.uint32)
    _check_case(ops, orc, torch.from_numpy(raw32.view(np.int32)), "f32", [40, 50], [160], [32, 40], [1, 1],
                "128B_TR", "nan", [[0, 0], [12, 20], [-4, 30]])
    _say("128B_TR store direction")
    _store_case(ops, orc, "bf16", [72, 96], [144], [64, 32], [1, 1], "128B_TR", [[0, 0], [16, 80], [-8, -3]],
                False, 77)


@gpu
def test_random_descriptors(ops, orc):
    """Seeded random descriptors: rank 1..5, every element type, element strides, both fills,
    every swizzle the box allows."""
    rng = np.random.default_rng(1234)
    types = ["u8", "u16", "u32", "f16", "bf16", "f32"]
    npt = {"u8": np.uint8, "u16": np.uint16, "u32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "f32": np.uint32}
    tt = {"u8": torch.uint8, "u16": torch.int16, "u32": torch.int32, "f16": torch.int16, "bf16": torch.int16,
          "f32": torch.int32}
    done = 0
    while done < 60:
        dtype = types[int(rng.integers(0, len(types)))]
        es = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4}[dtype]
        rank = int(rng.integers(1, 6))
        dims = [int(rng.integers(1, 40)) for _ in range(rank)]
        # row pitch: a multiple of 16 bytes at least as long as a row
        pitch0 = ((dims[0] * es + 15) // 16) * 16 + 16 * int(rng.integers(0, 2))
        strides = []
        if rank > 1:
            strides.append(pitch0)
            for i in range(2, rank):
                strides.append(strides[-1] * dims[i - 1])
        total_bytes = (strides[-1] * dims[-1]) if rank > 1 else dims[0] * es
        box = [int(rng.integers(1, 17)) for _ in range(rank)]
        estr = [int(rng.integers(1, 9)) for _ in range(rank)]
        swizzle = "none"
        if rng.integers(0, 2):
            span = {"32B": 32, "64B": 64, "128B": 128, "128B_2ROW": 128}
            swizzle = ["32B", "64B", "128B", "128B_2ROW"][int(rng.integers(0, 4))]
            box[0] = max(1, span[swizzle] // es)
            estr[0] = 1
        n = [(b + e - 1) // e for b, e in zip(box, estr)]
        image = es * int(np.prod(n))
        if swizzle != "none":
            span = {"32B": 32, "64B": 64, "128B": 128, "128B_2ROW": 128}[swizzle]
            if image % span:
                continue
        if image > 65536:
            continue
        oob = "nan" if dtype in ("f16", "bf16", "f32") and rng.integers(0, 2) else "zero"
        raw = rng.integers(0, 1 << (8 * es), total_bytes // es, dtype=np.uint64).astype(npt[dtype])
        src = torch.from_numpy(raw.view(np.int8).copy()).view(tt[dtype])
        coords = [[int(rng.integers(-10, d + 5)) for d in dims] for _ in range(6)]
        _say(f"random copy {done}: {dtype} rank={rank} dims={dims} box={box} estr={estr} {swizzle} {oob}")
        _check_case(ops, orc, src, dtype, dims, strides, box, estr, swizzle, oob, coords, many=bool(done % 2))
        done += 1


@gpu
def test_copy_is_deterministic_and_leaves_source(ops):
    w = workloads.COPIES["c3_copy"]
    src = workloads.copy_source(w).cuda()
    before = src.clone()
    d = list(w.dims)
    strides = [d[0] * 2, d[0] * d[1] * 2, d[0] * d[1] * d[2] * 2, d[0] * d[1] * d[2] * d[3] * 2]
    desc = ops.encode(src, "bf16", d, strides, list(w.box), list(w.estr), "none", "nan")
    coords = torch.tensor([list(c) for c in w.coords], dtype=torch.int32, device="cuda")
    a = ops.tiled_copy_many(desc, coords)
    b = ops.tiled_copy_many(desc, coords)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(src.view(torch.int16), before.view(torch.int16))


# ---- store direction ("2 · Le Tensor Memory Accelerator" §2.5) -----------------------------------
def _store_case(ops, orc, dtype, dims, strides, box, estr, swizzle, coords_list, many, seed):
    """Store random images into a tensor of sentinel bytes on the GPU, one box after another (or
    all at once), and compare every byte of the tensor with the oracle's stores."""
    es = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4}[dtype]
    rank = len(dims)
    total_bytes = (strides[-1] * dims[-1]) if rank > 1 else dims[0] * es
    rng = np.random.default_rng(seed)
    d_tensor = torch.full((total_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    desc = ops.encode(d_tensor, dtype, dims, strides, box, estr, swizzle, "zero")
    nb = tbg_box_bytes(desc)
    images = rng.integers(0, 256, nb * len(coords_list), dtype=np.uint8)
    d_images = torch.from_numpy(images).cuda()
    if many:
        d_coords = torch.tensor(coords_list, dtype=torch.int32, device="cuda")
        ops.tiled_store_many(desc, d_coords, d_images)
    else:
        for b, c in enumerate(coords_list):
            ops.tiled_store(desc, c, d_images[b * nb:(b + 1) * nb].clone())  # own, 16-byte aligned buffer
    torch.cuda.synchronize()
    want = np.full(total_bytes, 0xA5, dtype=np.uint8)
    for b, c in enumerate(coords_list):
        want = orc.tiled_store(want, dtype, dims, strides, box, estr, swizzle, c, images[b * nb:(b + 1) * nb])
    got = d_tensor.cpu().numpy()
    bad = int((got != want).sum())
    assert bad == 0, f"{bad} tensor bytes differ"


def tbg_box_bytes(desc):
    import tiled_bf16_gemm_amd as tbg
    return tbg.box_bytes(desc)


@gpu
def test_store_c1_and_c3_boxes(ops, orc):
    _say("store: c1 box {64,128} bf16 128B swizzle, in bounds, overhanging and negative")
    for c in ([0, 0], [64, 128], [224, 192], [-32, -64]):
        _store_case(ops, orc, "bf16", [256, 256], [512], [64, 128], [1, 1], "128B", [c], False, 11)
    _say("store: c3 5-D boxes {64,16,4,2,2}, element strides {1,2,1,1,1}, 432 boxes in one call")
    coords = [[x, y, z, w, v] for v in (0, 2) for w in (0, 2, 4) for z in (0, 4) for y in range(0, 129, 16)
              for x in (0, 64, 128, 192)]
    assert len(coords) == 432
    _store_case(ops, orc, "bf16", [200, 129, 7, 5, 3], [400, 51600, 361200, 1806000], [64, 16, 4, 2, 2],
                [1, 2, 1, 1, 1], "none", coords, True, 12)


@gpu
def test_store_random_descriptors(ops, orc):
    """Seeded random descriptors for the store: rank 1..5, every element type, element strides,
    every swizzle the box allows, coordinates inside, overhanging and negative."""
    rng = np.random.default_rng(4321)
    types = ["u8", "u16", "u32", "f16", "bf16", "f32"]
    done = 0
    while done < 60:
        dtype = types[int(rng.integers(0, len(types)))]
        es = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4}[dtype]
        rank = int(rng.integers(1, 6))
        dims = [int(rng.integers(1, 40)) for _ in range(rank)]
        pitch0 = ((dims[0] * es + 15) // 16) * 16 + 16 * int(rng.integers(0, 2))
        strides = []
        if rank > 1:
            strides.append(pitch0)
            for i in range(2, rank):
                strides.append(strides[-1] * dims[i - 1])
        box = [int(rng.integers(1, 17)) for _ in range(rank)]
        estr = [int(rng.integers(1, 9)) for _ in range(rank)]
        swizzle = "none"
        span = {"32B": 32, "64B": 64, "128B": 128, "128B_2ROW": 128}
        if rng.integers(0, 2):
            swizzle = ["32B", "64B", "128B", "128B_2ROW"][int(rng.integers(0, 4))]
            box[0] = max(1, span[swizzle] // es)
            estr[0] = 1
        n = [(b + e - 1) // e for b, e in zip(box, estr)]
        image = es * int(np.prod(n))
        if (swizzle != "none" and image % span[swizzle]) or image > 65536:
            continue
        coords = [[int(rng.integers(-10, d + 5)) for d in dims] for _ in range(3)]
        many = bool(done % 2)
        if many:
            coords = coords[:1]  # one box per call: overlapping boxes are written in no set order
        _say(f"random store {done}: {dtype} rank={rank} dims={dims} box={box} estr={estr} {swizzle}")
        _store_case(ops, orc, dtype, dims, strides, box, estr, swizzle, coords, many, 100 + done)
        done += 1


@gpu
def test_interleaved_copies(ops, orc):
    """NC/xHWCx tensors ("H100 · cuTensorMap" §12): 16-byte slices (NC/8HW8 bf16) with and without
    a swizzle, 32-byte slices (NC/16HW16 bf16, NC/8HW8 f32) with the 32B swizzle, zero and NaN
    fill, boxes overhanging every edge; images byte for byte against the oracle."""
    import tiled_bf16_gemm_amd as tbg
    rng = np.random.default_rng(505)
    cases = [("bf16", 8, 16, "16B", "none", "zero"), ("bf16", 8, 16, "16B", "128B", "zero"),
             ("bf16", 16, 32, "32B", "32B", "nan"), ("f32", 8, 32, "32B", "32B", "zero")]
    for dtype, x, width, il, swz, oob in cases:
        N, CS, H, W = 2, 3, 9, 13
        es = width // x
        vals = torch.randn(N * CS * H * W * x)
        src = (vals.to(torch.bfloat16) if dtype == "bf16" else vals).contiguous()
        dims = [x, W, H, CS, N]
        strides = [width, width * W, width * W * H, width * W * H * CS]
        box = [x, 8, 4, 2, 1]
        d = src.cuda()
        desc = tbg.encode_tiled_interleaved(dtype, 5, d.data_ptr(), dims, strides, box, [1] * 5, il, swz, "none", oob)
        nbytes = tbg.box_bytes(desc)
        coords = [[0, int(rng.integers(-4, W)), int(rng.integers(-2, H)), int(rng.integers(-1, CS)),
                   int(rng.integers(0, N))] for _ in range(24)] + [[0, W - 3, H - 2, CS - 1, N - 1], [0, -7, -3, 0, 0]]
        _say(f"interleave {il} {dtype} swizzle {swz} {oob}: {len(coords)} boxes of {nbytes} bytes")
        out = torch.full((len(coords) * nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        ops.tiled_copy_many(desc, torch.tensor(coords, dtype=torch.int32, device="cuda"), out=out)
        torch.cuda.synchronize()
        host = out.cpu().numpy()
        assert np.all(host[len(coords) * nbytes:] == SENTINEL), "write past the last image"
        srcb = _src_bytes(src)
        for i, c in enumerate(coords):
            want = orc.tiled_copy(srcb, dtype, dims, strides, box, [1] * 5, swz, oob == "nan", c)
            assert np.array_equal(host[i * nbytes:(i + 1) * nbytes], want), (il, c)
