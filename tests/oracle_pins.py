"""Pins of the CPU oracle against what the pages and plain mathematics fix.

Each pin takes an ``oracle.Oracle`` handle and raises AssertionError when the oracle disagrees,
so ``test_oracle_pins.py`` can run them on the oracle as committed and on deliberately broken
builds of it (every broken build must fail at least one pin).  None of these checks retypes the
oracle's own formula: each goes through another route (per-bit statements, numpy slicing,
index decoding, exact rationals, integer matmul, closed forms).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pages_worked_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------------------
# Swizzle ("H100 · cuTensorMap" §11.2–§11.4)
# ---------------------------------------------------------------------------------------------
# The library's gfx950 extension modes, stated bit by bit (pairs [destination bit, source bit]):
# 128B_2ROW a[6:4] ^= a[10:8]; 128B_TR (the layout read back with the transposing 8-byte read)
# a[4] ^= a[9], a[5] ^= a[8], a[6] ^= a[10].
EXT_RULES = {"128B_2ROW": [[6, 10], [5, 9], [4, 8]], "128B_TR": [[4, 9], [5, 8], [6, 10]]}
# 128B_TR worked by hand from its row/unit statement (unit c of 128-byte row r moves to
# c ^ (4·r[3] + 2·r[1] + r[2])): e.g. 1973 is row 15, unit 3, byte 5 -> unit 3 ^ 7 = 4 -> 1989.
EXT_HAND_EXAMPLES = {"128B_TR": [(0, 0), (128, 128), (256, 288), (512, 528), (1024, 1088), (1973, 1989),
                                 (2304, 2336), (2047, 1935), (3072, 3136)]}


def _per_bit(a: np.ndarray, rules) -> np.ndarray:
    a = a.astype(np.uint64)
    out = a.copy()
    for dst, src in rules:
        bit = ((a >> np.uint64(dst)) ^ (a >> np.uint64(src))) & np.uint64(1)
        out = (out & ~np.uint64(1 << dst)) | (bit << np.uint64(dst))
    return out


def pin_swizzle_bit_rules(o):
    g = golden()["swizzle_bit_rules"]
    a = np.arange(1 << 14, dtype=np.uint64)
    big = np.array([(1 << 40) + 12345, (1 << 33) - 1, 0xFFFF_FFF0], dtype=np.uint64)
    a = np.concatenate([a, big])
    assert np.array_equal(o.swizzle(a, "none"), a)
    for mode in ("32B", "64B", "128B"):
        assert np.array_equal(o.swizzle(a, mode), _per_bit(a, g[mode])), mode
    for mode, rules in EXT_RULES.items():
        assert np.array_equal(o.swizzle(a, mode), _per_bit(a, rules)), mode
    # 128B_TR as the GEMM's K×N layout states it: row r = a >> 7 keeps its place, its 16-byte
    # unit c = a[6:4] moves to c ^ (4·r[3] + 2·r[1] + r[2])
    r, c, b = a >> np.uint64(7), (a >> np.uint64(4)) & np.uint64(7), a & np.uint64(15)
    x = (((r >> np.uint64(3)) & np.uint64(1)) << np.uint64(2)) | (((r >> np.uint64(1)) & np.uint64(1)) << np.uint64(1)) \
        | ((r >> np.uint64(2)) & np.uint64(1))
    assert np.array_equal(o.swizzle(a, "128B_TR"), (r << np.uint64(7)) | ((c ^ x) << np.uint64(4)) | b)
    # a[3:0] never changes (§11.3)
    for mode in ("32B", "64B", "128B", "128B_2ROW", "128B_TR"):
        s = o.swizzle(a, mode)
        assert np.array_equal(s & np.uint64(15), a & np.uint64(15))


def pin_swizzle_hand_examples(o):
    ex = golden()["swizzle_hand_examples"]
    for mode in ("32B", "64B", "128B"):
        for a, want in ex[mode]:
            assert int(o.swizzle([a], mode)[0]) == want, (mode, a, want)
    for mode, pairs in EXT_HAND_EXAMPLES.items():
        for a, want in pairs:
            assert int(o.swizzle([a], mode)[0]) == want, (mode, a, want)


def pin_swizzle_structure(o):
    """Involution; bijection inside each atom (rows of 128 B × the rows the mode reads its
    bits from); 16-byte units move whole; the permutation never leaves its span block."""
    atoms = {"32B": 256, "64B": 512, "128B": 1024, "128B_2ROW": 2048, "128B_TR": 2048}
    spans = {"32B": 32, "64B": 64, "128B": 128, "128B_2ROW": 128, "128B_TR": 128}
    a = np.arange(1 << 15, dtype=np.uint64)
    for mode, atom in atoms.items():
        s = o.swizzle(a, mode)
        assert np.array_equal(o.swizzle(s, mode), a), mode
        blocks = a.reshape(-1, atom)
        sb = s.reshape(-1, atom)
        for b, t in zip(blocks, sb):
            assert np.array_equal(np.sort(t), b), mode
        # whole 16-byte units: offsets of one unit stay together and in order
        u = s.reshape(-1, 16)
        assert np.all(u[:, 1:] - u[:, :-1] == 1), mode
        span = spans[mode]
        assert np.array_equal(s // np.uint64(span), a // np.uint64(span)), mode


def pin_bank_spread(o):
    """§11.2 bank = (a'/4) % 32: in 128B mode the same logical 16-byte column of 8 consecutive
    128-byte rows lands in 8 distinct 16-byte bank groups, covering all 32 banks.  For the
    library's 2-row mode, 16 consecutive rows fill a 64-bank (256-byte) window."""
    g = golden()["bank_equation"]
    for col in range(8):
        offs = np.array([r * 128 + col * 16 for r in range(8)], dtype=np.uint64)
        s = o.swizzle(offs, "128B")
        banks = set()
        for x in s:
            for w in range(4):
                banks.add(int((int(x) + 4 * w) // g["bank_bytes"]) % g["banks"])
        assert banks == set(range(g["banks"])), col
        # without a swizzle every row hits the same 4 banks
        assert len({int(x // 4) % 32 for x in offs}) == 1
    for col in range(8):
        offs = np.array([r * 128 + col * 16 for r in range(16)], dtype=np.uint64)
        s = o.swizzle(offs, "128B_2ROW")
        assert len({int(x // 16) % 16 for x in s}) == 16, col
    # 128B_TR: the transposing 8-byte read takes 32 bytes (an aligned pair of 16-byte units, pair p)
    # from each of the rows {r0 + 8t + 4h + e : t < 2, e < 4} per 32 lanes, which the LDS serves from
    # one 256-byte window (64 banks of 4 bytes); the eight pieces must fall on eight distinct
    # 32-byte bank groups.  The 128B and 2-row modes put two of them on one group.
    for r0 in (0, 16, 32):
        for h in (0, 1):
            rows = [r0 + 8 * t + 4 * h + e for t in range(2) for e in range(4)]
            for p in range(4):
                offs = np.array([r * 128 + p * 32 for r in rows], dtype=np.uint64)
                groups = {mode: {int(x // 32) % 8 for x in o.swizzle(offs, mode)} for mode in
                          ("128B_TR", "128B", "128B_2ROW")}
                assert len(groups["128B_TR"]) == 8, (r0, h, p)
                assert len(groups["128B"]) < 8 and len(groups["128B_2ROW"]) < 8, (r0, h, p)
                # the two 16-byte units of a pair stay an aligned pair
                both = np.concatenate([offs, offs + np.uint64(16)])
                s = o.swizzle(both, "128B_TR")
                assert np.array_equal(s[:len(offs)] // np.uint64(32), s[len(offs):] // np.uint64(32))


# ---------------------------------------------------------------------------------------------
# Tiled copy ("2 · Le Tensor Memory Accelerator" §2.2–§2.5; "H100 · cuTensorMap" §8–§9, §14)
# ---------------------------------------------------------------------------------------------
def _bf16_matrix(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    t = (torch.rand((rows, cols), generator=g) * 2 - 1).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def pin_worked_descriptor(o):
    """The page's creer_descripteur on a 256×256 bf16 matrix: the image is the 128×64 LDS
    tile of §2.4 (16384 bytes, the byte count the barrier expects), swizzled in 16-byte units;
    undoing the swizzle gives A[y:y+128, x:x+64] with zeros past the edges."""
    g = golden()["tma_worked_descriptor"]
    rows = cols = 256
    A = _bf16_matrix(rows, cols, 11)
    dims = [cols, rows]
    strides = [cols * g["stride_bytes_per_col"]]
    want_bytes = g["smem_tile_rows"] * g["smem_tile_cols"] * g["smem_tile_elsize"]
    assert want_bytes == g["image_bytes"] == golden()["mbarrier_expect_tx_bytes"]["bytes"]
    bits = golden()["swizzle_bit_rules"]["128B"]
    for (x, y) in [(0, 0), (64, 0), (192, 128), (128, 64), (224, 192), (-32, -64), (250, 250), (-64, 0)]:
        img = o.tiled_copy(A, "bf16", dims, strides, g["box"], g["element_strides"], g["swizzle"],
                           g["oob"] == "nan", [x, y])
        assert img.size == g["image_bytes"]
        # undo the swizzle with the per-bit statement (an involution), element by element
        offs = np.arange(img.size, dtype=np.uint64)
        logical = np.empty_like(img)
        logical[offs] = img[_per_bit(offs, bits)]
        tile = logical.view(np.uint16).reshape(g["smem_tile_rows"], g["smem_tile_cols"])
        want = np.zeros((128, 64), dtype=np.uint16)
        ys, xs = max(y, 0), max(x, 0)
        ye, xe = min(y + 128, rows), min(x + 64, cols)
        if ye > ys and xe > xs:
            want[ys - y:ye - y, xs - x:xe - x] = A[ys:ye, xs:xe]
        assert np.array_equal(tile, want), (x, y)


def _index_tensor(dims_inner_first, dtype):
    total = int(np.prod(dims_inner_first))
    npdt = {"u8": np.uint8, "u16": np.uint16, "u32": np.uint32, "f16": np.uint16, "bf16": np.uint16,
            "f32": np.uint32}[dtype]
    return np.arange(total, dtype=np.uint64).astype(npdt)


def _decode_case(o, dims, box, estr, coords, dtype, oob, padded_rows=0, swz="none"):
    """Fill a tensor with its own linear index, copy one box, and check every image element
    against the coordinates it must come from (or the fill)."""
    rank = len(dims)
    elsize = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4}[dtype]
    # row pitch of dim 1 padded by `padded_rows` elements, rounded so strides are 16-byte multiples
    pitch = [elsize * (dims[0] + padded_rows)]
    for i in range(2, rank):
        pitch.append(pitch[-1] * dims[i - 1])
    total_elems = (pitch[-1] * dims[rank - 1]) // elsize if rank > 1 else dims[0]
    npdt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[elsize]
    src = np.zeros(total_elems, dtype=npdt)
    # linear index of coordinate x under these strides
    idx = np.indices(dims[::-1]).reshape(rank, -1)[::-1]  # idx[i] = coordinate along dim i
    lin = idx[0].astype(np.int64)
    for i in range(1, rank):
        lin = lin + idx[i].astype(np.int64) * (pitch[i - 1] // elsize)
    tag = (np.arange(lin.size, dtype=np.int64) + 1)      # element tags 1..count
    src[lin] = tag.astype(npdt)
    before = src.copy()
    img = o.tiled_copy(src, dtype, dims, pitch[:rank - 1], box, estr, swz, oob == "nan", coords)
    assert np.array_equal(src, before), "source modified"
    n = [(b + e - 1) // e for b, e in zip(box, estr)]
    img_e = img.view(npdt)
    if swz != "none":
        # the swizzle permutes whole bytes; undo it and compare against the unswizzled copy
        plain = o.tiled_copy(src, dtype, dims, pitch[:rank - 1], box, estr, "none", oob == "nan", coords)
        offs = np.arange(img.size, dtype=np.uint64)
        assert np.array_equal(img[o.swizzle(offs, swz)], plain)
        return
    jj = np.indices(n[::-1]).reshape(rank, -1)[::-1]
    x = np.stack([coords[i] + jj[i] * estr[i] for i in range(rank)])
    inside = np.all([(x[i] >= 0) & (x[i] < dims[i]) for i in range(rank)], axis=0)
    # tag of an inside element: 1 + its rank among all elements in innermost-first order
    t = x[0].astype(np.int64)
    mul = 1
    for i in range(1, rank):
        mul *= dims[i - 1]
        t = t + x[i].astype(np.int64) * mul
    want_tag = (t + 1).astype(np.int64)
    got = img_e.astype(np.int64)
    if oob == "nan":
        fill = {"f16": 0x7E00, "bf16": 0x7FC0, "f32": 0x7FC00000}[dtype]
    else:
        fill = 0
    modv = 1 << (8 * elsize)
    assert np.array_equal(got[inside], want_tag[inside] % modv)
    assert np.all(got[~inside] == fill)


def pin_copy_decode(o):
    rng = np.random.default_rng(7)
    # hand-picked cases: ragged edges, negative coordinates, element strides at each position
    _decode_case(o, [40, 9, 3], [16, 4, 2], [1, 2, 1], [32, -2, 1], "u16", "zero")
    _decode_case(o, [17, 5, 4, 3, 2], [8, 3, 2, 2, 2], [3, 1, 2, 1, 1], [-5, 3, 2, 2, 1], "f16", "nan")
    _decode_case(o, [33], [20], [4], [20], "f32", "nan")
    _decode_case(o, [64, 64], [64, 16], [1, 8], [0, 3], "u32", "zero")
    _decode_case(o, [7, 6, 5, 4, 3], [8, 8, 8, 8, 8], [8, 7, 6, 5, 4], [-1, -2, 0, 1, -3], "u8", "zero")
    _decode_case(o, [64, 10], [64, 8], [1, 1], [-8, -4], "bf16", "nan")
    for _ in range(40):
        rank = int(rng.integers(1, 6))
        dims = [int(rng.integers(1, 12)) for _ in range(rank)]
        box = [int(rng.integers(1, 10)) for _ in range(rank)]
        estr = [int(rng.integers(1, 9)) for _ in range(rank)]
        coords = [int(rng.integers(-6, d + 3)) for d in dims]
        dtype = ["u8", "u16", "u32", "f16", "bf16", "f32"][int(rng.integers(0, 6))]
        oob = "nan" if dtype in ("f16", "bf16", "f32") and rng.integers(0, 2) else "zero"
        _decode_case(o, dims, box, estr, coords, dtype, oob, padded_rows=int(rng.integers(0, 3)) * 8)
    # swizzled images are the same bytes permuted by the swizzle
    _decode_case(o, [64, 20], [64, 16], [1, 1], [0, 8], "bf16", "zero", swz="128B")
    _decode_case(o, [32, 20], [32, 8], [1, 2], [0, 3], "bf16", "nan", swz="64B")
    _decode_case(o, [16, 20], [16, 8], [1, 1], [0, -3], "u16", "zero", swz="32B")
    _decode_case(o, [64, 40], [64, 32], [1, 1], [0, 5], "bf16", "zero", swz="128B_2ROW")


def pin_fill_and_source(o):
    """§14: the fill is written to the destination only; zero fill gives zero bytes, NaN fill a
    NaN of the element type; the source is not modified."""
    for dtype, npdt in (("bf16", np.uint16), ("f16", np.uint16), ("f32", np.uint32)):
        src = np.arange(64, dtype=npdt)
        before = src.copy()
        img = o.tiled_copy(src, dtype, [8, 8], [8 * src.itemsize], [4, 4], [1, 1], "none", True, [100, 100])
        vals = img.view(npdt)
        if dtype == "bf16":
            f = (vals.astype(np.uint32) << 16).view(np.float32)
        elif dtype == "f16":
            f = vals.view(np.float16)
        else:
            f = vals.view(np.float32)
        assert np.all(np.isnan(f)), dtype
        img0 = o.tiled_copy(src, dtype, [8, 8], [8 * src.itemsize], [4, 4], [1, 1], "none", False, [100, 100])
        assert np.all(img0 == 0)
        assert np.array_equal(src, before)


def _store_case(o, dims, box, estr, coords, dtype, padded_rows=0):
    """Store an image of distinct tags into a tensor of sentinels; every box position inside the
    tensor must land at the coordinates it names, and nothing else may change."""
    rank = len(dims)
    elsize = {"u8": 1, "u16": 2, "u32": 4, "f16": 2, "bf16": 2, "f32": 4}[dtype]
    npdt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[elsize]
    pitch = [elsize * (dims[0] + padded_rows)]
    for i in range(2, rank):
        pitch.append(pitch[-1] * dims[i - 1])
    total = (pitch[-1] * dims[rank - 1]) // elsize if rank > 1 else dims[0]
    sentinel = {1: 0xAB, 2: 0xABCD, 4: 0xABCDEF01}[elsize]
    tensor = np.full(total, sentinel, dtype=npdt)
    n = [(b + e - 1) // e for b, e in zip(box, estr)]
    count = int(np.prod(n))
    tags = ((np.arange(count, dtype=np.int64) % (sentinel - 1)) + 1).astype(npdt)  # never the sentinel
    out = o.tiled_store(tensor, dtype, dims, pitch[:rank - 1], box, estr, "none", coords, tags).view(npdt)
    want = tensor.copy()
    jj = np.indices(n[::-1]).reshape(rank, -1)[::-1]
    x = np.stack([coords[i] + jj[i] * estr[i] for i in range(rank)])
    inside = np.all([(x[i] >= 0) & (x[i] < dims[i]) for i in range(rank)], axis=0)
    lin = x[0].astype(np.int64)
    for i in range(1, rank):
        lin = lin + x[i].astype(np.int64) * (pitch[i - 1] // elsize)
    want[lin[inside]] = tags[inside]
    assert np.array_equal(out, want)


def pin_store_decode(o):
    """"2 · Le Tensor Memory Accelerator" §2.5, the store direction with the same descriptor:
    brute-force index decoding of every box position, edges not written."""
    rng = np.random.default_rng(17)
    _store_case(o, [40, 9, 3], [16, 4, 2], [1, 2, 1], [32, -2, 1], "u16")
    _store_case(o, [17, 5, 4, 3, 2], [8, 3, 2, 2, 2], [3, 1, 2, 1, 1], [-5, 3, 2, 2, 1], "f16")
    _store_case(o, [33], [20], [4], [20], "f32")
    _store_case(o, [64, 10], [64, 8], [1, 1], [-8, -4], "bf16", padded_rows=8)
    for _ in range(40):
        rank = int(rng.integers(1, 6))
        dims = [int(rng.integers(1, 12)) for _ in range(rank)]
        box = [int(rng.integers(1, 10)) for _ in range(rank)]
        estr = [int(rng.integers(1, 9)) for _ in range(rank)]
        coords = [int(rng.integers(-6, d + 3)) for d in dims]
        dtype = ["u8", "u16", "u32", "f16", "bf16", "f32"][int(rng.integers(0, 6))]
        _store_case(o, dims, box, estr, coords, dtype, padded_rows=int(rng.integers(0, 3)) * 8)


def pin_store_hand_example(o):
    """A 4×4 u16 tensor (row pitch 16 bytes after padding to 8 elements), box {2, 2} at (-1, 3):
    of the four positions only j = (1, 0) is inside, at x = (0, 3)."""
    t = np.zeros(4 * 8, dtype=np.uint16)
    out = o.tiled_store(t, "u16", [4, 4], [16], [2, 2], [1, 1], "none", [-1, 3],
                        np.array([10, 11, 12, 13], dtype=np.uint16)).view(np.uint16)
    want = np.zeros(4 * 8, dtype=np.uint16)
    want[3 * 8 + 0] = 11
    assert np.array_equal(out, want)


def pin_store_swizzle_and_roundtrip(o):
    """A swizzled image stores like its unswizzled permutation (logical element k sits at image
    byte swizzle(k)); storing an image and loading the same box back returns the image at the
    positions inside the tensor and the fill elsewhere."""
    rng = np.random.default_rng(23)
    for swz, box0 in (("128B", 64), ("64B", 32), ("32B", 16), ("128B_2ROW", 64)):
        dims, box, coords = [box0 + 8, 20], [box0, 16], [0, 7]
        t = np.zeros((dims[1], dims[0]), dtype=np.uint16)
        img = rng.integers(1, 60000, box0 * 16).astype(np.uint16)
        out_s = o.tiled_store(t, "bf16", dims, [dims[0] * 2], box, [1, 1], swz, coords, img)
        offs = np.arange(img.size * 2, dtype=np.uint64)
        plain = img.view(np.uint8)[o.swizzle(offs, swz)]
        out_p = o.tiled_store(t, "bf16", dims, [dims[0] * 2], box, [1, 1], "none", coords, plain)
        assert np.array_equal(out_s, out_p), swz
    for _ in range(30):
        rank = int(rng.integers(1, 5))
        dims = [int(rng.integers(1, 10)) for _ in range(rank)]
        box = [int(rng.integers(1, 8)) for _ in range(rank)]
        estr = [int(rng.integers(1, 4)) for _ in range(rank)]
        coords = [int(rng.integers(-4, d + 2)) for d in dims]
        strides = [2 * dims[0]]
        for i in range(2, rank):
            strides.append(strides[-1] * dims[i - 1])
        total = int(np.prod(dims))
        n = [(b + e - 1) // e for b, e in zip(box, estr)]
        img = rng.integers(1, 60000, int(np.prod(n))).astype(np.uint16)
        t = np.zeros(total, dtype=np.uint16)
        stored = o.tiled_store(t, "u16", dims, strides[:rank - 1], box, estr, "none", coords, img)
        back = o.tiled_copy(stored.view(np.uint16), "u16", dims, strides[:rank - 1], box, estr, "none", False,
                            coords).view(np.uint16)
        jj = np.indices(n[::-1]).reshape(rank, -1)[::-1]
        inside = np.all([(coords[i] + jj[i] * estr[i] >= 0) & (coords[i] + jj[i] * estr[i] < dims[i])
                         for i in range(rank)], axis=0)
        assert np.array_equal(back[inside], img[inside])
        assert np.all(back[~inside] == 0)


# ---------------------------------------------------------------------------------------------
# GEMM ("GEMM: la moltiplicazione di matrici sull'hardware")
# ---------------------------------------------------------------------------------------------
def _bits_of(values: np.ndarray) -> np.ndarray:
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_gemm_exact_rationals(o):
    """Brute force on tiny shapes: each C_ij against Σ_k A_ik B_kj in exact rational arithmetic.
    Every bf16 product is exact and these sums stay exact in binary64, so the binary64 result
    must equal the rational exactly and the binary32 result is its correct rounding."""
    rng = np.random.default_rng(3)
    for (M, N, K, lda_pad, ldb_pad) in [(3, 4, 5, 0, 0), (7, 1, 9, 3, 0), (1, 1, 1, 0, 0), (5, 6, 17, 0, 5),
                                        (2, 9, 33, 7, 1), (4, 3, 64, 0, 0)]:
        lda, ldn = K + lda_pad, N + ldb_pad
        A = _bits_of(rng.standard_normal((M, lda)).astype(np.float32))
        Bkn = _bits_of(rng.standard_normal((K, ldn)).astype(np.float32))
        Af, Bf = _f64(A), _f64(Bkn)
        exact = [[sum((Fraction(Af[m, k]) * Fraction(Bf[k, n]) for k in range(K)), Fraction(0))
                  for n in range(N)] for m in range(M)]
        c32, c64 = o.gemm(A, Bkn, M, N, K, lda, ldn, "kn", want64=True)
        for m in range(M):
            for n in range(N):
                assert Fraction(c64[m, n]) == exact[m][n], (M, N, K, m, n)
                assert c32[m, n] == np.float32(float(exact[m][n]))
        # the same product with B stored N×K (K contiguous)
        ldk = K + ldb_pad
        Bnk = np.zeros((N, ldk), dtype=np.uint16)
        Bnk[:, :K] = Bkn[:K, :N].T
        c32n = o.gemm(A, Bnk, M, N, K, lda, ldk, "nk")
        assert np.array_equal(c32n, c32)
        # sampled points agree with whole rows
        ms = rng.integers(0, M, 5)
        ns = rng.integers(0, N, 5)
        p32 = o.gemm_points(A, Bkn, K, lda, ldn, ms, ns, "kn")
        assert np.array_equal(p32, c32[ms, ns])
        p32n = o.gemm_points(A, Bnk, K, lda, ldk, ms, ns, "nk")
        assert np.array_equal(p32n, c32[ms, ns])


def pin_gemm_closed_forms(o):
    """A·I = A; all-ones gives C = K; integer-valued operands give exact integer products that
    must equal numpy's integer matmul (exact for these magnitudes)."""
    rng = np.random.default_rng(5)
    M, K = 37, 29
    A = _bits_of(rng.uniform(-1, 1, (M, K)).astype(np.float32))
    I = _bits_of(np.eye(K, dtype=np.float32))
    c = o.gemm(A, I, M, K, K, K, K, "kn")
    assert np.array_equal(c, _f64(A).astype(np.float32))
    c = o.gemm(A, I, M, K, K, K, K, "nk")
    assert np.array_equal(c, _f64(A).astype(np.float32))
    ones = _bits_of(np.ones((64, 64), dtype=np.float32))
    for K1 in (1, 7, 64):
        c = o.gemm(ones, ones, 5, 6, K1, 64, 64, "kn")
        assert np.all(c == K1)
    for (M, N, K, bl) in [(31, 45, 777, "kn"), (16, 9, 300, "nk"), (64, 64, 64, "kn")]:
        Ai = rng.integers(-8, 9, (M, K))
        Bi = rng.integers(-8, 9, (K, N))
        want = (Ai.astype(np.int64) @ Bi.astype(np.int64)).astype(np.float64)
        A = _bits_of(Ai.astype(np.float32))
        if bl == "kn":
            c = o.gemm(A, _bits_of(Bi.astype(np.float32)), M, N, K, K, N, "kn")
        else:
            c = o.gemm(A, _bits_of(np.ascontiguousarray(Bi.T).astype(np.float32)), M, N, K, K, K, "nk")
        assert np.array_equal(c.astype(np.float64), want), (M, N, K, bl)


def pin_gemm_tiled_equals_direct(o):
    """The GEMM page's NumPy example: a T=32 tiled product of A (96,80) and B (80,64) equals the
    direct product.  Tiles are cut with the oracle's own tiled copy (zero fill past the edges,
    so the ragged K=80 edge contributes nothing), multiplied with numpy and summed over K."""
    g = golden()["tiled_matmul_numpy_example"]
    (M, K), (_, N), T = g["A_shape"], g["B_shape"], g["T"]
    rng = np.random.default_rng(9)
    A = _bits_of(rng.standard_normal((M, K)).astype(np.float32))
    B = _bits_of(rng.standard_normal((K, N)).astype(np.float32))
    _, c64 = o.gemm(A, B, M, N, K, K, N, "kn", want64=True)
    C = np.zeros((M, N))
    for i in range(0, M, T):
        for j in range(0, N, T):
            acc = np.zeros((T, T))
            for k in range(0, K, T):
                a = o.tiled_copy(A, "bf16", [K, M], [K * 2], [T, T], [1, 1], "none", False, [k, i])
                b = o.tiled_copy(B, "bf16", [N, K], [N * 2], [T, T], [1, 1], "none", False, [j, k])
                acc += _f64(a.view(np.uint16).reshape(T, T)) @ _f64(b.view(np.uint16).reshape(T, T))
            C[i:i + T, j:j + T] = acc[:min(T, M - i), :min(T, N - j)]
    assert np.allclose(C, c64, rtol=1e-12, atol=1e-12) == g["allclose"]
    # and against numpy's direct product of the widened operands
    assert np.allclose(_f64(A) @ _f64(B), c64, rtol=1e-12, atol=1e-12)


def pin_f32_to_bf16(o):
    """Round to nearest even against torch's conversion, on ties of every exponent, specials and
    a dense random sample; NaN stays NaN."""
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    ties = (np.arange(1 << 16, dtype=np.uint32) << 16) | np.uint32(0x8000)
    near = (np.arange(1 << 16, dtype=np.uint32) << 16) | np.uint32(0x7FFF)
    specials = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001, 0x7FC00000,
                         0x7F800001, 0x3F808000, 0x3F818000], dtype=np.uint32)
    u = np.concatenate([u, ties, near, specials])
    f = u.view(np.float32)
    got = o.f32_to_bf16(f)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], want[~nan])
    back = (got[nan].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(back))


def pin_gemm_ex(o):
    """C <- alpha·A·B + beta·C ("GEMM" page, tensor-core section: the BLAS form).  alpha = 1,
    beta = 0 is the plain product; beta = 0 does not read C (NaN there stays out); alpha = 0 gives
    beta·C; on small-integer operands the result is exact and equals integer arithmetic."""
    rng = np.random.default_rng(31)
    M, N, K = 7, 9, 13
    A = _bits_of(rng.normal(size=(M, K)))
    B = _bits_of(rng.normal(size=(K, N)))
    plain = o.gemm(A, B, M, N, K, K, N, "kn")
    assert np.array_equal(o.gemm_ex(A, B, M, N, K, K, N, "kn", 1.0, 0.0), plain)
    nanC = np.full((M, N), np.nan, dtype=np.float32)
    assert np.array_equal(o.gemm_ex(A, B, M, N, K, K, N, "kn", 1.0, 0.0, nanC), plain)
    Cold = rng.normal(size=(M, N)).astype(np.float32)
    assert np.array_equal(o.gemm_ex(A, B, M, N, K, K, N, "kn", 0.0, 0.5, Cold), Cold * np.float32(0.5))
    Ai = rng.integers(-8, 9, (M, K))
    Bi = rng.integers(-8, 9, (N, K))
    Ci = rng.integers(-100, 101, (M, N))
    got = o.gemm_ex(_bits_of(Ai.astype(np.float64)), _bits_of(Bi.astype(np.float64)), M, N, K, K, K, "nk", 2.0,
                    -3.0, Ci.astype(np.float32))
    want = 2 * (Ai @ Bi.T) - 3 * Ci
    assert np.array_equal(got.astype(np.int64), want)


def pin_f16_decode(o):
    """binary16 decoding against numpy's float16 for all 65536 bit patterns (NaN where numpy
    has NaN; infinities, subnormals and signed zeros exact)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f64(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_gemm_f16(o):
    """fp16 inputs: small integers (products and sums exact) against numpy's integer matmul, both
    layouts; values with fractions and the extreme exponents of binary16 (2^-24 subnormals, 2^15)
    against exact rationals."""
    rng = np.random.default_rng(61)
    M, N, K = 33, 29, 71
    Ai = rng.integers(-16, 17, (M, K))
    Bi = rng.integers(-16, 17, (K, N))
    Ab = Ai.astype(np.float16).view(np.uint16)
    Bb = Bi.astype(np.float16).view(np.uint16)
    want = (Ai @ Bi).astype(np.float64)
    assert np.array_equal(o.gemm(Ab, Bb, M, N, K, K, N, "kn", ab="f16"), want.astype(np.float32))
    BbT = np.ascontiguousarray(Bi.T).astype(np.float16).view(np.uint16)
    assert np.array_equal(o.gemm(Ab, BbT, M, N, K, K, K, "nk", ab="f16"), want.astype(np.float32))
    vals = np.array([2.0 ** -24, 3 * 2.0 ** -24, 2.0 ** -14, 1.0 / 3, 0.1, 65504.0, -2.0 ** 15, 1.5], dtype=np.float16)
    a = rng.choice(vals, (5, 8))
    b = rng.choice(vals, (8, 4))
    got = o.gemm(a.view(np.uint16), b.view(np.uint16), 5, 4, 8, 8, 4, "kn", want64=True, ab="f16")[1]
    for i in range(5):
        for j in range(4):
            ex = sum(Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(8))
            assert Fraction(got[i, j]) == ex or abs(Fraction(got[i, j]) - ex) <= abs(ex) * Fraction(1, 2 ** 52)


def pin_f8_decode(o):
    """OCP E4M3 and E5M2 decoding for all 256 patterns against torch's float8_e4m3fn and
    float8_e5m2 conversions, and the formats' landmarks: E4M3 max 448 (0x7E), NaN 0x7F, smallest
    subnormal 2^-9; E5M2 max 57344 (0x7B), infinity 0x7C, smallest subnormal 2^-16."""
    bits = np.arange(256, dtype=np.uint8)
    for fmt, tdt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        got = o.f8_to_f64(bits, fmt)
        want = torch.from_numpy(bits.copy()).view(tdt).double().numpy()
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), fmt
        assert np.array_equal(got[~nan], want[~nan]), fmt
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), fmt
    e4 = o.f8_to_f64(bits, "e4m3")
    assert e4[0x7E] == 448.0 and np.isnan(e4[0x7F]) and e4[0x01] == 2.0 ** -9 and e4[0x08] == 2.0 ** -6
    e5 = o.f8_to_f64(bits, "e5m2")
    assert e5[0x7B] == 57344.0 and e5[0x7C] == np.inf and e5[0x01] == 2.0 ** -16 and np.isnan(e5[0x7D])


def pin_f8_nan_fill(o):
    """NaN fill of 8-bit float tensors (tiled and im2col copies): every out-of-bounds byte decodes
    to NaN under torch's float8_e4m3fn / float8_e5m2 conversions, every in-bounds byte is the
    source's, and a zero fill stays zero."""
    rng = np.random.default_rng(88)
    src = rng.integers(0, 0x70, 6 * 5, dtype=np.uint8)  # finite patterns of both formats
    for dt, tdt in (("f8e4m3", torch.float8_e4m3fn), ("f8e5m2", torch.float8_e5m2)):
        img = o.tiled_copy(src, dt, [6, 5], [6], [16, 4], [1, 1], "none", True, [-3, 2])
        inb = np.zeros((4, 16), dtype=bool)
        inb[:3, 3:9] = True  # rows 2..4 of 5, columns 0..5 of 6
        vals = torch.from_numpy(img.copy()).view(tdt).float().numpy().reshape(4, 16)
        assert np.isnan(vals[~inb]).all(), dt
        assert np.array_equal(img.reshape(4, 16)[inb], src.reshape(5, 6)[2:5, 0:6].reshape(-1)), dt
        zero = o.tiled_copy(src, dt, [6, 5], [6], [16, 4], [1, 1], "none", False, [-3, 2])
        assert (zero.reshape(4, 16)[~inb] == 0).all(), dt
        im = o.im2col_copy(src, dt, [6, 5, 1, 1], [6, 30, 30], [1, 1], [1, 1], [1, 1], [1, 1], [3, 3], 16, 3, "none",
                           True, [0, 0, 0, 1])  # tap r = 1: the image row; tap s = 0: pixel 0 in the padding
        v = torch.from_numpy(im.copy()).view(tdt).float().numpy().reshape(3, 16)
        assert np.isnan(v[:, 6:]).all() and np.isnan(v[0]).all(), dt  # channels past C; pixel 0 in the padding
        assert np.array_equal(im.reshape(3, 16)[1, :6], src[0:6]), dt
        assert np.array_equal(im.reshape(3, 16)[2, :6], src[6:12]), dt


def _f8_bits(values: np.ndarray, fmt: str) -> np.ndarray:
    tdt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(tdt).view(torch.uint8).numpy().copy()


def pin_gemm_f8(o):
    """8-bit inputs: small integers (exact in both formats) against numpy's integer matmul, and
    values with fractions and subnormals against exact rationals."""
    rng = np.random.default_rng(81)
    M, N, K = 21, 19, 150
    for fmt, lim in (("e4m3", 16), ("e5m2", 8)):
        Ai = rng.integers(-lim, lim + 1, (M, K))
        Bi = rng.integers(-lim, lim + 1, (N, K))
        got = o.gemm_f8(_f8_bits(Ai, fmt), _f8_bits(Bi, fmt), M, N, K, K, K, fmt)
        assert np.array_equal(got, (Ai @ Bi.T).astype(np.float32)), fmt
        vals = np.array([2.0 ** -9, 2.0 ** -6, 0.375, -1.75, 3.5, 40.0], dtype=np.float32) if fmt == "e4m3" else \
            np.array([2.0 ** -16, 2.0 ** -14, 0.75, -1.5, 3.0, 96.0], dtype=np.float32)
        a = rng.choice(vals, (4, 9))
        b = rng.choice(vals, (3, 9))
        ab, bb = _f8_bits(a, fmt), _f8_bits(b, fmt)
        g64 = o.gemm_f8(ab, bb, 4, 3, 9, 9, 9, fmt, want64=True)[1]
        av, bv = o.f8_to_f64(ab, fmt), o.f8_to_f64(bb, fmt)
        for i in range(4):
            for j in range(3):
                ex = sum(Fraction(float(av[i, k])) * Fraction(float(bv[j, k])) for k in range(9))
                assert Fraction(g64[i, j]) == ex, (fmt, i, j)


def _nc_x_hwcx(nchw: np.ndarray, x: int) -> np.ndarray:
    """NCHW -> NC/xHWCx by numpy: channels cut into slices of x (the last one zero-padded), each
    slice stored per position: array (N, C/x, H, W, x)."""
    N, C, H, W = nchw.shape
    cs = -(-C // x)
    padded = np.zeros((N, cs * x, H, W), dtype=nchw.dtype)
    padded[:, :C] = nchw
    return np.ascontiguousarray(padded.reshape(N, cs, x, H, W).transpose(0, 1, 3, 4, 2))


def pin_interleaved_boxes(o):
    """"H100 · cuTensorMap" §12: a box of an NC/xHWCx tensor (dimension 0 one channel slice, read
    whole) is the numpy slice of the interleaved array, and a box over every slice of a spatial
    window, reordered (h, w, slice, x), is that window of the NHWC tensor with the padded
    channels zero."""
    rng = np.random.default_rng(71)
    N, C, H, W, x = 2, 21, 9, 11, 8
    nchw = rng.integers(1, 60000, (N, C, H, W)).astype(np.uint16)
    t = _nc_x_hwcx(nchw, x)
    cs = t.shape[1]
    dims = [x, W, H, cs, N]
    strides = [2 * x, 2 * x * W, 2 * x * W * H, 2 * x * W * H * cs]
    for coords in ([0, 0, 0, 0, 0], [0, 3, 2, 1, 1], [0, 8, 6, 2, 0], [0, -2, -1, 0, 1]):
        box = [x, 5, 4, cs, 1]
        img = o.tiled_copy(t, "u16", dims, strides, box, [1] * 5, "none", False, coords).view(np.uint16)
        img = img.reshape(1, cs, 4, 5, x)
        want = np.zeros((1, cs, 4, 5, x), dtype=np.uint16)
        for n in range(1):
            for c in range(cs):
                for h in range(4):
                    for w in range(5):
                        hh, ww, cc, nn = coords[2] + h, coords[1] + w, coords[3] + c, coords[4] + n
                        if 0 <= hh < H and 0 <= ww < W and 0 <= cc < cs:
                            want[n, c, h, w] = t[nn, cc, hh, ww]
        assert np.array_equal(img, want), coords
        if coords[1] >= 0 and coords[2] >= 0 and coords[1] + 5 <= W and coords[2] + 4 <= H and coords[3] == 0:
            nhwc = img[0].transpose(1, 2, 0, 3).reshape(4, 5, cs * x)
            ref = nchw[coords[4], :, coords[2]:coords[2] + 4, coords[1]:coords[1] + 5].transpose(1, 2, 0)
            assert np.array_equal(nhwc[:, :, :C], ref) and not nhwc[:, :, C:].any()


# ---------------------------------------------------------------------------------------------
# im2col copy and 2-D convolution ("2 · Le Tensor Memory Accelerator", section "im2col": the
# convolution becomes a GEMM over an im2col matrix formed during the copy)
# ---------------------------------------------------------------------------------------------
def _im2col_numpy(X, R, S, pad, stride, dil):
    """Textbook im2col through explicit zero padding and slicing (no bounds tests): X (N,H,W,C)
    -> (N*OH*OW, R, S, C)."""
    N, H, W, C = X.shape
    top, left, bottom, right = pad
    Xp = np.pad(X, ((0, 0), (top, bottom), (left, right), (0, 0)))
    OH = (H + top + bottom - dil[0] * (R - 1) - 1) // stride[0] + 1
    OW = (W + left + right - dil[1] * (S - 1) - 1) // stride[1] + 1
    out = np.zeros((N, OH, OW, R, S, C), dtype=X.dtype)
    for r in range(R):
        for s_ in range(S):
            h0, w0 = r * dil[0], s_ * dil[1]
            out[:, :, :, r, s_, :] = Xp[:, h0:h0 + stride[0] * (OH - 1) + 1:stride[0],
                                        w0:w0 + stride[1] * (OW - 1) + 1:stride[1], :]
    return out.reshape(N * OH * OW, R, S, C), OH, OW


def pin_conv_out_dim(o):
    """Output extents against torch's convolution shapes and two hand values (56×56 with a 3×3
    filter and padding 1 keeps 56; 7 with a 3-tap window at stride 2 gives 3)."""
    assert o.conv_out_dim(56, 1, 1, 1, 1, 3) == 56
    assert o.conv_out_dim(7, 0, 0, 2, 1, 3) == 3
    assert o.conv_out_dim(2, 0, 0, 1, 1, 3) == 0
    rng = np.random.default_rng(5)
    for _ in range(40):
        n = int(rng.integers(1, 20)); p = int(rng.integers(0, 4)); st = int(rng.integers(1, 4))
        d = int(rng.integers(1, 3)); f = int(rng.integers(1, 5))
        if n + 2 * p < d * (f - 1) + 1:
            continue
        t = torch.nn.functional.conv1d(torch.zeros(1, 1, n), torch.zeros(1, 1, f), stride=st, padding=p, dilation=d)
        assert o.conv_out_dim(n, p, p, st, d, f) == t.shape[-1], (n, p, st, d, f)


def pin_im2col_hand_example(o):
    """A 3×3 single-channel image holding 1..9, a 2×2 filter, stride 1, no padding: the four
    im2col rows are the four 2×2 windows read row by row."""
    X = np.arange(1, 10, dtype=np.uint32).reshape(1, 3, 3, 1)
    want = np.array([[1, 2, 4, 5], [2, 3, 5, 6], [4, 5, 7, 8], [5, 6, 8, 9]], dtype=np.uint32)
    got = np.zeros((4, 4), dtype=np.uint32)
    for r in range(2):
        for s_ in range(2):
            img = o.im2col_copy(X, "u32", [1, 3, 3, 1], [4, 12, 36], [0, 0], [0, 0], [1, 1], [1, 1], [2, 2], 1, 4,
                                "none", False, [0, 0, s_, r])
            got[:, 2 * r + s_] = img.view(np.uint32)
    assert np.array_equal(got, want)


def pin_im2col_decode(o):
    """Every image slot of random im2col copies decodes to the element the textbook im2col (zero
    padding by np.pad, windows by slicing) puts there, or to the fill."""
    rng = np.random.default_rng(11)
    cases = [((2, 6, 7, 5), 3, 3, (1, 1, 1, 1), (1, 1), (1, 1)), ((1, 9, 8, 3), 3, 2, (0, 2, 1, 0), (2, 1), (1, 2)),
             ((3, 5, 5, 4), 1, 1, (0, 0, 0, 0), (2, 2), (1, 1)), ((1, 7, 6, 2), 2, 3, (2, 0, 0, 3), (1, 2), (2, 1))]
    for (N, H, W, C), R, S, pad, stride, dil in cases:
        X = (np.arange(N * H * W * C, dtype=np.uint32) + 1).reshape(N, H, W, C)
        cols, OH, OW = _im2col_numpy(X, R, S, pad, stride, dil)
        M = N * OH * OW
        for _ in range(6):
            ch = int(rng.integers(1, 9)); px = int(rng.integers(1, 12))
            c0 = int(rng.integers(-2, C + 1)); m0 = int(rng.integers(-3, M + 2))
            r = int(rng.integers(0, R)); s_ = int(rng.integers(0, S))
            img = o.im2col_copy(X, "u32", [C, W, H, N], [4 * C, 4 * C * W, 4 * C * W * H], [pad[1], pad[0]],
                                [pad[3], pad[2]], [stride[1], stride[0]], [dil[1], dil[0]], [S, R], ch, px, "none",
                                False, [c0, m0, s_, r]).view(np.uint32).reshape(px, ch)
            for i in range(px):
                for j in range(ch):
                    m, c = m0 + i, c0 + j
                    want = cols[m, r, s_, c] if (0 <= m < M and 0 <= c < C) else 0
                    assert img[i, j] == want, ((N, H, W, C), R, S, pad, stride, dil, c0, m0, r, s_, i, j)
    # NaN fill of a bf16 tensor, and the swizzle of a 64-channel (128-byte) row
    X = np.ones((1, 4, 4, 64), dtype=np.uint16) * 0x3F80
    img = o.im2col_copy(X, "bf16", [64, 4, 4, 1], [128, 512, 2048], [1, 1], [1, 1], [1, 1], [1, 1], [3, 3], 64, 8,
                        "none", True, [0, 0, 0, 0]).view(np.uint16).reshape(8, 64)
    assert np.all(img[0] == 0x7FC0) and np.all(img[1:4] == 0x7FC0) and np.all(img[4] == 0x7FC0)
    assert np.all(img[5:8] == 0x3F80)
    X = (np.arange(2 * 4 * 4 * 64, dtype=np.uint32) % 65521).astype(np.uint16).reshape(2, 4, 4, 64)
    plain = o.im2col_copy(X, "u16", [64, 4, 4, 2], [128, 512, 2048], [1, 1], [1, 1], [1, 1], [1, 1], [3, 3], 64,
                          16, "none", False, [0, 3, 1, 2])
    swz = o.im2col_copy(X, "u16", [64, 4, 4, 2], [128, 512, 2048], [1, 1], [1, 1], [1, 1], [1, 1], [3, 3], 64, 16,
                        "128B", False, [0, 3, 1, 2])
    perm = o.swizzle(np.arange(plain.size, dtype=np.uint64), "128B")
    assert np.array_equal(swz[perm.astype(np.int64)], plain)


def _conv_case(rng, N, H, W, C, K, R, S, integer):
    if integer:
        Xv = rng.integers(-4, 5, (N, H, W, C)).astype(np.float32)
        Wv = rng.integers(-4, 5, (K, R, S, C)).astype(np.float32)
    else:
        Xv = rng.standard_normal((N, H, W, C)).astype(np.float32)
        Wv = rng.standard_normal((K, R, S, C)).astype(np.float32)
    Xb = _bits_of(Xv)
    Wb = _bits_of(Wv)
    return Xb, Wb


def pin_conv_torch(o):
    """The convolution against torch's float64 conv2d on the CPU (a library routine, NCHW):
    bit for bit on small integers (every sum exact in any order), within 1e-12 relative on
    random values; padding is applied with F.pad so it may be asymmetric."""
    rng = np.random.default_rng(21)
    cases = [(2, 7, 6, 5, 4, 3, 3, (1, 1, 1, 1), (1, 1), (1, 1)), (1, 9, 8, 3, 2, 3, 2, (0, 2, 1, 0), (2, 1), (1, 2)),
             (2, 5, 5, 4, 3, 1, 1, (0, 0, 0, 0), (2, 2), (1, 1)), (1, 7, 6, 2, 5, 2, 3, (2, 0, 0, 3), (1, 2), (2, 1))]
    for integer in (True, False):
        for N, H, W, C, K, R, S, pad, stride, dil in cases:
            Xb, Wb = _conv_case(rng, N, H, W, C, K, R, S, integer)
            got32, got64 = o.conv2d(Xb, Wb, N, H, W, C, K, R, S, pad, stride, dil, want64=True)
            xt = torch.from_numpy(_f64(Xb).reshape(N, H, W, C)).permute(0, 3, 1, 2)
            wt = torch.from_numpy(_f64(Wb).reshape(K, R, S, C)).permute(0, 3, 1, 2)
            xt = torch.nn.functional.pad(xt, (pad[1], pad[3], pad[0], pad[2]))
            yt = torch.nn.functional.conv2d(xt, wt, stride=stride, dilation=dil)
            ref = yt.permute(0, 2, 3, 1).reshape(-1, K).numpy()
            assert got64.shape == ref.shape
            if integer:
                assert np.array_equal(got64, ref) and np.array_equal(got32, ref.astype(np.float32))
            else:
                assert np.allclose(got64, ref, rtol=1e-12, atol=1e-12)


def pin_conv_1x1_is_gemm(o):
    """A 1×1 convolution at stride 1 without padding is the GEMM X(NHW × C) · W(K × C)ᵀ: the
    same sums in the same order, so the binary32 results agree bit for bit."""
    rng = np.random.default_rng(31)
    N, H, W, C, K = 2, 5, 7, 24, 9
    Xb, Wb = _conv_case(rng, N, H, W, C, K, 1, 1, False)
    y = o.conv2d(Xb, Wb, N, H, W, C, K, 1, 1)
    g = o.gemm(Xb, Wb, N * H * W, K, C, C, C, "nk")
    assert np.array_equal(y, g)


def pin_conv_equals_im2col_gemm(o):
    """The page's identity: the convolution equals the GEMM of its im2col matrix (built from
    im2col copies, one per tap and channel block) with the filters as a K × (R·S·C) matrix; the
    sums run in the same (r, s, c) order, so the results agree bit for bit."""
    rng = np.random.default_rng(41)
    N, H, W, C, K, R, S = 2, 6, 7, 10, 6, 3, 2
    pad, stride, dil = (1, 0, 2, 1), (2, 1), (1, 2)
    Xb, Wb = _conv_case(rng, N, H, W, C, K, R, S, False)
    OH = o.conv_out_dim(H, pad[0], pad[2], stride[0], dil[0], R)
    OW = o.conv_out_dim(W, pad[1], pad[3], stride[1], dil[1], S)
    M = N * OH * OW
    cols = np.zeros((M, R, S, C), dtype=np.uint16)
    for r in range(R):
        for s_ in range(S):
            for m0 in range(0, M, 16):
                for c0 in range(0, C, 4):
                    img = o.im2col_copy(Xb.reshape(N, H, W, C), "bf16", [C, W, H, N], [2 * C, 2 * C * W, 2 * C * W * H],
                                        [pad[1], pad[0]], [pad[3], pad[2]], [stride[1], stride[0]],
                                        [dil[1], dil[0]], [S, R], 4, 16, "none", False, [c0, m0, s_, r])
                    blk = img.view(np.uint16).reshape(16, 4)
                    rows = min(16, M - m0); chs = min(4, C - c0)
                    cols[m0:m0 + rows, r, s_, c0:c0 + chs] = blk[:rows, :chs]
    y = o.conv2d(Xb, Wb, N, H, W, C, K, R, S, pad, stride, dil)
    g = o.gemm(cols.reshape(M, -1), Wb.reshape(K, -1), M, K, R * S * C, R * S * C, R * S * C, "nk")
    assert np.array_equal(y, g)


ALL_PINS = [pin_swizzle_bit_rules, pin_swizzle_hand_examples, pin_swizzle_structure, pin_bank_spread,
            pin_worked_descriptor, pin_copy_decode, pin_fill_and_source, pin_store_decode, pin_store_hand_example,
            pin_store_swizzle_and_roundtrip, pin_gemm_exact_rationals, pin_gemm_closed_forms,
            pin_gemm_tiled_equals_direct, pin_gemm_ex, pin_f32_to_bf16, pin_conv_out_dim, pin_im2col_hand_example,
            pin_im2col_decode, pin_conv_torch, pin_conv_1x1_is_gemm, pin_conv_equals_im2col_gemm,
            pin_f16_decode, pin_gemm_f16, pin_interleaved_boxes, pin_f8_decode, pin_gemm_f8, pin_f8_nan_fill]
