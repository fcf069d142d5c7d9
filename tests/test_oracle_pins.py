"""The CPU oracle against the pages' worked examples and plain mathematics (no GPU).

Also checks the pins' strength: each deliberately broken copy of ``oracle/oracle.c`` (a dropped
term, a wrong sign, index or bound, a transposed operand) must fail at least one pin.
"""
import os
import subprocess
import sys

import pytest

import oracle
from oracle import build as oracle_build
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


# (description, text in oracle.c, replacement)
MUTANTS = [
    ("128B mask drops bit 9", "oracle_swizzle_general(a, 0x380u, 3)", "oracle_swizzle_general(a, 0x180u, 3)"),
    ("64B shift off by one", "oracle_swizzle_general(a, 0x180u, 3)", "oracle_swizzle_general(a, 0x180u, 2)"),
    ("2-row mode uses 128B bits", "oracle_swizzle_general(a, 0x700u, 4)", "oracle_swizzle_general(a, 0x380u, 3)"),
    ("transposing-read mode uses the 2-row bits",
     "case 5: return a ^ (((a >> 9) & 1u) << 4) ^ (((a >> 8) & 1u) << 5) ^ (((a >> 10) & 1u) << 6);",
     "case 5: return oracle_swizzle_general(a, 0x700u, 4);"),
    ("transposing-read mode swaps its low two bits",
     "case 5: return a ^ (((a >> 9) & 1u) << 4) ^ (((a >> 8) & 1u) << 5) ^ (((a >> 10) & 1u) << 6);",
     "case 5: return a ^ (((a >> 8) & 1u) << 4) ^ (((a >> 9) & 1u) << 5) ^ (((a >> 10) & 1u) << 6);"),
    ("transposing-read mode drops row bit 3",
     "case 5: return a ^ (((a >> 9) & 1u) << 4) ^ (((a >> 8) & 1u) << 5) ^ (((a >> 10) & 1u) << 6);",
     "case 5: return a ^ (((a >> 9) & 1u) << 4) ^ (((a >> 8) & 1u) << 5);"),
    ("negative coordinate counted inside", "if (x < 0 || (uint64_t)x >= dim[i]) inside = 0;",
     "if ((uint64_t)x >= dim[i] && x >= 0) inside = 0;"),
    ("upper bound off by one", "(uint64_t)x >= dim[i]", "(uint64_t)x > dim[i]"),
    ("element stride dropped", "int64_t x = c[i] + (int64_t)j[i] * (int64_t)estr[i];", "int64_t x = c[i] + (int64_t)j[i];"),
    ("floor instead of ceil", "n[i] = (box[i] + estr[i] - 1) / estr[i];", "n[i] = box[i] / estr[i] + (box[i] < estr[i]);"),
    ("image index uses wrong extent", "j[0] + n[0] * (j[1] + n[1] *", "j[0] + n[1] * (j[1] + n[1] *"),
    ("bf16 NaN bytes swapped", "fill[0] = 0xC0; fill[1] = 0x7F;", "fill[0] = 0x7F; fill[1] = 0xC0;"),
    ("swizzle skipped on the image", "uint64_t off = oracle_swizzle(lin * (uint64_t)elsize, swizzle);",
     "uint64_t off = lin * (uint64_t)elsize;"),
    ("KN product reads B with lda", "const uint16_t* brow = B + k * ldb;", "const uint16_t* brow = B + k * lda;"),
    ("wrong sign in accumulation", "acc[n] += a * in_to_f64(brow[n], ab_kind);", "acc[n] -= a * in_to_f64(brow[n], ab_kind);"),
    ("NK operand transposed", "acc += in_to_f64(A[m * lda + k], ab_kind) * in_to_f64(B[n * ldb + k], ab_kind);",
     "acc += in_to_f64(A[m * lda + k], ab_kind) * in_to_f64(B[k * ldb + n], ab_kind);"),
    ("first term dropped", "for (int64_t k = 0; k < K; ++k) {\n                    double a", "for (int64_t k = 1; k < K; ++k) {\n                    double a"),
    ("ties rounded up", "u += 0x7FFFu + lsb;", "u += 0x8000u;"),
    ("points use the wrong layout", "uint16_t b = b_layout == 0 ? B[k * ldb + n] : B[n * ldb + k];",
     "uint16_t b = b_layout == 0 ? B[k * ldb + n] : B[k * ldb + n];"),
    ("store writes positions outside the tensor", "if (!inside) continue;", "if (0) continue;"),
    ("store skips the swizzle", "uint64_t off = oracle_swizzle(lin * (uint64_t)elsize, swizzle);\n        if (off + (uint64_t)elsize > size)",
     "uint64_t off = lin * (uint64_t)elsize;\n        if (off + (uint64_t)elsize > size)"),
    ("store drops the element stride", "int64_t x = c[i] + (int64_t)j[i] * (int64_t)estr[i];\n            if (x < 0 || (uint64_t)x >= dim[i]) inside = 0;\n            else dst_off",
     "int64_t x = c[i] + (int64_t)j[i];\n            if (x < 0 || (uint64_t)x >= dim[i]) inside = 0;\n            else dst_off"),
    ("im2col tap ignores the dilation", "ih = oh * cstride[1] - pad_lo[1] + tap_r * dil[1];",
     "ih = oh * cstride[1] - pad_lo[1] + tap_r;"),
    ("im2col pixel order transposed", "const int64_t ow = m % OW, oh = (m / OW) % OH;\n            n = m / (OW * OH);",
     "const int64_t oh = m % OH, ow = (m / OH) % OW;\n            n = m / (OW * OH);"),
    ("im2col padding added instead of subtracted", "iw = ow * cstride[0] - pad_lo[0] + tap_s * dil[0];",
     "iw = ow * cstride[0] + pad_lo[0] + tap_s * dil[0];"),
    ("im2col channel bound off by one", "if (row_inside && c >= 0 && c < C) {", "if (row_inside && c >= 0 && c <= C) {"),
    ("im2col image rows use the pixel count", "(uint64_t)elsize * (j + (uint64_t)channels * i)",
     "(uint64_t)elsize * (j + (uint64_t)pixels * i)"),
    ("output extent loses the last position", "return span / stride + 1;", "return span / stride;"),
    ("convolution flips the filter", "const uint16_t* wp = Wt + ((k * R + r) * S + s) * C;",
     "const uint16_t* wp = Wt + ((k * R + (R - 1 - r)) * S + (S - 1 - s)) * C;"),
    ("convolution ignores the stride", "const int64_t ih = oh * sh - ph + r * dh;", "const int64_t ih = oh - ph + r * dh;"),
    ("f16 exponent bias off by one", "else v = ldexp((double)(1024 + f), e - 25);",
     "else v = ldexp((double)(1024 + f), e - 24);"),
    ("f16 subnormals scaled like normals", "if (e == 0) v = ldexp((double)f, -24);", "if (e == 0) v = ldexp((double)f, -25);"),
    ("f16 inputs decoded as bf16", "return kind == 1 ? f16_to_f64(h) : bf16_to_f64(h);", "return bf16_to_f64(h);"),
    ("e4m3 exponent bias off by one", "r = e == 0 ? ldexp((double)f, -9) : ldexp((double)(8 + f), e - 10);",
     "r = e == 0 ? ldexp((double)f, -9) : ldexp((double)(8 + f), e - 11);"),
    ("e4m3 top exponent read as NaN", "if (e == 15 && f == 7) return NAN;", "if (e == 15) return NAN;"),
    ("e5m2 subnormals scaled like e4m3", "r = e == 0 ? ldexp((double)f, -16) : ldexp((double)(4 + f), e - 17);",
     "r = e == 0 ? ldexp((double)f, -9) : ldexp((double)(4 + f), e - 17);"),
    ("f8 product reads B transposed", "acc += f8_to_f64(A[m * lda + k], fmt) * f8_to_f64(B[n * ldb + k], fmt);",
     "acc += f8_to_f64(A[m * lda + k], fmt) * f8_to_f64(B[k * ldb + n], fmt);"),
    ("convolution drops the last channel", "for (int64_t c = 0; c < C; ++c) acc +=", "for (int64_t c = 0; c + 1 < C; ++c) acc +="),
    ("e5m2 NaN fill writes infinity", "else if (nan_kind == 5) { fill[0] = 0x7E; }", "else if (nan_kind == 5) { fill[0] = 0x7C; }"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_broken_oracle_fails_a_pin(tmp_path, desc, old, new):
    src = open(oracle_build.SRC).read()
    assert old in src, f"mutation site not found: {desc}"
    mutated = src.replace(old, new, 1)
    csrc = tmp_path / "oracle.c"
    csrc.write_text(mutated)
    out = str(tmp_path / "liboracle_mut.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", str(csrc), "-o", out],
                   check=True)
    # The broken build runs in a child process: a wrong index can write past the image.
    child = (
        "import sys; sys.path.insert(0, %r)\n"
        "import oracle\n"
        "from tests import oracle_pins\n"
        "o = oracle.Oracle(%r)\n"
        "bad = []\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    try:\n"
        "        pin(o)\n"
        "    except (AssertionError, ValueError, IndexError):\n"
        "        bad.append(pin.__name__)\n"
        "print('FAILED_PINS', ','.join(bad))\n"
    ) % (ROOT, out)
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        # the broken build crashed inside a pin: it is caught, but only as a crash
        assert "FAILED_PINS" not in r.stdout
        return
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED_PINS")][0]
    failures = [x for x in line.split(" ", 1)[1].split(",") if x]
    assert failures, f"no pin catches: {desc}"


def test_oracle_under_sanitizers(tmp_path):
    """Every pin against a build of ``oracle.c`` with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only): an out-of-bounds access, a use of freed memory, a signed overflow or a shift
    out of range anywhere the pins reach aborts the child and fails the test."""
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    libubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    if not (os.path.isabs(libasan) and os.path.exists(libasan) and os.path.isabs(libubsan)):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    out = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
                    oracle_build.SRC, "-o", out], check=True)
    child = (
        "import sys; sys.path.insert(0, %r)\n"
        "import oracle\n"
        "from tests import oracle_pins\n"
        "o = oracle.Oracle(%r)\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    pin(o)\n"
        "print('ALL_PINS_PASSED', len(oracle_pins.ALL_PINS))\n"
    ) % (ROOT, out)
    env = dict(os.environ, LD_PRELOAD=f"{libasan}:{libubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, timeout=900, env=env)
    assert r.returncode == 0 and "ALL_PINS_PASSED" in r.stdout, (r.stdout[-2000:] + r.stderr[-4000:])
