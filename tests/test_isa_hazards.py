"""Static check of the kernels' AMD assembly (CPU only): every direct-to-LDS buffer load written as
inline assembly has its scalar operands settled.

gfx9 needs 5 wait states between a vector instruction that writes a scalar register (for example
v_readfirstlane_b32) and a vector-memory instruction that reads that register (the buffer
descriptor, M0).  The compiler inserts them in front of its own memory instructions but cannot see
inside inline assembly, so a descriptor built with v_readfirstlane right before an asm buffer load
is read stale, and a stale descriptor can address memory outside the operand.  The load's
scalar offset register, where it has one, counts as one of its scalar operands.  This test compiles
every kernel source (product build and hand-off checking build) to assembly and requires that no
such load has a vector write of one of its scalar operands within the 5 preceding wait states
(each instruction counts 1, s_nop N counts N + 1).

The same listings also fix the ring's stage hand-off: the wait before each barrier of a barrier-ring
kernel is an immediate built by hand (vmcnt split over bits 3:0 and 15:14), and a wrong field
would let a barrier pass before its tile landed.  Every barrier of each ring instance must wait
for vmcnt T·(S−1) (the prologue: tile 0 landed), T·(S−2) (the loop: tile kt+1 landed) or 0, with T
the instance's copy atoms per wave and K tile and S its stages, and the hand-off checking build
for 0 everywhere.  Those counts hold only if the copy atoms are the only vector-memory instructions
a wave has in flight before its drain: in every barrier-ring, fp8, im2col- and halo-convolution
instance (the kernels whose waves all copy and compute), no other
vector-memory instruction (a load or store of the compiler's, a register spill) may be reachable
from the kernel's entry without passing a full drain (`vmcnt(0)` and a barrier), walked over the
listing's basic blocks and branches, since the blocks' order in the listing is not the order they
run in.  The same walk requires every vmcnt wait met there to be a barrier's (or a vmcnt(0) that
settles the copies right before the drain): a wait the compiler places for loads of its own counts
the copies too and would hold them back without any sign but time."""
import concurrent.futures
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_bf16_gemm_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def _sregs(tok):
    tok = tok.strip()
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.match(r"s\d+$", tok) or tok in ("m0", "vcc"):
        return {tok}
    return set()


def _vector_sgpr_writes(ins):
    """Scalar registers a vector instruction writes (empty for any other instruction)."""
    op, _, rest = ins.partition(" ")
    if not op.startswith("v_"):
        return set()
    ops = [o.strip() for o in rest.split(",")]
    out = set()
    if op.startswith(("v_readfirstlane", "v_readlane")) or (op.startswith("v_cmp") and op.endswith("_e64")):
        out |= _sregs(ops[0])
    if op.startswith(("v_add_co", "v_sub_co", "v_subrev_co", "v_addc_co", "v_subb_co", "v_mad_u64", "v_mad_i64",
                      "v_div_scale")) and len(ops) > 1:
        out |= _sregs(ops[1])
    return out


def scan(text):
    """Hazards in one assembly listing: (load, offending instruction, wait states between)."""
    ins = []
    for line in text.splitlines():
        t = line.strip()
        if not t or t.startswith((".", ";", "//")) or t.endswith(":"):
            continue
        ins.append(t.split(";")[0].strip())
    found = []
    for i, t in enumerate(ins):
        if not (t.startswith("buffer_load") and t.endswith(" lds")):
            continue
        ops = [o.strip() for o in t.partition(" ")[2].split(",")]
        if ops[1].startswith("v"):
            found.append((t, "descriptor in vector registers", 0))
            continue
        need = _sregs(ops[1]) | {"m0"} | (_sregs(ops[2].split()[0]) if len(ops) > 2 else set())
        ws = 0
        for prev in reversed(ins[max(0, i - 8):i]):
            if _vector_sgpr_writes(prev) & need:
                found.append((t, prev, ws))
                break
            m = re.match(r"s_nop\s+(\d+)", prev)
            ws += int(m.group(1)) + 1 if m else 1
            if ws >= 5:
                break
    return found


def test_scan_flags_a_planted_hazard_and_passes_settled_code():
    """The scanner itself: a readfirstlane straight into a descriptor register is flagged; the same
    with s_nop 4 in between, or with the descriptor written by scalar instructions, is not."""
    bad = "v_readfirstlane_b32 s43, v70\n s_mov_b32 m0, s2\n buffer_load_dwordx4 v1, s[40:43], 0 offen lds\n"
    assert len(scan(bad)) == 1
    ok = "v_readfirstlane_b32 s43, v70\n s_nop 4\n buffer_load_dwordx4 v1, s[40:43], 0 offen lds\n"
    assert scan(ok) == []
    ok2 = "s_mov_b32 s43, 0x20000\n buffer_load_dwordx4 v1, s[40:43], 0 offen lds\n"
    assert scan(ok2) == []
    far = "v_readfirstlane_b32 s43, v70\n" + "s_add_i32 s1, s1, 1\n" * 5 + "buffer_load_dwordx4 v1, s[40:43], 0 offen lds\n"
    assert scan(far) == []
    m0 = "v_readfirstlane_b32 m0, v3\n buffer_load_dwordx4 v1, s[40:43], 0 offen lds\n"
    assert len(scan(m0)) == 1
    so = "v_readlane_b32 s7, v9, 3\n buffer_load_dwordx4 v1, s[40:43], s7 offen lds\n"
    assert len(scan(so)) == 1
    so_ok = "v_readlane_b32 s7, v9, 3\n buffer_load_dwordx4 v1, s[40:43], s8 offen lds\n"
    assert scan(so_ok) == []


RING = re.compile(r"^(_ZN3tbg16gemm_ring_kernelI((?:Li\d+E)+)EEvNS_10GemmParamsE):", re.M)


def _vmcnt(ins):
    """The vmcnt of an s_waitcnt instruction (None when it does not wait on vmcnt)."""
    m = re.match(r"s_waitcnt\b.*\bvmcnt\((\d+)\)", ins)
    return int(m.group(1)) if m else None


def barrier_waits(text):
    """Per barrier-ring kernel instance: (BM, BN, S, CLK) and the vmcnt of the nearest s_waitcnt
    before each of its s_barrier instructions (None when none precedes it since the last barrier)."""
    out = {}
    heads = list(RING.finditer(text))
    for i, h in enumerate(heads):
        args = [int(a) for a in re.findall(r"Li(\d+)E", h.group(2))]
        body = text[h.end():heads[i + 1].start() if i + 1 < len(heads) else len(text)]
        end = body.find(".Lfunc_end")
        ins = [t.strip().split(";")[0].strip() for t in body[:end if end >= 0 else len(body)].splitlines()]
        ins = [t for t in ins if t and not t.startswith((".", "//")) and not t.endswith(":")]
        waits = []
        for j, t in enumerate(ins):
            if t != "s_barrier":
                continue
            v = None
            for prev in reversed(ins[max(0, j - 12):j]):
                if prev == "s_barrier":
                    break
                if _vmcnt(prev) is not None:
                    v = _vmcnt(prev)
                    break
            waits.append(v)
        out[h.group(1)] = (args, waits)
    return out


def ring_wait_problems(text, check):
    """Barriers of ring instances whose wait is not the intended count (see the module text)."""
    problems = []
    for name, (args, waits) in barrier_waits(text).items():
        bm, bn, s = args[0], args[1], args[2]
        atoms = bm // 32 + bn // 32
        allowed = {0} if check else {0, atoms * (s - 2), atoms * (s - 1)}
        bad = [w for w in waits if w not in allowed]
        if bad:
            problems.append(f"{name}: barrier waits {sorted(set(map(str, bad)))} outside {sorted(allowed)}")
        if not check and not ({atoms * (s - 1), atoms * (s - 2)} <= set(waits)):
            problems.append(f"{name}: no prologue or loop hand-off found among waits {sorted(set(map(str, waits)))}")
    return problems


def test_ring_wait_check_flags_wrong_counts():
    """The checker itself on a small listing: the intended counts pass, a wait with a wrong count
    or none at all is flagged, and the hand-off checking build accepts only 0."""
    head = "_ZN3tbg16gemm_ring_kernelILi128ELi128ELi3ELi0ELi0ELi1ELi0ELi0EEEvNS_10GemmParamsE:\n"
    good = head + ("s_waitcnt vmcnt(16) lgkmcnt(0)\ns_barrier\nv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]\n"
                   "s_waitcnt vmcnt(8) lgkmcnt(0)\nv_add_u32 v1, v1, v2\ns_barrier\n"
                   "s_waitcnt vmcnt(0) lgkmcnt(0)\ns_barrier\n.Lfunc_end3:\n")
    assert [a for a, _ in barrier_waits(good).values()] == [[128, 128, 3, 0, 0, 1, 0, 0]]
    assert ring_wait_problems(good, 0) == []
    assert ring_wait_problems(good, 1) != []
    assert ring_wait_problems(good.replace("vmcnt(8)", "vmcnt(12)"), 0) != []
    assert ring_wait_problems(good.replace("s_waitcnt vmcnt(8) lgkmcnt(0)\n", ""), 0) != []
    drained = re.sub(r"vmcnt\(\d+\)", "vmcnt(0)", good)
    assert ring_wait_problems(drained, 1) == []


KERNEL = re.compile(r"^(_ZN3tbg(?:16gemm_ring_kernel|21gemm_conv_halo_kernel|15gemm_fp8_kernel|16gemm_conv_kernel)I\w+):",
                    re.M)


def _blocks(lines):
    """Basic blocks of one kernel's listing: [label or None, [instructions]] in listing order."""
    blocks, cur = [], [None, []]
    for raw in lines:
        t = raw.split(";")[0].strip()
        if not t or t.startswith("//"):
            continue
        m = re.match(r"^(\.LBB\d+_\d+):", t)
        if m:
            blocks.append(cur)
            cur = [m.group(1), []]
            continue
        if t.startswith("."):
            continue
        cur[1].append(t)
        if re.match(r"s_(c?branch|endpgm)", t):
            blocks.append(cur)
            cur = [None, []]
    blocks.append(cur)
    return [b for b in blocks if b[0] is not None or b[1]]


def _guarded_barrier(ins, j):
    """Whether the s_waitcnt at ins[j] is the wait of a barrier: an s_barrier follows within 12
    instructions with no other vmcnt wait in between."""
    for t in ins[j + 1:j + 13]:
        if t == "s_barrier":
            return True
        if _vmcnt(t) is not None:
            return False
    return False


def _settles_drain(ins, j):
    """Whether the wait at ins[j] only settles the copies right before the drain: the next vmcnt
    wait, within 12 instructions and with no memory instruction or product in between, is a
    barrier's vmcnt(0)."""
    for k in range(j + 1, min(j + 13, len(ins))):
        t = ins[k]
        if _vmcnt(t) is not None:
            return _vmcnt(t) == 0 and _guarded_barrier(ins, k)
        if re.match(r"(buffer|global|flat|scratch|ds)_|v_mfma", t):
            return False
    return False


def early_vmem(lines):
    """Walk the blocks reachable from the entry without passing a full drain (an s_waitcnt with
    vmcnt(0) that is a barrier's wait).  Returns the vector-memory instructions met there that are
    not direct-to-LDS copy atoms, the number of copy atoms met, the number of barriers met (each
    leaving copies in flight) and the vmcnt waits met that are no barrier's wait (a wait the
    compiler placed for loads it cannot tell apart from the copies would hold them back), except a
    vmcnt(0) right before the drain."""
    bl = _blocks(lines)
    at = {b[0]: i for i, b in enumerate(bl) if b[0]}

    def succ(i):
        last = bl[i][1][-1] if bl[i][1] else ""
        m = re.match(r"s_branch (\.LBB\d+_\d+)", last)
        if m:
            return [at[m.group(1)]]
        if last.startswith("s_endpgm"):
            return []
        out = []
        m = re.match(r"s_cbranch_\w+ (\.LBB\d+_\d+)", last)
        if m:
            out.append(at[m.group(1)])
        return out + ([i + 1] if i + 1 < len(bl) else [])

    seen, todo, bad, copies, barriers, stray = set(), [0], [], 0, 0, []
    while todo:
        i = todo.pop()
        if i in seen:
            continue
        seen.add(i)
        ins, stop = bl[i][1], False
        for j, t in enumerate(ins):
            if t == "s_barrier":
                barriers += 1
            v = _vmcnt(t)
            if v is not None:
                if _guarded_barrier(ins, j):
                    if v == 0:
                        stop = True
                        break
                elif not (v == 0 and _settles_drain(ins, j)):
                    stray.append(t)
            if re.match(r"(buffer|global|flat|scratch)_", t):
                if t.startswith("buffer_load_dwordx4") and t.endswith(" lds"):
                    copies += 1
                else:
                    bad.append(t)
        if not stop:
            todo += succ(i)
    return bad, copies, barriers, stray


def early_vmem_problems(text, check):
    problems = []
    heads = list(KERNEL.finditer(text))
    for i, h in enumerate(heads):
        body = text[h.end():heads[i + 1].start() if i + 1 < len(heads) else len(text)]
        end = body.find(".Lfunc_end")
        bad, copies, barriers, stray = early_vmem(body[:end if end >= 0 else len(body)].splitlines())
        if bad:
            problems.append(f"{h.group(1)}: {bad[:3]} before the drain")
        if stray:
            problems.append(f"{h.group(1)}: vmcnt waits {stray[:3]} that no barrier follows, before the drain")
        # (in the hand-off checking build every barrier drains: there the walk ends at the first)
        if copies == 0 or (barriers == 0 and not check):
            problems.append(f"{h.group(1)}: the walk met {copies} copy atoms and {barriers} barriers before the drain")
    return problems


def test_early_vmem_walk_flags_loads_among_the_copies():
    """The walk on small listings: a compiler load inside the K loop (before a barrier that leaves
    copies in flight) is flagged, and so is a register spill; the same load after the drain is not,
    nor an epilogue block laid out in the listing ahead of the loop's remainder block but reached
    only after the drain, while a branch that falls through into the epilogue before the drain
    is; a vmcnt wait that guards no barrier is reported."""
    copy = "buffer_load_dwordx4 v1, s[8:11], 0 offen lds"
    loop = [".LBB0_1:", copy, "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
            "s_waitcnt vmcnt(8) lgkmcnt(0)", "s_barrier", "s_cbranch_scc1 .LBB0_1"]
    drain = ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier"]
    store = "global_store_dwordx4 v[2:3], v[4:7], off nt"
    load = "global_load_dword v9, v[2:3], off"
    ok = [copy] + loop + drain + [store, "s_endpgm"]
    assert early_vmem(ok) == ([], 2, 1, [])
    planted = [copy] + loop[:2] + [load] + loop[2:] + drain + [store, "s_endpgm"]
    assert early_vmem(planted)[0] == [load]
    spill = [copy, "scratch_store_dword off, v5, s0 offset:16"] + loop + drain + ["s_endpgm"]
    assert early_vmem(spill)[0] == ["scratch_store_dword off, v5, s0 offset:16"]
    # listing order: loop, then an epilogue block, then the remainder block that jumps back to it
    laid_out = [copy] + loop + ["s_branch .LBB0_3", ".LBB0_2:", store, "s_endpgm", ".LBB0_3:", copy,
                                "s_waitcnt vmcnt(4) lgkmcnt(0)", "s_barrier"] + drain + ["s_branch .LBB0_2"]
    assert early_vmem(laid_out)[0] == []
    falls = [copy] + loop + ["s_cbranch_scc0 .LBB0_3", ".LBB0_2:", store, "s_endpgm", ".LBB0_3:"] + drain + \
        ["s_branch .LBB0_2"]
    assert early_vmem(falls)[0] == [store]
    # a wait of the compiler's at the loop head (no barrier follows it) is flagged; the kernel's own
    # vmcnt(0) right before the drain is not
    throttled = [copy, loop[0], "s_waitcnt vmcnt(1)"] + loop[1:] + drain + [store, "s_endpgm"]
    assert early_vmem(throttled)[3] == ["s_waitcnt vmcnt(1)"]
    settle = [copy] + loop + ["s_waitcnt vmcnt(0)", "v_cvt_pk_bf16_f32 v21, v21, v30"] + drain + [store, "s_endpgm"]
    assert early_vmem(settle)[3] == []
    early = [copy] + loop[:2] + ["s_waitcnt vmcnt(0)"] + loop[2:] + drain + [store, "s_endpgm"]
    assert early_vmem(early)[3] == ["s_waitcnt vmcnt(0)"]
    leaked = laid_out[:laid_out.index(".LBB0_3:") + 1] + [load] + laid_out[laid_out.index(".LBB0_3:") + 1:]
    assert early_vmem(leaked)[0] == [load]


def _compile(src, check):
    out = tempfile.NamedTemporaryFile(suffix=".s", delete=False).name
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wno-unused-command-line-argument",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC,
           f"-DTBG_HANDOFF_CHECK={check}", "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    try:
        if r.returncode != 0:
            return src, check, None, r.stderr[-2000:], []
        with open(out) as f:
            text = f.read()
        return src, check, scan(text), "", ring_wait_problems(text, check) + early_vmem_problems(text, check)
    finally:
        os.unlink(out)


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_inline_buffer_loads_have_settled_scalar_operands_and_ring_waits():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = [(s, c) for s in srcs for c in (0, 1)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs))
    problems = []
    rings = 0
    for src, check, found, err, waits in results:
        problems += [f"{os.path.basename(src)} (hand-off check {check}): {w}" for w in waits]
        if os.path.basename(src).startswith("gemm_ring_") and found is not None:
            rings += 1
        name = f"{os.path.basename(src)} (hand-off check {check})"
        if found is None:
            problems.append(f"{name}: hipcc failed: {err}")
        for load, prev, ws in found or []:
            problems.append(f"{name}: {load!r} after {prev!r} ({ws} wait states)")
    assert rings == 8, "every ring source compiled in both builds"
    assert not problems, "\n".join(problems[:20])
