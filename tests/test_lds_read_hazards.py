"""The LDS reads the kernels issue as inline assembly, checked in the ISA.

The hot LDS reads (ds_read_b128, ds_read_b64_tr_b16 and friends) are inline
asm: the compiler's own LDS reads would first wait for every direct
global->LDS copy in flight (it cannot tell that those target other stages),
which drains the copy pipelines. An asm read is issued without waiting; a
later `s_waitcnt lgkmcnt(N)` that names its destination registers makes its
result usable. The compiler, however, takes such an output as written when
the asm statement issues. If it read, wrote or reallocated those registers
before the wait, the value would be stale or the late-arriving data would
overwrite a register that holds something else.

This test compiles every kernel for gfx950 and checks that this never
happens in the code that ships. In each basic block it tracks the LDS
operations in flight. LDS operations complete in issue order, so a
`s_waitcnt lgkmcnt(N)` retires all but the youngest N. Scalar loads share
the counter and complete in any order, but they can only make the real wait
stricter, so ignoring them keeps the check sound. It requires that:

* no instruction reads or writes a register of an LDS read still in flight;
* no LDS read is still in flight at a branch, a label or the end of the
  kernel.

The compiler's own LDS reads (outside the ;;#ASMSTART .. ;;#ASMEND markers
of the listing) count towards the in-order completion but are not checked:
the compiler tracks their registers itself.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_blockwise_attention_amd import build

CSRC = build.CSRC
KERNEL_SOURCES = ["ra_fwd.hip", "ra_bwd.hip", "ra_dq.hip", "ra_dqds.hip", "ra_misc.hip", "ra_gemm.hip"]

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
LGKM = re.compile(r"lgkmcnt\((\d+)\)")


def regs_of(text):
    """The vector (v) and accumulation (a) registers an operand list names."""
    out = set()
    for m in REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            for r in range(int(m.group(2)), int(m.group(3)) + 1):
                out.add((kind, r))
    return out


BRANCH = re.compile(r"^s_(cbranch_\w+|branch)$")
ENDS = ("s_endpgm", "s_setpc_b64", "s_swappc_b64")


def check_function(name, lines):
    """Returns the hazards found in one kernel's instruction lines.

    The in-flight list of each straight-line stretch follows the control
    flow: a forward branch hands its list to its target label, where the
    lists of all incoming paths must agree (or hold no asm read); a loop's
    back edge, a label reached by one, and the kernel's end must hold no asm
    read in flight. Dropping older entries from a list keeps it a suffix of
    the hardware's queue, so the retirement rule stays sound."""
    items = []  # (line, op, operands, issued by inline asm)
    in_asm = False  # inside an inline-asm statement (;;#ASMSTART .. ;;#ASMEND)
    for n, raw in lines:
        if "#ASMSTART" in raw:
            in_asm = True
        elif "#ASMEND" in raw:
            in_asm = False
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            items.append((n, "label", line[:-1], False))
            continue
        op, _, rest = line.partition(" ")
        items.append((n, op, rest.strip(), in_asm))
    label_pos = {rest: i for i, (_, op, rest, _) in enumerate(items) if op == "label"}
    back_targets = {rest.split()[0] for i, (_, op, rest, _) in enumerate(items)
                    if BRANCH.match(op) and rest.split()[0] in label_pos and label_pos[rest.split()[0]] < i}

    problems = []
    inflight = []  # LDS operations in flight, oldest first: (line, dest registers of asm reads)
    pending = {}  # label -> in-flight lists handed over by forward branches
    reachable = True

    def asm_pending(lst):
        return [ln for ln, regs in lst if regs]

    for i, (n, op, rest, asm) in enumerate(items):
        if op == "label":
            incoming = pending.pop(rest, []) + ([list(inflight)] if reachable else [])
            if rest in back_targets:
                for lst in incoming:
                    if asm_pending(lst):
                        problems.append(f"{name}: LDS read(s) at {asm_pending(lst)[:3]} in flight into loop head {rest}")
                inflight = []
            elif incoming and all(lst == incoming[0] for lst in incoming):
                inflight = list(incoming[0])
            else:
                for lst in incoming:
                    if asm_pending(lst):
                        problems.append(f"{name}: LDS read(s) at {asm_pending(lst)[:3]} in flight into {rest}, "
                                        "whose incoming paths disagree")
                inflight = []
            reachable = True
            continue
        if not reachable:
            continue
        if op.startswith("s_waitcnt"):
            m = LGKM.search(rest)
            if m:
                keep = int(m.group(1))
                del inflight[:max(0, len(inflight) - keep)]
            continue
        if BRANCH.match(op):
            target = rest.split()[0]
            if target in label_pos and label_pos[target] > i:
                pending.setdefault(target, []).append(list(inflight))
            elif asm_pending(inflight):
                problems.append(f"{name}: LDS read(s) at {asm_pending(inflight)[:3]} in flight at the back edge "
                                f"{op} {target} (line {n})")
            if op == "s_branch":
                reachable = False
                inflight = []
            continue
        if op in ENDS:
            if asm_pending(inflight):
                problems.append(f"{name}: LDS read(s) at {asm_pending(inflight)[:3]} in flight at {op} (line {n})")
            reachable = False
            inflight = []
            continue
        used = regs_of(rest)
        busy = set()
        for _, regs in inflight:
            busy |= regs
        clash = used & busy
        if clash:
            problems.append(f"{name}: line {n} `{op} {rest}` touches {sorted(clash)[:4]} of an LDS read in flight")
        if op.startswith("ds_"):
            # a read's destination is its first operand; writes and atomics
            # without a return value have none (the compiler's own reads are
            # counted, for the order, but it tracks their registers itself)
            is_read = op.startswith(("ds_read", "ds_load")) or "_rtn" in op
            inflight.append((n, regs_of(rest.split(",")[0]) if is_read and asm else set()))
    if asm_pending(inflight) and reachable:
        problems.append(f"{name}: LDS read(s) at {asm_pending(inflight)[:3]} in flight at the end of the kernel")
    return problems


def kernels_of(asm):
    """(name, [(line number, text)]) for every kernel in an assembly listing."""
    funcs, cur, body = [], None, []
    for n, line in enumerate(asm.splitlines(), 1):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur and line.startswith(".Lfunc_end"):
            funcs.append((cur, body))
            cur = None
            continue
        if cur:
            body.append((n, line))
    return funcs


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    cc = build.hipcc()
    if not cc or not shutil.which(cc) and not os.path.exists(cc):
        pytest.skip("hipcc is not available")
    out = tmp_path_factory.mktemp("isa")
    res = {}
    for src in KERNEL_SOURCES:
        path = out / (src + ".s")
        cmd = [cc, *build.HIP_FLAGS, "--cuda-device-only", "-S", "-I", build.INCLUDE, "-I", CSRC,
               os.path.join(CSRC, src), "-o", str(path)]
        subprocess.run(cmd, check=True, capture_output=True)
        res[src] = path.read_text()
    return res


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_register_touches_an_lds_read_in_flight(listings, src):
    funcs = kernels_of(listings[src])
    assert funcs, f"no kernels found in {src}"
    problems = []
    for name, lines in funcs:
        problems += check_function(name, lines)
    assert not problems, "\n".join(problems[:20])


def test_the_checker_finds_planted_hazards():
    """Listings with a use before the wait, a wait that retires too little and
    a read left in flight across a branch are all flagged; the right order
    is not."""
    good = [(1, "ds_read_b128 v[4:7], v1 offset:16"), (2, "ds_read_b128 v[8:11], v1"),
            (3, "s_waitcnt lgkmcnt(1)"), (4, "v_mov_b32_e32 v20, v4"),
            (5, "s_waitcnt lgkmcnt(0)"), (6, "v_mov_b32_e32 v21, v8"), (7, "s_endpgm")]
    good = asm_marked([(n, t, t.startswith("ds_")) for n, t in good])
    assert check_function("good", good) == []
    early = [(1, "ds_read_b128 v[4:7], v1"), (2, "v_add_f32_e32 v5, v5, v5"), (3, "s_waitcnt lgkmcnt(0)")]
    assert check_function("early", asm_marked([(n, t, t.startswith("ds_")) for n, t in early]))
    short = [(1, "ds_read_b128 v[4:7], v1"), (2, "ds_read_b128 v[8:11], v1"),
             (3, "s_waitcnt lgkmcnt(1)"), (4, "v_mov_b32_e32 v20, v8")]
    assert check_function("short", asm_marked([(n, t, t.startswith("ds_")) for n, t in short]))
    across = [(0, ".LBB0_2:"), (1, "ds_read_b64_tr_b16 v[2:3], v1"), (2, "s_cbranch_scc1 .LBB0_2"),
              (3, "s_waitcnt lgkmcnt(0)"), (4, "s_endpgm")]
    assert check_function("across", asm_marked([(n, t, t.startswith("ds_")) for n, t in across]))
    clobber = [(1, "ds_read_b64_tr_b16 v[2:3], v1"), (2, "v_mov_b32_e32 v3, 0"), (3, "s_waitcnt lgkmcnt(0)")]
    assert check_function("clobber", asm_marked([(n, t, t.startswith("ds_")) for n, t in clobber]))
    mfma = [(1, "ds_read_b128 v[4:7], v1"),
            (2, "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"), (3, "s_waitcnt lgkmcnt(0)")]
    assert check_function("mfma", asm_marked([(n, t, t.startswith("ds_")) for n, t in mfma]))
    # a compiler read counts for the order: the asm read behind it is only
    # retired when both are
    order = [(1, "ds_read_b32 v30, v1", False), (2, "ds_read_b128 v[4:7], v1", True),
             (3, "s_waitcnt lgkmcnt(1)"), (4, "v_mov_b32_e32 v20, v4")]
    assert check_function("order", asm_marked(order))
    order_ok = [(1, "ds_read_b32 v30, v1", False), (2, "ds_read_b128 v[4:7], v1", True),
                (3, "s_waitcnt lgkmcnt(0)"), (4, "v_mov_b32_e32 v20, v4"), (5, "s_endpgm")]
    assert check_function("order_ok", asm_marked(order_ok)) == []
    # a read in flight over a skip branch: fine while nothing on either path
    # touches it, flagged when the skipped block does, or when the paths
    # reach the join with different reads in flight
    skip = [(1, "ds_read_b128 v[4:7], v1", True), (2, "s_cbranch_execz .LBB0_9"), (3, "v_mov_b32_e32 v20, v2"),
            (4, ".LBB0_9:"), (5, "s_waitcnt lgkmcnt(0)"), (6, "v_mov_b32_e32 v21, v4"), (7, "s_endpgm")]
    assert check_function("skip", asm_marked(skip)) == []
    skip_bad = [(1, "ds_read_b128 v[4:7], v1", True), (2, "s_cbranch_execz .LBB0_9"), (3, "v_mov_b32_e32 v5, v2"),
                (4, ".LBB0_9:"), (5, "s_waitcnt lgkmcnt(0)"), (6, "s_endpgm")]
    assert check_function("skip_bad", asm_marked(skip_bad))
    split = [(1, "ds_read_b128 v[4:7], v1", True), (2, "s_cbranch_execz .LBB0_9"), (3, "s_waitcnt lgkmcnt(0)"),
             (4, ".LBB0_9:"), (5, "v_mov_b32_e32 v21, v4"), (6, "s_endpgm")]
    assert check_function("split", asm_marked(split))


def asm_marked(items):
    """A listing in which entries flagged True are inline-asm statements."""
    out = []
    for it in items:
        if len(it) == 3 and it[2]:
            out += [(it[0], ";;#ASMSTART"), (it[0], it[1]), (it[0], ";;#ASMEND")]
        else:
            out.append((it[0], it[1]))
    return out


KINFO = re.compile(r"^\s*\.set\s+(_Z\w+)\.private_seg_size,\s*(\d+)")


def scratch_of(asm):
    """kernel -> bytes of scratch per lane, from the listing's kernel info."""
    out, cur = {}, None
    for line in asm.splitlines():
        m = KINFO.match(line)
        if m:
            cur = m.group(1)
            out[cur] = int(m.group(2))
            continue
        if cur and line.startswith("; ScratchSize:"):
            out[cur] = max(out[cur], int(line.split(":")[1]))
            cur = None
    return out


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_kernel_spills_to_scratch(listings, src):
    """Every kernel, the fp32 correctness kernels included, fits its
    registers at the occupancy its launch bounds ask for: a spill would show
    as scratch and turn the hot loops' register traffic into memory
    traffic."""
    scratch = scratch_of(listings[src])
    assert scratch, f"no kernel info in {src}"
    spilled = {k: v for k, v in scratch.items() if v}
    assert not spilled, f"{src}: scratch bytes per lane {spilled}"
