"""The C ABI's host-side validation and workspace layout (csrc/ra_host.h),
built with g++ under the address and undefined-behaviour sanitizers and
driven with the invalid-argument table of the ABI tests plus a seeded fuzz
of shapes, strides and pointers.

The driver reads one call per line and prints the status (or workspace
size) the library's entry point would return; it also checks the workspace
layouts it computes (aligned, disjoint, inside the total). Every answer is
compared with libra.so's own answer to the same call wherever that call is
rejected before anything is enqueued (the only calls that may run without a
GPU), and with the workspace size libra.so reports for every problem. Any
sanitizer report aborts the driver and fails the test.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import exact_blockwise_attention_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_blockwise_attention_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

DRIVER = r"""
#include <cstdio>
#include <cstring>
#include <string>
#include "ra_host.h"
using namespace ra::host;

static void* P(long long x) { return reinterpret_cast<void*>(static_cast<uintptr_t>(x)); }

// a sequence read as 5 numbers; ptr -1: the ra_seq pointer itself is NULL
static const ra_seq* read_seq(ra_seq* s) {
  long long p, a, b, c, d;
  if (scanf("%lld %lld %lld %lld %lld", &p, &a, &b, &c, &d) != 5) return nullptr;
  if (p == -1) return nullptr;
  s->ptr = P(p); s->s_blk = a; s->s_batch = b; s->s_tok = c; s->s_head = d;
  return s;
}

static bool inside(size_t off, size_t len, size_t total) { return off % kAlign == 0 && off + len <= total; }

int main() {
  char op[16];
  ra_problem pb{};
  bool have_pb = false;
  while (scanf("%15s", op) == 1) {
    std::string o(op);
    if (o == "P") {
      long long bl;
      int isnull;
      if (scanf("%d %d %d %d %d %lld %d %d %f %d %d", &isnull, &pb.batch, &pb.heads, &pb.head_dim, &pb.ring_size,
                &bl, &pb.layout, &pb.causal, &pb.scale, &pb.dtype, &pb.kv_heads) != 11) return 3;
      pb.block_len = bl;
      have_pb = !isnull;
    } else if (o == "WS") {
      int rb, re, cp, bw;
      if (scanf("%d %d %d %d", &rb, &re, &cp, &bw) != 4) return 3;
      size_t bytes = 0;
      if (have_pb && check_problem(&pb, rb, re) == RA_OK) {
        const int n = re - rb;
        if (bw) {
          const BwdWs w = bwd_ws_layout(&pb, n);
          const size_t rows = (size_t)n * pb.batch * pb.heads * pb.block_len;
          if (!inside(w.dsum, rows * 4, w.lse2) || !inside(w.lse2, rows * 4, w.small_total)) printf("BAD bwd layout\n");
          if (w.total > w.small_total) {
            const size_t kt = (size_t)((pb.block_len + 127) / 128);
            const size_t kop = (size_t)pb.batch * kv_heads_of(&pb) * pb.ring_size * kt * 128 * pb.head_dim * 2;
            const size_t ds = (size_t)n * pb.batch * pb.heads * pb.ring_size * (size_t)w.ds_stride * 64 * 128 * 2;
            if (!inside(w.kop, kop, w.ds) || !inside(w.ds, ds, w.total) || w.kop < w.small_total || w.ds_stride < 1)
              printf("BAD stored-dS layout\n");
          }
          bytes = bw == 2 ? w.small_total : w.total;
        } else {
          const FwdWs w = fwd_ws_layout(&pb, n, cp);
          if (cp) {
            const size_t blk = (size_t)pb.batch * pb.block_len * kv_heads_of(&pb) * pb.head_dim * elem_bytes(pb.dtype);
            const size_t rows = (size_t)n * pb.batch * pb.heads * pb.block_len;
            if (!inside(w.kbuf[0], blk, w.vbuf[0]) || !inside(w.vbuf[0], blk, w.kbuf[1]) ||
                !inside(w.kbuf[1], blk, w.vbuf[1]) || !inside(w.vbuf[1], blk, w.st_o) ||
                !inside(w.st_o, rows * pb.head_dim * 4, w.st_lse) || !inside(w.st_lse, rows * 4, w.total))
              printf("BAD copy layout\n");
          } else if (w.n_split > 1) {
            const size_t rows = (size_t)w.n_split * n * pb.batch * pb.heads * pb.block_len;
            if (w.n_split > pb.ring_size || !inside(w.st_o, rows * pb.head_dim * 4, w.st_lse) ||
                !inside(w.st_lse, rows * 4, w.total))
              printf("BAD split layout\n");
          } else if (w.total != 0) {
            printf("BAD unsplit workspace\n");
          }
          bytes = w.total;
        }
      }
      printf("%zu\n", bytes);
    } else if (o == "FWD") {
      int rb, re, cp;
      ra_seq s[4];
      const ra_seq* sp[4];
      long long lse, ws, wsb;
      if (scanf("%d %d", &rb, &re) != 2) return 3;
      for (int i = 0; i < 4; ++i) sp[i] = read_seq(&s[i]);
      if (scanf("%lld %lld %lld %d", &lse, &ws, &wsb, &cp) != 4) return 3;
      const FwdPlan pl = plan_forward(have_pb ? &pb : nullptr, rb, re, sp[0], sp[1], sp[2], sp[3],
                                      static_cast<const float*>(P(lse)), P(ws), (size_t)wsb, cp != 0);
      printf("%d\n", (int)pl.st);
    } else if (o == "BWD") {
      int rb, re;
      ra_seq s[8];
      const ra_seq* sp[8];
      long long lse, ws, wsb;
      if (scanf("%d %d", &rb, &re) != 2) return 3;
      for (int i = 0; i < 8; ++i) sp[i] = read_seq(&s[i]);
      if (scanf("%lld %lld %lld", &lse, &ws, &wsb) != 3) return 3;
      const BwdPlan pl = plan_backward(have_pb ? &pb : nullptr, rb, re, sp[0], sp[1], sp[2], sp[3], sp[4],
                                       static_cast<const float*>(P(lse)), sp[5], sp[6], sp[7], P(ws), (size_t)wsb);
      printf("%d\n", (int)pl.st);
    } else if (o == "MRG") {
      long long rows, p[6];
      int hd;
      if (scanf("%lld %d %lld %lld %lld %lld %lld %lld", &rows, &hd, &p[0], &p[1], &p[2], &p[3], &p[4], &p[5]) != 8)
        return 3;
      const float* f[6];
      for (int i = 0; i < 6; ++i) f[i] = static_cast<const float*>(P(p[i]));
      printf("%d\n", (int)check_merge(rows, hd, f[0], f[1], f[2], f[3], f[4], f[5]));
    } else if (o == "LC") {
      long long src, dst;
      if (scanf("%lld %lld", &src, &dst) != 2) return 3;
      printf("%d\n", (int)check_layout_copy(have_pb ? &pb : nullptr, P(src), P(dst)));
    } else {
      return 4;
    }
    fflush(stdout);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("g++ or the HIP headers are missing")
    d = tmp_path_factory.mktemp("host_sanitized")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    exe = d / "driver"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", CSRC, "-I", "/opt/rocm/include",
           str(src), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in (r.stderr + r.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return str(exe)


def run_driver(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"driver failed ({r.returncode}):\n{r.stderr[-3000:]}"
    out = r.stdout.split()
    assert "BAD" not in out, r.stdout
    return [int(x) for x in out]


def pb_line(pb):
    if pb is None:
        return "P 1 1 1 64 1 64 0 0 0 0 0"
    return (f"P 0 {pb.batch} {pb.heads} {pb.head_dim} {pb.ring_size} {pb.block_len} {pb.layout} {pb.causal} "
            f"{float(pb.scale)!r} {pb.dtype} {pb.kv_heads}")


def seq_fields(s):
    return "-1 0 0 0 0" if s is None else f"{s.ptr or 0} {s.s_blk} {s.s_batch} {s.s_tok} {s.s_head}"


def problem(**kw):
    base = dict(B=1, H=2, d=64, P=4, Bb=64, layout="striped", causal=True, dtype_code=ra.BF16, kv_heads=0)
    base.update(kw)
    return ra.make_problem(base["B"], base["H"], base["d"], base["P"], base["Bb"], base["layout"],
                           base["causal"], base["dtype_code"], kv_heads=base["kv_heads"])


def fake_seq(ptr=0x10000, s_blk=128, s_batch=1 << 20, s_tok=512, s_head=64):
    return ra.Seq(ptr, s_blk, s_batch, s_tok, s_head)


class Calls:
    """Calls for both the sanitized driver and libra.so."""

    def __init__(self):
        self.lines, self.lib_calls = [], []

    def fwd(self, pb, rb, re_, seqs, lse=0x20000, ws=0, ws_bytes=0, copy=False):
        self.lines.append(pb_line(pb))
        self.lines.append(f"FWD {rb} {re_} " + " ".join(seq_fields(s) for s in seqs) + f" {lse} {ws} {ws_bytes} "
                          f"{int(copy)}")
        lib = ra.library()
        self.lib_calls.append(lambda: lib.ra_forward(
            None if pb is None else ctypes.byref(pb), rb, re_, *[ra._ref(s) for s in seqs], lse or None,
            ws or None, ws_bytes, None, ctypes.c_void_p(0x1234) if copy else None))

    def bwd(self, pb, rb, re_, seqs, lse=0x20000, ws=0, ws_bytes=0):
        self.lines.append(pb_line(pb))
        self.lines.append(f"BWD {rb} {re_} " + " ".join(seq_fields(s) for s in seqs) + f" {lse} {ws} {ws_bytes}")
        lib = ra.library()
        self.lib_calls.append(lambda: lib.ra_backward(
            None if pb is None else ctypes.byref(pb), rb, re_, *[ra._ref(s) for s in seqs[:5]], lse or None,
            *[ra._ref(s) for s in seqs[5:]], ws or None, ws_bytes, None))

    def ws(self, pb, rb, re_, copy, bwd):
        self.lines.append(pb_line(pb))
        self.lines.append(f"WS {rb} {re_} {int(copy)} {int(bwd)}")
        self.lib_calls.append(lambda: ra.library().ra_workspace_bytes(
            None if pb is None else ctypes.byref(pb), rb, re_, int(copy), int(bwd)))

    def merge(self, rows, hd, ptrs):
        self.lines.append(f"MRG {rows} {hd} " + " ".join(str(p) for p in ptrs))
        self.lib_calls.append(lambda: ra.library().ra_merge_lse(rows, hd, *[p or None for p in ptrs], None))

    def layout_copy(self, pb, src, dst):
        self.lines.append(pb_line(pb))
        self.lines.append(f"LC {src} {dst}")
        self.lib_calls.append(lambda: ra.library().ra_layout_copy(
            None if pb is None else ctypes.byref(pb), src or None, dst or None, 0, None))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ra.library_path):
        pytest.skip("libra.so not built")
    return ra.library()


def test_invalid_argument_table(driver, lib):
    """The ABI tests' table of invalid arguments gives the same status from
    the sanitized host checks and from libra.so."""
    c, exp = Calls(), []
    s4 = lambda: [fake_seq() for _ in range(4)]  # noqa: E731
    for field, value, code in [("batch", 0, 2), ("heads", 0, 2), ("ring_size", 0, 2), ("block_len", 0, 2),
                               ("layout", 3, 2), ("causal", 3, 2), ("dtype", 7, 2), ("head_dim", 96, 3),
                               ("head_dim", 32, 3), ("kv_heads", 3, 2), ("kv_heads", -1, 2)]:
        pb = problem()
        setattr(pb, field, value)
        c.fwd(pb, 0, pb.ring_size if pb.ring_size > 0 else 1, s4())
        exp.append(code)
    pb = problem()
    pb.scale = float("nan")
    c.fwd(pb, 0, 4, s4())
    exp.append(2)
    for rb, re_ in ((-1, 2), (2, 2), (0, 5)):
        c.fwd(problem(), rb, re_, s4())
        exp.append(2)
    c.fwd(None, 0, 1, s4())
    exp.append(1)
    for idx, kw, code in ((2, None, 1), (0, dict(ptr=0), 1), (1, dict(ptr=0x10008), 5), (3, dict(s_tok=513), 5),
                          (0, dict(s_head=-64), 2), (1, dict(s_tok=(1 << 25) + 8), 3),
                          (2, dict(s_tok=(1 << 25) + 8), 3), (1, dict(s_tok=1 << 62), 2)):
        seqs = s4()
        seqs[idx] = None if kw is None else fake_seq(**kw)
        c.fwd(problem(), 0, 4, seqs)
        exp.append(code)
    c.fwd(problem(), 0, 4, s4(), lse=0)
    exp.append(1)
    c.fwd(problem(), 0, 4, s4(), lse=0x20002)
    exp.append(5)
    need = ra.workspace_bytes(problem(), 1, 2, True, False)
    for rb, re_, ws, nb, code in ((0, 2, 0, 0, 2), (1, 2, 0, 0, 4), (1, 2, 0x100000, need - 1, 4),
                                  (1, 2, 0x100010, need, 5)):
        c.fwd(problem(), rb, re_, s4(), ws=ws, ws_bytes=nb, copy=True)
        exp.append(code)
    pb3 = problem(d=64, P=3, Bb=300, H=2)
    c.fwd(pb3, 2, 3, s4(), ws=0x40010, ws_bytes=ra.workspace_bytes(pb3, 2, 3, False, False))
    exp.append(5)
    c.fwd(problem(layout="zigzag", Bb=63), 0, 4, s4())
    exp.append(2)
    s8 = lambda: [fake_seq() for _ in range(8)]  # noqa: E731
    bneed = ra.workspace_bytes(problem(), 0, 4, False, 2)
    c.bwd(problem(), 0, 4, s8())
    exp.append(4)
    c.bwd(problem(), 0, 4, s8(), ws=0x100000, ws_bytes=bneed - 4)
    exp.append(4)
    c.bwd(problem(), 0, 4, s8(), lse=0, ws=0x100000, ws_bytes=bneed)
    exp.append(1)
    c.bwd(problem(), 0, 4, s8(), ws=0x100040, ws_bytes=bneed)
    exp.append(5)
    seqs = s8()
    seqs[6] = None
    c.bwd(problem(), 0, 4, seqs, ws=0x100000, ws_bytes=bneed)
    exp.append(1)
    for idx in (0, 4):
        seqs = s8()
        seqs[idx] = fake_seq(s_tok=1 << 24)
        c.bwd(problem(), 0, 4, seqs)
        exp.append(3)
    seqs = s8()
    seqs[0] = fake_seq(s_tok=(1 << 24) - 8)
    c.bwd(problem(), 0, 4, seqs)
    exp.append(4)
    p = 0x10000
    for args, code in (((4, 64, [0, p, p, p, p, p]), 1), ((-1, 64, [p] * 6), 2), ((4, 0, [p] * 6), 2),
                       ((4, 2048, [p] * 6), 2), ((4, 64, [p + 8, p, p, p, p, p]), 5),
                       ((4, 64, [p, p + 2, p, p, p, p]), 5), ((1 << 40, 64, [p] * 6), 2)):
        c.merge(*args)
        exp.append(code)
    for src, dst, code in ((0, p, 1), (p + 4, p, 5)):
        c.layout_copy(problem(), src, dst)
        exp.append(code)
    c.layout_copy(None, p, p)
    exp.append(1)
    got = run_driver(driver, c.lines)
    assert got == exp
    for line_idx, (g, call) in enumerate(zip(got, c.lib_calls)):
        assert int(call()) == g, (line_idx, g)


def random_problem(rng):
    pick = lambda choices: choices[rng.integers(len(choices))]  # noqa: E731
    pb = ra.Problem()
    pb.batch = int(pick([1, 1, 2, 3, 0, -1, 1 << 30, 2 ** 31 - 1]))
    pb.heads = int(pick([1, 2, 8, 32, 0, -5, 1 << 20, 2 ** 31 - 1]))
    pb.head_dim = int(pick([64, 128, 128, 32, 96, 0, -64]))
    pb.ring_size = int(pick([1, 2, 4, 8, 16, 256, 0, -1, 2 ** 31 - 1]))
    pb.block_len = int(pick([1, 63, 64, 4096, 32768, 0, -4, (2 ** 31 - 1) // 2, 2 ** 30 + 1, 2 ** 62]))
    pb.layout = int(pick([0, 1, 2, 2, 3, -1]))
    pb.causal = int(pick([0, 1, 1, 2]))
    pb.scale = float(pick([0.0, 0.0, 0.125, -1.0, float("inf"), float("nan"), 1e30]))
    pb.dtype = int(pick([0, 1, 1, 5]))
    pb.kv_heads = int(pick([0, 0, 1, 2, 3, 8, -1, 2 ** 31 - 1]))
    return pb


def random_seq(rng):
    r = rng.integers(10)
    if r == 0:
        return None
    pick = lambda choices: int(choices[rng.integers(len(choices))])  # noqa: E731
    ptr = pick([0x10000, 0x10000, 0x10008, 0, 0x7fff0000])
    strides = [pick([0, 64, 128, 512, 4096, 1 << 20, 1 << 24, (1 << 25) + 8, 513, -64, 1 << 62, 2 ** 63 - 1])
               for _ in range(4)]
    return ra.Seq(ptr, *strides)


def test_seeded_fuzz(driver, lib):
    """Random problems, rank ranges, strides, pointers and workspaces, edge
    values included (zero, negative, 2^31 - 1, 2^62): no sanitizer report,
    consistent workspace layouts, and the same answers as libra.so."""
    rng = np.random.default_rng(20260)
    c = Calls()
    for _ in range(3000):
        pb = random_problem(rng) if rng.integers(20) else None
        P = pb.ring_size if pb is not None else 4
        rb = int(rng.integers(-1, max(2, min(P, 10) + 1)))
        re_ = int(rb + rng.integers(0, 4)) if rng.integers(4) else int(P)
        kind = rng.integers(5)
        if kind == 0:
            c.ws(pb, rb, re_, bool(rng.integers(2)), int(rng.integers(3)))
        elif kind in (1, 2):
            seqs = [random_seq(rng) for _ in range(4)]
            ws = int([0, 0x100000, 0x100010][rng.integers(3)])
            c.fwd(pb, rb, re_, seqs, lse=int([0x20000, 0x20002, 0][rng.integers(3)]), ws=ws,
                  ws_bytes=int(rng.integers(0, 1 << 40)) if ws else 0, copy=bool(rng.integers(2)))
        elif kind == 3:
            seqs = [random_seq(rng) for _ in range(8)]
            ws = int([0, 0x100000, 0x100010][rng.integers(3)])
            c.bwd(pb, rb, re_, seqs, ws=ws, ws_bytes=int(rng.integers(0, 1 << 40)) if ws else 0)
        else:
            rows = int([0, 1, 1000, -1, 1 << 40][rng.integers(5)])
            c.merge(rows, int([1, 37, 64, 128, 1024, 1025, 0][rng.integers(7)]),
                    [int([0x10000, 0x10004, 0][rng.integers(3)]) for _ in range(6)])
    got = run_driver(driver, c.lines)
    assert len(got) == len(c.lib_calls)
    compared = 0
    merge_or_ws = [ln.split()[0] for ln in c.lines if ln.split()[0] != "P"]
    for kind, g, call in zip(merge_or_ws, got, c.lib_calls):
        if kind == "WS" or g != 0:  # rejected calls enqueue nothing: safe to make without a GPU
            assert int(call()) == g, (kind, g)
            compared += 1
    assert compared > 1500
