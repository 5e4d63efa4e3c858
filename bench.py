"""Benchmark: causal striped blockwise ring attention, forward + backward, d=128.

Default workload (one GPU): B=1, H=32, L=32768, d=128, bf16, ring of P=8
blocks of 4096 tokens, causal, striped layout. One step = the forward over
all 8 ranks (every KV block visited in ring order, O and lse out) followed by
the backward (D = rowsum(dO*O), the ring walk recomputing P from lse with
dV/dP/dS/dQ/dK, dQ cast). Inputs are seeded synthetic N(0,1) tensors already
resident in HBM. Throughput is algorithmic: 4*d flop per visible
(query, key) pair forward and 10*d backward (masked pairs not counted).

Prints one JSON line. --workload picks one of the other workloads (for
profiling); the default is the forward+backward one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["exact_blockwise_attention_amd/csrc/" + f for f in
                  ("ra_fwd.hip", "ra_bwd.hip", "ra_dq.hip", "ra_dqds.hip", "ra_misc.hip", "ra_gemm.hip", "ra_api.cpp",
                   "ra_schedule.h", "ra_internal.h", "ra_lds.h", "ra_kvwalk.h", "ra_host.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5, 6, 7],
                    help="7: the Blockwise Parallel Transformer layer tail (W_o, LN, FFN, LN) at d_model 4096")
    ap.add_argument("--layout", default=None, help="workloads 3, 5 and 6: contiguous, striped or zigzag")
    ap.add_argument("--memory", default="original", choices=["blocked", "original"],
                    help="blocked: Q/K/V/dO resident as [P, B, Bb, H, d], each rank's block contiguous as a "
                         "device holds it (prepared before the timed region); original: [B, L, H, d] in token "
                         "order, the blocks read through strides")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-recompute", action="store_true",
                    help="give the backward its minimum workspace, so that the query-side walk recomputes S and dP "
                         "for dQ instead of reading the dS tiles the key-side walk stores")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (the library's layout copy with one block) three "
                         "times, as the reference for HBM byte counters")
    return ap.parse_args()


def calibrate_copy():
    """Copy 1 GiB once per launch with ra_layout_copy (P = 1: blocked order is
    the original order, so it is a plain copy): reads and writes 2**30 bytes."""
    import torch

    import exact_blockwise_attention_amd as ra
    B, L, H, d = 1, 131072, 32, 128  # bf16: 2**30 bytes
    x = torch.empty((B, L, H, d), dtype=torch.bfloat16, device="cuda").fill_(1.0)
    y = torch.empty((1, B, L, H, d), dtype=torch.bfloat16, device="cuda")
    pb = ra.make_problem(B, H, d, 1, L, "contiguous", True, ra.BF16)
    torch.cuda.synchronize()
    for _ in range(3):
        ra.layout_copy_raw(pb, x.data_ptr(), y.data_ptr(), False, ra._stream_handle(None))
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": 2 ** 30, "calibrate_copy_bytes_written": 2 ** 30,
                      "launches": 3}), flush=True)


def pair_count(layout, causal, P, Bb, ranks):
    """Visible (query, key) pairs of the given ranks' query blocks, per head:
    a striped block pair (i, j) sees b <= a - [j > i], a contiguous one all
    (j < i), the lower triangle (j == i) or nothing (j > i); a zigzag one the
    lower triangle (j == i) or Bb * Bb/2 pairs (j < i: every row sees the
    first half-block; j > i: the second half of the rows sees every key)."""
    total = 0
    for i in ranks:
        for kstep in range(P):
            j = (i - kstep) % P
            if not causal:
                total += Bb * Bb
            elif layout == "striped":
                total += Bb * (Bb + 1) // 2 if j <= i else Bb * (Bb - 1) // 2
            elif layout == "zigzag":
                total += Bb * (Bb + 1) // 2 if j == i else Bb * (Bb // 2)
            elif j < i:
                total += Bb * Bb
            elif j == i:
                total += Bb * (Bb + 1) // 2
    return total


def key_extent(layout, causal, i, j, Bb, a):
    """Keys 0 .. e-1 of block j that local row a of block i sees (the same
    relations as pair_count)."""
    if not causal:
        return Bb
    if layout == "striped":
        return max(0, min(Bb, a + 1 - (1 if j > i else 0)))
    if layout == "zigzag":
        h = Bb // 2
        return a + 1 if j == i else (h if j < i else (Bb if a >= h else 0))
    return Bb if j < i else (a + 1 if j == i else 0)


def stored_ds_tiles(layout, causal, P, Bb, ranks):
    """dS tiles (64 query rows x 128 keys, bf16) the backward stores and
    reads back, per (batch, head): for each query tile of each rank and each
    block, the 128-key tiles its last row sees."""
    total = 0
    for i in ranks:
        for j in range(P):
            for qt in range(-(-Bb // 64)):
                a_last = min(64 * qt + 63, Bb - 1)
                total += -(-key_extent(layout, causal, i, j, Bb, a_last) // 128)
    return total


def rank_work(layout, causal, P, Bb, i, rows_per_wg=256, keys_per_tile=64):
    """Per head: the KV tiles the forward executes for rank i (each
    256-row query tile walks, in each block, the tiles up to the last key its
    last row sees) and the KV blocks it visits (blocks with a visible key)."""
    tiles = 0
    for a0 in range(0, Bb, rows_per_wg):
        a_hi = min(a0 + rows_per_wg, Bb) - 1
        for j in range(P):
            tiles += -(-key_extent(layout, causal, i, j, Bb, a_hi) // keys_per_tile)
    blocks = sum(1 for j in range(P) if key_extent(layout, causal, i, j, Bb, Bb - 1) > 0)
    return tiles, blocks


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def workload_name(w, layout):
    """The workload's name with the layout actually run in it."""
    for other in ("contiguous", "striped", "zigzag"):
        if f"_{other}_" in w.name:
            return w.name.replace(f"_{other}_", f"_{layout}_")
    return w.name.replace("causal_", f"causal_{layout}_", 1) if w.causal else w.name


def hbm_row(ms, nbytes):
    """An HBM-bound launch: algorithmic bytes over its time, against 8 TB/s."""
    gbs = nbytes / ms / 1e6
    return {"ms": round(ms, 4), "bytes": int(nbytes), "GB/s": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def time_calls(torch, stream, fn, n=5, head_start=False):
    """Average ms of n back-to-back calls, HIP events on the launch stream
    (after one untimed call). With head_start the stream first runs a short
    device-side delay, so the calls are all queued before the first starts."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if head_start:
        with torch.cuda.stream(stream):
            torch.cuda._sleep(50_000_000)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def small_block_sweep(torch, ra, w, sh, stream):
    """One rank's share on the non-causal 16384-token shape (8 heads of 128)
    with query blocks of 64, 128 and 256 rows: the rank visits all L / rows
    ring blocks, so every K/V byte is used by only `rows` query rows (about
    `rows` flops per byte, below the MFMA/HBM ridge of 2500 / 8 = 312) and the
    share is bound by reading K and V from HBM. Algorithmic bytes: K and V of
    the whole sequence, the rank's Q and O rows, and its lse. The library
    splits the ring steps of such a share into parallel runs merged by
    log-sum-exp; the unsplit launch (one workgroup per head) is timed beside
    it. Each rate is the average of back-to-back calls queued behind a
    device-side delay, so the host's launch rate does not enter it. Those
    calls run warm: K and V (64 MiB) stay in the 256 MB last-level cache
    (MALL) between calls. `split_cold` is the median of single calls each
    preceded by a 512 MiB write that evicts them."""
    B, L, H, d = 1, w.seq_len, w.heads, w.head_dim
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1000 + w.wid)
    q, k, v = (torch.randn((B, L, H, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    out = {}
    for rows in (64, 128, 256):
        P = L // rows
        pb = ra.make_problem(B, H, d, P, rows, "contiguous", False, ra.BF16)
        need = ra.workspace_bytes(pb, 0, 1, False, False)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        o = torch.empty((B, rows, H, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((1, B, H, rows), dtype=torch.float32, device="cuda")
        qs = ra.Seq(q.data_ptr(), rows * H * d, L * H * d, H * d, d)
        os_ = ra.Seq(o.data_ptr(), rows * H * d, rows * H * d, H * d, d)
        ks = ra.Seq(k.data_ptr(), rows * H * d, L * H * d, H * d, d)
        vs = ra.Seq(v.data_ptr(), rows * H * d, L * H * d, H * d, d)
        nbytes = 2 * L * H * d * 2 + 2 * rows * H * d * 2 + rows * H * 4
        row = {"ring_size": P}
        for label, wsp, wsb in (("split", ws.data_ptr(), need), ("unsplit", None, 0)):
            call = lambda: ra.forward_raw(pb, 0, 1, qs, ks, vs, os_, lse.data_ptr(), wsp, wsb, sh, None)  # noqa: E731
            ms = time_calls(torch, stream, call, n=50, head_start=True)
            row[label] = {**hbm_row(ms, nbytes), "TFLOP/s": round(4 * d * rows * L * H / ms / 1e9, 2)}
            if label == "split":
                ms = cold_call_ms(torch, stream, call, flush)
                row["split_cold"] = {**hbm_row(ms, nbytes), "TFLOP/s": round(4 * d * rows * L * H / ms / 1e9, 2)}
        row["split_workspace_bytes"] = need
        out[f"q_rows_{rows}"] = row
        del ws, o, lse
    del flush
    return out


def cold_call_ms(torch, stream, fn, flush, n=20):
    """Median ms of single calls, each after writing `flush` (larger than the
    last-level cache) on the same stream, HIP events around the call only."""
    fn()
    times = []
    for _ in range(n):
        flush.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return sorted(times)[n // 2]


def memory_rows(torch, ra, w, q, sh, stream):
    """The HBM-bound calls on the workload's shapes, timed outside the step:
    the log-sum-exp merge of two fp32 partial results for every query row
    (read 2(4d+4), write 4d+4 bytes per row) and the layout gather of Q
    (read and write every byte once)."""
    d = w.head_dim
    rows = w.batch * w.heads * w.seq_len
    g = torch.Generator(device="cuda").manual_seed(w.wid)
    oa = torch.randn((rows, d), generator=g, device="cuda")
    ob = torch.randn((rows, d), generator=g, device="cuda")
    la = torch.randn((rows,), generator=g, device="cuda")
    lb = torch.randn((rows,), generator=g, device="cuda")
    oo, lo = torch.empty_like(oa), torch.empty_like(la)
    merge_ms = time_calls(torch, stream, lambda: ra.merge_lse_raw(rows, d, oa.data_ptr(), la.data_ptr(), ob.data_ptr(),
                                                                  lb.data_ptr(), oo.data_ptr(), lo.data_ptr(), sh))
    del oa, ob, oo
    q = q.reshape(w.batch, w.seq_len, w.heads, d)  # blocked (zigzag) copies hold the same bytes
    B, L, H, _ = q.shape
    P = w.ring_size
    blk = torch.empty((P, B, L // P, H, d), dtype=q.dtype, device="cuda")
    pb = ra.make_problem(B, H, d, P, L // P, "striped", True, ra.BF16 if w.dtype == "bf16" else ra.F32)
    copy_ms = time_calls(torch, stream, lambda: ra.layout_copy_raw(pb, q.data_ptr(), blk.data_ptr(), False, sh))
    del blk
    return {"F7_merge_lse": hbm_row(merge_ms, rows * (3 * 4 * d + 3 * 4)),
            "F0_layout_copy_striped_q": hbm_row(copy_ms, 2 * q.numel() * q.element_size())}


def receive_overlap(torch, ra, w, t, pb, rb, re_, so, sk, o, lse, sh, stream, total_ms):
    """One device's share with the next KV block copied on a second stream:
    c = compute per ring step (the same rank's ring in one launch, KV read in
    place, divided by P), m = the copy per step (the library's striped gather
    of the whole K, then V, divided by P: per step one K and one V block, read
    and written once), and how close the overlapped call comes to P max(c, m)."""
    P = w.ring_size
    c_all = time_calls(torch, stream, lambda: ra.forward_raw(pb, rb, re_, so(t["q"]), sk(t["k"]), sk(t["v"]), so(o),
                                                            lse.data_ptr(), None, 0, sh, None), n=2)
    B, L, Hk, d = t["k"].shape
    blk = torch.empty((P, B, L // P, Hk, d), dtype=t["k"].dtype, device="cuda")
    pbk = ra.make_problem(B, Hk, d, P, L // P, "striped", True, ra.BF16)
    gk = time_calls(torch, stream, lambda: ra.layout_copy_raw(pbk, t["k"].data_ptr(), blk.data_ptr(), False, sh), n=2)
    gv = time_calls(torch, stream, lambda: ra.layout_copy_raw(pbk, t["v"].data_ptr(), blk.data_ptr(), False, sh), n=2)
    del blk
    c, m = c_all / P, (gk + gv) / P
    step_bytes = 2 * 2 * (t["k"].numel() // P) * t["k"].element_size()
    return {"c_ms": round(c, 4), "m_ms": round(m, 4), "m_GB/s": round(step_bytes / m / 1e6, 1),
            "overlapped_ms": round(total_ms, 4), "serial_bound_ms": round(P * (c + m), 4),
            "overlap_efficiency": round(P * max(c, m) / total_ms, 4)}


def balance_report(torch, ra, w, layout, t, pb, blocked, o, lse, sh, stream):
    """Each rank's forward launched alone (its query block against the whole
    ring): kernel time, exact unmasked pairs, executed KV tiles and KV blocks
    visited, and the max/min ratios. Every device of a ring waits for the
    slowest one at each step, so the largest rank sets the pace."""
    P, Bb = w.ring_size, w.block_len
    per = []
    for r in range(P):
        if blocked:
            q_s, o_s = ra.seq_blocked(t["q"], block_offset=r), ra.seq_blocked(o, block_offset=r)
            k_s, v_s = ra.seq_blocked(t["k"]), ra.seq_blocked(t["v"])
        else:
            q_s, o_s = (ra.seq_original(x, P, layout, block_offset=r) for x in (t["q"], o))
            k_s, v_s = (ra.seq_original(x, P, layout) for x in (t["k"], t["v"]))
        ms = time_calls(torch, stream, lambda: ra.forward_raw(pb, r, r + 1, q_s, k_s, v_s, o_s, lse[r].data_ptr(),
                                                             None, 0, sh, None), n=3)
        tiles, blocks = rank_work(layout, w.causal, P, Bb, r)
        bh = w.batch * w.heads
        per.append({"rank": r, "ms": round(ms, 4), "pairs": pair_count(layout, w.causal, P, Bb, [r]) * bh,
                    "kv_tiles": tiles * bh, "kv_blocks_visited": blocks})
    ratio = lambda key: round(max(x[key] for x in per) / max(1e-12, min(x[key] for x in per)), 4)  # noqa: E731
    return {"per_rank": per, "ms_max_over_min": ratio("ms"), "pairs_max_over_min": ratio("pairs"),
            "kv_tiles_max_over_min": ratio("kv_tiles"),
            "slowest_rank_ms_over_mean": round(max(x["ms"] for x in per) / (sum(x["ms"] for x in per) / P), 4)}


def cpu_baseline(w):
    """Oracle (float64 numpy) on a bounded sample of the workload."""
    import numpy as np
    import oracle
    from exact_blockwise_attention_amd import synthetic as syn
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    d = w.head_dim
    if "bwd" in w.passes:
        # of the full 32768-token sequence (the workload's own tensors),
        # forward + backward: heads 0 and H-1 (about 10 s on 16 host cores),
        # or with shared K/V heads the query heads of K/V head 0 (about 20 s)
        G = w.heads // (w.kv_heads or w.heads)
        heads = [0, w.heads - 1] if G == 1 else list(range(G))
        t = {}
        for n in ("q", "k", "v", "do"):
            pay = syn.make_payload(w.wid, n, syn.workload_shape(w, n), w.dtype)
            sel = [0] if (G > 1 and n in ("k", "v")) else heads
            t[n] = syn.to_f64(np.ascontiguousarray(pay[:, :, sel]))
            del pay
        L = w.seq_len
        t0 = time.perf_counter()
        dq_r, dk_r, dv_r, o_r, lse_r = oracle.attention_bwd(t["q"], t["k"], t["v"], t["do"], True)  # runs the forward inside
        dt = time.perf_counter() - t0
        ref = {"heads": heads, "kv_heads": [0] if G > 1 else heads,
               "O": o_r, "lse": lse_r, "dQ": dq_r, "dK": dk_r, "dV": dv_r}
        flops = len(heads) * L * (L + 1) // 2 * (4 + 10) * d
        which = f"heads 0 and {w.heads - 1} of {w.heads}" if G == 1 else \
            f"query heads 0..{G - 1} of {w.heads} (the ones sharing K/V head 0)"
        sample = f"{which}, all {L} tokens, forward+backward (causal, " \
                 "contiguous order: the oracle's mask is on token positions, so the layout does not change it)"
    else:
        Ls = 4096 if w.causal else 2048
        shape = (1, Ls, 1, d)
        t = {n: syn.to_f64(syn.make_payload(w.wid, n, shape, w.dtype)) for n in ("q", "k", "v")}
        t0 = time.perf_counter()
        oracle.attention_fwd(t["q"], t["k"], t["v"], w.causal)
        dt = time.perf_counter() - t0
        pairs = Ls * (Ls + 1) // 2 if w.causal else Ls * Ls
        flops = pairs * 4 * d
        sample = f"one head, first {Ls} tokens, forward"
        ref = None  # a stand-alone sample, not the workload's own tensors
    rec = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": sample, "seconds": round(dt, 3), "cpu_model": cpu_model()}
    return rec, ref


def cpu_model():
    """The host CPU's model name (as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


BAND = 4.0  # below it a bf16 output meets the plain bar; above it, plus its own rounding


def half_bf16_spacing(x):
    import numpy as np
    ax = np.abs(x)
    _, e = np.frexp(ax)
    return np.where(ax > 0, np.ldexp(1.0, e - 9), 0.0)


def parity_report(torch, ra, w, layout, blocked, outs, ref):
    """The timed run's last outputs against the oracle results the CPU
    baseline computed (same tensors, the oracle's head subset): max |GPU -
    oracle| per output, max |oracle|, and whether every element meets the
    bar (2e-2 for bf16 inputs: plainly below |ref| = 4, plus the output's
    own bf16 rounding at and above it; 1e-4 for fp32)."""
    import numpy as np
    P, Bb = w.ring_size, w.block_len
    tol = 2e-2 if w.dtype == "bf16" else 1e-4

    def original(x):  # a [B, L, H, d] device tensor in token order
        return ra.layout_copy(x, P, layout, inverse=True) if blocked else x

    def f64(x):
        return x.float().cpu().numpy().astype(np.float64)

    got = {}
    hq, hk = ref["heads"], ref["kv_heads"]
    for name, key, hs in (("O", "o", hq), ("dQ", "dq", hq), ("dK", "dk", hk), ("dV", "dv", hk)):
        got[name] = f64(original(outs[key])[:, :, hs])
    lse = outs["lse"].cpu().numpy().astype(np.float64)  # [P, B, H, Bb], local row order
    x = np.arange(Bb)
    if layout == "striped":
        pos = np.concatenate([x * P + i for i in range(P)])
    elif layout == "zigzag":
        h = Bb // 2
        pos = np.concatenate([np.where(x < h, i * h + x, (2 * P - 1 - i) * h + (x - h)) for i in range(P)])
    else:
        pos = np.concatenate([i * Bb + x for i in range(P)])
    flat = lse.transpose(1, 0, 3, 2).reshape(w.batch, P * Bb, w.heads)[:, :, hq]
    tok = np.empty_like(flat)
    tok[:, pos] = flat
    got["lse"] = tok
    err, val, ok = {}, {}, True
    for name in ("O", "lse", "dQ", "dK", "dV"):
        e = np.abs(got[name] - ref[name])
        r = np.abs(ref[name])
        err[name] = float(e.max())
        val[name] = float(r.max())
        if name == "lse" or w.dtype != "bf16":
            ok = ok and err[name] <= tol
        else:
            band = r >= BAND
            ok = ok and float(e[~band].max(initial=0.0)) <= tol
            if band.any():
                mag = np.maximum(np.abs(got[name][band]), r[band] + tol)
                ok = ok and float((e[band] - half_bf16_spacing(mag)).max()) <= tol
    return {"max_abs_err": {k: float(f"{v:.4g}") for k, v in err.items()},
            "max_abs_val": {k: float(f"{v:.4g}") for k, v in val.items()},
            "bar": tol, "within_bar": bool(ok), "heads": hq, "rows": "all"}


class ClockSampler:
    """Samples the GPU's graphics clock (amdsmi) on a host thread while the
    timed steps run; reports the median in MHz, or None where amdsmi or the
    device's handle is not available."""

    def __init__(self, torch):
        import threading
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            bus = None
            try:
                pr = torch.cuda.get_device_properties(0)
                bus = (int(pr.pci_domain_id), int(pr.pci_bus_id), int(pr.pci_device_id))
            except Exception:  # noqa: BLE001
                pass
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, b, rest = bdf.split(":")
                if bus is not None and (int(dom, 16), int(b, 16), int(rest.split(".")[0], 16)) == bus:
                    self._handle = h
            if self._handle is None and len(handles) == 1:
                self._handle = handles[0]
            self._amdsmi = amdsmi
        except Exception:  # noqa: BLE001
            self._handle = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        if clks:
            return sum(clks) / len(clks)
        c = m.get("current_gfxclk") or m.get("average_gfxclk_frequency")
        return float(c) if isinstance(c, (int, float)) and 0 < c < 10000 else None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v:
                    self.samples.append(v)
            except Exception:  # noqa: BLE001
                return
            self._stop.wait(0.005)

    def start(self):
        if self._handle is not None:
            import threading
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=2)
        return list(self.samples)


def measure_clock(torch, step, seconds=2.5):
    """The graphics clock while the step repeats (untimed, right after the
    timed steps, so under the same load): the firmware refreshes the metrics
    about once a second, so readings from before the first refresh under load
    are dropped. Median over XCDs' mean clock, in MHz; None if unavailable."""
    cs = ClockSampler(torch)
    if cs._handle is None:
        return None
    cs.start()
    t0 = time.time()
    while time.time() - t0 < seconds:
        step()
        torch.cuda.synchronize()
    samples = cs.stop()
    if not samples:
        return None
    first = 0
    while first < len(samples) and samples[first] == samples[0]:
        first += 1
    loaded = sorted(samples[first:])
    if not loaded:
        return None
    return {"median_mhz": round(loaded[len(loaded) // 2], 1), "min_mhz": round(loaded[0], 1),
            "max_mhz": round(loaded[-1], 1), "samples": len(loaded),
            "source": "amdsmi gpu metrics: mean of the per-XCD current gfx clocks while the step repeats, "
                      "untimed, for 2.5 s after the timed steps"}


def bench_bpt(args):
    """The BPT layer after attention over a 32768-row sequence, 4096 rows at
    a time: algorithmic flops 2 d^2 (W_o) + 4 d d_ff (FFN) per row; the
    products' kernel against the bf16 MFMA peak, layer norm against HBM."""
    import numpy as np
    import torch

    import exact_blockwise_attention_amd as ra
    from exact_blockwise_attention_amd import synthetic as syn
    w = syn.BPT_WORKLOAD
    rows, dm, dff, br = w["rows"], w["d_model"], w["d_ff"], w["block_rows"]

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(x).to("cuda")

    attn = dev(syn.make_payload(w["wid"], "attn", (rows, dm), "bf16"))
    x = dev(syn.make_payload(w["wid"], "x", (rows, dm), "bf16"))
    prm = {k: dev(v) for k, v in syn.bpt_params(w["wid"], dm, dff).items()}
    out = torch.empty_like(x)
    pb = ra.BptProblem(rows, dm, dff, br, 0.0)
    wts = ra.BptWeights(*(prm[n].data_ptr() for n in ra.BPT_WEIGHT_NAMES))
    need = ra.bpt_workspace_bytes(pb)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sh = ra._stream_handle(stream)
    torch.cuda.synchronize()
    call = lambda: ra.bpt_ffn_raw(pb, attn.data_ptr(), x.data_ptr(), wts, out.data_ptr(), ws.data_ptr(), need, sh)  # noqa: E731
    for _ in range(args.warmup):
        call()
    ms = time_calls(torch, stream, call, n=args.steps)
    flops = rows * (2 * dm * dm + 4 * dm * dff)
    value = flops / ms / 1e9
    # each product shape of one block, and one layer norm, timed alone
    a_blk = torch.empty((br, dff), dtype=torch.bfloat16, device="cuda").normal_()
    o32 = torch.empty((br, max(dm, dff)), dtype=torch.float32, device="cuda")
    shapes = {"W_o": (dm, dm, prm["w_o"], prm["b_o"]), "W_1": (dff, dm, prm["w_1"], prm["b_1"]),
              "W_2": (dm, dff, prm["w_2"], prm["b_2"])}
    gem = {}
    for name, (n, k, wt, bias) in shapes.items():
        gms = time_calls(torch, stream, lambda: ra.linear_raw(br, n, k, a_blk.data_ptr(), a_blk.stride(0),
                                                             wt.data_ptr(), k, bias.data_ptr(), None, 0, 0,
                                                             o32.data_ptr(), o32.stride(0), 1, sh), n=5)
        gem[name] = {"m": br, "n": n, "k": k, "ms": round(gms, 4), "tflops": round(2 * br * n * k / gms / 1e9, 2)}
    z = torch.empty((br, dm), dtype=torch.float32, device="cuda").normal_()
    lms = time_calls(torch, stream, lambda: ra.layer_norm_raw(br, dm, z.data_ptr(), prm["ln1_g"].data_ptr(),
                                                             prm["ln1_b"].data_ptr(), 0.0, out.data_ptr(), sh), n=5)
    ln = hbm_row(lms, br * dm * (4 + 2) + 2 * dm * 4)
    dom = max(gem.values(), key=lambda g: g["ms"])
    peak = PEAK_BF16_TFLOPS
    roof = {"bound": "mfma", "kernel": "gemm_bf16_kernel", "achieved": dom["tflops"], "peak": peak,
            "unit": "TFLOP/s", "frac": round(dom["tflops"] / peak, 4), "traffic": read_traffic("gemm_bf16_kernel"),
            "launch_ms": dom["ms"], "shape": [dom["m"], dom["n"], dom["k"]]}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.bpt as ob
        sel = np.arange(16384)  # the first 16384 rows of the tail (rows are independent); about 10 s
        p64 = {k: syn.to_f64(v) for k, v in syn.bpt_params(w["wid"], dm, dff).items()}
        a64 = syn.to_f64(syn.make_payload(w["wid"], "attn", (rows, dm), "bf16")[sel])
        x64 = syn.to_f64(syn.make_payload(w["wid"], "x", (rows, dm), "bf16")[sel])
        t0 = time.perf_counter()
        ob.ffn_block(a64, x64, p64)
        dt = time.perf_counter() - t0
        cpu = {"value": round(len(sel) * (2 * dm * dm + 4 * dm * dff) / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": int(os.cpu_count() or 1), "kind": "oracle", "sample": f"{len(sel)} rows of the tail",
               "seconds": round(dt, 3)}
    print(json.dumps({
        "metric": f"BPT layer tail TFLOP/s ({w['name']})", "value": round(value, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "rows": rows, "d_model": dm, "d_ff": dff, "block_rows": br},
        "frac_of_peak": round(value / peak, 4), "roofline": roof, "cpu_baseline": cpu,
        "details": {"products": gem, "layer_norm": ln, "workspace_bytes": need},
        "device": torch.cuda.get_device_name(0)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the ring across GPUs is not "
              "implemented; it times one GPU's share of the ring at its real shape", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import exact_blockwise_attention_amd as ra
    from exact_blockwise_attention_amd import synthetic as syn

    ra.library()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload == 7:
        bench_bpt(args)
        return
    w = syn.WORKLOADS[args.workload]
    layout = args.layout or w.layouts[-1]
    P, Bb, d = w.ring_size, w.block_len, w.head_dim
    ranks = list(range(*w.q_ranks)) if w.q_ranks else list(range(P))
    rb, re_ = ranks[0], ranks[-1] + 1
    names = ("q", "k", "v", "do") if "bwd" in w.passes else ("q", "k", "v")

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(x).to("cuda")

    # zigzag blocks are not strided slices of the token order, and a device
    # holds its block contiguously in any layout: keep blocked copies resident
    # (the one-device share of workload 4 holds its query rows in local order)
    blocked = layout == "zigzag" or (args.memory == "blocked" and not w.q_ranks)
    if layout == "zigzag" and w.q_ranks:
        raise SystemExit("the one-device share is run in the striped layout")
    t = {}
    for n in names:
        pay = syn.make_payload(w.wid, n, syn.workload_shape(w, n), w.dtype)
        if n == "q" and w.q_ranks:
            # one device's share: only its query block is resident, in local row order
            x = np.arange(Bb)
            pos = x * P + rb if layout == "striped" else rb * Bb + x
            pay = np.ascontiguousarray(pay[:, pos])
        if blocked:
            # blocked order [P, B, Bb, H, d]: block s holds tokens s, s + P, ...
            # (striped), half-blocks s and 2P-1-s (zigzag), or s Bb .. (contiguous)
            if layout == "zigzag":
                hb = Bb // 2
                perm = np.concatenate([np.r_[s_ * hb:(s_ + 1) * hb, (2 * P - 1 - s_) * hb:(2 * P - s_) * hb]
                                       for s_ in range(P)])
            elif layout == "striped":
                perm = np.concatenate([np.arange(s_, P * Bb, P) for s_ in range(P)])
            else:
                perm = np.arange(P * Bb)
            pay = np.ascontiguousarray(pay[:, perm].reshape(w.batch, P, Bb, pay.shape[2], d).transpose(1, 0, 2, 3, 4))
        t[n] = dev(pay)
        del pay
    torch.cuda.synchronize()

    code = ra.BF16 if w.dtype == "bf16" else ra.F32
    pb = ra.make_problem(w.batch, w.heads, d, P, Bb, layout, w.causal, code, kv_heads=w.kv_heads)
    stream = torch.cuda.current_stream()
    sh = ra._stream_handle(stream)
    copy_stream = torch.cuda.Stream() if w.prefetch else None
    ch = ra._stream_handle(copy_stream) if copy_stream is not None else None
    if blocked:
        so = lambda x: ra.seq_blocked(x, block_offset=rb)  # noqa: E731
        sk = ra.seq_blocked
    elif w.q_ranks:
        so = lambda x: ra._seq_rank_rows(x, re_ - rb, layout, P)  # noqa: E731
    else:
        so = lambda x: ra.seq_original(x, P, layout, block_offset=rb)  # noqa: E731
    if not blocked:
        sk = lambda x: ra.seq_original(x, P, layout)  # noqa: E731
    o = torch.empty_like(t["q"])
    nr = re_ - rb
    lse = torch.empty((nr, w.batch, w.heads, Bb), dtype=torch.float32, device="cuda")
    fws = ra.workspace_bytes(pb, rb, re_, w.prefetch, False)
    fwd_ws = torch.empty(max(fws, 256), dtype=torch.uint8, device="cuda")
    bwd = "bwd" in w.passes
    if bwd:
        dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
        bws = ra.workspace_bytes(pb, rb, re_, False, 2 if args.bwd_recompute else True)
        stores_ds = bws > ra.workspace_bytes(pb, rb, re_, False, 2)
        bwd_ws = torch.empty(bws, dtype=torch.uint8, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def mark(timing, key):
        if timing is not None:
            e = ev()
            e.record(stream)
            timing[key].append(e)

    def step(timing=None):
        mark(timing, "f0")
        ra.forward_raw(pb, rb, re_, so(t["q"]), sk(t["k"]), sk(t["v"]), so(o), lse.data_ptr(),
                       fwd_ws.data_ptr() if fws else None, fws, sh, ch)
        mark(timing, "f1")
        if bwd:
            args_ = (pb, rb, re_, so(t["q"]), sk(t["k"]), sk(t["v"]), so(o), so(t["do"]), lse.data_ptr(), so(dq),
                     sk(dk), sk(dv), bwd_ws.data_ptr(), bws, sh)
            ra.backward_stage_raw(0, *args_)
            mark(timing, "b0")
            ra.backward_stage_raw(1, *args_)
            mark(timing, "b1")
            ra.backward_stage_raw(2, *args_)
            mark(timing, "b2")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timing = {"f0": [], "f1": [], "b0": [], "b1": [], "b2": []}
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step(timing)
    stop.record(stream)
    torch.cuda.synchronize()
    sclk = measure_clock(torch, step)
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps

    def span(a, b):
        return sum(x.elapsed_time(y) for x, y in zip(timing[a], timing[b])) / args.steps

    pairs = pair_count(layout, w.causal, P, Bb, ranks) * w.batch * w.heads
    d_ = d
    fwd_flops = 4 * d_ * pairs
    bwd_flops = 10 * d_ * pairs if bwd else 0
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    fwd_ms = span("f0", "f1")
    # per kernel: (ms, algorithmic flops it performs, tag). The dK/dV walk does
    # the S recompute, dP, dV and dK products (8d per pair); the dQ walk adds
    # only dQ (2d per pair) to the method's work, its S/dP recompute is extra.
    kern = {"fwd": (fwd_ms, fwd_flops, "fwd_bf16_kernel" if w.dtype == "bf16" else "fwd_f32_kernel")}
    details = {"pairs": pairs, "fwd_ms": round(fwd_ms, 4), "fwd_tflops": round(fwd_flops / fwd_ms / 1e9, 2)}
    if bwd:
        pre_ms, dkdv_ms, dq_ms = span("f1", "b0"), span("b0", "b1"), span("b1", "b2")
        kern["dkdv"] = (dkdv_ms, 8 * d_ * pairs, "dkdv_bf16_kernel")
        details.update({"bwd_pre_ms": round(pre_ms, 4), "dkdv_ms": round(dkdv_ms, 4), "dq_ms": round(dq_ms, 4),
                        "dkdv_tflops": round(8 * d_ * pairs / dkdv_ms / 1e9, 2),
                        "dq_tflops_alg": round(2 * d_ * pairs / dq_ms / 1e9, 2),
                        "bwd_ms": round(pre_ms + dkdv_ms + dq_ms, 4),
                        "bwd_tflops": round(bwd_flops / (pre_ms + dkdv_ms + dq_ms) / 1e9, 2)})
        if stores_ds:
            # dQ = scale dS K from the stored tiles: bound by reading them
            tiles = stored_ds_tiles(layout, w.causal, P, Bb, ranks) * w.batch * w.heads
            dq_bytes = tiles * 64 * 128 * 2 + len(ranks) * w.batch * w.heads * Bb * d_ * 2
            kern["dq"] = (dq_ms, 2 * d_ * pairs, "dq_from_ds_kernel")
            details["dq_path"] = "stored dS (written by the dK/dV walk, read by dq_from_ds_kernel)"
            details["stored_ds_tiles"] = tiles
            details["workspace_bytes"] = bws
            details["memory_rows_dq"] = hbm_row(dq_ms, dq_bytes)
        else:
            kern["dq"] = (dq_ms, 2 * d_ * pairs, "dq_bf16_kernel")
            details["dq_path"] = "recompute of S and dP in the query-side walk (dq_bf16_kernel)"
            details["dq_tflops_mfma"] = round(6 * d_ * pairs / dq_ms / 1e9, 2)
    dom = max(kern, key=lambda k_: kern[k_][0])
    dom_ms, dom_flops, tag = kern[dom]
    achieved = dom_flops / dom_ms / 1e9
    value = (fwd_flops + bwd_flops) / ms / 1e9
    roof = {"bound": "mfma", "kernel": tag, "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": read_traffic(tag), "launch_ms": round(dom_ms, 4)}
    if w.prefetch:
        roof["note"] = "one call of 8 step launches plus the side-stream copies, timed as a whole"
    if bwd:
        B_, H_ = w.batch, w.heads
        # D = rowsum(dO * O): reads O and dO rows, writes one fp32 per row
        pre_bytes = len(ranks) * B_ * H_ * Bb * (2 * d_ * t["q"].element_size() + 4)
        # stage 0 alone with the minimum workspace: D = rowsum(dO * O) only
        # (with the full workspace it also arranges K for the dQ product)
        small = ra.workspace_bytes(pb, rb, re_, False, 2)
        pre_args = (pb, rb, re_, so(t["q"]), sk(t["k"]), sk(t["v"]), so(o), so(t["do"]), lse.data_ptr(), so(dq),
                    sk(dk), sk(dv), bwd_ws.data_ptr(), small, sh)
        pre_ms = time_calls(torch, stream, lambda: ra.backward_stage_raw(0, *pre_args))
        details["memory_rows"] = {"B1_rowsum_dO_O": hbm_row(pre_ms, pre_bytes),
                                  **memory_rows(torch, ra, w, t["q"], sh, stream)}
    if w.wid == 2:
        details["small_block_sweep"] = small_block_sweep(torch, ra, w, sh, stream)
    if w.wid == 3:
        details["balance"] = balance_report(torch, ra, w, layout, t, pb, blocked, o, lse, sh, stream)
    if w.prefetch:
        details["receive_overlap"] = receive_overlap(torch, ra, w, t, pb, rb, re_, so, sk, o, lse, sh, stream, ms)
    cpu, ref = (None, None) if args.no_cpu_baseline else cpu_baseline(w)
    parity = None
    if ref is not None and bwd:
        parity = parity_report(torch, ra, w, layout, blocked,
                               {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, ref)
    gqa_tag = f", {w.heads} query heads on {w.kv_heads} K/V heads" if w.kv_heads else ""
    out = {
        "metric": f"attention TFLOP/s fwd+bwd (causal {layout}{gqa_tag}, d=128) and % of bf16 MFMA peak" if bwd else
                  f"attention forward TFLOP/s ({workload_name(w, layout)})",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": workload_name(w, layout), "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len, "head_dim": d,
                   "kv_heads": w.kv_heads or w.heads,
                   "ring_size": P, "block_len": Bb, "layout": layout, "causal": w.causal,
                   "ranks": [rb, re_], "passes": list(w.passes), "prefetch": w.prefetch,
                   "memory": "blocked" if blocked else "original"},
        "frac_of_peak": round(value / peak, 4),
        "roofline": roof, "cpu_baseline": cpu, "parity": parity, "gpu_clock": sclk, "details": details,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
