"""Throughput of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
fa_fwd (the forward kernel) followed by fa_bwd's three stages (the
query-tile kernel computing dQ and storing the row terms -D_i and
-LSE_i / scale; the key-block kernel computing dK and dV; the sum of split
dK / dV partials, which enqueues nothing at these shapes), all through the
C ABI on torch's current stream, inputs resident in HBM.

Default workload: causal attention B=1, Hq=Hkv=32, N=4096, d=128, bf16
(the pages' 4096-token, 32-head case). ``value`` is the step's algorithmic
throughput: forward 4*B*Hq*N_q*N_kv*d FLOP, backward 2.5x that, both halved
for causal, divided by the measured time per step.

The roofline objects price each kernel's algorithmic FLOP per launch against
the published bf16/fp16 dense matrix-core peak. The backward's five products
of two N x d operands (S, dP, dV, dK, dQ) split as four in the key-block
kernel and one (dQ = dS K) in the query-tile kernel; the S and dP that the
query-tile kernel recomputes are an implementation cost and are not counted.

Warm-up: the GPU reaches its steady clock only after some tens of
milliseconds under load; at the default workload the first ~50 steps run up
to ~15 % slower than the later ones. Before the ``--warmup`` untimed steps
the bench therefore runs untimed steps for ``--settle-ms`` milliseconds of
wall time (default 150; 0 turns it off), so that a short warm-up (say 5
steps) does not leave the clock still rising inside the timed region. The
settle time and the number of steps it ran are reported in the JSON line.

Timing: the K timed steps run back to back between two events (no event
between kernels), bracketed by synchronizations; ``ms_per_step`` and
``value`` come from that region. Then each kernel runs K times back to back
between two events of its own: its mean launch duration (``kernel_ms``, the
roofline objects). Last, K steps with an event after every kernel give each
kernel's median and minimum launch time (``kernel_ms_median``,
``kernel_ms_min``). Event records between kernels add a few microseconds
each, so they are kept out of the step time and the means. Decode workloads
time each call between its own events instead (see below).

Prints ONE JSON line. ``--workload`` selects another synthetic workload for
development measurements (decode workloads report HBM GB/s, each timed call
starting from cold caches unless --warm-cache).
``--copy-mib M`` runs one plain device copy of M MiB before the warmup, so a
rocprofv3 counter run of this command also holds a copy kernel of known size
to calibrate FETCH_SIZE / WRITE_SIZE against.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak (published)
METRIC = "attention fwd/bwd TFLOP/s & % bf16 MFMA peak, causal N=4096 d=128"
CSRC = os.path.join(ROOT, "exact_attention_115_amd", "csrc")
COMMON = ["fa_device.h", "fa_tile.h", "fa_internal.h"]
# Sources each kernel is built from; a counter summary is only used while
# their hash matches the one it was taken on.
KERNEL_SOURCES = {
    "fwd": ["fa_fwd.hip"] + COMMON,
    "bwd_dkdv": ["fa_bwd.hip"] + COMMON,
    "bwd_dq": ["fa_bwd_dq.hip"] + COMMON,
    "decode": ["fa_decode.hip"] + COMMON,
}
TRAFFIC_SUMMARY = {
    "fwd": "fwd_causal_b1h32n4096d128_bf16_hbm_traffic.md",
    "bwd_dkdv": "bwd_dkdv_causal_b1h32n4096d128_bf16_hbm_traffic.md",
    "bwd_dq": "bwd_dq_causal_b1h32n4096d128_bf16_hbm_traffic.md",
    # split + combine kernels of one decode call, B=16 Hq=32 Hkv=8 N_kv=8192 d=128
    "decode": "decode_b16h32kv8n8192d128_bf16_hbm_traffic.md",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed steps for this many ms of wall time before the warm-up, so "
                         "the GPU clock has settled (0: none)")
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB before the warmup")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability on P (fa_fwd_dropout / fa_bwd_dropout); the "
                         "backward is then timed as one pass")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 (E4M3) forward (fa_fwd_fp8) on the workload's shape, "
                         "forward only")
    ap.add_argument("--warm-cache", action="store_true",
                    help="decode workloads: skip the cache flush before each timed call")
    ap.add_argument("--inputs", choices=("randn", "const"), default="randn",
                    help="development measurement only: 'const' sets every element of q, k, v, "
                         "dO to 0.5 (the same instruction stream with operands that do not "
                         "toggle, to see how much of the time is the clock the chip holds "
                         "under power); the metric is defined on the default N(0,1) draws")
    return ap.parse_args()


def code_only(text):
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that the hash below changes with the code but not with its comments.
    String and character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(kernel_key):
    """sha256 (first 16 hex digits) of the code, comments aside, of the
    files the kernel is built from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel_key]:
        h.update(code_only(open(os.path.join(CSRC, name), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the summary is missing or was taken on another kernel source."""
    name = TRAFFIC_SUMMARY.get(kernel_key)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per launch:\s*`?([0-9.eE+]+)", text)
    if not m_hash or not m_bytes:
        return None
    if m_hash.group(1) != source_hash(kernel_key):
        return None
    return float(m_bytes.group(1))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s):
    """Time the float64 oracle (as it stands) on a bounded sample of whole
    heads of the workload; returns the throughput in the bench's unit."""
    import oracle
    from synth import make_inputs, to_f64

    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q, k, v, do = make_inputs(w)
    G = w.Hq // w.Hkv
    per_head_flop = (w.fwd_flop() + (w.bwd_flop() if w.backward else 0.0)) / (w.B * w.Hq)
    done = 0
    t0 = time.perf_counter()
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    for b, h in heads:
        qh, kh, vh = to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G])
        oracle.head_forward(qh, kh, vh, w.causal, w.scale)
        if w.backward:
            oracle.head_backward(qh, kh, vh, to_f64(do[b, h]), w.causal, w.scale)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if w.Nq == 1:
        nbytes = decode_bytes(w) * done / (w.B * w.Hq)
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
                "cpu": cpu_model(), "host_cpus": os.cpu_count(),
                "sample": f"{done} of {w.B * w.Hq} (batch, head) rows of {w.name}, forward, "
                          f"float64 numpy, {dt:.1f} s"}
    return {"value": per_head_flop * done / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{done} of {w.B * w.Hq} heads of {w.name} "
                      f"({'forward + backward' if w.backward else 'forward'}), float64 numpy, "
                      f"{dt:.1f} s; algorithmic FLOP counted as on the GPU"}


def decode_bytes(w):
    e = 2 if w.dtype != "f32" else 4
    return (w.B * w.Hq * w.Nq * w.d * e * 2 + 2 * w.B * w.Hkv * w.Nkv * w.d * e
            + 4 * w.B * w.Hq * w.Nq)


def mfma_roofline(kernel, flop, ms, traffic, peak=PEAK_BF16_TFLOPS):
    ach = flop / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
            "kernel": kernel, "avg_launch_ms": round(ms, 4),
            "algorithmic_flop_per_launch": flop}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; multi-GPU runs are not "
                                   "implemented (heads would shard across GPUs with no "
                                   "communication)", "n_gpus": args.gpus}))
        return 2

    import torch

    import exact_attention_115_amd as fa
    from synth import WORKLOADS, make_inputs

    # A trailing "p" on a decode workload (c5dgp, c5dmp) runs it over a paged
    # K/V cache: 128-key pages in a shuffled pool, every sequence full.
    paged = args.workload.endswith("p") and args.workload[:-1] in WORKLOADS
    w = WORKLOADS[args.workload[:-1] if paged else args.workload]
    if paged and w.Nq != 1:
        raise SystemExit("paged workloads are decode workloads")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    q, k, v, do = make_inputs(w)
    if args.inputs == "const":
        for t in (q, k, v, do):
            if t is not None:
                t.fill_(0.5)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    do = do.to(dev) if do is not None else None
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    fws = fa.fa_fwd_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, q.dtype)
    fwd_ws = torch.empty(fws, dtype=torch.uint8, device=dev) if fws else None
    if paged:
        PS = 128
        mp = (w.Nkv + PS - 1) // PS
        npages = w.B * mp
        pad = mp * PS - w.Nkv
        kpad = torch.nn.functional.pad(k, (0, 0, 0, pad))
        vpad = torch.nn.functional.pad(v, (0, 0, 0, pad))
        perm = torch.randperm(npages, generator=torch.Generator().manual_seed(w.seed)).to(dev)
        k_pool = torch.empty((npages, w.Hkv, PS, w.d), dtype=k.dtype, device=dev)
        v_pool = torch.empty_like(k_pool)
        # Logical page p of sequence b goes to pool page perm[b * mp + p].
        k_pool[perm] = kpad.reshape(w.B, w.Hkv, mp, PS, w.d).permute(0, 2, 1, 3, 4).reshape(
            npages, w.Hkv, PS, w.d)
        v_pool[perm] = vpad.reshape(w.B, w.Hkv, mp, PS, w.d).permute(0, 2, 1, 3, 4).reshape(
            npages, w.Hkv, PS, w.d)
        table = perm.reshape(w.B, mp).to(torch.int32).contiguous()
        lens = torch.full((w.B,), w.Nkv, dtype=torch.int32, device=dev)
        del kpad, vpad
        pws = fa.fa_fwd_paged_workspace_size(w.B, w.Hq, w.Hkv, PS, mp, w.d, q.dtype)
        fwd_ws = torch.empty(pws, dtype=torch.uint8, device=dev)
    bwd = w.backward
    if bwd:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d, q.dtype)
        bwd_ws = torch.empty(bws, dtype=torch.uint8, device=dev)

    drop = args.dropout > 0.0
    if drop and (paged or w.Nq == 1):
        raise SystemExit("--dropout applies to the prefill workloads")
    fp8 = args.fp8
    if fp8:
        if paged or w.Nq == 1 or w.d != 128 or drop:
            raise SystemExit("--fp8 applies to the d = 128 prefill workloads, without dropout")
        # E4M3 codes of the same draws (descale 1), bf16 output.
        q8 = q.float().to(torch.float8_e4m3fn).view(torch.uint8)
        k8 = k.float().to(torch.float8_e4m3fn).view(torch.uint8)
        v8 = v.float().to(torch.float8_e4m3fn).view(torch.uint8)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        bwd = False
    if drop:
        names = ["fwd"] + (["bwd"] if bwd else [])
    else:
        # Stage 2 (the sum of split dK / dV partials) enqueues nothing unless
        # the query-head group is split; it is timed with stage 1.
        names = ["fwd"] + (["bwd_dq", "bwd_dkdv"] if bwd else [])
    seed = 1234

    # The step's parts, in order, one per entry of `names`: each part is one
    # kernel launch, or one library call where a call runs several kernels.
    # The parts call the C entry points with their arguments marshalled once
    # (device pointers, sizes, the stream), so that the Python binding's
    # per-call checks add no host time between launches; the library still
    # checks every call's arguments on the host.
    import ctypes

    lib = fa.load()
    S = ctypes.c_void_p(stream.cuda_stream)

    def ptr(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    def nbytes(t):
        return 0 if t is None else t.numel() * t.element_size()

    def raw(fn, *a):
        f = getattr(lib, fn)

        def call():
            st = f(*a)
            if st != 0:
                raise fa.FAError(st, fn)
        return call

    dt = {torch.float32: fa.FA_F32, torch.float16: fa.FA_F16, torch.bfloat16: fa.FA_BF16}[q.dtype]
    shape = (w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.d)
    sc, cz = float(w.scale), int(bool(w.causal))
    if fp8:
        parts = [raw("fa_fwd_fp8", ptr(q8), ptr(k8), ptr(v8), ptr(o), ptr(lse), *shape, sc, cz,
                     1.0, 1.0, 1.0, S)]
    elif drop:
        parts = [raw("fa_fwd_dropout", ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), ptr(fwd_ws),
                     nbytes(fwd_ws), *shape, sc, cz, args.dropout, seed, 0, dt, S)]
        if bwd:
            parts.append(raw("fa_bwd_dropout", ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), ptr(do),
                             ptr(dq), ptr(dk), ptr(dv), ptr(bwd_ws), nbytes(bwd_ws), *shape, sc,
                             cz, args.dropout, seed, 0, dt, S))
    else:
        if paged:
            parts = [raw("fa_fwd_paged", ptr(q), ptr(k_pool), ptr(v_pool), ptr(table), ptr(lens),
                         ptr(o), ptr(lse), ptr(fwd_ws), nbytes(fwd_ws), w.B, w.Hq, w.Hkv,
                         k_pool.shape[0], k_pool.shape[2], table.shape[1], w.d, sc, dt, S)]
        else:
            parts = [raw("fa_fwd", ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), ptr(fwd_ws),
                         nbytes(fwd_ws), *shape, sc, cz, dt, S)]
        if bwd:
            stage = [raw("fa_bwd_stage", s_, ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), ptr(do),
                         ptr(dq), ptr(dk), ptr(dv), ptr(bwd_ws), nbytes(bwd_ws), *shape, sc, cz,
                         dt, S) for s_ in range(3)]
            parts += [stage[0], lambda: (stage[1](), stage[2]())]
    assert len(parts) == len(names)

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        for j, part in enumerate(parts):
            part()
            if events is not None:
                events[j + 1].record(stream)

    settle_steps = 0
    if args.settle_ms > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
            for _ in range(8):
                step()
            settle_steps += 8
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # Decode streams K and V once per call: unless --warm-cache, each timed
    # call starts from cold caches (a 1 GiB write, more than the 256 MiB
    # last-level cache and the L2s, runs before it, outside its events).
    cold = w.Nq == 1 and not args.warm_cache
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if cold else None
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        if cold:
            flush.fill_(i & 0xFF)
        step(evs[i] if cold else None)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps
    per_kernel_ms = {}
    if not cold:
        if w.Nq > 1:
            # Each kernel's mean launch duration: K launches of that kernel
            # alone, back to back between two events.
            for j, n in enumerate(names):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(args.steps):
                    parts[j]()
                e1.record(stream)
                torch.cuda.synchronize()
                per_kernel_ms[n] = e0.elapsed_time(e1) / args.steps
        # Median and minimum per launch: K steps with an event after every
        # kernel (the event records add a few microseconds to each).
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
    per_call = {n: sorted(e[j].elapsed_time(e[j + 1]) for e in evs) for j, n in enumerate(names)}
    for n, t in per_call.items():
        per_kernel_ms.setdefault(n, sum(t) / args.steps)
    if w.Nq == 1:
        # Decode: time per call between its own events. From cold caches the
        # flushes are not counted; with warm caches a call (about 20 us at
        # Hkv = 1) is shorter than the host's time to enqueue the next one,
        # so the wall time between the first and last event would measure
        # the host, not the GPU.
        ms_per_step = sum(per_kernel_ms.values())

    fwd_flop, bwd_flop = w.fwd_flop(), (w.bwd_flop() if bwd else 0.0)
    out = {
        "metric": (METRIC if args.workload == "c3" and not drop and not fp8 and args.inputs == "randn"
                   else f"attention throughput, {args.workload}"
                   + (f" with dropout p={args.dropout}" if drop else "")
                   + (" FP8 (E4M3) forward" if fp8 else "")
                   + (" on constant inputs (development measurement)"
                      if args.inputs == "const" else "")),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"ms": args.settle_ms, "untimed_steps": settle_steps},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 (bf16 out)" if fp8 else w.dtype,
        "data": ("synthetic: seeded i.i.d. N(0,1) q, k, v, dO rounded to the storage dtype"
                 if args.inputs == "randn" else "synthetic: every element of q, k, v, dO = 0.5"),
        "config": {"workload": f"{'causal' if w.causal else 'non-causal'} attention "
                               f"{'forward+backward' if bwd else 'forward'} B={w.B} Hq={w.Hq} "
                               f"Hkv={w.Hkv} N_q={w.Nq} N_kv={w.Nkv} d={w.d} {w.dtype}"
                               + (" over a paged K/V cache (128-key pages, shuffled pool)"
                                  if paged else "")
                               + (f" with dropout p={args.dropout} on P" if drop else "")
                               + (" as E4M3 inputs, P rounded to E4M3, bf16 output" if fp8 else ""),
                   "name": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N_q": w.Nq,
                   "N_kv": w.Nkv, "d": w.d, "causal": w.causal, "parallelism": "single GPU"},
        "wall_s_timed": round(wall, 4),
        "kernel_ms": {n: round(t, 4) for n, t in per_kernel_ms.items()},
        "kernel_ms_median": {n: round(t[len(t) // 2], 4) for n, t in per_call.items()},
        "kernel_ms_min": {n: round(t[0], 4) for n, t in per_call.items()},
    }
    if w.Nq == 1:
        # Decode: HBM-bound, reported as algorithmic bytes per second.
        nbytes = decode_bytes(w) + ((table.numel() + lens.numel()) * 4 if paged else 0)
        gbs = nbytes / (ms_per_step * 1e-3) / 1e9
        out.update({"value": round(gbs, 2), "unit": "GB/s", "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
                    "cache": "cold (1 GiB write before each timed call)" if cold else "warm"})
        out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                           "traffic": read_traffic("decode") if args.workload == "c5dg" else None,
                           "kernel": "decode split + combine (one fa_fwd" + ("_paged" if paged else "") + " call)",
                           "algorithmic_bytes": nbytes}
    else:
        tflops = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12
        fwd_t = fwd_flop / (per_kernel_ms["fwd"] * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
        out.update({"value": round(tflops, 2), "unit": "TFLOP/s",
                    "pct_peak": round(100 * tflops / peak, 2),
                    "fwd_tflops": round(fwd_t, 2),
                    "fwd_pct_peak": round(100 * fwd_t / peak, 2)})
        flop = {"fwd": fwd_flop}
        if bwd and drop:
            bwd_t = bwd_flop / (per_kernel_ms["bwd"] * 1e-3) / 1e12
            out.update({"bwd_tflops": round(bwd_t, 2), "bwd_pct_peak": round(100 * bwd_t / PEAK_BF16_TFLOPS, 2)})
            flop["bwd"] = bwd_flop
        elif bwd:
            bwd_ms = per_kernel_ms["bwd_dq"] + per_kernel_ms["bwd_dkdv"]
            bwd_t = bwd_flop / (bwd_ms * 1e-3) / 1e12
            out.update({"bwd_tflops": round(bwd_t, 2), "bwd_pct_peak": round(100 * bwd_t / PEAK_BF16_TFLOPS, 2)})
            flop.update({"bwd_dkdv": 0.8 * bwd_flop, "bwd_dq": 0.2 * bwd_flop})
        on_profiled = args.workload == "c3" and not drop and not fp8
        lines = {kname: mfma_roofline(kname, f, per_kernel_ms[kname],
                                      read_traffic(kname) if on_profiled else None, peak)
                 for kname, f in flop.items()}
        # The dominant kernel is the one with the longest average launch.
        dom = max(lines, key=lambda kname: per_kernel_ms[kname])
        out["roofline"] = lines[dom]
        out["roofline_all"] = lines
    if not args.no_cpu_baseline and not drop and not fp8:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
