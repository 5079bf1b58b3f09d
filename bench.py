"""Benchmark of the SplitZip codec on one MI355X.

Workload: a streaming KV cache of 32 layers x (K, V) tensors [1, 8, 32768, 128]
bf16 (64 tensors, 2^31 elements, 4 GiB), N(0, 0.02) values (seed 5, stream
2*layer + kv), one codebook per tensor.  A step is one pass of the whole hot
path: calibrate all 64 tensors, encode all 64, decode all 64 (inputs already
resident in HBM).  The per-phase times come from HIP events on the stream the
kernels are launched on.

Prints ONE JSON line.  ``value`` is the end-to-end raw-BF16 throughput of the
step (4 GiB / step time); the line also carries per-phase throughput, the
compression ratio, the roofline of the dominant call, the rate of a
reference stream with each phase's access pattern (its practical ceiling) and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "encode/decode GB/s of raw BF16 + % HBM roofline; compression ratio"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
LAYERS, HEADS, SEQ, HEAD_DIM = 32, 8, 32768, 128
N = HEADS * SEQ * HEAD_DIM       # elements per tensor


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle budget for the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 512 MiB device to device once (a "
                         "reference for hardware byte counters)")
    ap.add_argument("--no-h2d", action="store_true", help="skip the host-to-device pipeline")
    ap.add_argument("--no-small", action="store_true", help="skip the small single-tensor configs")
    ap.add_argument("--h2d-tensors", type=int, default=8,
                    help="KV tensors in the host-to-device pipeline sample")
    ap.add_argument("--small-only", metavar="WORKLOAD", nargs="?", const="all",
                    help="instead of the benchmark, run the smaller single-tensor workloads only "
                         "(or the one named) and print them as one JSON line")
    ap.add_argument("--sizes", action="store_true",
                    help="instead of the benchmark, time single-tensor calls of N(0, 0.02) values "
                         "at 2^16, 2^18, ..., 2^30 elements and print them as one JSON line")
    ap.add_argument("--probes", action="store_true",
                    help="instead of the benchmark, run the probes of the part's costs that the "
                         "design rests on (reference-stream library) and print them as one JSON line")
    return ap.parse_args()


def d2d_copy(x_all, stream):
    """Device-to-device copy of the 4 GiB workload with torch's copy kernel
    (a library reference; the access-pattern ceilings are pattern_ceilings)."""
    import torch

    dst = torch.empty_like(x_all)
    dst.copy_(x_all)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        dst.copy_(x_all)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    moved = 2 * x_all.numel() * 2
    del dst
    return {"ms": round(ms, 4), "bytes_moved": moved, "GBps": round(moved / ms / 1e6, 1),
            "hbm_frac": round(moved / ms / 1e6 / HBM_PEAK_GBPS, 4), "kernel": "torch copy_"}


def pattern_ceilings(S, x_all, phases, stream, reps):
    """The reference memory streams (the codec kernels' loads and stores with
    XORs for the coding) over the bytes of one batched launch of each phase:
    the ceiling of each access pattern, timed in the same run, and each
    phase's algorithmic rate as a fraction of it."""
    import torch

    lib = S._abi.ceiling_lib()
    sh = int(stream.cuda_stream)
    # the batched calibrate launch of this size runs one workgroup per compute unit
    cus = torch.cuda.get_device_properties(x_all.device).multi_processor_count
    n = x_all[:32].numel()                       # elements of one 32-tensor launch
    x = x_all[:32].reshape(-1)
    scratch = torch.empty(n // 2 + n + 2 * n, dtype=torch.uint8, device=x_all.device)
    pk, sm = scratch[: n // 2], scratch[n // 2: n // 2 + n]
    out = scratch[n // 2 + n:]
    sink = torch.zeros(1, dtype=torch.int32, device=x_all.device)

    def ok(rc):
        if rc:
            raise S._abi.SplitZipError("reference stream", rc)

    runs = {
        "calibrate": ("k_read_shape", 2 * n,
                      lambda: ok(lib.splitzip_ceiling_read(x.data_ptr(), 2 * n, cus,
                                                           sink.data_ptr(), sh))),
        "encode": ("k_encode_shape", 2 * n + n // 2 + n,
                   lambda: ok(lib.splitzip_ceiling_encode_shape(x.data_ptr(), n, pk.data_ptr(),
                                                                sm.data_ptr(), sh))),
        "decode": ("k_decode_shape", n // 2 + n + 2 * n,
                   lambda: ok(lib.splitzip_ceiling_decode_shape(pk.data_ptr(), sm.data_ptr(),
                                                                out.data_ptr(), n, sh))),
    }
    res = {}
    for phase, (kernel, moved, fn) in runs.items():
        fn()
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rate = moved / ms / 1e6
        res[phase] = {"kernel": kernel, "bytes_per_launch": moved, "ms_per_launch": round(ms, 4),
                      "GBps": round(rate, 1), "hbm_frac": round(rate / HBM_PEAK_GBPS, 4),
                      "phase_frac_of_ceiling": round(phases[phase]["alg_GBps"] / rate, 4)}
    del scratch
    res["note"] = ("same loads, stores, workgroup shapes and data map as the codec kernel, "
                   "XORs in place of the coding; 2^30 elements per launch, mean of %d" % reps)
    return res


def design_probes(S, dev):
    """Costs of the part that the codec's design rests on, measured with the
    reference-stream library (HIP events on the launch stream, mean over the
    timed launches after two untimed ones):

    * access shapes: the encode / decode patterns with 8-element units per
      thread (the codec's) against thread-contiguous 32-element units, over
      2^30 elements per launch, and over one 2^25-element tensor per launch
      (64 launches back to back over 32 tensors' worth of memory: the
      single-call ceiling);
    * the encode pattern with a fused arrival (count store, s_waitcnt,
      two-level arrival counter), and with an agent-scope fence per
      workgroup;
    * both patterns with `run` consecutive tiles per XCD in turn against the
      plain order of tiles (TB/s);
    * device-scope atomics: dependent adds by one thread (latency), one add
      by each of 8,192 workgroups on one address against 64 spread ones;
    * 64 launches of an almost empty kernel, ordinary and cooperative;
    * the in-place decode's forms alone and beside a long kernel on another
      stream (slot_contention)."""
    import torch

    lib = S._abi.ceiling_lib()
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)

    def ok(rc):
        if rc:
            raise S._abi.SplitZipError("probe", rc)

    def timed(fn, reps):
        fn()
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps   # ms

    res = {}
    big = 1 << 30
    x = torch.empty(big, dtype=torch.int16, device=dev)
    x.random_(-32768, 32767)
    pk = torch.empty(big // 2, dtype=torch.uint8, device=dev)
    sm = torch.empty(big, dtype=torch.uint8, device=dev)
    out = torch.empty(big, dtype=torch.int16, device=dev)
    tiles = big // 8192
    counts = torch.zeros(tiles, dtype=torch.int32, device=dev)
    ctrs = torch.zeros(8 * (1 + (tiles + 15) // 16), dtype=torch.int64, device=dev)
    ready = torch.zeros(4, dtype=torch.int32, device=dev)
    epoch = [0]

    def ptrs(n, k):
        """Element offset k * n of every buffer (the per-call runs cycle through
        32 different tensors' worth of memory, so that nothing is cache-resident)."""
        o = k * n
        return (x.data_ptr() + 2 * o, pk.data_ptr() + o // 2, sm.data_ptr() + o, out.data_ptr() + 2 * o)

    def arrive(n, k):
        epoch[0] += 1
        xp, pp, sp, _ = ptrs(n, k)
        ok(lib.splitzip_ceiling_encode_arrive(xp, n, pp, sp, counts.data_ptr(), ctrs.data_ptr(),
                                              ready.data_ptr(), epoch[0], sh))

    def call(fn, enc_side):
        def run(n, k):
            xp, pp, sp, op = ptrs(n, k)
            ok(fn(xp, n, pp, sp, sh) if enc_side else fn(pp, sp, op, n, sh))
        return run

    enc = {
        "shape_8": call(lib.splitzip_ceiling_encode_shape, True),
        "wide_32": call(lib.splitzip_ceiling_encode_wide, True),
        "fused_arrival": arrive,
        "fence_per_workgroup": call(lib.splitzip_ceiling_encode_fenced, True),
    }
    dec = {
        "shape_8": call(lib.splitzip_ceiling_decode_shape, False),
        "wide_32": call(lib.splitzip_ceiling_decode_wide, False),
    }
    one = 1 << 25   # one KV tensor
    slices = big // one
    for name, table in (("encode", enc), ("decode", dec)):
        res[name] = {}
        for k, fn in table.items():
            ms_big = timed(lambda: fn(big, 0), 5)
            turn = [0]

            def next_call():
                fn(one, turn[0] % slices)
                turn[0] += 1
            ms_one = timed(next_call, 64)
            moved = 3.5   # bytes per element, both patterns
            res[name][k] = {
                "per_2^30_launch": {"ms": round(ms_big, 4),
                                    "TBps": round(moved * big / ms_big / 1e9, 3)},
                "per_2^25_call": {"us": round(ms_one * 1e3, 2),
                                  "TBps": round(moved * one / ms_one / 1e9, 3)}}
    torch.cuda.synchronize()
    assert int(ready[0].item()) == epoch[0], "fused arrival: the last arrival was not seen"

    # order of tiles over the XCDs: `run` consecutive tiles per XCD in turn
    # (0: the plain order), both patterns, per 2^30 launch and per 2^25 call
    res["tile_order"] = {}
    for name, dec_side in (("encode", 0), ("decode", 1)):
        res["tile_order"][name] = {}
        for n, runs in ((big, (0, 8, 16, 32, 64, 128, 256, 512, big // 8192 // 8)),
                        (one, (0, 8, 16, 32, 64, 128, 256, 512))):
            key = "per_2^30_launch" if n == big else "per_2^25_call"
            row = {}
            for run in runs:
                turn = [0]

                def order_call(run=run, n=n):
                    k = turn[0] % (big // n)
                    turn[0] += 1
                    xp, pp, sp, op = ptrs(n, k)
                    ok(lib.splitzip_ceiling_order(dec_side, run, xp, pp, sp, op, n, sh))
                ms = timed(order_call, 5 if n == big else 64)
                row["plain" if run == 0 else "run_%d" % run] = round(3.5 * n / ms / 1e9, 3)
            res["tile_order"][name][key] = row
    del x, pk, sm, out, counts

    ac = torch.zeros(8 * 64, dtype=torch.int64, device=dev)
    lat_ms = timed(lambda: ok(lib.splitzip_ceiling_atomics(ac.data_ptr(), 1, 1, 4096, sh)), 3)
    one_ms = timed(lambda: ok(lib.splitzip_ceiling_atomics(ac.data_ptr(), 8192, 1, 1, sh)), 5)
    spread_ms = timed(lambda: ok(lib.splitzip_ceiling_atomics(ac.data_ptr(), 8192, 64, 1, sh)), 5)
    res["atomics"] = {
        "dependent_add_latency_us": round(lat_ms * 1e3 / 4096, 3),
        "8192_workgroups_one_address_us": round(one_ms * 1e3, 2),
        "8192_workgroups_64_addresses_us": round(spread_ms * 1e3, 2),
        "one_address_ns_per_add": round(one_ms * 1e6 / 8192, 2)}
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    res["launch"] = {}
    for coop in (0, 1):
        ms = timed(lambda: ok(lib.splitzip_ceiling_launch(coop, 64, sink.data_ptr(), sh)), 64)
        res["launch"]["cooperative" if coop else "ordinary"] = {"us_per_launch": round(ms * 1e3, 2)}
    res["slot_contention"] = slot_contention(S, dev)
    return res


def slot_contention(S, dev):
    """In-place decode of one KV-stream tensor (33,554,432 elements) on its
    own and while a long elementwise kernel (a multiply over 2^28 floats,
    small workgroups) runs on another stream, in the multi-pass form (the
    default) and the resident form (ordinary and cooperative launch).  The
    multiply is enqueued first and a 200,000-cycle spin on the decode's
    stream lets it take the GPU before the decode starts; HIP events on the
    decode's stream, median of 5 after one untimed call."""
    import os
    import statistics

    import torch
    import workloads as W

    x = W.kv_cache_tensor(0, 0, device=dev).reshape(-1)
    n = x.numel()
    ws = S.Workspace(n, dev)
    cb = S.calibrate(x, ws)
    payload, meta = S.encode(x, cb, ws)
    comp = S.read_meta(meta).comp_bytes
    pay = payload[:comp].clone()
    del payload
    slot = torch.empty(2 * n, dtype=torch.uint8, device=dev)
    stash = torch.empty(comp, dtype=torch.uint8, device=dev)
    big = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sa, sb = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    res = {}
    old = os.environ.pop("SPLITZIP_SLOT_LAUNCH", None)
    try:
        for form in ("multi_pass", "resident", "resident_cooperative"):
            if form == "resident_cooperative":
                os.environ["SPLITZIP_SLOT_LAUNCH"] = "coop"
            row = {}
            for contend in (False, True):
                ts = []
                for k in range(6):
                    slot[:comp].copy_(pay)
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    if contend:
                        with torch.cuda.stream(sb):
                            big.mul_(1.0000001)
                    with torch.cuda.stream(sa):
                        if contend:
                            torch.cuda._sleep(200_000)
                        e0.record(sa)
                        S.decode_slot(slot, meta, cb, n, stash, stream=sa, resident=form != "multi_pass")
                        e1.record(sa)
                    torch.cuda.synchronize()
                    if k:
                        ts.append(e0.elapsed_time(e1))
                assert torch.equal(slot.view(torch.int16), x.view(torch.int16)), form
                row["beside_multiply_ms" if contend else "alone_ms"] = round(statistics.median(ts), 4)
            res[form] = row
    finally:
        os.environ.pop("SPLITZIP_SLOT_LAUNCH", None)
        if old is not None:
            os.environ["SPLITZIP_SLOT_LAUNCH"] = old
    return res

def single_call_sizes(S, W, dev, stream):
    """Single-tensor calls by size: one N(0, 0.02) tensor of 2^k elements
    (k = 16, 18, ..., 30), median event time of 10 calls per phase after 3
    warm-up calls (calibrate, encode into a payload of the tensor's own
    size, decode into one output buffer), round trip checked."""
    import statistics

    import torch

    out = {}
    ws = S.Workspace(1 << 30, device=dev)
    for k in range(16, 31, 2):
        n = 1 << k
        x = W.gaussian_weight(n, seed=7, device=dev)
        cb = S.calibrate(x, ws)
        payload = S.payload_for(cb, n)
        meta = S.codec.new_meta(dev)
        dst = torch.empty(n, dtype=torch.bfloat16, device=dev)

        def med(fn):
            for _ in range(3):
                fn()
            ts = []
            for _ in range(10):
                torch.cuda._sleep(100_000)      # keep the GPU busy while the call is enqueued
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            return statistics.median(ts)

        us = {"calibrate": med(lambda: S.calibrate(x, ws, cb=cb)),
              "encode": med(lambda: S.encode(x, cb, ws, payload=payload, meta=meta)),
              "decode": med(lambda: S.decode(payload, meta, cb, n, out=dst))}
        if S.read_meta(meta).status != 0 or not torch.equal(dst.view(torch.int16),
                                                            x.view(torch.int16)):
            raise AssertionError("round trip failed at 2^%d elements" % k)
        out["2^%d" % k] = {ph: {"us": round(v, 1), "raw_GBps": round(2 * n / v / 1e3, 1)}
                          for ph, v in us.items()}
        del x, payload, dst
    return out


def small_configs(S, W, dev, stream, host_inputs=None, only=None):
    """The smaller single-tensor workloads: one call per phase, median GPU
    time of 20 calls (100 decodes into one output buffer for the linear
    weight), warm (after 3 warm-up calls; they fit the 256 MB last-level
    cache), cold (a 512 MiB buffer is read before each call, so the caches
    hold other, clean data) and cold_dirty (it is written instead: the call
    also pays for writing that buffer's dirty lines back); rates on
    raw and on algorithmic bytes (calibrate 2n, encode and decode 2n plus the
    payload).  With ``host_inputs`` (a dict), each workload's bits are also
    copied to it for the oracle; ``only`` names the one workload to run."""
    import statistics

    import torch

    cfgs = {
        "weight_1m_odd": [W.gaussian_weight(1_000_003, seed=0, device=dev)],
        "kv_layer_8x4096x128": [W.kv_layer(seed=2, stream=kv, device=dev) for kv in (0, 1)],
        "stress_16m_log_uniform": [W.log_uniform_stress(1 << 24, seed=3, stream=0, device=dev)],
        "stress_16m_subnormal": [W.subnormal_gaussian(1 << 24, seed=3, stream=1, device=dev)],
        "linear_weight_12288x3072": [W.weight_with_outliers(seed=4, device=dev)],
    }
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ws = S.Workspace(1 << 26, device=dev)

    def gpu_time(fn, reps, mode):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            if mode == "cold":
                scrub.view(torch.int64).sum()
            elif mode == "cold_dirty":
                scrub.fill_(1)
            torch.cuda._sleep(100_000)      # keep the GPU busy while the call is enqueued
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(ts)

    out = {}
    for name, xs in cfgs.items():
        if only and name != only:
            continue
        rec = {"tensors": len(xs), "elements": sum(x.numel() for x in xs)}
        comp = esc = 0
        for mode in ("warm", "cold", "cold_dirty"):
            us = {"calibrate": 0.0, "encode": 0.0, "decode": 0.0}
            for x in xs:
                cb = S.calibrate(x, ws)
                payload, meta = S.encode(x, cb, ws)
                dst = torch.empty(x.numel(), dtype=torch.bfloat16, device=dev)
                reps = 100 if name.startswith("linear") else 20
                us["calibrate"] += gpu_time(lambda: S.calibrate(x, ws, cb=cb), 20, mode)
                us["encode"] += gpu_time(lambda: S.encode(x, cb, ws, payload=payload, meta=meta),
                                         20, mode)
                us["decode"] += gpu_time(lambda: S.decode(payload, meta, cb, x.numel(), out=dst),
                                         reps, mode)
                if not torch.equal(dst.view(torch.int16), x.reshape(-1).view(torch.int16)):
                    raise AssertionError("round trip failed on " + name)
                if mode == "warm":
                    m = S.read_meta(meta)
                    comp += m.comp_bytes
                    esc += m.n_esc
            raw = 2 * rec["elements"]
            alg = {"calibrate": raw, "encode": raw + comp, "decode": comp + raw}
            rec[mode] = {k: {"us": round(v, 2), "raw_GBps": round(raw / v / 1e3, 1),
                             "alg_GBps": round(alg[k] / v / 1e3, 1),
                             "hbm_frac": round(alg[k] / v / 1e3 / HBM_PEAK_GBPS, 4)}
                         for k, v in us.items()}
        rec["payload_over_raw"] = round(comp / (2 * rec["elements"]), 6)
        rec["escape_fraction"] = round(esc / rec["elements"], 6)
        out[name] = rec
        if host_inputs is not None:
            host_inputs[name] = [x.reshape(-1).view(torch.int16).cpu() for x in xs]
    del scrub
    return out


def cpu_small_configs(host_inputs):
    """The oracle (one core) on each smaller workload, per phase: the median
    of 3 runs of each tensor's calibrate, encode and decode."""
    import statistics

    import numpy as np

    import oracle

    o = oracle.default()
    res = {}
    for name, xs in host_inputs.items():
        ms = {"calibrate": 0.0, "encode": 0.0, "decode": 0.0}
        elems = 0
        for xt in xs:
            a = xt.numpy().view(np.uint16)
            elems += a.size
            ts = {k: [] for k in ms}
            for _ in range(3):
                t0 = time.perf_counter()
                cb = o.calibrate(a)
                t1 = time.perf_counter()
                payload, meta = o.encode(a, cb)
                t2 = time.perf_counter()
                back = o.decode(payload, meta, cb.dec_lut)
                t3 = time.perf_counter()
                for k, dt in zip(ms, (t1 - t0, t2 - t1, t3 - t2)):
                    ts[k].append(dt * 1e3)
            if not np.array_equal(back, a):
                raise AssertionError("oracle round trip failed on " + name)
            for k in ms:
                ms[k] += statistics.median(ts[k])
        res[name] = {k: {"ms": round(v, 3), "raw_GBps": round(2 * elems / v / 1e6, 3)}
                     for k, v in ms.items()}
    return res


def slot_decode_phase(S, batch, metas_h, x_all, stream, passes):
    """In-place decode of every tensor: each payload is first copied into the
    head of the tensor's output buffer (untimed, all 64 before the timed
    region, so the payloads are not cache-resident), then the 64 slot decodes
    are timed with HIP events on the stream they run on (the GPU kept busy
    while the host enqueues them, so the host's marshalling is not timed):
    one call per tensor, then all 64 as one group (32 per launch), in the
    library's default multi-pass form (as many passes as still fill the
    GPU: two per call, six per group of 32 here); the same in the resident
    form (the GPU has nothing else to run here); and groups in the resident
    form with its first kernel launched cooperatively.  Copies and sleep on
    the same stream; `torch.cuda._sleep` spins 10M cycles."""
    import os
    import torch

    T = len(batch.xs)
    comp = [m.comp_bytes for m in metas_h]
    stash = torch.empty(max(comp), dtype=torch.uint8, device=x_all.device)
    stashes = [torch.empty(c, dtype=torch.uint8, device=x_all.device) for c in comp]
    slots = [o.view(torch.uint8) for o in batch.outs]

    def timed(grouped, resident):
        ms = 0.0
        for k in range(passes + 1):   # the first pass untimed (first use of a launch form)
            for i in range(T):
                slots[i][: comp[i]].copy_(batch.payloads[i][: comp[i]])
            # keep the GPU busy while the host marshals and enqueues the calls
            torch.cuda._sleep(10_000_000)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if grouped:
                S.decode_slots(slots, batch.metas, batch.cbs, batch.ns, stashes, stream=stream,
                               resident=resident)
            else:
                for i in range(T):
                    S.decode_slot(slots[i], batch.metas[i], batch.cbs[i], batch.ns[i], stash,
                                  stream=stream, resident=resident)
            e1.record(stream)
            torch.cuda.synchronize()
            if k:
                ms += e0.elapsed_time(e1)
        assert torch.equal(torch.stack(batch.outs).view(torch.int16), x_all.view(torch.int16)), \
            "in-place round trip failed"
        return ms / passes

    raw = 2 * sum(batch.ns)
    alg = raw + sum(comp)

    def rec(ms):
        return {"ms": round(ms, 4), "raw_GBps": round(raw / ms / 1e6, 1),
                "alg_GBps": round(alg / ms / 1e6, 1), "hbm_frac": round(alg / ms / 1e6 / 8000.0, 4)}

    old = os.environ.pop("SPLITZIP_SLOT_LAUNCH", None)
    try:
        ms, ms_b = timed(False, False), timed(True, False)
        msr, msr_b = timed(False, True), timed(True, True)
        os.environ["SPLITZIP_SLOT_LAUNCH"] = "coop"
        msc_b = timed(True, True)
    finally:
        if old is None:
            os.environ.pop("SPLITZIP_SLOT_LAUNCH", None)
        else:
            os.environ["SPLITZIP_SLOT_LAUNCH"] = old
    del stashes
    return dict(rec(ms), calls=T, form="multi-pass form (two kernels per call)",
                batched=dict(rec(ms_b), launches=(T + 31) // 32,
                             form="multi-pass form, six kernels per 32 slots"),
                resident=dict(rec(msr), form="resident form, ordinary launch (+ a finishing "
                                             "kernel) per call"),
                batched_resident=dict(rec(msr_b), form="resident form, one ordinary launch per "
                                                       "32 slots (+ a finishing kernel)"),
                batched_cooperative=rec(msc_b),
                note="payload at the head of the output buffer; resident form: the inputs of "
                     "the tiles whose output overlaps it wait in registers across a grid "
                     "barrier; multi-pass form: the packed nibbles of those tiles, and the "
                     "sign/mantissa bytes of the last pass's tiles, are stashed first (written "
                     "and read once more), the other tiles decoded in passes ordered so that no "
                     "output overwrites an input still to be read")


def h2d_pipeline(S, batch, metas_h, x_all, dev, count):
    """Host-to-device transfer of `count` KV tensors: raw BF16 copies from
    pinned memory, against payload copies into the slot heads on a copy
    stream with the in-place decodes on a second stream (each waits on its
    copy's event).  Rates count raw BF16 bytes delivered to HBM."""
    import torch

    count = min(count, len(batch.xs))
    comp = [metas_h[i].comp_bytes for i in range(count)]
    host_raw = [torch.empty(batch.ns[i], dtype=torch.bfloat16, pin_memory=True)
                for i in range(count)]
    host_pay = [torch.empty(c, dtype=torch.uint8, pin_memory=True) for c in comp]
    for i in range(count):
        host_raw[i].copy_(x_all[i])
        host_pay[i].copy_(batch.payloads[i][: comp[i]])
    slots = [batch.outs[i].view(torch.uint8) for i in range(count)]
    stash = torch.empty(max(comp), dtype=torch.uint8, device=dev)
    copy_s, dec_s = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    raw = 2 * sum(batch.ns[:count])

    def run_raw():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(copy_s)
        with torch.cuda.stream(copy_s):
            for i in range(count):
                batch.outs[i].copy_(host_raw[i], non_blocking=True)
        e1.record(copy_s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def run_pipe():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(copy_s)
        dec_s.wait_event(e0)
        for i in range(count):
            with torch.cuda.stream(copy_s):
                slots[i][: comp[i]].copy_(host_pay[i], non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(copy_s)
            dec_s.wait_event(ev)
            S.decode_slot(slots[i], batch.metas[i], batch.cbs[i], batch.ns[i], stash, stream=dec_s)
        e1.record(dec_s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def run_zero_copy():
        # the payloads stay in pinned host memory; the decode reads them over
        # the link while it decodes (one kernel per tensor, no slot, no copy)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(dec_s)
        for i in range(count):
            S.decode(host_pay[i], batch.metas[i], batch.cbs[i], batch.ns[i], out=batch.outs[i],
                     stream=dec_s)
        e1.record(dec_s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run_raw(), run_pipe(), run_zero_copy()     # warm up
    raw_ms = min(run_raw() for _ in range(3))
    zc_ms = min(run_zero_copy() for _ in range(3))
    ok_zc = all(torch.equal(batch.outs[i].view(torch.int16), x_all[i].view(torch.int16))
                for i in range(count))
    assert ok_zc, "decode from pinned host memory failed"
    pipe_ms = min(run_pipe() for _ in range(3))

    # the other direction: raw copies to pinned host memory, against encoding
    # straight into it (the kernels write the payload over the link)
    host_enc = [torch.empty(c + 64, dtype=torch.uint8, pin_memory=True) for c in comp]
    enc_metas = [torch.zeros_like(batch.metas[i]) for i in range(count)]
    ws = S.Workspace(max(batch.ns[:count]), device=dev)

    def run_raw_d2h():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(copy_s)
        with torch.cuda.stream(copy_s):
            for i in range(count):
                host_raw[i].copy_(x_all[i], non_blocking=True)
        e1.record(copy_s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def run_encode_to_host():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(dec_s)
        for i in range(count):
            S.encode(x_all[i], batch.cbs[i], ws, payload=host_enc[i], meta=enc_metas[i],
                     stream=dec_s)
        e1.record(dec_s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run_raw_d2h(), run_encode_to_host()
    d2h_ms = min(run_raw_d2h() for _ in range(3))
    enc_host_ms = min(run_encode_to_host() for _ in range(3))
    for i in range(count):
        m = S.read_meta(enc_metas[i])
        assert m.status == 0 and m.comp_bytes == comp[i], "encode into host memory failed"
        assert torch.equal(host_enc[i][: comp[i]], host_pay[i]), "encode into host memory differs"
    ok = all(torch.equal(batch.outs[i].view(torch.int16), x_all[i].view(torch.int16))
             for i in range(count))
    assert ok, "pipelined in-place round trip failed"
    return {"tensors": count, "raw_bytes": raw, "payload_bytes": sum(comp),
            "raw_h2d_ms": round(raw_ms, 3), "raw_h2d_GBps": round(raw / raw_ms / 1e6, 1),
            "splitzip_ms": round(pipe_ms, 3),
            "splitzip_effective_GBps": round(raw / pipe_ms / 1e6, 1),
            "speedup": round(raw_ms / pipe_ms, 3),
            "zero_copy_decode_ms": round(zc_ms, 3),
            "zero_copy_decode_effective_GBps": round(raw / zc_ms / 1e6, 1),
            "zero_copy_speedup": round(raw_ms / zc_ms, 3),
            "raw_d2h_GBps": round(raw / d2h_ms / 1e6, 1),
            "encode_to_host_effective_GBps": round(raw / enc_host_ms / 1e6, 1),
            "encode_to_host_speedup": round(d2h_ms / enc_host_ms, 3),
            "note": "pinned host memory; PCIe-inclusive; best of 3"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark runs on exactly one GPU; --gpus %d is not supported "
              "(the codec shards across GPUs by tensor or by chunk range; that path is not built)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import lossless_bf16_tensor_splitzip_amd as S
    from lossless_bf16_tensor_splitzip_amd import _abi
    import workloads as W

    lib = S.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    if args.probes:
        print(json.dumps({"probes": design_probes(S, dev), "device": torch.cuda.get_device_name(dev)}))
        return
    if args.sizes:
        print(json.dumps({"single_call_sizes": single_call_sizes(S, W, dev, stream)}))
        return
    if args.small_only:
        only = None if args.small_only == "all" else args.small_only
        line = {"small_configs": small_configs(S, W, dev, stream, only=only)}
        if args.copy_calibration:
            copy_calibration(torch, dev)
            line["copy_calibration_bytes"] = 512 << 20
        print(json.dumps(line))
        return
    T = 2 * LAYERS

    # inputs, generated on the GPU, resident in HBM
    x_all = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
    for layer in range(LAYERS):
        for kv in range(2):
            x_all[2 * layer + kv] = W.kv_cache_tensor(layer, kv, device=dev).reshape(-1)
    # payload buffers sized by a first (untimed) calibrate: each tensor's
    # payload under its own codebook, not the all-escape bound (3.2 GB
    # instead of 18 GB for the workload)
    batch = S.Batch([x_all[i] for i in range(T)], capacities=[16] * T)
    ws = S.Workspace(N, device=dev, batch_ns=batch.ns)
    batch.calibrate(ws)
    batch.fit_payloads()
    torch.cuda.synchronize()

    items, wsp, wsb = batch.items, ws.ptr(), ws.nbytes
    cal_b, enc_b, dec_b = (lib.splitzip_calibrate_batch, lib.splitzip_encode_batch,
                           lib.splitzip_decode_batch)

    def check(name, rc):
        if rc:
            raise _abi.SplitZipError(name, rc)

    def step(evs=None):
        """One pass of the hot path over the workload: calibrate all, encode
        all, decode all (batched calls, up to 32 tensors per launch)."""
        if evs:
            evs[0].record(stream)
        check("splitzip_calibrate_batch", cal_b(items, T, wsp, wsb, sh))
        if evs:
            evs[1].record(stream)
        check("splitzip_encode_batch", enc_b(items, T, wsp, wsb, sh))
        if evs:
            evs[2].record(stream)
        check("splitzip_decode_batch", dec_b(items, T, None, sh))
        if evs:
            evs[3].record(stream)

    xp = [batch.xs[i].data_ptr() for i in range(T)]
    pp = [batch.payloads[i].data_ptr() for i in range(T)]
    op = [batch.outs[i].data_ptr() for i in range(T)]
    cp = [batch.cbs[i].data_ptr() for i in range(T)]
    mp = [batch.metas[i].data_ptr() for i in range(T)]
    caps = [batch.payloads[i].numel() for i in range(T)]
    lut_off = _abi.DEC_LUT_OFFSET
    cal, enc, dec = lib.splitzip_calibrate, lib.splitzip_encode, lib.splitzip_decode

    def step_per_call(evs=None):
        """The same pass with one single-tensor call per tensor and phase."""
        if evs:
            evs[0].record(stream)
        for i in range(T):
            check("splitzip_calibrate", cal(xp[i], N, cp[i], wsp, wsb, sh))
        if evs:
            evs[1].record(stream)
        for i in range(T):
            check("splitzip_encode", enc(xp[i], N, cp[i], pp[i], caps[i], mp[i], wsp, wsb, sh))
        if evs:
            evs[2].record(stream)
        for i in range(T):
            check("splitzip_decode", dec(pp[i], caps[i], mp[i], cp[i] + lut_off, op[i], N, 0, sh))
        if evs:
            evs[3].record(stream)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            fn(evs[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = {"calibrate": 0.0, "encode": 0.0, "decode": 0.0}
        for e in evs:
            ms["calibrate"] += e[0].elapsed_time(e[1])
            ms["encode"] += e[1].elapsed_time(e[2])
            ms["decode"] += e[2].elapsed_time(e[3])
        return {k: v / steps for k, v in ms.items()}, wall / steps

    def verify():
        # correctness of the timed work: every tensor round-trips bit for bit
        assert torch.equal(torch.stack(batch.outs).view(torch.int16),
                           x_all.view(torch.int16)), "round trip failed"
        ms_ = [S.read_meta(batch.metas[i]) for i in range(T)]
        assert all(m.status == 0 for m in ms_)
        return ms_

    per_call_ms, _ = timed(step_per_call, max(2, args.steps // 2), 1)
    verify()
    for o in batch.outs:
        o.zero_()
    phase_ms, wall = timed(step, args.steps, args.warmup)
    metas_h = verify()
    step_ms = sum(phase_ms.values())
    comp_total = sum(m.comp_bytes for m in metas_h)
    esc_total = sum(m.n_esc for m in metas_h)
    covered = sum(m.covered for m in metas_h)
    raw_bytes = 2 * N * T

    def gbps(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    # algorithmic bytes (what the method must move) per phase
    alg = {"calibrate": raw_bytes, "encode": raw_bytes + comp_total, "decode": comp_total + raw_bytes}
    launches = (T + 31) // 32           # tensors share launches 32 at a time
    phases = {}
    for k, ms in phase_ms.items():
        phases[k] = {"ms": round(ms, 4), "launches": launches,
                     "ms_per_launch": round(ms / launches, 4),
                     "raw_GBps": round(gbps(raw_bytes, ms), 1),
                     "alg_bytes_per_launch": alg[k] // launches,
                     "alg_GBps": round(gbps(alg[k], ms), 1),
                     "hbm_frac": round(gbps(alg[k], ms) / HBM_PEAK_GBPS, 4)}
    per_call = {k: {"ms": round(v, 4), "raw_GBps": round(gbps(raw_bytes, v), 1),
                    "alg_GBps": round(gbps(alg[k], v), 1)} for k, v in per_call_ms.items()}
    # Roofline of the dominant kernel: the decode kernel and the main encode
    # kernel are the two longest of the step, about equally long; the decode
    # phase is that one kernel, so its event time is the kernel's time (the
    # encode phase is three launches: main, count sums, escape placement).
    dom = "decode"
    achieved = gbps(alg[dom], phase_ms[dom])
    roofline = {"bound": "hbm", "kernel": "k_decode<4>", "phase": dom,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": counted_traffic("k_decode<4>"),
                "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                "alg_bytes_per_launch": alg[dom] // launches,
                "ms_per_launch": round(phase_ms[dom] / launches, 4)}
    # The main encode kernel is as long as the decode kernel (the longer of
    # the two in the kernel trace).  Its phase also holds the placement
    # launches, so the event-timed figure below is a lower bound for the
    # kernel itself; the kernel trace's duration of the same source, when
    # the committed summary matches it, gives the kernel's own rate.
    enc_trace = traced_duration_us("k_encode", 131072)
    roofline_encode = {
        "bound": "hbm", "kernel": "k_encode", "phase": "encode", "peak": HBM_PEAK_GBPS,
        "unit": "GB/s", "alg_bytes_per_launch": alg["encode"] // launches,
        "phase_achieved": round(gbps(alg["encode"], phase_ms["encode"]), 1),
        "phase_frac": round(gbps(alg["encode"], phase_ms["encode"]) / HBM_PEAK_GBPS, 4),
        "phase_ms_per_launch": round(phase_ms["encode"] / launches, 4),
        "kernel_trace_us": enc_trace,
        "kernel_trace_frac": (round(alg["encode"] / launches / (enc_trace * 1e-6) / 1e9
                                    / HBM_PEAK_GBPS, 4) if enc_trace else None),
        "traffic": counted_traffic("k_encode")}

    slot = slot_decode_phase(S, batch, metas_h, x_all, stream, max(2, args.steps // 2))
    copy = d2d_copy(x_all, stream)
    ceilings = pattern_ceilings(S, x_all, phases, stream, max(3, args.steps))
    small_inputs = None if args.no_cpu_baseline else {}
    small = None if args.no_small else small_configs(S, W, dev, stream, small_inputs)
    h2d = None if args.no_h2d else h2d_pipeline(S, batch, metas_h, x_all, dev, args.h2d_tensors)
    if h2d:
        # the decode must outrun the link it sits behind (raw bytes per second)
        h2d["decode_over_raw_h2d"] = round(phases["decode"]["raw_GBps"] / h2d["raw_h2d_GBps"], 1)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x_all, args.cpu_seconds)
        if small_inputs:
            cpu["small_configs"] = cpu_small_configs(small_inputs)

    line = {
        "metric": METRIC,
        "value": round(gbps(raw_bytes, step_ms), 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": "kv_stream_32x2x8x32768x128", "tensors": T,
                   "elements_per_tensor": N, "raw_bytes": raw_bytes,
                   "values": "N(0,0.02) bf16, seed 5, stream 2*layer+kv",
                   "codebook": "one per tensor",
                   "step": "calibrate all, encode all, decode all (batched calls)"},
        "encode_GBps": phases["encode"]["raw_GBps"],
        "decode_GBps": phases["decode"]["raw_GBps"],
        "calibrate_GBps": phases["calibrate"]["raw_GBps"],
        "payload_over_raw": round(comp_total / raw_bytes, 6),
        "raw_over_payload": round(raw_bytes / comp_total, 4),
        "n_esc_total": esc_total,
        "coverage": round(covered / (N * T), 6),
        "phases": phases,
        "per_call_phases": per_call,
        "d2d_copy": copy,
        "pattern_ceilings": ceilings,
        "slot_decode": slot,
        "small_configs": small,
        "h2d_pipeline": h2d,
        "roofline": roofline,
        "roofline_encode": roofline_encode,
        "cpu_baseline": cpu,
        "context_h200": {"encode_GBps": 613, "decode_GBps": 2182,
                         "note": "pages' figures on LLM KV activations, other hardware"},
    }
    if args.copy_calibration:
        copy_calibration(torch, dev)
        line["copy_calibration_bytes"] = 512 << 20
    print(json.dumps(line))


def copy_calibration(torch, dev):
    """One 512 MiB device-to-device copy, the last dispatch of the run: the
    reference for scaling hardware byte counters."""
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def counted_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel source has changed since it was taken."""
    import hashlib

    src = os.path.join(ROOT, "lossless_bf16_tensor_splitzip_amd", "csrc", "splitzip.hip")
    summary = os.path.join(ROOT, "profiles", "kv_stream_4gib_hbm_counters.md")
    try:
        lines = open(summary).read().splitlines()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    recorded = [ln.split()[1] for ln in lines if ln.startswith("source_sha256 ")]
    if not recorded or recorded[0] != sha:
        return None
    for ln in lines:
        parts = ln.split()
        if len(parts) == 3 and parts[0] == "traffic_bytes_per_launch" and parts[1] == kernel:
            return int(parts[2])
    return None


def traced_duration_us(kernel, workgroups):
    """Mean duration of `kernel` at that launch shape from the committed
    kernel-trace summary, or None when the kernel source has changed since
    it was taken."""
    import hashlib

    src = os.path.join(ROOT, "lossless_bf16_tensor_splitzip_amd", "csrc", "splitzip.hip")
    summary = os.path.join(ROOT, "profiles", "kv_stream_4gib_kernel_trace.md")
    try:
        lines = open(summary).read().splitlines()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    recorded = [ln.split()[1] for ln in lines if ln.startswith("source_sha256 ")]
    if not recorded or recorded[0] != sha:
        return None
    for ln in lines:
        parts = ln.split()
        if (len(parts) == 4 and parts[0] == "duration_us" and parts[1] == kernel
                and parts[2] == str(workgroups)):
            return float(parts[3])
    return None


def cpu_baseline(x_all, budget_s):
    """The oracle as it stands (plain single-threaded C), on whole tensors of
    the same workload until the time budget is spent."""
    import numpy as np
    import torch

    import oracle

    o = oracle.default()
    done, t_cpu = 0, 0.0
    t_ph = [0.0, 0.0, 0.0]
    while done < x_all.shape[0] and (t_cpu < budget_s or done == 0):
        xs = x_all[done].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        cb = o.calibrate(xs)
        t1 = time.perf_counter()
        payload, meta = o.encode(xs, cb)
        t2 = time.perf_counter()
        out = o.decode(payload, meta, cb.dec_lut)
        t3 = time.perf_counter()
        t_cpu += t3 - t0
        for k, dt in enumerate((t1 - t0, t2 - t1, t3 - t2)):
            t_ph[k] += dt
        if not np.array_equal(out, xs):
            raise AssertionError("oracle round trip failed on tensor %d" % done)
        done += 1
    raw = 2 * N * done
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(raw / t_cpu / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d of 64 tensors (calibrate+encode+decode each), %.1f s" % (done, t_cpu),
            "phases_GBps": {k: round(raw / t / 1e9, 3)
                            for k, t in zip(("calibrate", "encode", "decode"), t_ph)},
            "host": {"nproc": os.cpu_count(), "cpu": model}}


if __name__ == "__main__":
    main()
