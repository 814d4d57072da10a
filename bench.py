"""Decode throughput of a stack of quantised MoE layers on one MI355X.

One step = one token through the whole stack (router, top-k, packed gate|up dequant-GEMV with
SwiGLU, down dequant-GEMV, weighted combine with the shared expert, for every layer, the layers
chained by the RMS glue), i.e. one moe_stack_decode call. The default workload is the
Qwen3.6-35B-A3B-shaped 4-bit stack: 40 layers, H 2048, 256 experts, top-8, I 512, shared
expert 512, group-64 bf16 scale/bias, seeded synthetic weights resident in HBM; each step gets a
fresh seeded input so routing changes every step.

Prints one JSON line with the throughput, the HBM roofline of the decode kernel (algorithmic
bytes per launch / its average launch duration, timed with HIP events on the launch stream),
the fp64 CPU oracle timed on a bounded sample, and a "batched" leg: the same weights with a
Zipf(1.1) router bias, T = 512 tokens per layer call through moe_layer_batched, reporting its
MFMA utilisation against the fp16 dense peak.
"""
import argparse
import dataclasses
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tokens/s and achieved HBM GB/s (% of peak), 4-bit 35B shape"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
FP16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, published


# The sources the decode kernel is compiled from (its device code and the launch-plan header):
# counter figures taken on the decode kernel stay valid while these are unchanged.
DECODE_SOURCES = ("decode.hip", "moe_device.hpp", "moe_internal.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "quantized_moe_decode_router_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel: str):
    """Per-launch HBM bytes from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _oracle_rate(layers, wl, budget_s: float):
    """Layer-tokens per second of the oracle on `layers`, tokens chained through them."""
    import numpy as np
    import torch

    import oracle
    import synth
    layer_tokens = 0
    tokens = 0
    t0 = time.perf_counter()
    while True:
        xb = synth.make_x(wl.shape, 1, wl.seed, step=10_000 + tokens).view(torch.int16).numpy().view(np.uint16)
        for L in layers:
            out = oracle.layer_forward(L, xb)
            xb = oracle.rms_glue(out["y"][0], 1e-6)[None, :]
            layer_tokens += 1
        tokens += 1
        el = time.perf_counter() - t0
        if el >= budget_s and tokens >= 2:
            break
    return layer_tokens / el, tokens, el


def cpu_baseline(stack, wl, budget_s: float):
    """The oracle as it stands, on this host's cores (every core, then one thread), on a bounded
    sample: the first `n` layers of the same stack, tokens chained through them for ~budget_s each;
    tokens/s = 1 / (time per layer-token x the stack's layers)."""
    import oracle
    from tests.helpers import host_layer

    n = min(8, wl.n_layers)
    layers = [host_layer(stack, l) for l in range(n)]
    threads = oracle.num_threads()
    rate, tokens, el = _oracle_rate(layers, wl, budget_s)
    oracle.set_num_threads(1)
    try:
        rate1, tokens1, el1 = _oracle_rate(layers, wl, budget_s)
    finally:
        oracle.set_num_threads(threads)
    return {"value": rate / wl.n_layers, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{tokens} tokens x first {n} of {wl.n_layers} layers (T=1, chained by the glue), "
                      f"{el:.1f} s on {threads} threads; tokens/s = 1 / (time per layer-token x {wl.n_layers} layers)",
            "single_thread": {"value": rate1 / wl.n_layers, "unit": "tokens/s", "cores": 1,
                              "sample": f"{tokens1} tokens x first {n} layers, {el1:.1f} s"}}


def batched_leg(stack, steps: int, warmup: int):
    """T = 512 tokens through every layer of the stack (each layer called on the step's input)
    with moe_layer_batched; the Zipf(1.1) router bias of the batched workload is attached to the
    same weights. Reports the MFMA utilisation (algorithmic flops, router included, over the fp16
    dense peak) and the fraction of the attainable roofline max(t_HBM, t_MFMA) / t, with t_HBM the
    algorithmic bytes (touched experts of every layer, shared expert, router, x, y) over 8 TB/s."""
    import torch

    import quantized_moe_decode_router_amd as moe
    import synth

    wl = synth.QWEN35B_BATCHED
    shape, T, L = wl.shape, wl.tokens, stack.n_layers
    H, E, K, I, Is = shape.hidden, shape.num_experts, shape.top_k, shape.inter, shape.shared_inter
    dev = stack.router.device
    sb = synth.with_zipf_bias(stack, wl.seed, wl.zipf_s)
    layers = [sb.layer(l) for l in range(L)]
    n = warmup + steps
    xs = [synth.make_x(shape, T, wl.seed, step=s, device=dev) for s in range(n)]
    y = torch.empty(T, H, dtype=torch.float32, device=dev)
    idx = torch.empty(L, T, K, dtype=torch.int32, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_BATCHED, dev)
    stream = torch.cuda.current_stream()

    def step(s):
        for l in range(L):
            moe.moe_layer_batched(shape, layers[l], xs[s], T, y, idx[l], workspace=ws, stream=stream)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for s in range(warmup, n):
        step(s)
    b.record(stream)
    torch.cuda.synchronize()
    if moe.moe_read_status(ws) != 0:
        raise SystemExit("batched leg: device status is not OK")
    ms = a.elapsed_time(b) / steps
    per_layer_us = ms * 1e3 / L
    flops = 2.0 * T * (E + 1) * H + 6.0 * T * K * I * H + 6.0 * T * Is * H
    tflops = flops / (per_layer_us * 1e-6) / 1e12
    touched = [int((torch.bincount(idx[l].view(-1).long(), minlength=E) > 0).sum().item()) for l in range(L)]
    counts = torch.bincount(idx[L - 1].view(-1).long(), minlength=E)
    bytes_layer = (sum(touched) / L * shape.expert_bytes() + shape.expert_bytes(Is) + 4 * (E + 1) * H
                   + 2 * T * H + 4 * T * H)
    t_hbm = bytes_layer / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (FP16_PEAK_TFLOPS * 1e12)
    return {"workload": wl.name, "tokens_per_call": T, "layers": L, "steps": steps,
            "ms_per_step": round(ms, 4), "us_per_layer": round(per_layer_us, 2),
            "layer_tokens_per_s": round(T * L / (ms / 1e3), 1),
            "mfma": {"dtype": "fp16", "algorithmic_tflop_per_layer": round(flops / 1e12, 4),
                     "achieved_tflops": round(tflops, 1), "peak_tflops": FP16_PEAK_TFLOPS,
                     "utilisation": round(tflops / FP16_PEAK_TFLOPS, 4)},
            "roofline": {"algorithmic_bytes_per_layer": int(bytes_layer), "t_hbm_us": round(t_hbm * 1e6, 2),
                         "t_mfma_us": round(t_mfma * 1e6, 2),
                         "attainable_frac": round(max(t_hbm, t_mfma) / (per_layer_us * 1e-6), 4)},
            "experts_touched_mean": round(sum(touched) / L, 1),
            "last_layer_experts_touched": touched[-1],
            "last_layer_max_load": int(counts.max().item())}


SWEEP_TOKENS = list(range(1, 17)) + [32, 64, 128, 512]


def crossover_sweep(stack, reps: int):
    """One layer (layer 0 of the stack, no router bias) through moe_layer_decode (T <= 8) and
    moe_layer_batched for every T of SWEEP_TOKENS: the mean time per call over `reps` calls after
    a warm-up, and the largest T at which the decode path is the faster one (below it every
    decode-capable T is faster too)."""
    import torch

    import quantized_moe_decode_router_amd as moe
    import synth

    shape, dev = stack.shape, stack.router.device
    layer = stack.layer(0)
    stream = torch.cuda.current_stream()
    rows = []
    for T in SWEEP_TOKENS:
        x = synth.make_x(shape, T, 7, step=T, device=dev)
        y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
        row = {"tokens": T}
        paths = [("batched", moe.MOE_WS_BATCHED, moe.moe_layer_batched)]
        if T <= 8:
            paths.insert(0, ("decode", moe.MOE_WS_DECODE, moe.moe_layer_decode))
        for name, kind, fn in paths:
            ws = moe.workspace(shape, T, kind, dev)
            for _ in range(5):
                fn(shape, layer, x, T, y, workspace=ws, stream=stream)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn(shape, layer, x, T, y, workspace=ws, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            row[name + "_us"] = round(us, 2)
            row[name + "_us_per_token"] = round(us / T, 3)
        rows.append(row)
        print(f"[sweep] T={T}: " + ", ".join(f"{k} {v}" for k, v in row.items() if k != "tokens"),
              file=sys.stderr, flush=True)
    cross = 0
    for row in rows:
        if "decode_us" in row and row["decode_us"] <= row["batched_us"]:
            cross = row["tokens"]
        elif "decode_us" in row:
            break
    return {"workload": stack_name(stack), "layer": 0, "reps": reps, "rows": rows, "crossover": cross}


RESIDENCY_FRACTIONS = [0.0, 0.05, 0.1, 0.25, 0.5, 1.0]


def residency_sweep(stack, wl, warmup: int, steps: int, zipf_s):
    """The decode stack with its routed experts in a fixed-stride container in pinned host memory
    and a bounded HBM pool (LFU + recency) in front of it, for each pool size in
    RESIDENCY_FRACTIONS (fraction of the L * E experts): per token one moe_stack_decode_table call,
    the routing read back, and moe_cache_update (policy, admissions copied into the pool, table
    rewritten). Reports tokens/s of that loop (host work and copies included), the kernel's own
    time per call, the hit rate over the timed tokens and the bytes copied per token, with and
    without a landing buffer (misses written through by the decode, admitted device to device), for each
    router bias in zipf_s: None (no bias: every expert equally likely, the least locality) or a
    Zipf(s) bias per layer, standing in for the expert popularity skew of real text. Every layer
    routes the step's own token (MOE_STACK_INDEPENDENT): chained through the weightless RMS glue,
    these random-weight layers lose the token's identity within a few layers and from about the
    ninth on route every token to the same experts, which would make any cache look perfect."""
    import ctypes

    import torch

    import quantized_moe_decode_router_amd as moe
    import synth

    shape, T, L = wl.shape, wl.tokens, wl.n_layers
    E, K = shape.num_experts, shape.top_k
    dev = stack.router.device
    stride = moe.moe_expert_stride(shape)
    nbytes = L * E * stride
    hip = ctypes.CDLL("libamdhip64.so")
    hbuf = ctypes.c_void_p()
    if hip.hipHostMalloc(ctypes.byref(hbuf), ctypes.c_size_t(nbytes + 4096), ctypes.c_uint(0)) != 0:
        raise SystemExit("hipHostMalloc of the expert container failed")
    base = (hbuf.value + 4095) // 4096 * 4096
    container = (base, nbytes)
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    moe.moe_pack_experts(shape, stack, L, container, stream=stream)
    torch.cuda.synchronize()
    print(f"[residency] packed {nbytes / 1e9:.2f} GB into pinned host memory in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    nsteps = warmup + steps
    xs = torch.stack([synth.make_x(shape, T, wl.seed, step=s, device=dev) for s in range(nsteps)])
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    idx = torch.empty(L, T, K, dtype=torch.int32, device=dev)
    idx_h = torch.empty(L, T, K, dtype=torch.int32, pin_memory=True)
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    table = torch.empty(L * E, dtype=torch.int64, device=dev)
    rows = []
    # the same loop's decode with every expert resident in its stacked arrays (no table, no cache)
    for s in range(warmup):
        moe.moe_stack_decode(shape, stack, L, xs[s], T, y, workspace=ws, stream=stream, flags=moe.MOE_STACK_INDEPENDENT)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for s in range(warmup, nsteps):
        moe.moe_stack_decode(shape, stack, L, xs[s], T, y, workspace=ws, stream=stream, flags=moe.MOE_STACK_INDEPENDENT)
    b.record(stream)
    torch.cuda.synchronize()
    resident_ms = a.elapsed_time(b) / steps
    print(f"[residency] all experts resident, no table: {resident_ms:.3f} ms per token", file=sys.stderr, flush=True)
    # the table decode with every block in device memory: a copy of the container in HBM
    dbuf = torch.empty(nbytes + 4096, dtype=torch.uint8, device=dev)
    doff = (-dbuf.data_ptr()) % 4096
    moe.moe_pack_experts(shape, stack, L, dbuf[doff:doff + nbytes], stream=stream)
    dtab = (dbuf.data_ptr() + doff + torch.arange(L * E, dtype=torch.int64, device=dev) * stride).contiguous()
    nost0 = dataclasses.replace(stack, w13_codes=None, w13_scales=None, w13_biases=None, w2_codes=None,
                                w2_scales=None, w2_biases=None)
    for s in range(warmup):
        moe.moe_stack_decode_table(shape, nost0, L, dtab, xs[s], T, y, workspace=ws, stream=stream,
                                   flags=moe.MOE_STACK_INDEPENDENT)
    torch.cuda.synchronize()
    a.record(stream)
    for s in range(warmup, nsteps):
        moe.moe_stack_decode_table(shape, nost0, L, dtab, xs[s], T, y, workspace=ws, stream=stream,
                                   flags=moe.MOE_STACK_INDEPENDENT)
    b.record(stream)
    torch.cuda.synchronize()
    table_hbm_ms = a.elapsed_time(b) / steps
    del dbuf, dtab
    print(f"[residency] table decode, every block in HBM: {table_hbm_ms:.3f} ms per token", file=sys.stderr,
          flush=True)
    try:
        land_t = torch.empty(L * T * K * stride + 4096, dtype=torch.uint8, device=dev)
        loff = (-land_t.data_ptr()) % 4096
        land = land_t[loff:loff + L * T * K * stride]
        for zs, through in [(z, f) for z in zipf_s for f in (False, True)]:
            st = stack if zs is None else synth.with_zipf_bias(stack, wl.seed, zs)
            nost = dataclasses.replace(st, w13_codes=None, w13_scales=None, w13_biases=None, w2_codes=None,
                                       w2_scales=None, w2_biases=None)
            for frac in RESIDENCY_FRACTIONS:
                slots = int(round(frac * L * E))
                pool = torch.empty(max(slots, 1) * stride + 4096, dtype=torch.uint8, device=dev)
                off = (-pool.data_ptr()) % 4096
                lnd = land if through else None
                cache = moe.MoeCache(shape, L, container, pool[off:off + max(slots, 1) * stride] if slots else None,
                                     slots, table, stream=stream, landing=lnd)
                kern_ms, hits, misses = 0.0, 0, 0
                b0 = cache.stats()[2]
                for s in range(nsteps):
                    if s == warmup:
                        torch.cuda.synchronize()
                        w0 = time.perf_counter()
                        b0 = cache.stats()[2]
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    moe.moe_stack_decode_table(shape, nost, L, table, xs[s], T, y, topk_idx_all=idx, workspace=ws,
                                               stream=stream, flags=moe.MOE_STACK_INDEPENDENT, landing=lnd)
                    b.record(stream)
                    idx_h.copy_(idx, non_blocking=True)
                    stream.synchronize()
                    h, m = cache.update(idx_h, T, K, stream=stream)
                    if s >= warmup:
                        kern_ms += a.elapsed_time(b)
                        hits, misses = hits + h, misses + m
                torch.cuda.synchronize()
                wall = time.perf_counter() - w0
                if moe.moe_read_status(ws) != 0:
                    raise SystemExit("device status after the residency steps is not OK")
                copied = cache.stats()[2] - b0
                cache.close()
                del pool
                row = {"zipf_s": zs, "write_through": through, "pool_fraction": frac, "slots": slots, "pool_gb": round(slots * stride / 1e9, 2),
                       "tokens_per_s": round(steps * T / wall, 2), "ms_per_token": round(wall * 1e3 / steps, 3),
                       "kernel_ms": round(kern_ms / steps, 3), "hit_rate": round(hits / max(hits + misses, 1), 4),
                       "copied_mb_per_token": round(copied / steps / 1e6, 1)}
                rows.append(row)
                print(f"[residency] {row}", file=sys.stderr, flush=True)
        # prefill through the table: one batched layer (T = 512, Zipf(1.1) router bias) with every
        # routed block read from the pinned container, against the same layer resident in HBM
        Tb = 512
        stb = synth.with_zipf_bias(stack, wl.seed, 1.1)
        nob = dataclasses.replace(stb, w13_codes=None, w13_scales=None, w13_biases=None, w2_codes=None,
                                  w2_scales=None, w2_biases=None)
        xb = synth.make_x(shape, Tb, wl.seed, step=1 << 16, device=dev)
        yb = torch.empty(Tb, shape.hidden, dtype=torch.float32, device=dev)
        wsb = moe.workspace(shape, Tb, moe.MOE_WS_BATCHED, dev)
        row0 = (base + torch.arange(E, dtype=torch.int64, device=dev) * stride).contiguous()
        prefill = {}
        for name, fn in (("resident", lambda: moe.moe_layer_batched(shape, stb.layer(0), xb, Tb, yb, workspace=wsb,
                                                                      stream=stream)),
                         ("from_host", lambda: moe.moe_layer_batched_table(shape, nob.layer(0), row0, xb, Tb, yb,
                                                                            workspace=wsb, stream=stream))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(10):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            prefill[name + "_us_per_layer"] = round(a.elapsed_time(b) * 100, 1)
        # the better order: route, admit the selected experts (one read each), then the layer
        lgb = torch.empty(Tb, E, dtype=torch.float32, device=dev)
        idxb = torch.empty(Tb, K, dtype=torch.int32, device=dev)
        wb = torch.empty(Tb, K, dtype=torch.float32, device=dev)
        poolb = torch.empty(E * stride + 4096, dtype=torch.uint8, device=dev)
        pofb = (-poolb.data_ptr()) % 4096
        tab1 = torch.empty(E, dtype=torch.int64, device=dev)
        tms = []
        for rep in range(4):
            cache = moe.MoeCache(shape, 1, (base, E * stride), poolb[pofb:pofb + E * stride], E, tab1, stream=stream)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            moe.moe_route(shape, stb.layer(0), xb, Tb, lgb, idxb, wb, stream=stream)
            keys = torch.unique(idxb).cpu().numpy()
            cache.admit(keys, stream=stream)
            moe.moe_layer_batched_table(shape, nob.layer(0), tab1, xb, Tb, yb, workspace=wsb, stream=stream)
            torch.cuda.synchronize()
            tms.append(time.perf_counter() - t0)
            cache.close()
        prefill["admit_first_us_per_layer"] = round(min(tms[1:]) * 1e6, 1)
        prefill["experts_admitted"] = int(len(keys))
        print(f"[residency] prefill layer T=512: {prefill}", file=sys.stderr, flush=True)
    finally:
        torch.cuda.synchronize()
        hip.hipHostFree(hbuf)
    return {"workload": wl.name, "resident_kernel_ms": round(resident_ms, 3), "table_all_hbm_kernel_ms": round(table_hbm_ms, 3), "prefill_T512": prefill, "expert_stride": stride, "container_gb": round(nbytes / 1e9, 2),
            "warmup": warmup, "steps": steps, "rows": rows}


PHASE_NAMES = ["layer", "input", "router_rows", "logits_put", "x_limbs", "logits_got", "topk", "shared_gu",
               "routed_issued", "routed_landed", "gu_units", "gu_barrier", "gu_put", "routed_done", "down_issued",
               "h_polled", "h_got", "down_units", "down_done", "y_put", "layer_end"]
REALTIME_HZ = 100e6  # s_memrealtime counts at 100 MHz


def phase_profile(stack, wl, T: int, warmup: int, steps: int, chained: bool):
    """Per-phase timing of the decode kernel from the phase-timer build of the library: every
    workgroup's wave 0 stamps the 100 MHz real-time counter at each phase mark of every layer. For a
    mark m of a layer, crit(m) is the time the last workgroup passed it; the critical-path share of
    phase m is crit(m) - crit(m - 1) (from crit(layer_end) of the previous layer for the first mark),
    the typical share the median over workgroups of their own t(m) - t(m - 1), and the skew the
    spread of the workgroups' t(m). Medians over the steps and the layers 1 .. L-1."""
    import numpy as np
    import torch

    import quantized_moe_decode_router_amd as moe
    import synth

    assert moe.LIB_PATH.endswith("libmoe_amd_phase.so"), "the phase-timer library is not loaded"
    shape, L = wl.shape, stack.n_layers
    dev = stack.router.device
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    nm = len(PHASE_NAMES)
    ph = ws[256:256 + 8 * L * 1024 * nm].view(torch.int64)[: L * grid * nm]
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    flags = 0 if chained else moe.MOE_STACK_INDEPENDENT
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    crit, typ, skew, layer_us, ratio = [], [], [], [], []
    for s in range(warmup + steps):
        x = synth.make_x(shape, T, wl.seed, step=s, device=dev)
        a.record(stream)
        moe.moe_stack_decode(shape, stack, L, x, T, y, workspace=ws, stream=stream, flags=flags)
        b.record(stream)
        torch.cuda.synchronize()
        if s < warmup:
            continue
        t = ph.cpu().numpy().reshape(L, grid, nm).astype(np.float64) / REALTIME_HZ * 1e6  # us
        c = t.max(axis=1)  # [L][nm]: the last workgroup at each mark
        span = t[L - 1, :, nm - 1].max() - t[0, :, 0].min()
        ratio.append(span / (a.elapsed_time(b) * 1e3))
        for l in range(1, L):
            prev = c[l - 1, nm - 1]
            cl = np.concatenate([[prev], c[l]])
            crit.append(np.diff(cl))
            d = np.diff(t[l], axis=1)
            typ.append(np.concatenate([[np.median(t[l, :, 0] - t[l - 1, :, nm - 1])], np.median(d, axis=0)]))
            skew.append(t[l].max(axis=0) - t[l].min(axis=0))
            layer_us.append(c[l, nm - 1] - prev)
    crit, typ, skew = np.median(crit, axis=0), np.median(typ, axis=0), np.median(skew, axis=0)
    rows = [{"phase": f"{PHASE_NAMES[m - 1] if m else 'layer_end(prev)'} -> {PHASE_NAMES[m]}",
             "critical_us": round(float(crit[m]), 3), "typical_us": round(float(typ[m]), 3),
             "skew_at_mark_us": round(float(skew[m]), 3)} for m in range(nm)]
    return {"workload": wl.name, "tokens_per_step": T, "layers": L, "chained": chained, "grid": grid,
            "steps": steps, "layer_us_median": round(float(np.median(layer_us)), 3),
            "stamp_span_over_event_time": round(float(np.median(ratio)), 4), "phases": rows}


def stack_name(stack) -> str:
    s = stack.shape
    return f"H{s.hidden}_E{s.num_experts}_K{s.top_k}_I{s.inter}_Is{s.shared_inter}_{s.bits}bit"


def main():
    import synth
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=0,
                    help="tokens per decode step (1..8; default: the workload's own, 1)")
    ap.add_argument("--workload", default=synth.QWEN35B_4BIT.name,
                    choices=[w.name for w in synth.ALL.values() if w.tokens <= 8 and w.n_layers > 1])
    ap.add_argument("--independent", action="store_true",
                    help="unchained layers (every layer takes the step's input): an upper bound, not decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--batched-steps", type=int, default=10,
                    help="steps of the batched leg (0 skips it)")
    ap.add_argument("--batched-only", action="store_true",
                    help="run only the batched leg (T = 512 per layer call) and print its result")
    ap.add_argument("--residency", action="store_true",
                    help="only the expert-residency sweep over pool sizes (one JSON line)")
    ap.add_argument("--residency-steps", type=int, default=100)
    ap.add_argument("--residency-warmup", type=int, default=100)
    ap.add_argument("--sweep", action="store_true",
                    help="only the decode / batched crossover sweep of one layer (one JSON line)")
    ap.add_argument("--phases", action="store_true",
                    help="only the per-phase timing of the decode kernel, from the phase-timer build (one JSON line)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MoE decode path here is single-GPU (no sharding or "
              "collectives are built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.phases:
        os.environ["MOE_AMD_PHASE_TIMER"] = "1"  # before the binding is imported
    import torch
    import quantized_moe_decode_router_amd as moe

    dev = torch.device("cuda:0")
    wl = synth.ALL[args.workload]
    shape, T, L = wl.shape, wl.tokens, wl.n_layers
    if args.tokens:
        T = args.tokens
    t0 = time.perf_counter()
    stack = synth.make_workload(wl, dev)
    torch.cuda.synchronize()
    print(f"[bench] {wl.describe()}: {stack.nbytes() / 1e9:.2f} GB generated in "
          f"{time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    if args.sweep:
        print(json.dumps({"sweep": crossover_sweep(stack, reps=50)}), flush=True)
        return
    if args.phases:
        print(json.dumps({"phases": phase_profile(stack, wl, T, warmup=args.warmup, steps=args.steps,
                                                  chained=not args.independent)}), flush=True)
        return
    if args.batched_only:
        print(json.dumps({"batched": batched_leg(stack, max(args.batched_steps, 1), 2)}), flush=True)
        return
    if args.residency:
        print(json.dumps({"residency": residency_sweep(stack, wl, warmup=args.residency_warmup,
                                                       steps=args.residency_steps,
                                                       zipf_s=[None, 0.5, 1.1])}), flush=True)
        return
    nsteps = args.warmup + args.steps
    xs = torch.stack([synth.make_x(shape, T, wl.seed, step=s, device=dev) for s in range(nsteps)])
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    flags = moe.MOE_STACK_INDEPENDENT if args.independent else 0
    stream = torch.cuda.current_stream()
    # for T > 1 the routing of every timed step is kept: the bytes a step must move count each
    # distinct routed expert of a layer once
    idx_steps = (torch.empty(args.steps, L, T, shape.top_k, dtype=torch.int32, device=dev) if T > 1 else None)

    def step(s, i=None):
        idx = idx_steps[i] if (idx_steps is not None and i is not None) else None
        moe.moe_stack_decode(shape, stack, L, xs[s], T, y, topk_idx_all=idx, workspace=ws, stream=stream,
                             flags=flags)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    assert moe.moe_read_status(ws) == 0
    # one event pair around every launch: their mean is the kernel's average launch duration
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i, s in enumerate(range(args.warmup, nsteps)):
        evs[i][0].record(stream)
        step(s, i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    status = moe.moe_read_status(ws)
    if status != 0:
        raise SystemExit(f"device status {moe.status_string(status)} after the timed steps")
    total_ms = evs[0][0].elapsed_time(evs[-1][1])
    launch = sorted(a.elapsed_time(b) for a, b in evs)
    launch_ms = sum(launch) / args.steps
    ms_per_step = total_ms / args.steps
    tokens_per_s = args.steps * T / (total_ms / 1e3)
    # trials: the timed steps in (up to) five contiguous runs, tokens/s of each
    ntr = min(5, args.steps)
    bounds = [round(k * args.steps / ntr) for k in range(ntr + 1)]
    trial_tps = sorted((bounds[k + 1] - bounds[k]) * T /
                       (evs[bounds[k]][0].elapsed_time(evs[bounds[k + 1] - 1][1]) / 1e3) for k in range(ntr))

    bytes_per_launch = decode_step_bytes(shape, L, T, idx_steps)
    achieved = bytes_per_launch / (launch_ms / 1e3) / 1e9
    kernel = "decode_kernel"
    traffic = recorded_traffic(wl.name, kernel) if T == 1 else None
    result = {
        "metric": METRIC, "value": round(tokens_per_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded counter-based weights and inputs; no checkpoints)",
        "config": {"workload": wl.name, "layers": L, "tokens_per_step": T, "hidden": shape.hidden,
                   "experts": shape.num_experts, "top_k": shape.top_k, "inter": shape.inter,
                   "shared_inter": shape.shared_inter, "bits": shape.bits, "group": shape.group_size,
                   "stack_gb": round(stack.nbytes() / 1e9, 2), "kernel": kernel,
                   "chained": not args.independent},
        "hbm_gbps": round(achieved, 1), "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "avg_launch_us": round(launch_ms * 1e3, 3)},
        "spread": {"launch_us": {"median": round(_pct(launch, 50) * 1e3, 3), "p10": round(_pct(launch, 10) * 1e3, 3),
                                 "p90": round(_pct(launch, 90) * 1e3, 3)},
                   "trials_tokens_per_s": [round(v, 1) for v in trial_tps],
                   "trial_median": round(_pct(trial_tps, 50), 1), "trial_p10": round(_pct(trial_tps, 10), 1),
                   "trial_p90": round(_pct(trial_tps, 90), 1)},
        "run": run_metadata(wl.seed),
        "cpu_baseline": None,
        "batched": None,
    }
    if args.batched_steps > 0 and shape == synth.QWEN35B_BATCHED.shape:
        result["batched"] = batched_leg(stack, args.batched_steps, 2)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(stack, wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _pct(sorted_vals, q: float) -> float:
    """The q-th percentile of an ascending list (linear interpolation)."""
    n = len(sorted_vals)
    if n == 1:
        return float(sorted_vals[0])
    pos = (n - 1) * q / 100.0
    lo = int(pos)
    hi = min(lo + 1, n - 1)
    return float(sorted_vals[lo] + (sorted_vals[hi] - sorted_vals[lo]) * (pos - lo))


def decode_step_bytes(shape, L: int, T: int, idx_steps=None) -> float:
    """Algorithmic bytes of one decode step of T tokens through L layers, averaged over the timed
    steps: per layer the router, the shared-gate vector and the shared expert once, every distinct
    routed expert the step's tokens selected once (K per layer at T = 1), and x (bf16) and y (fp32)
    per token."""
    E, H = shape.num_experts, shape.hidden
    once = 4 * E * H
    if shape.shared_inter:
        once += 4 * H + shape.expert_bytes(shape.shared_inter)
    per_token = 2 * H + 4 * H
    if idx_steps is None:
        distinct = L * T * shape.top_k  # T == 1: a token's K experts are distinct
    else:
        import torch
        n = idx_steps.shape[0]
        flat = idx_steps.view(n * L, -1).long()
        seen = torch.zeros(n * L, E, dtype=torch.bool, device=flat.device)
        seen.scatter_(1, flat, True)
        distinct = seen.sum().item() / n
    return L * (once + T * per_token) + distinct * shape.expert_bytes()


def run_metadata(seed: int) -> dict:
    """What identifies the run: source revision, device, runtime versions, clocks, seed. Read from
    files only: this process has initialised the GPU, so it starts no other program."""
    import torch
    meta = {"seed": seed, "kernel_source_hash": kernel_source_hash(), "git": _git_head(),
            "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        props = torch.cuda.get_device_properties(0)
        meta["gpu"] = props.name
        meta["arch"] = getattr(props, "gcnArchName", None)
        meta["compute_units"] = props.multi_processor_count
    except Exception:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            meta["rocm"] = f.read().strip()
    except Exception:
        pass
    clocks = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [l.split(":", 1)[1].strip(" *\n") for l in f if l.rstrip().endswith("*")]
                if cur:
                    clocks[f"{os.path.basename(os.path.dirname(dev))}.{name[3:]}"] = cur[0]
            except OSError:
                pass
    meta["clocks"] = clocks or None
    return meta


def _git_head():
    """The checked-out commit from .git (None where the tree was copied without it)."""
    try:
        with open(os.path.join(ROOT, ".git", "HEAD")) as f:
            head = f.read().strip()
        if not head.startswith("ref:"):
            return head[:7]
        ref = head.split(None, 1)[1]
        p = os.path.join(ROOT, ".git", ref)
        if os.path.exists(p):
            with open(p) as f:
                return f.read().strip()[:7]
        with open(os.path.join(ROOT, ".git", "packed-refs")) as f:
            for line in f:
                if line.strip().endswith(ref):
                    return line.split()[0][:7]
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
