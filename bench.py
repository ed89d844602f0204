#!/usr/bin/env python3
"""Benchmark of the signaling-GEMM hot path on one MI355X.

One step = one pass of the whole path over one batch: the signaling GEMM
(stream A) with the consumer and the post-communication reorder (stream B)
running beside it, linked only by the device signals.  Inputs are seeded and
synthetic and already resident in HBM when the timed region starts.

Default workload: the profiled GEMM shape of the pages' wave-pattern figure,
M = 2048, N = K = 8192, bf16, 256 x 128 tiles, 512 tiles over 256 CUs (two
waves).  Schedules: partitions (2) and (1, 1), the consumer gated in the
stream's queue or polling on the CUs, the post-reorder whole or group by
group.  The schedule is chosen from interleaved blocks; then, five times,
W warm-up passes and exactly K timed passes (synchronised on both sides,
host clock, with device events around the region, and every GEMM bracketed
by events on its own stream for the roofline); ``value`` is useful
GEMM TFLOP/s of the whole step (2 M N K per step / step time) of the median
region.

Prints one JSON line.  Extra fields: the signaling and plain GEMMs measured
alone (alternating blocks), their ratio, the consumer's and the
post-reorder's HBM GB/s (MALL flushed before each timed launch; also on the
224 MiB MoE layout), per-schedule pass times, the same pass without overlap,
the other workloads, a check of the partition search, and the oracle timed
on the host cores as a CPU baseline (rank 0, N = 1).
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="profiled")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (prefill, decode, ReduceScatter, MoE All-to-All)")
    ap.add_argument("--no-search", action="store_true",
                    help="skip the check of the predictive partition search against measured partitions")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc passes: the calibration copy and each kernel launched alone on one "
                         "stream (counter collection serialises dispatches, which the two-stream pipeline "
                         "cannot run under)")
    return ap.parse_args()


class _HipEvent:
    """A HIP event for timing on a given stream, created with hipEventDisableSystemFence: recording it does
    no system-scope memory fence (which only matters to a host reading device memory right after the event;
    every read here follows a device synchronisation).  Recording a torch event, which does the fence, in
    front of each GEMM delayed every pass by about 4.5 us; this one by about 0.3 us."""
    _lib = None
    _live = []
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if _HipEvent._lib is None:
            _HipEvent._lib = ctypes.CDLL("libamdhip64.so")
        self._c = ctypes
        self.h = ctypes.c_void_p()
        if _HipEvent._lib.hipEventCreateWithFlags(ctypes.byref(self.h), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)):
            raise RuntimeError("hipEventCreateWithFlags failed")
        _HipEvent._live.append(self)

    def record(self, stream=None):
        import torch
        st = stream if stream is not None else torch.cuda.current_stream()
        if _HipEvent._lib.hipEventRecord(self.h, self._c.c_void_p(int(st.cuda_stream))):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        ms = self._c.c_float()
        if _HipEvent._lib.hipEventElapsedTime(self._c.byref(ms), self.h, end.h):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    @classmethod
    def destroy_all(cls):
        for e in cls._live:
            cls._lib.hipEventDestroy(e.h)
        cls._live = []


def _event_pairs(torch, n):
    return [(_HipEvent(), _HipEvent()) for _ in range(n)]


def _flush_mall(torch, scratch):
    scratch.fill_(1)        # writes 512 MiB: evicts the 256 MB memory-side cache


def wave_pattern_of(t_sig, W, tick_us, bins=40):
    """Tile completion times grouped by wave (deep-dive 三 › wave 模式; the summary page's wave figure).

    t_sig[s] is the device wall clock at slot s's signal; slot s belongs to
    wave s // W.  Times are relative to the first signal of the launch.
    Returns each wave's first / median / last completion, the gap between
    the end of one wave and the start of the next, and a histogram of
    completions per wave over the launch.
    """
    t = (np.asarray(t_sig, dtype=np.int64) - int(np.min(t_sig))) * tick_us
    T = (len(t) + W - 1) // W
    per = []
    for wv in range(T):
        x = t[wv * W:(wv + 1) * W]
        per.append({"tiles": int(x.size), "first_us": round(float(x.min()), 2),
                    "median_us": round(float(np.median(x)), 2), "last_us": round(float(x.max()), 2)})
    edges = np.linspace(0.0, float(t.max()) + 1e-9, bins + 1)
    hist = [np.histogram(t[wv * W:(wv + 1) * W], bins=edges)[0].tolist() for wv in range(T)]
    return {"waves": per,
            "gap_us": [round(per[i + 1]["first_us"] - per[i]["last_us"], 2) for i in range(T - 1)],
            "bin_us": round(float(edges[1] - edges[0]), 3), "histogram": hist}



def configs_check(torch, fo, Pipeline, dev, streams, scratch, steps=20, warmup=5):
    """The other workloads beside the headline: signaling and plain GEMM alone, and the pipeline at each
    workload's first partition (one wave per group if it names none) under the schedule that runs fastest
    (consumer gated or polling, post-reorder per group or whole; interleaved blocks of passes): its time per
    pass (host clock over K passes) and the signaling GEMM inside it (events on the GEMM's stream).

    Inputs are drawn on the device from the workload's distribution (the parity tests use the seeded host
    inputs; throughput does not depend on the exact values).  MoE: useful FLOP count the routed rows only;
    its 224 MiB buffers also give the consumer's and the post-reorder's bandwidth beyond the MALL.
    """
    from workloads import WORKLOADS, moe_routing
    out = []
    s = streams[0]
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    # the prefill, ReduceScatter and MoE shapes keep two or more waves with 256 x 256 tiles as well; on the
    # profiled shape that tile leaves a single wave (one group, nothing to overlap), and its line compares the
    # GEMM with the library's on the same operands
    runs = [("profiled", (256, 256)), ("ar_prefill", None), ("ar_prefill", (256, 256)), ("ar_decode", None),
            ("rs", None), ("rs", (256, 256)), ("moe_a2a", None), ("moe_a2a", (256, 256))]
    for name, tile in runs:
        w = WORKLOADS[name]
        BM, BN = tile or (w.BM, w.BN)
        if w.experts:
            m_per, tok = moe_routing(w)
            row_dest = tok // (w.tokens // w.ranks)
        else:
            m_per, row_dest = [w.M], None
        M = sum(m_per)
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed_base)
        std = w.dist[1] if w.dist[0] == "normal" else 1.0
        dA = (torch.randn(M * w.K, device=dev, generator=g) * std).to(td[w.dtype]).view(torch.int16)
        dB = (torch.randn(len(m_per) * w.N * w.K, device=dev, generator=g) * std).to(td[w.dtype]).view(torch.int16)
        dpeer = (torch.randn(M * w.N, device=dev, generator=g) * std).to(td[w.dtype]).view(torch.int16)
        comp = w.compositions[0] if w.compositions and tile is None else None
        plan = fo.Plan(m_per, w.N, w.K, w.dtype, BM=BM, BN=BN, swizzle=w.S, wave_size=w.W, composition=comp,
                       mode=w.mode, ranks=w.ranks, row_dest=row_dest)
        flops = 2.0 * M * w.N * w.K
        alg_bytes = 2.0 * (M * w.K + len(m_per) * w.N * w.K + M * w.N)
        C = torch.empty(M * w.N, dtype=torch.int16, device=dev)
        sig = plan.new_sig(dev)
        ep = [0]

        def _sig(st):
            ep[0] += 1
            plan.gemm_signal(dA, dB, C, sig, ep[0], stream=st)
        launches = [_sig, lambda st: plan.gemm_plain(dA, dB, C, stream=st)]
        if not w.experts:
            # context only: the library GEMM (hipBLASLt through torch) on the same operands, C = A . B^T
            a_mat = dA.view(td[w.dtype]).view(M, w.K)
            b_mat = dB.view(td[w.dtype]).view(w.N, w.K)
            c_mat = torch.empty(M, w.N, dtype=td[w.dtype], device=dev)

            def _lib(st):
                with torch.cuda.stream(st):
                    torch.mm(a_mat, b_mat.t(), out=c_mat)
            launches.append(_lib)
        times = _time_blocks(torch, launches, s, 10)
        sig_ms, plain_ms = times[0], times[1]
        lib_tflops = round(flops / (times[2] * 1e-3) / 1e12, 1) if len(times) > 2 else None
        if not w.experts:
            del a_mat, b_mat, c_mat
        # the matrix pipe's ceiling on this workload's A values (fo_mfma_rate), after the clock settles
        pr_out = torch.empty(n_cu * 512, dtype=torch.float32, device=dev)

        def _rate(st):
            fo.mfma_rate(dA, pr_out, n_cu, 320, dtype=w.dtype, stream=st)
        for _ in range(200):
            _rate(s)
        rate_tflops = fo.mfma_rate_flops(n_cu, 320) / (_time_kernel(torch, _rate, s, 20) * 1e-3) / 1e12
        del pr_out
        # the schedule: gated or polling consumer, post-reorder per group or whole, chosen from
        # interleaved blocks of passes as for the headline
        scheds = []
        for consumer in ("gated", "poll"):
            for per_group in ((True, False) if plan.P > 1 else (False,)):
                scheds.append(dict(consumer=consumer, per_group=per_group, ms=[],
                                   pipe=Pipeline(plan, dA, dB, dpeer, streams=streams, consumer=consumer,
                                                 post_per_group=per_group)))
        for r in scheds:
            for _ in range(warmup):
                r["pipe"].step()
            r["pipe"].join()
        torch.cuda.synchronize()
        for _ in range(3):
            for r in scheds:
                pipe = r["pipe"]
                for _ in range(3):
                    pipe.step()
                pipe.join()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(steps):
                    pipe.step()
                pipe.join()
                torch.cuda.synchronize()
                r["ms"].append((time.perf_counter() - t0) * 1e3 / steps)
                if int(pipe.status.item()) != 0:
                    raise SystemExit(f"consumer reported {fo.status_string(int(pipe.status.item()))}")
        best = min(scheds, key=lambda r: float(np.median(r["ms"])))
        pipe = best["pipe"]
        gev = _event_pairs(torch, steps)
        for e in gev:
            pipe.step(events={"gemm": e})
        pipe.join()
        torch.cuda.synchronize()
        if int(pipe.status.item()) != 0:
            raise SystemExit(f"consumer reported {fo.status_string(int(pipe.status.item()))}")
        gemm_pipe_ms = float(np.median([s_.elapsed_time(e_) for s_, e_ in gev]))
        pass_ms = float(np.median(best["ms"]))
        post = "post-reorder per group" if best["per_group"] else "post-reorder whole"
        rec = {"workload": f"{name}: M={M} N={w.N} K={w.K}, {BM}x{BN} tiles, {plan.NT} tiles, T={plan.T}, "
                           f"mode {w.mode}, groups {list(comp) if comp else [1] * plan.T}, "
                           f"{best['consumer']} consumer, {post}",
               "signal_gemm_alone_tflops": round(flops / (sig_ms * 1e-3) / 1e12, 1),
               "plain_gemm_alone_tflops": round(flops / (plain_ms * 1e-3) / 1e12, 1),
               "signal_over_plain_alone": round(plain_ms / sig_ms, 4),
               "signal_gemm_in_pass_tflops": round(flops / (gemm_pipe_ms * 1e-3) / 1e12, 1),
               "signal_in_pass_over_plain": round(plain_ms / gemm_pipe_ms, 4),
               "frac_of_peak": round(flops / (gemm_pipe_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "mfma_rate_workload_operands_tflops": round(rate_tflops, 1),
               "context_library_gemm_tflops": lib_tflops,
               # which roof bounds this shape: its arithmetic intensity (FLOP per algorithmic HBM byte:
               # A, every problem's B and C once each) against the ridge of the two peaks
               "flop_per_byte": round(flops / alg_bytes, 1),
               "bound": "mfma" if flops / alg_bytes >= PEAK_BF16_TFLOPS / PEAK_HBM_GBPS * 1e3 else "hbm",
               "gemm_in_pass_hbm_gbps": round(alg_bytes / (gemm_pipe_ms * 1e-3) / 1e9, 1),
               "gemm_in_pass_frac_hbm": round(alg_bytes / (gemm_pipe_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
               "pass_ms": round(pass_ms, 4),
               "pass_tflops": round(flops / (pass_ms * 1e-3) / 1e12, 1),
               "schedules_ms": {f"{r['consumer']}, {'per group' if r['per_group'] else 'whole'}":
                                round(float(np.median(r["ms"])), 4) for r in scheds}}
        if w.experts and tile is None:
            mn = M * w.N
            status = torch.zeros(1, dtype=torch.int32, device=dev)
            ready = plan.new_sig(dev)
            plan.flag_of(ready).fill_(1)
            recv = torch.empty_like(C)
            cons_ms = _time_kernel(torch, lambda st: plan.consume_group(C, dpeer, recv, ready, 1, status, stream=st),
                                   s, 10, scratch)
            gated_ms = _time_kernel(torch, lambda st: plan.consume_group_gated(C, dpeer, recv, ready, 1, status,
                                                                               stream=st), s, 10, scratch)
            post_ms = _time_kernel(torch, lambda st: plan.reorder_post(recv, C, stream=st), s, 10, scratch)
            rec.update(consumer_alone_gbps=round(6.0 * mn / (cons_ms * 1e-3) / 1e9, 1),
                       consumer_gated_alone_gbps=round(6.0 * mn / (gated_ms * 1e-3) / 1e9, 1),
                       post_reorder_alone_gbps=round(4.0 * mn / (post_ms * 1e-3) / 1e9, 1),
                       hbm_note=f"{2 * mn / 2 ** 20:.0f} MiB per buffer, MALL flushed, event-timed")
        out.append(rec)
        for r in scheds:
            r["pipe"].close()
        plan.close()
        del dA, dB, dpeer, C
    return out


def _time_partitions(torch, Pipeline, plans, dA, dB, dpeer, streams, steps, rounds=3, warmup=2):
    """Median end of communication (GEMM start to the consumer's end, ms) of each plan's pipeline, timed in
    `rounds` interleaved rounds whose order rotates, after a common warm-up: a partition timed first after
    another workload's passes ran up to 8% slow."""
    pipes = [Pipeline(p, dA, dB, dpeer, streams=streams) for p in plans]
    for _ in range(3 * warmup):
        for pipe in pipes:
            pipe.step()
    per = [[] for _ in pipes]
    n = len(pipes)
    for r in range(rounds):
        for k in range(n):
            i = (k + r * max(1, n // rounds)) % n
            pipe = pipes[i]
            for _ in range(warmup):
                pipe.step()
            evs = [{key: _event_pairs(torch, 1)[0] for key in ("gemm", "consume", "post")} for _ in range(steps)]
            for e in evs:
                pipe.step(events=e)
            pipe.join()
            torch.cuda.synchronize()
            if int(pipe.status.item()) != 0:
                raise SystemExit(f"consumer reported status {int(pipe.status.item())}")
            per[i].append(float(np.median([e["gemm"][0].elapsed_time(e["consume"][1]) for e in evs])))
    for pipe in pipes:
        pipe.close()
    return [float(np.median(x)) for x in per]


def _cut_mask(comp) -> int:
    """Waves per group -> cut mask (bit i: a group ends after wave i + 1), the index of fo_plan_search's
    per-partition predictions."""
    mask, end = 0, 0
    for c in comp[:-1]:
        end += c
        mask |= 1 << (end - 1)
    return mask


def moe_search_check(torch, fo, Pipeline, dev, streams, steps=10, warmup=3, samples=8):
    """Predictive partition search on the MoE shape, whose waves leave too many partitions to run them all
    (deep-dive 三 › 调优挑战: the tuning cost grows as 2^(T-1); 四 › 在线阶段: the search replaces it).

    fo_plan_search scores every partition from the GEMM's duration and a consumer latency curve (sampled up to
    the MoE output's size, at the MoE row width); its choice then runs in the pipeline beside a fixed set of
    partitions (one group; one wave per group; even groups of 2, 4 and 8 waves; one small group first or last)
    and `samples` random ones, and the measured end of communication (GEMM start to the consumer's end) ranks
    them.  Inputs are drawn on the device (throughput does not depend on the values)."""
    from workloads import WORKLOADS, moe_routing
    w = WORKLOADS["moe_a2a"]
    m_per, tok = moe_routing(w)
    row_dest = tok // (w.tokens // w.ranks)
    M = sum(m_per)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed_base)
    std = w.dist[1]
    dA = (torch.randn(M * w.K, device=dev, generator=g) * std).to(torch.bfloat16).view(torch.int16)
    dB = (torch.randn(len(m_per) * w.N * w.K, device=dev, generator=g) * std).to(torch.bfloat16).view(torch.int16)
    dpeer = (torch.randn(M * w.N, device=dev, generator=g) * std).to(torch.bfloat16).view(torch.int16)
    s = streams[0]

    def plan_of(comp=None):
        return fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=comp,
                       mode=w.mode, ranks=w.ranks, row_dest=row_dest)
    base = plan_of()
    T = base.T
    C = torch.empty(M * w.N, dtype=torch.int16, device=dev)
    for _ in range(3):
        base.gemm_plain(dA, dB, C, stream=s)
    gemm_ms = float(np.median([_time_kernel(torch, lambda st: base.gemm_plain(dA, dB, C, stream=st), s, 1)
                               for _ in range(5)]))
    del C
    curve_b, curve_s = [], []
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for rows in (64, 256, 1024, 2048, 4096, 8192):
        probe = fo.Plan(rows, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W)
        cp = fo.Plan(rows, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=(probe.T,))
        probe.close()
        x = torch.zeros(cp.M * cp.N, dtype=torch.int16, device=dev)
        y = torch.empty_like(x)
        ready = cp.new_sig(dev)
        cp.flag_of(ready).fill_(1)
        ms = float(np.median([_time_kernel(torch, lambda st: cp.consume_group_gated(x, x, y, ready, 1, status,
                                                                                    stream=st),
                                           s, 1) for _ in range(5)]))
        curve_b.append(2.0 * cp.M * cp.N)
        curve_s.append(ms * 1e-3)
        cp.close()
        del x, y
    pred, pred_s, all_s = base.search(gemm_ms * 1e-3, curve_b, curve_s, with_all=True)
    base.close()
    fixed = [(T,), (1,) * T, (2,) * (T // 2) + (1,) * (T % 2), (4,) * (T // 4) + ((T % 4,) if T % 4 else ()),
             (8,) * (T // 8) + ((T % 8,) if T % 8 else ()), (1, T - 1), (T - 1, 1)]
    rng = np.random.Generator(np.random.PCG64(w.seed_base + 5))
    rand = []
    for _ in range(samples):
        cuts = rng.integers(0, 2, size=T - 1)
        comp, run = [], 0
        for i in range(T):
            run += 1
            if i == T - 1 or cuts[i]:
                comp.append(run)
                run = 0
        rand.append(tuple(comp))
    cands = []
    for c in [tuple(pred)] + fixed + rand:
        if c not in cands:
            cands.append(c)
    plans = [plan_of(c) for c in cands]
    meas = _time_partitions(torch, Pipeline, plans, dA, dB, dpeer, streams, steps, warmup=warmup)
    for p_ in plans:
        p_.close()
    rows_out = [(c, all_s[_cut_mask(c)] * 1e3, m) for c, m in zip(cands, meas)]
    del dA, dB, dpeer
    best = min(rows_out, key=lambda r: r[2])
    pick = rows_out[0]
    order = sorted(rows_out, key=lambda r: r[2])
    return {
        "workload": f"{w.name}: M={M} N={w.N} K={w.K}, {w.BM}x{w.BN} tiles, T={T}, {1 << (T - 1)} partitions, "
                    f"gated consumer",
        "gemm_plain_us": round(gemm_ms * 1e3, 1),
        "curve_bytes": curve_b, "curve_us": [round(x * 1e6, 2) for x in curve_s],
        "predicted_best": list(pred), "predicted_us": round(pred_s * 1e6, 1),
        "measured": len(rows_out), "best_of_measured": list(best[0]), "best_of_measured_us": round(best[2] * 1e3, 1),
        "predicted_choice_measured_us": round(pick[2] * 1e3, 1),
        "regret_vs_best_of_measured": round(pick[2] / best[2] - 1.0, 4),
        "rank_of_predicted_choice": 1 + [r[0] for r in order].index(pick[0]),
        "candidates": [{"groups": list(c), "predicted_us": round(p * 1e3, 1), "measured_us": round(m * 1e3, 1)}
                       for c, p, m in rows_out],
    }


def search_check(torch, fo, Pipeline, dev, streams, steps=20, warmup=5):
    """Predictive partition search against measurement on the 4-wave prefill workload.

    The search's offline inputs, as the pages describe them (deep-dive
    四 › 离线阶段 / 在线阶段): the GEMM's duration (the plain GEMM alone) and a
    latency-versus-size curve of the communication -- here its one-GPU
    stand-in, the consumer, run on a single group of each sampled size with
    the flag already raised (HIP events, so a call's fixed cost is included).
    fo_plan_search scores all 2^(T-1) partitions; every partition then runs in
    the pipeline (gated consumer), and the measured end of communication (GEMM
    start to the consumer's end) is set against the prediction.
    """
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["ar_prefill"]
    A, B, peer, m_per, rd = make_inputs(w)
    dA = torch.from_numpy(A.view(np.int16).reshape(-1).copy()).to(dev)
    dB = torch.from_numpy(np.concatenate([b.reshape(-1) for b in B]).view(np.int16).copy()).to(dev)
    dpeer = torch.from_numpy(peer.view(np.int16).copy()).to(dev)
    s = streams[0]
    base = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W)
    C = torch.empty(w.M * w.N, dtype=torch.int16, device=dev)
    gemm_ms = float(np.median([_time_kernel(torch, lambda st: base.gemm_plain(dA, dB, C, stream=st), s, 1)
                               for _ in range(10)]))
    curve_b, curve_s = [], []
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for rows in (16, 64, 256, 1024, 2048, 4096):
        probe = fo.Plan(rows, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W)
        cp = fo.Plan(rows, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=(probe.T,))
        probe.close()
        x = torch.zeros(cp.M * cp.N, dtype=torch.int16, device=dev)
        y = torch.empty_like(x)
        ready = cp.new_sig(dev)
        cp.flag_of(ready).fill_(1)
        ms = float(np.median([_time_kernel(torch, lambda st: cp.consume_group_gated(x, x, y, ready, 1, status,
                                                                                    stream=st),
                                           s, 1) for _ in range(10)]))
        curve_b.append(2.0 * cp.M * cp.N)
        curve_s.append(ms * 1e-3)
        cp.close()
    pred, pred_s, all_s = base.search(gemm_ms * 1e-3, curve_b, curve_s, with_all=True)

    def comp_of(mask, T):     # cut mask -> waves per group (bit i: a group ends after wave i+1)
        out, run = [], 0
        for wv in range(T):
            run += 1
            if wv == T - 1 or (mask >> wv) & 1:
                out.append(run)
                run = 0
        return tuple(out)

    comps = [comp_of(mask, base.T) for mask in range(1 << (base.T - 1))]
    plans = [fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W, composition=c)
             for c in comps]
    meas = _time_partitions(torch, Pipeline, plans, dA, dB, dpeer, streams, steps, warmup=warmup)
    for p_ in plans:
        p_.close()
    rows = [(c, all_s[mask] * 1e3, m) for mask, (c, m) in enumerate(zip(comps, meas))]
    T = base.T
    base.close()
    best_m = min(rows, key=lambda r: r[2])
    pick = next(r for r in rows if r[0] == pred)
    order = sorted(rows, key=lambda r: r[2])
    return {
        "workload": f"{w.name}: M={w.M} N={w.N} K={w.K}, {w.BM}x{w.BN} tiles, wave {w.W}, T={T}, gated consumer",
        "gemm_plain_us": round(gemm_ms * 1e3, 1),
        "curve_bytes": curve_b, "curve_us": [round(x * 1e6, 2) for x in curve_s],
        "predicted_best": list(pred), "predicted_us": round(pred_s * 1e6, 1),
        "measured_best": list(best_m[0]), "measured_best_us": round(best_m[2] * 1e3, 1),
        "predicted_choice_measured_us": round(pick[2] * 1e3, 1),
        "regret": round(pick[2] / best_m[2] - 1.0, 4),
        "rank_of_predicted_choice": 1 + [r[0] for r in order].index(pred),
        "candidates": [{"groups": list(c), "predicted_us": round(p * 1e3, 1), "measured_us": round(m * 1e3, 1)}
                       for c, p, m in rows],
    }


def _time_blocks(torch, launches, stream, n, rounds=3, warmup=30):
    """Average durations (ms) of several launches timed in alternating blocks of n (median block of each over
    `rounds` rounds), after `warmup` untimed launches of each in turn, so that the clock has settled under
    their load and drift falls on all alike (a kernel timed first after lighter work ran up to 15% slower)."""
    for _ in range(warmup):
        for f in launches:
            f(stream)
    t = [[] for _ in launches]
    for _ in range(rounds):
        for i, f in enumerate(launches):
            t[i].append(_time_kernel(torch, f, stream, n))
    return [float(np.median(x)) for x in t]


def _time_kernel(torch, launch, stream, n, scratch=None):
    """Average duration (ms) of ``launch(stream)`` over n launches, HIP events on that stream."""
    ev = _event_pairs(torch, n)
    for i in range(n):
        if scratch is not None:
            with torch.cuda.stream(stream):
                _flush_mall(torch, scratch)
        ev[i][0].record(stream)
        launch(stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def kernel_source_hash() -> str:
    """sha256 over the GEMM kernel's sources and build flags: ties committed traffic counters to the code they measured."""
    import hashlib
    h = hashlib.sha256()
    for rel in ("gemm_tile_signaling_amd/csrc/kernels/gemm.hip", "gemm_tile_signaling_amd/csrc/kernels/buffer.h",
                "gemm_tile_signaling_amd/csrc/fo_internal.h", "gemm_tile_signaling_amd/build.py"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str):
    """HBM bytes per launch of the signaling GEMM from the committed rocprofv3 counter passes, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"signal_gemm_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_info():
    """The board's clock limits, memory clock and power cap, read through amdsmi (read-only); None where it is
    not available.  The clock the GEMM actually runs at comes from the counter passes in profiles/ (GPU-active
    cycles over the kernel's duration): the sampled clock reading does not follow a load this short."""
    try:
        import amdsmi
    except ImportError:
        return None
    try:
        amdsmi.amdsmi_init()
        try:
            h = amdsmi.amdsmi_get_processor_handles()[0]
            gfx = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            mem = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)
            cap = amdsmi.amdsmi_get_power_cap_info(h)
            return dict(sclk_min_mhz=gfx.get("min_clk"), sclk_max_mhz=gfx.get("max_clk"), mclk_mhz=mem.get("clk"),
                        power_cap_w=round(cap.get("power_cap", 0) / 1e6, 1) if cap.get("power_cap") else None)
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception as e:  # noqa: BLE001 -- a monitoring read must never stop the benchmark
        return dict(error=f"{type(e).__name__}: {e}")


def cpu_baseline(w, A, B, peer, m_per, row_dest, comp, min_seconds=10.0):
    """The oracle pipeline (fp64 GEMM, pre-reorder, consumer, post-reorder) on the host cores.

    Threaded: the full workload, repeated until about ``min_seconds`` of CPU
    work have been timed, with the BLAS thread pool at the host's CPU count.
    Single-threaded: one pass over the first 512 rows of A (a quarter of the
    profiled workload's rows, the same B), the BLAS pool at one thread.
    """
    import oracle
    from oracle.tiles import make_plan
    from threadpoolctl import threadpool_info, threadpool_limits
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)

    def run(rows, limit, min_s, max_reps):
        Ar = A[:rows]
        plan = make_plan([rows], w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W,
                         composition=comp if rows == w.M else None, mode=w.mode, ranks=w.ranks, row_dest=row_dest)
        pr = peer[:rows * w.N]
        with threadpool_limits(limits=limit):
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.run_pipeline(Ar, B, pr, plan, w.dtype)
                reps += 1
                dt = time.perf_counter() - t0
                if dt >= min_s or reps >= max_reps:
                    break
        return 2.0 * rows * w.N * w.K * reps / dt / 1e12, threads, reps, dt

    v, threads, reps, dt = run(w.M, nproc, min_seconds, 50)
    v1, _, reps1, dt1 = run(min(512, w.M), 1, 0.0, 1)
    # one more threaded pass, stage by stage (seconds), as the oracle times its own steps
    stages = {}
    with threadpool_limits(limits=nproc):
        oracle.run_pipeline(A, B, peer, make_plan([w.M], w.N, BM=w.BM, BN=w.BN, S=w.S, W=w.W, composition=comp,
                                                  mode=w.mode, ranks=w.ranks, row_dest=row_dest),
                            w.dtype, stage_seconds=stages)
    mn = w.M * w.N
    stage_rates = {"gemm_tflops": 2.0 * w.M * w.N * w.K / stages["gemm"] / 1e12,
                   "consume_gbps": 6.0 * mn / stages["consume"] / 1e9,
                   "pre_reorder_gbps": 4.0 * mn / stages["pre_reorder"] / 1e9,
                   "post_reorder_gbps": 4.0 * mn / stages["post_reorder"] / 1e9}
    return dict(value=round(v, 4), unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"full workload (M={w.M}, N={w.N}, K={w.K}, groups {tuple(comp)}) x {reps} passes, "
                       f"{dt:.1f} s, BLAS pool {threads} threads",
                single_thread=dict(value=round(v1, 4), unit="TFLOP/s",
                                   sample=f"first {min(512, w.M)} rows x 1 pass, {dt1:.1f} s, 1 thread"),
                nproc=int(nproc), cpu_model=_cpu_model(),
                stages_s={k: round(t, 4) for k, t in stages.items()},
                stage_rates={k: round(r, 3) for k, r in stage_rates.items()})


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {a.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import gemm_tile_signaling_amd as fo
    from gemm_tile_signaling_amd.pipeline import Pipeline
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[a.workload]
    if w.experts:
        raise SystemExit("the benchmark line is quoted on a single-problem workload")
    A, B, peer, m_per, row_dest = make_inputs(w)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A.view(np.int16).reshape(-1).copy()).to(dev)
    dB = torch.from_numpy(np.concatenate([b.reshape(-1) for b in B]).view(np.int16).copy()).to(dev)
    dpeer = torch.from_numpy(peer.view(np.int16).copy()).to(dev)
    flops = 2.0 * w.M * w.N * w.K
    comps = list(w.compositions) or [None]
    scratch = torch.empty(512 * 2 ** 20 // 4, dtype=torch.int32, device=dev)
    # a plain copy of known size (256 MiB read, 256 MiB written): the reference that
    # scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters of the other kernels
    cal_src = torch.ones(256 * 2 ** 20 // 4, dtype=torch.int32, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    if a.counters:
        plan = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W,
                       composition=comps[0], mode=w.mode, ranks=w.ranks, row_dest=row_dest)
        buf = torch.empty(w.M * w.N, dtype=torch.int16, device=dev)
        out = torch.empty_like(buf)
        sig = plan.new_sig(dev)
        ready = plan.new_sig(dev)
        plan.flag_of(ready).fill_(1)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        for e in range(1, a.steps + 1):
            plan.gemm_signal(dA, dB, buf, sig, e)
        for _ in range(a.steps):
            plan.gemm_plain(dA, dB, out)
        for _ in range(a.steps):
            plan.consume_group(buf, dpeer, out, ready, 1, status)
        for _ in range(a.steps):
            plan.consume_group_gated(buf, dpeer, out, ready, 1, status)
        for _ in range(a.steps):
            plan.reorder_post(buf, out)
        # the library GEMM on the same operands, for context (hipBLASLt through torch)
        tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]
        tA, tB = dA.view(tdt).view(w.M, w.K), dB.view(tdt).view(w.N, w.K)
        for _ in range(a.steps):
            torch.mm(tA, tB.t())
        torch.cuda.synchronize()
        print(json.dumps({"counters_pass": w.name, "launches_per_kernel": a.steps,
                          "calibration_copy_bytes": 256 * 2 ** 20, "status": int(status.item())}), flush=True)
        plan.close()
        return

    # one pair of streams, each with a hardware queue of its own, for every pipeline and every kernel
    # timed alone: the device has few hardware queues, and streams created per pipeline would share
    # them in an order that changes the timings from one schedule to the next
    streams = (fo.stream_create(), fo.stream_create())
    plans, scheds = [], []   # schedules: a partition, the consumer, the post-reorder whole or per group
    for comp in comps:
        plan = fo.Plan(m_per, w.N, w.K, w.dtype, BM=w.BM, BN=w.BN, swizzle=w.S, wave_size=w.W,
                       composition=comp, mode=w.mode, ranks=w.ranks, row_dest=row_dest)
        plans.append(plan)
        for consumer in ("gated", "poll"):
            for per_group in ((False, True) if plan.P > 1 else (False,)):
                scheds.append(dict(plan=plan, pipe=Pipeline(plan, dA, dB, dpeer, post_per_group=per_group,
                                                            streams=streams, consumer=consumer),
                                   comp=comp or tuple([1] * plan.T), per_group=per_group, consumer=consumer))
    launches = [0]   # signaling-GEMM launches so far (locates the timed region in a kernel trace)
    regions = 5
    # every event is created and recorded once here: torch creates the HIP event at its first
    # record, and a few hundred creations inside a timed loop stall the host for milliseconds;
    # the GPU idling that long drops its clock, and the passes after it run in the ramp back up
    gemm_ev = [_event_pairs(torch, a.steps) for _ in range(regions)]
    region_ev = _event_pairs(torch, regions)
    pick_ev = _event_pairs(torch, a.steps)
    br_ev = [{k: _event_pairs(torch, a.steps) for k in ("gemm", "consume", "post")} for _ in scheds]
    for pair in ([p for r in gemm_ev for p in r] + region_ev + pick_ev
                 + [p for d in br_ev for v in d.values() for p in v]):
        pair[0].record()
        pair[1].record()
    torch.cuda.synchronize()
    # no garbage collection pause inside the measured phases either
    gc.collect()
    gc.disable()

    def check(pipe):
        if int(pipe.status.item()) != 0:
            raise SystemExit(f"consumer reported {fo.status_string(int(pipe.status.item()))}")

    def passes(pipe, n, **kw):
        for _ in range(n):
            pipe.step(**kw)
        launches[0] += n
        pipe.join()
        torch.cuda.synchronize()
        check(pipe)

    # choose the schedule: blocks of K passes (each GEMM bracketed by events, as in the timed
    # region), every schedule in turn, three rounds, so that clock and power drift falls on all of
    # them alike; the serial schedule (GEMM, consumer, post-reorder on one queue) is measured alike
    passes(scheds[0]["pipe"], a.warmup)
    order = [(i, False) for i in range(len(scheds))] + [(0, True)]
    picks = {k: [] for k in order}
    for _ in range(3):
        for i, serial in order:
            pipe = scheds[i]["pipe"]
            passes(pipe, 5, serial=serial)
            t0 = time.perf_counter()
            for j in range(a.steps):
                pipe.step(events={"gemm": pick_ev[j]}, serial=serial)
            pipe.join()
            torch.cuda.synchronize()
            picks[(i, serial)].append((time.perf_counter() - t0) * 1e3 / a.steps)
            launches[0] += a.steps
            check(pipe)
    for i, r in enumerate(scheds):
        r["pick_ms"] = float(np.median(picks[(i, False)]))
    serial_ms = float(np.median(picks[(0, True)]))
    best = min(scheds, key=lambda r: r["pick_ms"])
    plan, pipe = best["plan"], best["pipe"]

    # timed: five regions, each W warm-up passes then exactly K passes of the chosen schedule,
    # synchronised on both sides; a device event pair brackets each region (first GEMM's start to
    # the last post-reorder's end) beside the host clock; the GEMM of every pass is bracketed by
    # events on its own stream for the roofline.  The value is the median region.  Before the
    # first region the chosen schedule runs 100 untimed passes, so no region starts in a clock ramp.
    passes(pipe, 100)
    reg = []
    for r in range(regions):
        passes(pipe, a.warmup)
        first = launches[0]
        t0 = time.perf_counter()
        region_ev[r][0].record(pipe.next_gemm_stream())
        for i in range(a.steps):
            pipe.step(events={"gemm": gemm_ev[r][i]})
        region_ev[r][1].record(pipe.post_stream)
        pipe.join()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3 / a.steps
        launches[0] += a.steps
        check(pipe)
        each = [s.elapsed_time(e) for s, e in gemm_ev[r]]
        dev_ms = region_ev[r][0].elapsed_time(region_ev[r][1]) / a.steps
        reg.append(dict(host_ms=host_ms, device_ms=dev_ms, gemm_ms=float(np.mean(each)),
                        gemm_q=np.percentile(each, [10, 50, 90]).tolist(), launches=[first, launches[0]]))
    mid = sorted(range(regions), key=lambda r: reg[r]["host_ms"])[regions // 2]
    best.update(step_ms=reg[mid]["host_ms"], gemm_ms=reg[mid]["gemm_ms"], gemm_q=reg[mid]["gemm_q"])
    timed_range = reg[mid]["launches"]

    # untimed: every kernel of every schedule bracketed, for the breakdown
    for r, evs in zip(scheds, br_ev):
        for i in range(a.steps):
            r["pipe"].step(events={k: v[i] for k, v in evs.items()})
        launches[0] += a.steps
        r["pipe"].join()
        torch.cuda.synchronize()
        check(r["pipe"])
        avg = {k: float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in evs.items()}
        r.update(br_gemm_ms=avg["gemm"], consume_ms=avg["consume"], post_ms=avg["post"])

    gc.enable()

    # one traced pass: device wall-clock stamps of every tile's signal and of each group's consumer start
    gtr = torch.zeros(2 * plan.NT + plan.P, dtype=torch.int64, device=dev)
    ctr = torch.zeros(plan.P, dtype=torch.int64, device=dev)
    pipe.step(trace=gtr, consumer_trace=ctr)
    pipe.join()
    torch.cuda.synchronize()
    check(pipe)
    g = gtr.cpu().numpy().view(np.uint64).astype(np.int64)
    c = ctr.cpu().numpy().view(np.uint64).astype(np.int64)
    tick_us = 1e3 / plan.info["clock_khz"]
    grp = np.array(plan.tables()["group_of_slot"])
    t_sig = g[0:2 * plan.NT:2]
    last = np.array([t_sig[grp == j].max() for j in range(plan.P)])
    signal_to_consume_us = [round(float(x) * tick_us, 2) for x in (c - last)]
    first_consume_before_gemm_end_us = round(float(last[-1] - c[0]) * tick_us, 2)
    wave_pattern = wave_pattern_of(t_sig, plan.W, tick_us)

    # kernels alone (same plan), each timed with HIP events on its own stream
    s = streams[0]
    n_alone = max(10, min(a.steps, 50))
    C = torch.empty(w.M * w.N, dtype=torch.int16, device=dev)
    sig = plan.new_sig(dev)
    ep = [0]

    def _sig(st):
        ep[0] += 1
        plan.gemm_signal(dA, dB, pipe.buf, sig, ep[0], stream=st)
    # context only: the library GEMM (hipBLASLt through torch) on the same operands, C = A . B^T, timed in
    # the same alternating blocks as the two GEMMs
    a_mat = dA.view(torch.bfloat16 if w.dtype == "bf16" else torch.float16).view(w.M, w.K)
    b_mat = dB.view(a_mat.dtype).view(w.N, w.K)
    c_mat = torch.empty(w.M, w.N, dtype=a_mat.dtype, device=dev)

    def _lib(st):
        with torch.cuda.stream(st):
            torch.mm(a_mat, b_mat.t(), out=c_mat)
    signal_ms, plain_ms, lib_ms = _time_blocks(torch, [_sig, lambda st: plan.gemm_plain(dA, dB, C, stream=st), _lib],
                                               s, max(10, n_alone // 3))
    del c_mat
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ready = plan.new_sig(dev)
    plan.flag_of(ready).fill_(1)
    recv = torch.empty_like(pipe.buf)
    consume_ms = _time_kernel(torch, lambda st: plan.consume_group(pipe.buf, dpeer, recv, ready, 1, status, stream=st),
                              s, n_alone, scratch)
    gated_ms = _time_kernel(torch, lambda st: plan.consume_group_gated(pipe.buf, dpeer, recv, ready, 1, status,
                                                                       stream=st), s, n_alone, scratch)
    post_ms = _time_kernel(torch, lambda st: plan.reorder_post(recv, C, stream=st), s, n_alone, scratch)
    bias = (torch.randn(plan.num_problems * w.N, device=dev) * 0.02).to(torch.bfloat16 if w.dtype == "bf16"
                                                                        else torch.float16).view(torch.int16)
    post_ep_ms = _time_kernel(torch, lambda st: plan.reorder_post_ep(recv, C, bias=bias, act="silu", stream=st), s,
                              n_alone, scratch)
    # context: torch's own device copy of the same bytes (read M*N, write M*N elements), MALL flushed alike
    cp_src = torch.ones(w.M * w.N, dtype=torch.int16, device=dev)

    def _copy(st):
        with torch.cuda.stream(st):
            C.copy_(cp_src)
    for _ in range(3):   # first launches load the kernel's code
        _copy(s)
    copy_ms = _time_kernel(torch, _copy, s, n_alone, scratch)
    # and torch's elementwise add of two such buffers into a third (the consumer's bytes)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    add_a, add_b, add_c = pipe.buf.view(tdt), dpeer.view(tdt), C.view(tdt)

    def _add(st):
        with torch.cuda.stream(st):
            torch.add(add_a, add_b, out=add_c)
    for _ in range(3):
        _add(s)
    add_ms = _time_kernel(torch, _add, s, n_alone, scratch)
    del cp_src, add_a, add_b, add_c
    # the matrix pipe's ceiling on this data (fo_mfma_rate: the 256 x 128 tile's MFMAs only, no loads, LDS
    # or epilogue; one workgroup of eight waves per CU), on operand values read from A (the GEMM's own
    # distribution) and on zeros (no multiplier toggles); each after 200 untimed launches of about the GEMM's
    # length, so the clock has settled under that load
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    pr_iters = 320
    pr_out = torch.empty(n_cu * 512, dtype=torch.float32, device=dev)
    pr_zero = torch.zeros(4096, dtype=torch.int16, device=dev)
    mfma_rate = {}
    for key, ops in (("workload_operands_tflops", dA), ("zero_operands_tflops", pr_zero)):
        def _rate(st, ops=ops):
            fo.mfma_rate(ops, pr_out, n_cu, pr_iters, dtype=w.dtype, stream=st)
        for _ in range(200):
            _rate(s)
        mfma_rate[key] = round(fo.mfma_rate_flops(n_cu, pr_iters) / (_time_kernel(torch, _rate, s, n_alone) * 1e-3)
                               / 1e12, 1)
    del pr_out, pr_zero
    mn = w.M * w.N
    consume_gbps = 6.0 * mn / (consume_ms * 1e-3) / 1e9
    gated_gbps = 6.0 * mn / (gated_ms * 1e-3) / 1e9
    post_gbps = 4.0 * mn / (post_ms * 1e-3) / 1e9

    achieved = flops / (best["gemm_ms"] * 1e-3) / 1e12
    line = {
        "metric": "signaling-GEMM TFLOP/s (% of plain GEMM & MFMA peak); reorder HBM GB/s",
        "value": round(flops / (best["step_ms"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(best["step_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: GEMM M={w.M} N={w.N} K={w.K} {w.dtype}, {w.BM}x{w.BN} tiles, "
                               f"swizzle {w.S}, wave {w.W} tiles, groups {tuple(best['comp'])}, "
                               f"{best['consumer']} consumer copy+add, "
                               f"post-reorder{' per group' if best['per_group'] else ''}",
                   "M": w.M, "N": w.N, "K": w.K, "tile": [w.BM, w.BN], "swizzle": w.S, "wave": w.W,
                   "tiles": plan.NT, "waves": plan.T, "groups": list(best["comp"]), "consumer": best["consumer"],
                   "post_per_group": best["per_group"], "parallelism": "1 GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": committed_traffic(w.name),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes": 2 * (w.M * w.K + w.N * w.K + w.M * w.N),
                     "kernel": "signaling GEMM inside the timed passes (events on its own stream)"},
        "timed_regions": [{"host_ms_per_step": round(r["host_ms"], 4), "device_ms_per_step": round(r["device_ms"], 4),
                           "signal_gemm_ms": round(r["gemm_ms"], 4)} for r in reg],
        "timed_region_used": mid,
        "choice_block_ms_per_step": round(best["pick_ms"], 4),
        "signal_gemm_us_p10_p50_p90": [round(x * 1e3, 1) for x in best["gemm_q"]],
        "serial_pass_ms": round(serial_ms, 4),
        "overlap_speedup_over_serial": round(serial_ms / best["pick_ms"], 4),
        "signal_gemm_alone_tflops": round(flops / (signal_ms * 1e-3) / 1e12, 2),
        "plain_gemm_alone_tflops": round(flops / (plain_ms * 1e-3) / 1e12, 2),
        "signal_over_plain_alone": round(plain_ms / signal_ms, 4),
        "signal_with_consumer_over_plain": round(plain_ms / best["gemm_ms"], 4),
        "context_library_gemm_tflops": round(flops / (lib_ms * 1e-3) / 1e12, 2),
        "mfma_rate_probe": dict(mfma_rate, operands=f"A of the workload ({w.dist[0]}), and zeros",
                                signal_gemm_in_pass_over_workload_operands=round(
                                    achieved / mfma_rate["workload_operands_tflops"], 4)),
        "consumer_alone_gbps": round(consume_gbps, 1),
        "consumer_gated_alone_gbps": round(gated_gbps, 1),
        "post_reorder_alone_gbps": round(post_gbps, 1),
        "context_torch_copy_gbps": round(4.0 * w.M * w.N / (copy_ms * 1e-3) / 1e9, 1),
        "context_torch_add_gbps": round(6.0 * w.M * w.N / (add_ms * 1e-3) / 1e9, 1),
        "post_reorder_bias_silu_alone_gbps": round((4.0 * mn + 2.0 * plan.num_problems * w.N) / (post_ep_ms * 1e-3)
                                                   / 1e9, 1),
        "consumer_frac_hbm": round(max(consume_gbps, gated_gbps) / PEAK_HBM_GBPS, 4),
        "post_reorder_frac_hbm": round(post_gbps / PEAK_HBM_GBPS, 4),
        "signal_to_consume_us": signal_to_consume_us,
        "first_group_consumed_before_gemm_end_us": first_consume_before_gemm_end_us,
        "wave_pattern": wave_pattern,
        "schedules": [{"groups": list(r["comp"]), "consumer": r["consumer"], "post_per_group": r["per_group"],
                       "pick_step_ms": round(r["pick_ms"], 4),
                       "gemm_ms": round(r["br_gemm_ms"], 4), "consume_span_ms": round(r["consume_ms"], 4),
                       "post_ms": round(r["post_ms"], 4)} for r in scheds],
        "timed_signal_gemm_launches": timed_range,
        "gpu": gpu_info(),
        "cpu_baseline": None,
    }
    for r in scheds:
        r["pipe"].close()
    if not a.no_configs:
        line["configs"] = configs_check(torch, fo, Pipeline, dev, streams, scratch)
    if not a.no_search:
        line["search"] = search_check(torch, fo, Pipeline, dev, streams)
        line["search_moe"] = moe_search_check(torch, fo, Pipeline, dev, streams)
    # release every device object before the interpreter exits
    torch.cuda.synchronize()
    for st in streams:
        fo.stream_destroy(st)
    for p_ in plans:
        p_.close()
    del scheds, pipe, plan
    torch.cuda.synchronize()
    _HipEvent.destroy_all()
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, A, B, peer, m_per, row_dest, best["comp"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
