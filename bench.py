#!/usr/bin/env python3
"""Benchmark of the Key-Value Means layer on one MI355X.

A step is one kvm_prefill over the 350M-shaped workload (B=2, H=16, N=32768,
chunk 128, window 256, sqrt state with ceil(8 sqrt T) rows, 4 sinks, bf16):
absorption scan, fused attention over [state || window], ring refresh.  Each
timed step starts from an emptied state (kvm_state_reset, inside the timed
region).  The line also carries:

  roofline      the attention kernel (dominant flops): algorithmic MFMA FLOPs
                per launch / its mean launch time from HIP events recorded by
                the library around each launch on the stream it runs on,
                against the dense bf16/fp16 MFMA peak.  A prefill launches the
                attention in several pieces beside the absorption scan, so the
                per-launch figures are means over the pieces (total FLOPs /
                total kernel time).  `traffic` is the HBM bytes per launch
                from rocprofv3 FETCH_SIZE + WRITE_SIZE counters (scaled by the
                same counters on a plain copy of known size), taken from
                profiles/ only when they were measured on this kernel source.
  decode        the batched-decode workload (64 x 16 sequences, sqrt state
                prefilled with 16384 tokens): per-step time of the decode
                kernels and their algorithmic HBM bytes per step.
  scan          the absorption scan's time per chunk step and its input bytes against
                HBM (it is latency-bound: sequential over chunks).
  other_workloads  prefill time of the 120M-shaped and the long workloads (context).
  attn_alone    the attention kernel alone on the chip (serial prefill, outside the
                timed steps): context for the roofline, whose launches share the chip.
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload.

python bench.py [--steps K] [--warmup W] [--gpus 1]
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
sys.path.insert(0, ROOT)

METRIC = "KVM-layer prefill tokens/s (B*H*N) + % bf16 MFMA peak; decode HBM GB/s"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 (the fp32 path's backward contracts in fp32)
KERNEL_SRC = os.path.join(ROOT, "compressed_kv_state_amd", "csrc", "kvm_kernels.hip")
ATTN_KERNEL = "attn_dma_kernel"   # the bf16 attention kernel for chunks of 128 / 256
COUNTERS_MD = os.path.join(ROOT, "profiles", "attn_dma_kernel_350m_sqrt8_counters.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha() -> str:
    """Hash of the attention kernel's own source text (the counters describe that kernel only)."""
    src = open(KERNEL_SRC).read()
    a = src.index(f"void {ATTN_KERNEL}(")
    b = src.index("\n}\n", a)
    return hashlib.sha256(src[a:b].encode()).hexdigest()[:16]


def attn_flops(cfg, n: int) -> int:
    """Algorithmic MFMA FLOPs of one prefill attention launch over n tokens from position 0.

    Per query t of chunk c: 192 per state row (2*32 for q.k on the 32 live
    dims, 2*64 for p.v) and 256 per window key (2*64 + 2*64); masked and
    zero-padded work is not counted."""
    from compressed_kv_state_amd import schedule
    C, W = cfg.chunk, cfg.window
    nq = -(-n // C)
    rows = schedule(cfg, max(nq, 1))[2].tolist()
    total = 0
    for c in range(nq):
        j = c - W // C - 1
        S = rows[j] if j >= 0 else 0
        lo = max(0, c * C - W)
        for t in range(c * C, min(n, (c + 1) * C)):
            total += 192 * S + 256 * (t - lo + 1)
    return total * cfg.seqs


def backward_flops(cfg, n: int) -> int:
    """Algorithmic FLOPs of the attention part of one backward over n tokens from position 0: the
    five products of an attention backward (scores, dP, dq, dk, dv).  Per query t of chunk c:
    448 per state row (2*32 scores + 2*64 dP + 2*32 dq + 2*32 dk + 2*64 dv on the 32 live key
    dims) and 640 per window key (5 * 2*64); masked and zero-padded work is not counted."""
    from compressed_kv_state_amd import schedule
    C, W = cfg.chunk, cfg.window
    nq = -(-n // C)
    rows = schedule(cfg, max(nq, 1))[2].tolist()
    total = 0
    for c in range(nq):
        j = c - W // C - 1
        S = rows[j] if j >= 0 else 0
        lo = max(0, c * C - W)
        for t in range(c * C, min(n, (c + 1) * C)):
            total += 448 * S + 640 * (t - lo + 1)
    return total * cfg.seqs


def decode_bytes(cfg, rows: int, t: int) -> int:
    """Algorithmic HBM bytes of one decode step at position t (ring write + attention + combine).

    Per sequence: state rows read once (read-form key, 32 live dims x 2 B fp16,
    and read-form value rho * u, 64 x 2 B bf16: 192 B), window keys/values read
    once (2 x 64 x 2 B), q/k/v/gate in (3 x 128 + 4 B), ring write (2 x 128 + 4 B),
    output 128 B."""
    C, W = cfg.chunk, cfg.window
    c = t // C
    w = t - max(0, c * C - W) + 1
    return cfg.seqs * (192 * rows + 256 * w + 388 + 260 + 128)


def read_counters():
    """Traffic figures from profiles/, if they were measured on the current kernel source."""
    if not os.path.exists(COUNTERS_MD):
        return None
    txt = open(COUNTERS_MD).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_tr or m_sha.group(1) != kernel_sha():
        return None
    return float(m_tr.group(1))


def cpu_baseline(w, budget_s: float):
    """The oracle on a bounded sample: whole sequences of the workload until budget_s has passed,
    once with the BLAS library's default thread count and once with one thread."""
    import oracle.kvm_oracle as O
    from kvm_inputs import make_inputs
    from threadpoolctl import threadpool_info, threadpool_limits

    def blas_threads():
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])

    p = O.Params.of(w)

    def run(label):
        done, t_used = 0, 0.0
        while t_used < budget_s and done < w.seqs:
            inp = make_inputs(w, seqs=[done])
            arr = [t[0].double().numpy() for t in (inp.q, inp.k, inp.v, inp.gate_logits)]
            t0 = time.perf_counter()
            O.prefill(*arr, p)
            t_used += time.perf_counter() - t0
            done += 1
            log(f"cpu oracle ({label}): {done} sequence(s), {t_used:.1f}s")
        return done, t_used

    threads = blas_threads()
    done, t_used = run(f"{threads} BLAS threads")
    with threadpool_limits(limits=1):
        done1, t1 = run("1 thread")
    return {"value": done * w.n_tokens / t_used, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "sample": f"{done} of {w.seqs} sequences of {w.name} ({w.n_tokens} tokens each), full oracle prefill "
                      f"(absorption + attention), {t_used:.1f}s, NumPy fp64 with {threads} BLAS threads "
                      f"on a host with {os.cpu_count()} CPUs",
            "one_thread": {"value": done1 * w.n_tokens / t1, "unit": "tokens/s", "cores": 1,
                           "sample": f"{done1} sequences, {t1:.1f}s"}}


def bench_prefill(w, steps: int, warmup: int):
    import torch
    from compressed_kv_state_amd import KvmConfig, KvmState
    from kvm_inputs import make_inputs
    log(f"prefill workload {w.name}: generating inputs")
    inp = make_inputs(w)
    q, k, v, g = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.gate_logits))
    del inp
    cfg = KvmConfig.of(w, max_tokens=w.n_tokens)
    st = KvmState(cfg)
    out = torch.empty_like(q)
    log(f"warmup {warmup}")
    for _ in range(warmup):
        st.reset()
        st.prefill(q, k, v, g, out)
    torch.cuda.synchronize()
    st.profile_read()
    # inside the timed region only the attention launches carry event pairs
    # (the roofline kernel); the other phases are timed in two extra steps after it
    st.profile(2)
    log(f"timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.reset()
        st.prefill(q, k, v, g, out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = st.profile_read()
    st.check()
    assert torch.isfinite(out.float()).all(), "non-finite output"
    ms_step = (t1 - t0) * 1e3 / steps
    st.profile(True)
    for _ in range(2):
        st.reset()
        st.prefill(q, k, v, g, out)
    other = st.profile_read()
    st.profile(False)
    for key in ("scan", "ring", "prep"):
        prof[key + "_ms"] = other[key + "_ms"] * steps / 2   # per timed step, like attn_ms
    prof["final_rows"] = st.info()["rows"]
    prof["scan_groups"] = st.info()["scan_groups"]
    return cfg, ms_step, prof, (q, k, v, g)


def bench_attn_alone(w, tensors, steps: int):
    """The attention kernel with the chip to itself: the same prefill with KVM_FLAG_SERIAL_PREFILL
    (every absorption first, then the attention of all query chunks in one launch on the same
    stream).  Context for the main roofline, whose launches share the chip with the scan."""
    import torch
    from compressed_kv_state_amd import KvmConfig, KvmState
    q, k, v, g = tensors
    cfg = KvmConfig.of(w, max_tokens=w.n_tokens)
    cfg.serial_prefill = True
    st = KvmState(cfg)
    out = torch.empty_like(q)
    st.reset()
    st.prefill(q, k, v, g, out)
    torch.cuda.synchronize()
    st.profile(2)
    t0 = time.perf_counter()
    for _ in range(steps):
        st.reset()
        st.prefill(q, k, v, g, out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = st.profile_read()
    st.profile(False)
    st.check()
    launches = max(prof["attn_launches"], 1)
    ms = prof["attn_ms"] / launches
    flops = attn_flops(cfg, w.n_tokens) * steps / launches
    achieved = flops / (ms * 1e-3) / 1e12
    log(f"attention alone: {ms:.3f} ms per launch, {achieved:.0f} TFLOP/s")
    return {"kernel": ATTN_KERNEL, "ms_per_step": (t1 - t0) * 1e3 / steps, "ms_per_launch": ms,
            "launches_per_step": launches / steps, "flops_per_launch": flops, "achieved": achieved,
            "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_TFLOPS,
            "note": "serial prefill (KVM_FLAG_SERIAL_PREFILL): the attention runs after the absorption, "
                    "alone on the chip; not the timed line"}


def bench_other_workloads(steps: int):
    """Prefill time of the other prefill workloads (the 120M-shaped fixed state and the long
    saturating one): context beside the main line, not part of it."""
    import torch
    from compressed_kv_state_amd import KvmConfig, KvmState
    from kvm_inputs import WORKLOADS, make_inputs
    res = {}
    for w in (WORKLOADS[1], WORKLOADS[3]):
        inp = make_inputs(w)
        q, k, v, g = (t.cuda() for t in (inp.q, inp.k, inp.v, inp.gate_logits))
        del inp
        st = KvmState(KvmConfig.of(w, max_tokens=w.n_tokens))
        out = torch.empty_like(q)
        st.reset()
        st.prefill(q, k, v, g, out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.reset()
            st.prefill(q, k, v, g, out)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        # the attention launches of two more prefills, with events (as in the main line)
        st.profile_read()
        st.profile(2)
        for _ in range(2):
            st.reset()
            st.prefill(q, k, v, g, out)
        torch.cuda.synchronize()
        prof = st.profile_read()
        st.profile(False)
        st.check()
        info = st.info()
        launches = max(prof["attn_launches"], 1)
        a_ms = prof["attn_ms"] / launches
        a_flops = attn_flops(st.cfg, w.n_tokens) * 2 / launches
        a_tf = a_flops / (a_ms * 1e-3) / 1e12
        res[w.name] = {"ms_per_step": ms, "tokens_per_s": w.seqs * w.n_tokens / (ms * 1e-3),
                       "sequences": w.seqs, "n_tokens": w.n_tokens, "final_rows": info["rows"],
                       "scan_groups": info["scan_groups"],
                       "attention": {"kernel": ATTN_KERNEL, "ms_per_launch": a_ms,
                                     "launches_per_step": launches / 2, "flops_per_launch": a_flops,
                                     "achieved": a_tf, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                                     "frac": a_tf / PEAK_MFMA_TFLOPS,
                                     "note": "beside the scan, as in the main line"}}
        log(f"{w.name}: {ms:.3f} ms per prefill, attention {a_ms:.3f} ms per launch ({a_tf:.0f} TFLOP/s)")
        del st, out, q, k, v, g
    return res


def bench_backward(w, tensors, steps: int):
    """kvm_prefill_backward over the whole workload after one traced prefill: time per backward
    (HIP events on the stream it runs on) and its algorithmic fp32 contraction rate."""
    import torch
    from compressed_kv_state_amd import KvmConfig, KvmState
    q, k, v, g = tensors
    cfg = KvmConfig.of(w, max_tokens=w.n_tokens, trace=True)
    st = KvmState(cfg)
    out = st.prefill(q, k, v, g)
    gen = torch.Generator(device="cuda").manual_seed(7)
    d_out = torch.randn(out.shape, device="cuda", generator=gen).to(out.dtype)
    st.backward(q, k, v, g, d_out)      # warm-up (allocates the backward workspace once)
    torch.cuda.synchronize()
    import ctypes
    from compressed_kv_state_amd.kvm import library
    need = ctypes.c_size_t()
    library().kvm_backward_workspace_bytes(ctypes.byref(st._c), ctypes.byref(need))
    ws = torch.empty(int(need.value), dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        grads = st.backward(q, k, v, g, d_out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert all(torch.isfinite(t).all() for t in grads), "non-finite gradient"
    flops = backward_flops(cfg, w.n_tokens)
    achieved = flops / (ms * 1e-3) / 1e12
    bf = w.dtype == "bf16"
    peak = PEAK_MFMA_TFLOPS if bf else PEAK_FP32_MFMA_TFLOPS
    log(f"backward: {ms:.3f} ms, {achieved:.1f} TFLOP/s algorithmic")
    del st, grads, ws
    return {"ms_per_step": ms, "tokens_per_s": w.seqs * w.n_tokens / (ms * 1e-3), "flops": flops,
            "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "workspace_bytes": int(need.value),
            "note": "gradients of q, k, v and gate logits; time of the whole backward (six kernels) per "
                    "prefill of the workload; " + (
                        "bf16 path: products on bf16/fp16 MFMA operands with fp32 accumulation (the "
                        "second-stage products take fp32 factors as hi + lo bf16 pairs: up to three "
                        "MFMAs each), so the peak is the bf16 one" if bf else "fp32 contractions")}


def bench_projections(w, steps: int):
    """The block's projections at the workload's shapes (x [B, N, H*64], synthetic weights):
    kvm_project_in (q, k, v and the per-head gate logit) and kvm_project_out, HIP events on the
    stream they run on, against the dense bf16 MFMA peak."""
    import torch
    from compressed_kv_state_amd import KvmConfig, project_in, project_out
    cfg = KvmConfig.of(w, max_tokens=w.n_tokens)
    D, H = w.heads * 64, w.heads
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(w.batch, w.n_tokens, D, device="cuda", generator=g).bfloat16()
    w_in = (torch.randn(3 * D + H, D, device="cuda", generator=g) / D ** 0.5).bfloat16()
    b_gate = torch.zeros(H, device="cuda")
    w_out = (torch.randn(D, D, device="cuda", generator=g) / D ** 0.5).bfloat16()
    res = {}
    q, k, v, gl = project_in(cfg, x, w_in, b_gate)
    o = q.contiguous()
    for name, fn, flops in (("in", lambda: project_in(cfg, x, w_in, b_gate),
                             2 * w.batch * w.n_tokens * D * (3 * D + H)),
                            ("out", lambda: project_out(cfg, o, w_out), 2 * w.batch * w.n_tokens * D * D)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        achieved = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": ms, "flops": flops, "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_MFMA_TFLOPS}
        log(f"projection {name}: {ms:.3f} ms, {achieved:.0f} TFLOP/s")
    res["note"] = (f"x [{w.batch}, {w.n_tokens}, {D}] bf16; in: [{3 * D + H} x {D}] (q, k, v, one gate logit per "
                   f"head), out: [{D} x {D}]; fp32 accumulation; includes the scatter into the layer's layout")
    return res


VARIANTS = {"no_value_norm": dict(value_norm=False), "no_sink_protect": dict(sink_protect=False),
            "no_merge_gate": dict(merge_gate=False), "power_0.6_alpha3": dict(sched="power", alpha=3, exponent=0.6)}


def bench_variants(w, tensors, steps: int):
    """The layer variants (the pages' ablations, a power-law schedule) on the same workload and inputs:
    time per prefill step, as for the main line (reported beside it, not in `value`)."""
    import torch
    from compressed_kv_state_amd import KvmConfig, KvmState
    q, k, v, g = tensors
    res = {}
    for name, over in VARIANTS.items():
        cfg = KvmConfig.of(w.replace(**over), max_tokens=w.n_tokens)
        st = KvmState(cfg)
        out = torch.empty_like(q)
        st.reset()
        st.prefill(q, k, v, g, out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.reset()
            st.prefill(q, k, v, g, out)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        st.check()
        res[name] = {"ms_per_step": ms, "tokens_per_s": w.seqs * w.n_tokens / (ms * 1e-3),
                     "final_rows": st.info()["rows"]}
        log(f"variant {name}: {ms:.3f} ms/step")
        del st, out
    return res


def bench_decode(w, steps: int):
    """Decode steps of the batched-decode workload.  `steps` steps of one state (its ~285 MB of
    state rows and window fit the 256 MB last-level cache of the chip only in part), then the
    same number of steps alternating between that state and a second one prefilled with the same
    tokens (two working sets at different addresses, ~570 MB in all: each step's rows come from
    HBM, not from the cache).  Kernel time from HIP events around each decode kernel."""
    import torch
    from compressed_kv_state_amd import KvmConfig, KvmState, schedule
    from kvm_inputs import make_inputs
    warm = 8
    n = w.n_tokens + warm + 2 * steps
    log(f"decode workload {w.name}: generating inputs for {w.seqs} sequences")
    inp = make_inputs(w, n_total=n)
    cfg = KvmConfig.of(w, max_tokens=n)
    states = [KvmState(cfg), KvmState(cfg)]
    q, k, v, g = (t[:, :w.n_tokens].contiguous().cuda() for t in (inp.q, inp.k, inp.v, inp.gate_logits))
    log("decode workload: prefill of two states")
    for st in states:
        st.prefill(q, k, v, g)
    del q, k, v, g
    dq, dk, dv, dg = (t[:, w.n_tokens:].contiguous().cuda() for t in (inp.q, inp.k, inp.v, inp.gate_logits))
    del inp
    steps_in = [tuple(x[:, i].contiguous() for x in (dq, dk, dv, dg)) for i in range(warm + 2 * steps)]
    out = torch.empty_like(steps_in[0][0])
    for i in range(warm):
        for st in states:
            st.decode_step(*steps_in[i], out)
    torch.cuda.synchronize()
    sched_rows = schedule(cfg, (n - 1) // cfg.chunk + 1)[2].tolist()

    def step_bytes(t):
        absorbed = max(0, t // cfg.chunk - cfg.window // cfg.chunk)
        return decode_bytes(cfg, sched_rows[absorbed - 1] if absorbed else 0, t)

    # one state: positions [n0 + warm, n0 + warm + steps) of state 0
    a = states[0]
    a.profile(True)
    t0 = time.perf_counter()
    for i in range(warm, warm + steps):
        a.decode_step(*steps_in[i], out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = a.profile_read()
    a.profile(False)
    total_bytes = sum(step_bytes(w.n_tokens + i) for i in range(warm, warm + steps))
    attn_ms = prof["dec_attn_ms"]
    gbs = total_bytes / (attn_ms * 1e-3) / 1e9
    res = {
        "workload": w.name, "sequences": w.seqs, "prefilled": w.n_tokens, "steps": steps,
        "ms_per_step": (t1 - t0) * 1e3 / steps,
        "kernel_ms_per_step": attn_ms / max(prof["dec_attn_launches"], 1),
        "absorb_ms_per_merge": prof["dec_absorb_ms"] / max(prof["dec_absorb_launches"], 1),
        "merges": prof["dec_absorb_launches"],
        "bytes_per_step": total_bytes / steps,
        "achieved_GBs": gbs, "peak_GBs": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS,
        "note": "one state; its per-step working set (~285 MB) is re-read every step and partly cache-resident",
    }
    # two states alternating: state 0 continues at n0 + warm + steps, state 1 at n0 + warm
    b = states[1]
    for st in states:
        st.profile(16)
    t0 = time.perf_counter()
    for i in range(steps):
        a.decode_step(*steps_in[warm + steps + i], out)
        b.decode_step(*steps_in[warm + i], out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pa, pb = a.profile_read(), b.profile_read()
    for st in states:
        st.profile(False)
        st.check()
    two_bytes = sum(step_bytes(w.n_tokens + warm + steps + i) + step_bytes(w.n_tokens + warm + i)
                    for i in range(steps))
    two_ms = pa["dec_attn_ms"] + pb["dec_attn_ms"]
    launches = pa["dec_attn_launches"] + pb["dec_attn_launches"]
    gbs2 = two_bytes / (two_ms * 1e-3) / 1e9
    res["hbm_resident"] = {
        "states": 2, "steps_each": steps, "kernel_ms_per_step": two_ms / max(launches, 1),
        "ms_per_step": (t1 - t0) * 1e3 / (2 * steps), "bytes_per_step": two_bytes / (2 * steps),
        "achieved_GBs": gbs2, "peak_GBs": PEAK_HBM_GBS, "frac": gbs2 / PEAK_HBM_GBS,
        "note": "decode steps alternate between two states prefilled with the same tokens (~570 MB of rows "
                "and window read per pair of steps, twice the 256 MB last-level cache)",
    }
    log(f"decode: one state {res['kernel_ms_per_step'] * 1e3:.1f} us/step ({res['frac']:.3f} of HBM), "
        f"two states {res['hbm_resident']['kernel_ms_per_step'] * 1e3:.1f} us/step "
        f"({res['hbm_resident']['frac']:.3f})")
    del states, steps_in, dq, dk, dv, dg
    return res


def copy_calibration():
    """A plain device copy of known size, so counter readings can be scaled (profiling runs only)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {n} bytes")


def _counter_rows(path, counter, grid=None):
    """{kernel name: [values in dispatch order]} for one counter of a rocprofv3 --pmc CSV
    (only dispatches of `grid` threads when given; copy kernels always)."""
    import csv
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            if grid and "copy" not in row.get("Kernel_Name", "").lower() and row.get("Grid_Size") != str(grid):
                continue
            vals.setdefault(row.get("Kernel_Name", ""), []).append(float(row["Counter_Value"]))
    return vals


def _copy_scale(d):
    """KiB moved per KiB counted, from the 1 GiB device copies of --copy-calibration."""
    v = [x for k, xs in d.items() if "copyBuffer" in k or "copy" in k.lower() for x in xs]
    if not v:
        raise SystemExit("no copy-kernel dispatches in the counter CSV (run with --copy-calibration)")
    big = max(v)
    v = [x for x in v if x >= 0.5 * big]
    mean = sum(v) / len(v)
    return (1 << 30) / 1024.0 / mean, mean


def summarize_counters(fetch_csv: str, write_csv: str, out_md: str, command: str, kernel: str = ATTN_KERNEL,
                       title: str = "", grid=None):
    """Reduce two rocprofv3 --pmc counter CSVs (FETCH_SIZE run, WRITE_SIZE run) to a summary of `kernel`.

    Each counter is scaled by 1 GiB over its mean reading on the 1 GiB device copies of
    --copy-calibration (the copy's dispatches are the large ones of the copy kernel).  For the
    attention kernel the summary also carries the traffic figure bench.py reads, tied to a hash
    of the kernel's source text."""
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE", grid)
    write = _counter_rows(write_csv, "WRITE_SIZE", grid)
    sf, cf = _copy_scale(fetch)
    sw, cw = _copy_scale(write)

    def pick(d):
        v = [x for k, xs in d.items() if kernel in k for x in xs]
        if not v:
            raise SystemExit(f"no {kernel} dispatches in the counter CSV")
        return v

    fv, wv = pick(fetch), pick(write)
    f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
    traffic = (f_kib * sf + w_kib * sw) * 1024.0
    with open(out_md, "w") as f:
        f.write(f"# {kernel} HBM traffic per dispatch{': ' + title if title else ''}\n\n")
        if grid:
            f.write(f"Dispatches of {grid} threads only.\n\n")
        f.write(f"Command (one pass per counter): `{command}`\n\n")
        f.write(f"| counter | {kernel} KiB/dispatch (mean of {len(fv)}/{len(wv)}) | total KiB | copy kernel "
                f"KiB/dispatch (1 GiB moved) | scale |\n|---|---|---|---|---|\n")
        f.write(f"| FETCH_SIZE | {f_kib:.0f} | {sum(fv):.0f} | {cf:.0f} | {sf:.4f} |\n")
        f.write(f"| WRITE_SIZE | {w_kib:.0f} | {sum(wv):.0f} | {cw:.0f} | {sw:.4f} |\n\n")
        f.write(f"bytes per dispatch (scaled fetch + write): {traffic:.6e}\n")
        f.write(f"bytes over all dispatches: {(sum(fv) * sf + sum(wv) * sw) * 1024.0:.6e}\n")
        if kernel == ATTN_KERNEL:
            f.write("\nA prefill launches the attention in pieces beside the scan; the figures are means over\n"
                    "the pieces of the profiled prefills, like bench.py's per-launch FLOPs and time.\n\n")
            f.write(f"traffic_bytes_per_launch: {traffic:.6e}\n")
            f.write(f"kernel_source_sha256_16: {kernel_sha()}  (source text of {ATTN_KERNEL})\n")
    print(open(out_md).read())


def summarize_trace(db: str, out_md: str, command: str, title: str):
    """Per-kernel dispatch statistics from a rocprofv3 --kernel-trace database (rocpd sqlite)."""
    import sqlite3
    import statistics
    con = sqlite3.connect(db)
    rows = con.execute("select name, grid_x, workgroup_x, start, end from kernels order by start").fetchall()
    # the first workload's prefills end where another workload starts: a scan of another grid
    # (another sequence count or row split) or the first decode kernel
    scans = [(gx, t0) for name, gx, _, t0, _ in rows if "scan_kernel" in name]
    first_grid = scans[0][0] if scans else None
    ends = [t0 for gx, t0 in scans if gx != first_grid]
    ends += [t0 for name, _, _, t0, _ in rows if "dec_kernel" in name]
    dec0 = min(ends or [float("inf")])
    prefill_attn = [(t1 - t0) / 1e3 for name, _, _, t0, t1 in rows if ATTN_KERNEL in name and t0 < dec0]
    sel = {}
    for name, gx, wx, t0, t1 in rows:
        if "kvm" not in name:
            continue
        short = re.sub(r"^.*?(\w+_kernel)", r"\1", name.replace("(anonymous namespace)::", ""))
        short = re.sub(r"_ZN3kvm12_GLOBAL__N_1\d+", "", short)
        sel.setdefault((short[:60], gx, wx), []).append((t1 - t0) / 1e3)
    with open(out_md, "w") as f:
        f.write(f"# {title}\n\nCommand: `{command}`\n\n")
        f.write("| kernel | grid (threads) | block | calls | total us | avg us | min us | max us |\n"
                "|---|---|---|---|---|---|---|---|\n")
        for (short, gx, wx), d in sorted(sel.items(), key=lambda kv: -sum(kv[1])):
            f.write(f"| {short} | {gx} | {wx} | {len(d)} | {sum(d):.1f} | {statistics.mean(d):.1f} | "
                    f"{min(d):.1f} | {max(d):.1f} |\n")
        dec = [x for (k, _, _), d in sel.items() if k.startswith("dec_kernel") for x in d]
        if dec:
            f.write(f"\ndec_kernel (one fused decode step, all sequences): {len(dec)} dispatches, "
                    f"mean {statistics.mean(dec):.1f} us\n")
        if prefill_attn:
            f.write(f"\n{ATTN_KERNEL} in the first prefill workload (dispatches before the first scan of "
                    f"another workload or the first decode kernel): "
                    f"{len(prefill_attn)} dispatches, mean {statistics.mean(prefill_attn):.1f} us, "
                    f"total {sum(prefill_attn):.1f} us\n")
    print(open(out_md).read())


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-projections", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--no-attn-alone", action="store_true",
                    help="skip the serial-prefill attention measurement (e.g. for counter runs of the timed launches)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true", help="add a 1 GiB device copy (counter scaling)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"))
    ap.add_argument("--counter-kernel", default=ATTN_KERNEL, help="kernel the counter summary describes")
    ap.add_argument("--counter-out", default=COUNTERS_MD, help="where the counter summary goes")
    ap.add_argument("--counter-title", default="", help="workload line of the counter summary")
    ap.add_argument("--counter-grid", type=int, default=0, help="only dispatches of this many threads")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("DB", "OUT_MD", "COMMAND", "TITLE"))
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.counter_out,
                           args.summarize_counters[2], args.counter_kernel, args.counter_title,
                           args.counter_grid or None)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the KVM layer here is built and measured on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from kvm_inputs import WORKLOADS
    wp, wd = WORKLOADS[2], WORKLOADS[4]

    cfg, ms_step, prof, tensors = bench_prefill(wp, args.steps, args.warmup)
    launches = max(prof["attn_launches"], 1)
    attn_ms = prof["attn_ms"] / launches
    flops = attn_flops(cfg, wp.n_tokens) * args.steps / launches   # mean per launch
    achieved = flops / (attn_ms * 1e-3) / 1e12
    traffic = read_counters()
    tokens = wp.seqs * wp.n_tokens
    res = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wp.name, "batch": wp.batch, "heads": wp.heads, "n_tokens": wp.n_tokens,
                   "chunk": wp.chunk, "window": wp.window, "n_sinks": wp.n_sinks, "sched": "sqrt",
                   "alpha": wp.alpha, "final_rows": prof["final_rows"]},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_MFMA_TFLOPS, "traffic": traffic,
                     "kernel": ATTN_KERNEL, "flops_per_launch": flops, "ms_per_launch": attn_ms,
                     "launches_per_step": launches / args.steps},
        "phases_ms_per_step": {"scan": prof["scan_ms"] / args.steps, "attn": prof["attn_ms"] / args.steps,
                               "ring": prof["ring_ms"] / args.steps, "rope_prep": prof["prep_ms"] / args.steps,
                               "note": "scan and attention overlap on two streams; phases sum past the step; "
                                       "attn from the timed steps, the others from 2 profiled steps after them"},
    }
    # the absorption scan: sequential over chunks, so latency-bound; its input bytes per
    # absorbed token (live key 64 B + value 128 B + gate logit 4 B, bf16) against HBM
    absorbed = max(0, (wp.n_tokens - 1) // wp.chunk - wp.window // wp.chunk)   # chunks the prefill absorbs
    scan_ms = prof["scan_ms"] / args.steps
    in_bytes = wp.seqs * absorbed * wp.chunk * (64 + 128 + 4)
    res["scan"] = {"kernel": "scan_kernel", "bound": "latency (sequential over chunks)",
                   "ms_per_step": scan_ms, "chunk_steps": absorbed,
                   "us_per_chunk_step": scan_ms * 1e3 / max(absorbed, 1),
                   "workgroups_per_sequence": prof.get("scan_groups"),
                   "input_bytes_per_step": in_bytes, "achieved_GBs": in_bytes / (scan_ms * 1e-3) / 1e9,
                   "peak_GBs": PEAK_HBM_GBS, "frac": in_bytes / (scan_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if not args.no_attn_alone:
        res["attn_alone"] = bench_attn_alone(wp, tensors, 3)
    if not args.no_backward:
        res["backward"] = bench_backward(wp, tensors, 3)
    if not args.no_projections:
        res["projections"] = bench_projections(wp, 5)
    if not args.no_variants:
        res["variants"] = bench_variants(wp, tensors, 5)
    if not args.no_other:
        res["other_workloads"] = bench_other_workloads(3)
    del tensors
    if not args.no_decode:
        res["decode"] = bench_decode(wd, args.decode_steps)
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wp, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
