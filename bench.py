#!/usr/bin/env python3
"""Throughput of causal kernelized linear attention (rank-one PSD lift) on one
MI355X, with the dominant kernel's roofline fraction and the float64 CPU
oracle timed beside it.

Main line: bf16 prefill of 4 x 8 heads x 4096 tokens, d = 64 (D = 2080),
chunk 64 — one step is one kla_prefill call (lift, intra-chunk term,
cross-chunk state readout and update, combine). Secondary lines (in
"secondary"): the 16-head x 65536-token long-context prefill, the main
workload again through the quadratic (no state) form, both prefill workloads
with the multi-factor lift KATA-M2 (two concatenated factor lifts, chunked
state form), the main one in the quadratic form with KATA-M2 and KATA-Sigma-2
(two summed factors), its gradients (the quadratic-form backward), the decode + self-recall selection loop (4096
head-states, 128 steps), the hybrid prefill (2 x 16 x 16384) and the
token-by-token hybrid decode (4096 head-states, 128 steps after a 2048-token
fill). Inputs are seeded synthetic tensors resident in HBM before timing.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_VALU_TFLOPS = 157.3
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def phi_dim(d):
    return d * (d + 1) // 2


def measured_traffic(kernel_source, profile):
    """HBM bytes per launch of a kernel, from a committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by a plain-copy calibration).
    The summary records the sha256 of the kernel's source file; once the
    source has changed the counters no longer describe it and this returns
    None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    src = os.path.join(ROOT, "kernelized_linear_attention_02_amd", "csrc", kernel_source)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != digest:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, mib):
    """A plain device-to-device copy of a known size, for scaling the HBM
    byte counters (run under rocprofv3 --pmc)."""
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "bytes_read": n * 2, "bytes_written": n * 2}), flush=True)


def stream_ceiling(torch, mib):
    """Achievable HBM rates of plain streaming on this machine (HIP events):
    an in-place multiply (read and write one buffer, the decode state's 1:1
    pattern), a copy (1:1, two buffers) and an in-place add of a second
    buffer (2 reads : 1 write)."""
    n = mib * (1 << 20) // 4
    a = torch.rand(n, device="cuda")
    b = torch.rand(n, device="cuda")
    out = {}
    for name, fn, nbytes in (("rmw_mul", lambda: a.mul_(1.0000001), 2 * 4 * n),
                             ("copy", lambda: b.copy_(a), 2 * 4 * n),
                             ("add_inplace", lambda: a.add_(b), 3 * 4 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        out[name] = dict(ms=ms, tb_per_s=nbytes / (ms * 1e-3) / 1e12)
    print(json.dumps({"stream_ceiling_mib": mib, **out}), flush=True)


def timed_calls(torch, K, fn, steps, warmup):
    """Wall time per call (sync on both sides) and the library's own kernel
    timing of the dominant kernel (HIP events on the call's stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    K.profile_read()
    K.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    K.profile_enable(False)
    kms, nk, dropped = K.profile_read()
    return (t1 - t0) * 1e3 / steps, (kms / nk if nk else float("nan")), nk / steps


def bench_prefill(torch, K, S, name, steps, warmup, factors=1, factor_kind="concat"):
    """kla_prefill on a configuration (factors > 1: a multi-factor lift
    through kla_prefill_factors, the concatenated KATA-Mg or the summed
    KATA-Sigma-g, on the matrix path for bf16 inputs with d = 64)."""
    cfg = S.CONFIGS[name]
    c = S.prefill_case(name, cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], cfg["chunk"],
                       cfg["seed"])
    q, k, v = (torch.from_numpy(x).to("cuda", torch.bfloat16) for x in (c.q, c.k, c.v))
    del c
    o = torch.empty_like(v)
    step_ms, kern_ms, per_step = timed_calls(
        torch, K, lambda: K.prefill(q, k, v, chunk=cfg["chunk"], out=o, factors=factors, factor_kind=factor_kind),
        steps, warmup)
    B, H, T, d, dv = cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"]
    D = phi_dim(d) if factors == 1 else K.factor_phi_dim(d, factors, factor_kind)
    head_tokens = B * H * T
    # dominant kernel: cross-chunk readout phi(Q)[H|s] and update phi(K)^T[V|1]
    kern_flops = 4.0 * D * (dv + 1) * head_tokens
    # whole call: plus the causal intra-chunk term
    C = cfg["chunk"]
    call_flops = kern_flops + (C + 1) * (d + dv + 1) * head_tokens
    mfma = K.prefill_uses_matrix_cores()
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_F32_VALU_TFLOPS
    achieved = kern_flops / (kern_ms * 1e-3) / 1e12
    traffic = None
    if mfma and factors == 1:
        traffic = measured_traffic("prefill_mfma.hip", f"prefill_state_kernel_{name}_traffic.md")
    return dict(
        workload=name + ("" if factors == 1 else
                         f" (KATA-{'M' if factor_kind == 'concat' else 'Sigma-'}{factors}, chunked state form, "
                         f"D = {D}{'' if mfma else ', float32 vector path'})"),
        B=B, H=H, T=T, d_qk=d, d_v=dv, chunk=C, step_ms=step_ms,
        tokens_per_s=B * T / (step_ms * 1e-3), head_tokens_per_s=head_tokens / (step_ms * 1e-3),
        call_tflops=call_flops / (step_ms * 1e-3) / 1e12,
        roofline=dict(bound="mfma" if mfma else "alu", achieved=achieved, peak=peak, unit="TFLOP/s",
                      frac=achieved / peak, kernel_ms=kern_ms,
                      traffic=traffic,
                      kernel="prefill state/readout", flops_per_launch=kern_flops,
                      # the whole call (staging, state kernel, intra-chunk finish) against the same peak
                      call_frac=call_flops / (step_ms * 1e-3) / 1e12 / peak),
        arith="bf16" if mfma else "f32",
    )


def bench_prefill_quadratic(torch, K, S, name, steps, warmup, factors=1, factor_kind="concat"):
    """The same workload through the quadratic (no state) form; factors > 1
    selects a multi-factor lift (KATA-Mg "concat", KATA-Sigma-g "sum")."""
    cfg = S.CONFIGS[name]
    c = S.prefill_case(name, cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], cfg["chunk"],
                       cfg["seed"])
    q, k, v = (torch.from_numpy(x).to("cuda", torch.bfloat16) for x in (c.q, c.k, c.v))
    del c
    o = torch.empty_like(v)
    step_ms, kern_ms, per_step = timed_calls(
        torch, K, lambda: K.prefill_quadratic(q, k, v, out=o, factors=factors, factor_kind=factor_kind),
        steps, warmup)
    B, H, T, d, dv = cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"]
    # causal pairs x (the factor inner products: 2 d_qk flop, times g for the
    # g^2 crossed products of Sigma-g; weight times [v | 1]: 2 (d_v + 1) flop)
    score = d * (factors if factor_kind == "sum" else 1)
    kern_flops = B * H * T * (T + 1) / 2 * 2.0 * (score + dv + 1)
    achieved = kern_flops / (kern_ms * 1e-3) / 1e12
    variant = "" if factors == 1 else f", KATA-{'M' if factor_kind == 'concat' else 'Sigma-'}{factors}"
    return dict(
        workload=name + f" (quadratic form{variant})", B=B, H=H, T=T, d_qk=d, d_v=dv, step_ms=step_ms,
        tokens_per_s=B * T / (step_ms * 1e-3),
        roofline=dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=achieved / PEAK_BF16_TFLOPS, kernel_ms=kern_ms, traffic=None,
                      kernel="quadratic-form prefill", flops_per_launch=kern_flops),
        arith="bf16",
    )


def bench_prefill_backward(torch, K, S, name, steps, warmup):
    """Gradients of the main workload (quadratic-form backward), after one
    forward that stores the row denominators."""
    cfg = S.CONFIGS[name]
    c = S.prefill_case(name, cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], cfg["chunk"],
                       cfg["seed"])
    q, k, v = (torch.from_numpy(x).to("cuda", torch.bfloat16) for x in (c.q, c.k, c.v))
    del c
    g = torch.randn(v.shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(8)).to(
        torch.bfloat16)
    _, den = K.prefill_quadratic(q, k, v, return_den=True)
    step_ms, kern_ms, per_step = timed_calls(
        torch, K, lambda: K.prefill_quadratic_backward(q, k, v, den, g), steps, warmup)
    B, H, T, d, dv = cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"]
    # causal pairs x (S = q.k, dP = g.v, dV += P g, dK += dS q, dQ += dS k), 2 flop per multiply-add
    kern_flops = B * H * T * (T + 1) / 2 * 2.0 * (3 * d + 2 * dv)
    achieved = kern_flops / (kern_ms * 1e-3) / 1e12
    return dict(
        workload=name + " backward (quadratic form)", B=B, H=H, T=T, d_qk=d, d_v=dv, step_ms=step_ms,
        tokens_per_s=B * T / (step_ms * 1e-3),
        roofline=dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=achieved / PEAK_BF16_TFLOPS, kernel_ms=kern_ms, traffic=None,
                      kernel="quadratic-form backward (dQ and dK/dV kernels, one span)",
                      flops_per_launch=kern_flops),
        arith="bf16",
    )


def bench_decode(torch, K, S, steps_loop, reps, deferred=False):
    cfg = S.CONFIGS["decode_sre_4096x128"]
    N, d, T0, top, nf = cfg["N"], cfg["d"], cfg["T0"], cfg["top_k"], cfg["n_fresh"]
    nsteps = cfg["steps"] if steps_loop is None else steps_loop
    t = time.time()
    case = S.decode_case(N, d=d, T0=T0, steps=nsteps, top_k=top, n_fresh=nf, seed=cfg["seed"],
                         threads=16)
    log(f"[bench] decode inputs generated in {time.time() - t:.1f}s")
    dev = "cuda"
    pk = torch.from_numpy(case.prefix_k).to(dev)[None]
    pv = torch.from_numpy(case.prefix_v).to(dev)[None]
    H, s = K.prefill(pk, pk, pv, chunk=64, outputs=False)
    H, s = H[0].contiguous(), s[0].contiguous()
    del pk, pv
    n_cand = top + nf
    # candidate slabs per step: rows [0, top) = cache gathered by the previous step
    ck = torch.empty((nsteps + 1, N, n_cand, d), device=dev)
    cv = torch.empty((nsteps + 1, N, n_cand, d), device=dev)
    ck[0, :, :top] = torch.from_numpy(case.cache0_k).to(dev)
    cv[0, :, :top] = torch.from_numpy(case.cache0_v).to(dev)
    for i in range(nsteps):
        ck[i, :, top:] = torch.from_numpy(case.fresh_k[i]).to(dev)
        cv[i, :, top:] = torch.from_numpy(case.fresh_v[i]).to(dev)
    q = torch.from_numpy(case.q).to(dev)
    k = torch.from_numpy(case.k).to(dev)
    v = torch.from_numpy(case.v).to(dev)
    del case
    o = torch.empty((N, d), device=dev)
    sc = torch.empty((N, n_cand), device=dev)
    sel = torch.empty((N, top), dtype=torch.int32, device=dev)

    P = K.decode_pending_period()
    if deferred:
        pend_k, pend_v = K.decode_pending_slots(N, d, d)

    def loop():
        n_pend = 0
        for i in range(nsteps):
            out = dict(o=o, scores=sc, sel=sel, sel_k=ck[i + 1], sel_v=cv[i + 1], sel_stride=n_cand)
            if deferred:
                K.decode_step_deferred(H, s, pend_k, pend_v, n_pend, q[i], k[i], v[i], cand_k=ck[i],
                                       cand_v=cv[i], top_k=top, gather=True, out=out)
                n_pend = (n_pend + 1) % P
            else:
                K.decode_step(H, s, q[i], k[i], v[i], cand_k=ck[i], cand_v=cv[i], top_k=top, gather=True,
                              out=out)
        if deferred:
            K.decode_flush(H, s, pend_k, pend_v, n_pend)

    loop_ms, kern_ms, per_loop = timed_calls(torch, K, loop, reps, 1)
    D = phi_dim(d)
    state = D * d * 4 + D * 4
    # per step: q, k, v, o, the candidates' keys and values read, the kept
    # rows, scores and indices written
    io = 4 * d * 4 + 2 * n_cand * d * 4 + 2 * top * d * 4 + n_cand * 4 + top * 4
    step_ms = loop_ms / nsteps
    if not deferred:
        # one fused launch per step: H and s read and written
        step_bytes = N * (2 * state + io)
        achieved = step_bytes / (kern_ms * 1e-3) / 1e9
        return dict(
            workload="decode_sre_4096x128", N=N, steps=nsteps, step_ms=step_ms,
            steps_per_s=1e3 / step_ms, kernel_ms=kern_ms,
            roofline=dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                          frac=achieved / PEAK_HBM_GBS,
                          traffic=measured_traffic("decode_fused.hip",
                                                   "decode_sre_kernel_decode_sre_4096x128_traffic.md"),
                          kernel="decode step + SRE + top-k (fused)", bytes_per_launch=step_bytes),
        )
    # deferred folds: one launch per step. P - 1 of every P read H and s, the
    # pending slots in use (n_pend = 0 .. P - 2, on average (P - 2) / 2 of
    # them) and write the token's slot; the P-th reads and writes H and s
    # (adding the P - 1 slots and its token) and reads the slots
    slot = 2 * d * 4
    read_bytes = N * (state + io + (P - 2) / 2 * slot + slot)
    fold_bytes = N * (2 * state + io + (P - 1) * slot)
    avg_bytes = ((P - 1) * read_bytes + fold_bytes) / P
    achieved = avg_bytes / (kern_ms * 1e-3) / 1e9
    return dict(
        workload="decode_sre_4096x128 (deferred folds)", N=N, steps=nsteps, pending_period=P,
        step_ms=step_ms, steps_per_s=1e3 / step_ms, kernel_ms=kern_ms,
        bytes_read_only_launch=read_bytes, bytes_fold_launch=fold_bytes,
        roofline=dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=achieved / PEAK_HBM_GBS,
                      traffic=measured_traffic("decode_fused.hip",
                                               "decode_sre_kernel_decode_sre_4096x128_deferred_traffic.md"),
                      kernel="decode step + SRE + top-k with deferred folds (P - 1 read-only launches, "
                             "one folding launch, averaged)",
                      bytes_per_launch=avg_bytes),
    )


def bench_hybrid(torch, K, S, steps, warmup):
    cfg = S.CONFIGS["hybrid_2x16x16384"]
    c = S.hybrid_case("bench", cfg["B"], cfg["H"], cfg["T"], cfg["d"], cfg["window"],
                      cfg["cache_size"], cfg["refresh"], cfg["seed"], threads=16)
    q, k, v = (torch.from_numpy(x).to("cuda", torch.bfloat16) for x in (c.q, c.k, c.v))
    # the readouts run on a second stream of the caller's, overlapping the
    # refresh chain (kla_hybrid_prefill_streams)
    side = torch.cuda.Stream()
    fn = lambda: K.hybrid_prefill(q, k, v, cfg["window"], cfg["cache_size"], cfg["refresh"], aux_stream=side)
    # the call issues a few kernels and events per 64-token block, so the
    # library's timing hooks (two more events per refresh) would inflate the
    # wall time: the plain calls are timed, the hooked ones apart
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    hooked_ms, kern_ms, per_call = timed_calls(torch, K, fn, max(1, steps // 4), 1)
    B, T = cfg["B"], cfg["T"]
    work = hybrid_flops(B * cfg["H"], T, cfg["d"], cfg["window"], cfg["cache_size"], cfg["refresh"])
    achieved = work["total"] / (step_ms * 1e-3) / 1e12
    fp32_floor_ms = work["fp32_faithful"] / (PEAK_F32_MFMA_TFLOPS * 1e12) * 1e3
    return dict(workload="hybrid_2x16x16384", step_ms=step_ms, tokens_per_s=B * T / (step_ms * 1e-3),
                hooked_step_ms=hooked_ms, refresh_chain_ms_per_call=kern_ms * per_call,
                roofline=dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=achieved / PEAK_BF16_TFLOPS, traffic=None,
                              kernel="whole call (refresh chain, folds, readouts)",
                              flops_per_launch=work["total"], flops_fp32_faithful=work["fp32_faithful"],
                              fp32_faithful_floor_ms=fp32_floor_ms,
                              frac_of_fp32_faithful_floor=fp32_floor_ms / step_ms),
                arith="bf16 (scores, folds and readouts float32-faithful)")


def hybrid_flops(n_heads, T, d, W, lam, R):
    """Algorithmic work of the hybrid prefill, counted from its definition:
    the window and cache softmax terms (2 (d + d + 1) flop per query-key
    pair: the score, the weighted value and the weight), the linear readout
    phi(q)^T [H | s] per query (2 D (d + 1)), and per scored refresh the SRE
    of every candidate against [H | s] (2 D (d + 1)) and the fold of every
    rejected pair (2 D (d + 1) for H and s, less the D squares counted
    once). The scoring and the fold must be float32-faithful (a score error
    above the near-tie rule changes the selection chain)."""
    D = phi_dim(d)
    nb = -(-T // R)
    win_pairs = cache_pairs = lin_q = 0
    sre_c = fold_p = 0
    f_prev, n_cache = 0, 0
    for b in range(nb):
        b0, b1 = b * R, min(T, b * R + R)
        f = max(0, b0 - W)
        n_ev = f - f_prev
        if n_ev > 0:
            n_cand = n_cache + n_ev
            if n_cand <= lam:
                n_cache = n_cand
            else:
                sre_c += n_cand
                fold_p += n_cand - lam
                n_cache = lam
        f_prev = f
        for t in range(b0, b1):
            win_pairs += t - f + 1
            cache_pairs += n_cache
        if f > 0:
            lin_q += b1 - b0
    per_pair = 2 * (d + d + 1)
    readout = lin_q * 2 * D * (d + 1)
    sre = sre_c * 2 * D * (d + 1)
    fold = fold_p * (2 * D * (d + 1) - D)
    total = n_heads * ((win_pairs + cache_pairs) * per_pair + readout + sre + fold)
    faithful = n_heads * (sre + fold)
    return dict(total=float(total), fp32_faithful=float(faithful))


def hybrid_decode_step_bytes(N, d, W, lam, P, row_bytes):
    """Algorithmic HBM bytes of one steady-state token-by-token hybrid step
    (window full, cache full, one rejected pair), averaged over the P steps
    of a fold cycle: H and s read once, and written once every P steps (the
    rejected pairs wait in P pending slots and are folded together); the W
    older window rows and the lam cache rows read once (keys and values, in
    the tokens' type: row_bytes per element); the evicted row read and the
    replaced cache row and the new window row written; q, k, v (bf16) read
    and o (bf16) written."""
    D = phi_dim(d)
    row = 2 * d * row_bytes
    per = (1.0 + 1.0 / P) * (D * d * 4 + D * 4) + (W + lam) * row + 3 * row + 3 * d * 2 + d * 2 + 2 * 4
    return N * per


def bench_hybrid_decode(torch, K, S, steps=None, cpu_on=False):
    cfg = S.CONFIGS["hybrid_decode_4096"]
    N, d, W, lam, T0 = cfg["N"], cfg["d"], cfg["window"], cfg["cache_size"], cfg["T0"]
    nsteps = cfg["steps"] if steps is None else steps
    q, k, v = S.hybrid_decode_tokens(N, T0 + nsteps, d, cfg["seed"], cfg["dup_frac"])
    st = K.hybrid_decode_state(N, d, d, W, lam, "cuda", dtype=torch.bfloat16)
    o = torch.empty((N, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    t = time.time()
    for i in range(T0):  # untimed: fills the window and the cache
        K.hybrid_decode_step(st, i, q[i], k[i], v[i], W, lam, out=o, ws=ws)
    torch.cuda.synchronize()
    log(f"[bench] hybrid decode: {T0} warm-up tokens in {time.time() - t:.1f}s")

    def loop():
        for i in range(T0, T0 + nsteps):
            K.hybrid_decode_step(st, i, q[i], k[i], v[i], W, lam, out=o, ws=ws)

    loop_ms, span_ms, _ = timed_calls(torch, K, loop, 1, 0)
    step_ms = loop_ms / nsteps
    P = K.hybrid_decode_pending_slots()
    assert nsteps % P == 0, "time whole fold cycles"
    step_bytes = hybrid_decode_step_bytes(N, d, W, lam, P, 2)
    achieved = step_bytes / (span_ms * 1e-3) / 1e9
    cpu = None
    if cpu_on:
        # the oracle's hybrid at refresh = 1 over head-state 0's whole token
        # stream (the same values the GPU saw)
        import oracle as O
        hq, hk, hv = (x[:, 0].float().cpu().numpy() for x in (q, k, v))
        T = hq.shape[0]
        t = time.perf_counter()
        O.hybrid_prefill(hq, hk, hv, W, lam, 1, 1.0 / math.sqrt(d))
        el = time.perf_counter() - t
        cpu = _baseline(T / el / N, "steps/s",
                        f"1 of {N} head-states x {T} tokens ({T0} filling, then {nsteps}; from token "
                        f"{W + 1 + lam} on every token refreshes the cache), float64, refresh = 1, "
                        f"{el:.1f}s of CPU time, extrapolated x{N}")
    return dict(
        workload="hybrid_decode_4096", N=N, window=W, cache_size=lam, start_token=T0, steps=nsteps,
        step_ms=step_ms, steps_per_s=1e3 / step_ms, kernel_ms=span_ms,
        roofline=dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=achieved / PEAK_HBM_GBS,
                      traffic=measured_traffic("hybrid_decode.hip",
                                               "hybrid_decode_step_hybrid_decode_4096_traffic.md"),
                      kernel="hybrid decode step (state pass + mix; one span)",
                      bytes_per_launch=step_bytes),
        cpu_baseline=cpu,
    )


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([x.get("num_threads", 1) for x in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def _baseline(value, unit, sample):
    return dict(value=value, unit=unit, cores=_oracle_threads(), kind="oracle", sample=sample)


def cpu_baseline_heads(S, name, budget_s, run, what, max_tokens=None):
    """The oracle on the workload's heads, one at a time, until budget_s of
    CPU time has been spent, in tokens/s of the whole workload (B*T tokens
    over all heads; one head-token is 1/H of a token). ``run(O, q, k, v)``
    is the oracle function of the line; ``max_tokens`` cuts each head to its
    first tokens (for the linear-time forms, whose cost per token does not
    depend on T)."""
    import oracle as O
    cfg = S.CONFIGS[name]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    kind = cfg.get("gen", "normalised")
    heads = [(b, h) for b in range(B) for h in range(H)]
    Tr = T if max_tokens is None else min(T, max_tokens)
    done = 0
    elapsed = 0.0
    for (b, h) in heads:
        c = S.prefill_case(name, B, H, T, cfg["d_qk"], cfg["d_v"], cfg["chunk"], cfg["seed"], kind=kind,
                           heads=[(b, h)])
        q, k, v = c.q[0, 0, :Tr], c.k[0, 0, :Tr], c.v[0, 0, :Tr]
        t = time.perf_counter()
        run(O, q, k, v)
        elapsed += time.perf_counter() - t
        done += 1
        if elapsed >= budget_s:
            break
    tokens = done * Tr / H
    extra = "" if done == B * H else f", extrapolated x{B * H / done:g} to all heads"
    cut = "" if Tr == T else f" (the first {Tr} of each head's {T} tokens, scaled per token)"
    return _baseline(tokens / elapsed, "tokens/s",
                     f"{done} of {B * H} heads x {Tr} tokens{cut}, {what}, {elapsed:.1f}s of CPU time" + extra)


def cpu_baseline(S, name, budget_s):
    """The oracle's chunked form (float64) on a bounded sample of heads."""
    return cpu_baseline_heads(S, name, budget_s, lambda O, q, k, v: O.prefill_chunked(q, k, v, chunk=256),
                              "float64 chunked form")


def cpu_baseline_quadratic(S, name, budget_s, factors=1, kind="concat"):
    """The oracle's O(T^2) definition (float64): causal (q.k)^2 weights, or
    the factor variant's closed-form weights."""
    if factors == 1:
        return cpu_baseline_heads(S, name, budget_s, lambda O, q, k, v: O.prefill_bruteforce(q, k, v),
                                  "float64 quadratic form")
    return cpu_baseline_heads(S, name, budget_s,
                              lambda O, q, k, v: O.prefill_factors_bruteforce(q, k, v, factors, kind),
                              f"float64 quadratic form, {kind} of {factors} factors")


def cpu_baseline_factor_state(S, name, budget_s, factors, kind, max_tokens=None):
    """The oracle's recurrent state form of a factor lift (float64)."""
    return cpu_baseline_heads(S, name, budget_s,
                              lambda O, q, k, v: O.prefill_factors_recurrent(q, k, v, factors, kind),
                              f"float64 recurrent state form, {kind} of {factors} factors", max_tokens)


def cpu_baseline_backward(S, name, budget_s):
    """The oracle's gradients (float64, quadratic form) with an upstream
    gradient of the same shape (N(0,1), drawn on the host: timing only)."""
    import numpy as np

    def run(O, q, k, v):
        do = np.random.default_rng(8).standard_normal(v.shape)
        O.prefill_backward(q, k, v, do)
    return cpu_baseline_heads(S, name, budget_s, run, "float64 gradients dq, dk, dv")


def cpu_baseline_decode(S, budget_s):
    """The oracle's decode + self-recall selection chain (float64) over all
    128 steps for a bounded sample of head-states, in steps/s of the whole
    workload (4096 head-states). The initial state is not timed (on the GPU
    it is not either)."""
    import numpy as np

    import oracle as O
    cfg = S.CONFIGS["decode_sre_4096x128"]
    N, steps = cfg["N"], cfg["steps"]
    done, elapsed = 0, 0.0
    n = 0
    while elapsed < budget_s and n < N:
        c = S.decode_case(1, d=cfg["d"], T0=cfg["T0"], steps=steps, top_k=cfg["top_k"], n_fresh=cfg["n_fresh"],
                          seed=cfg["seed"], ids=[n], threads=1)
        fk = O.phi(c.prefix_k[0])
        H0, s0 = fk.T @ c.prefix_v[0].astype(np.float64), fk.sum(0)
        t = time.perf_counter()
        O.decode_sre_chain(H0, s0, c.q[:, 0], c.k[:, 0], c.v[:, 0], c.fresh_k[:, 0], c.fresh_v[:, 0],
                           c.cache0_k[0], c.cache0_v[0], cfg["top_k"])
        elapsed += time.perf_counter() - t
        done += 1
        n += 1 + (N // 64)  # head-states spread over the workload
    per_step_all = elapsed / done * N / steps
    return _baseline(1.0 / per_step_all, "steps/s",
                     f"{done} of {N} head-states x {steps} steps (update, readout, 64-candidate scoring, top-16), "
                     f"float64, {elapsed:.1f}s of CPU time, extrapolated x{N / done:g}")


def cpu_baseline_hybrid(S, budget_s):
    """The oracle's hybrid prefill (float64, block by block) on a bounded
    sample of heads, in tokens/s of the whole workload."""
    import oracle as O
    cfg = S.CONFIGS["hybrid_2x16x16384"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    done, elapsed = 0, 0.0
    for i in range(B * H):
        b, h = divmod(i, H)
        # the workload's own head (b, h): the generator is seeded per head
        q, k, v, _ = S.hybrid_head(cfg["seed"], b, h, T, cfg["d"])
        t = time.perf_counter()
        O.hybrid_prefill(q, k, v, cfg["window"], cfg["cache_size"], cfg["refresh"], 1.0 / math.sqrt(cfg["d"]))
        elapsed += time.perf_counter() - t
        done += 1
        if elapsed >= budget_s:
            break
    tokens = done * T / H
    return _baseline(tokens / elapsed, "tokens/s",
                     f"{done} of {B * H} heads x {T} tokens, float64 block-by-block refresh chain, "
                     f"{elapsed:.1f}s of CPU time, extrapolated x{B * H / done:g}")


def bench_tiny(torch, K, S, steps, warmup):
    """The tiny float32 configuration (1 x 1 x 256, d = 16, chunk 32): a
    launch-bound parity case, timed as a whole call."""
    cfg = S.CONFIGS["tiny_f32"]
    c = S.prefill_case("tiny_f32", cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], cfg["chunk"],
                       cfg["seed"], kind="tiny")
    q, k, v = (torch.from_numpy(x).to("cuda") for x in (c.q, c.k, c.v))
    o = torch.empty_like(v)
    step_ms, kern_ms, _ = timed_calls(torch, K, lambda: K.prefill(q, k, v, chunk=cfg["chunk"], out=o),
                                      max(steps, 20), warmup)
    D = phi_dim(cfg["d_qk"])
    flops = (4.0 * D * (cfg["d_v"] + 1) + (cfg["chunk"] + 1) * (cfg["d_qk"] + cfg["d_v"] + 1)) * cfg["T"]
    return dict(workload="tiny_f32", B=1, H=1, T=cfg["T"], d_qk=cfg["d_qk"], d_v=cfg["d_v"], chunk=cfg["chunk"],
                step_ms=step_ms, tokens_per_s=cfg["T"] / (step_ms * 1e-3), kernel_ms=kern_ms,
                flops_per_call=flops,
                roofline=dict(bound="alu", achieved=flops / (kern_ms * 1e-3) / 1e12, peak=PEAK_F32_VALU_TFLOPS,
                              unit="TFLOP/s", frac=flops / (kern_ms * 1e-3) / 1e12 / PEAK_F32_VALU_TFLOPS,
                              traffic=None, kernel="whole call (float32 vector path)",
                              flops_per_launch=flops),
                note="launch-bound: 2.65 MFLOP per call, a few microseconds of work in each launch",
                arith="f32")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true", help="main prefill line only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--decode-steps", type=int, default=None, help="steps of the decode loop (128)")
    ap.add_argument("--only", choices=["tiny_f32", "prefill_1x16x65536", "prefill_4x8x4096_quadratic",
                                       "prefill_4x8x4096_m2", "prefill_4x8x4096_sigma2",
                                       "prefill_4x8x4096_m2_state", "prefill_1x16x65536_m2_state",
                                       "prefill_4x8x4096_sigma2_state",
                                       "prefill_4x8x4096_backward", "decode_sre_4096x128",
                                       "decode_sre_4096x128_deferred", "hybrid_2x16x16384", "hybrid_decode_4096"],
                    help="run just this secondary workload and print its line (for profiling)")
    ap.add_argument("--stream-ceiling", type=int, default=0, metavar="MIB",
                    help="only time plain streaming (in-place multiply, copy, in-place add) over MIB-MiB buffers")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB bf16 copy three times (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); every head "
              f"is independent, so a multi-GPU run would shard heads with no exchange and is not "
              f"measured here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kernelized_linear_attention_02_amd as K
    from kernelized_linear_attention_02_amd import synth as S
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.stream_ceiling:
        stream_ceiling(torch, args.stream_ceiling)
        return
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    K.load_library()
    if args.only:
        if args.only == "tiny_f32":
            r = bench_tiny(torch, K, S, args.steps, args.warmup)
        elif args.only == "prefill_1x16x65536":
            r = bench_prefill(torch, K, S, args.only, args.steps, args.warmup)
        elif args.only == "prefill_4x8x4096_quadratic":
            r = bench_prefill_quadratic(torch, K, S, "prefill_4x8x4096", args.steps, args.warmup)
        elif args.only == "prefill_4x8x4096_sigma2_state":
            r = bench_prefill(torch, K, S, "prefill_4x8x4096", args.steps, args.warmup, factors=2, factor_kind="sum")
        elif args.only.endswith("_m2_state"):
            r = bench_prefill(torch, K, S, args.only[:-len("_m2_state")], args.steps, args.warmup, factors=2)
        elif args.only in ("prefill_4x8x4096_m2", "prefill_4x8x4096_sigma2"):
            kind = "concat" if args.only.endswith("m2") else "sum"
            r = bench_prefill_quadratic(torch, K, S, "prefill_4x8x4096", args.steps, args.warmup, 2, kind)
        elif args.only == "prefill_4x8x4096_backward":
            r = bench_prefill_backward(torch, K, S, "prefill_4x8x4096", args.steps, args.warmup)
        elif args.only == "decode_sre_4096x128":
            r = bench_decode(torch, K, S, args.decode_steps, max(1, args.steps // 10))
        elif args.only == "decode_sre_4096x128_deferred":
            r = bench_decode(torch, K, S, args.decode_steps, max(1, args.steps // 10), deferred=True)
        elif args.only == "hybrid_decode_4096":
            r = bench_hybrid_decode(torch, K, S, args.decode_steps)
        else:
            r = bench_hybrid(torch, K, S, args.steps, args.warmup)
        print(json.dumps(r), flush=True)
        return

    name = "prefill_4x8x4096"
    log("[bench] main: prefill_4x8x4096")
    main_r = bench_prefill(torch, K, S, name, args.steps, args.warmup)
    log(f"[bench] main done: {main_r['step_ms']:.3f} ms/step")
    secondary = []
    cpu_on = not args.no_cpu_baseline
    if not args.no_secondary:
        log("[bench] secondary: tiny_f32")
        r = bench_tiny(torch, K, S, args.steps, args.warmup)
        if cpu_on:
            r["cpu_baseline"] = cpu_baseline(S, "tiny_f32", 1.0)
        secondary.append(r)
        log("[bench] secondary: prefill_1x16x65536")
        r = bench_prefill(torch, K, S, "prefill_1x16x65536", max(3, args.steps // 4), 1)
        if cpu_on:
            log("[bench] cpu baseline (oracle): prefill_1x16x65536")
            r["cpu_baseline"] = cpu_baseline(S, "prefill_1x16x65536", args.cpu_seconds * 0.5)
        secondary.append(r)
        cs = args.cpu_seconds * 0.2  # the oracle budget of each of the lines below

        def with_cpu(r, f):
            if cpu_on:
                log(f"[bench] cpu baseline (oracle): {r['workload']}")
                r["cpu_baseline"] = f()
            return r
        log("[bench] secondary: prefill_4x8x4096 in the quadratic form")
        secondary.append(with_cpu(bench_prefill_quadratic(torch, K, S, name, args.steps, args.warmup),
                                  lambda: cpu_baseline_quadratic(S, name, cs)))
        log("[bench] secondary: prefill_4x8x4096 with the KATA-M2 lift (chunked state form)")
        secondary.append(with_cpu(bench_prefill(torch, K, S, name, args.steps, args.warmup, factors=2),
                                  lambda: cpu_baseline_factor_state(S, name, cs, 2, "concat")))
        log("[bench] secondary: prefill_4x8x4096 with the KATA-Sigma-2 lift (chunked state form)")
        secondary.append(with_cpu(
            bench_prefill(torch, K, S, name, args.steps, args.warmup, factors=2, factor_kind="sum"),
            lambda: cpu_baseline_factor_state(S, name, cs, 2, "sum")))
        log("[bench] secondary: prefill_1x16x65536 with the KATA-M2 lift (chunked state form)")
        secondary.append(with_cpu(
            bench_prefill(torch, K, S, "prefill_1x16x65536", max(3, args.steps // 4), 1, factors=2),
            lambda: cpu_baseline_factor_state(S, "prefill_1x16x65536", cs, 2, "concat", max_tokens=8192)))
        for g, kind in ((2, "concat"), (2, "sum")):
            log(f"[bench] secondary: prefill_4x8x4096 in the quadratic form, {kind} of {g} factors")
            secondary.append(with_cpu(bench_prefill_quadratic(torch, K, S, name, args.steps, args.warmup, g, kind),
                                      lambda: cpu_baseline_quadratic(S, name, cs, g, kind)))
        log("[bench] secondary: prefill_4x8x4096 backward")
        secondary.append(with_cpu(bench_prefill_backward(torch, K, S, name, args.steps, args.warmup),
                                  lambda: cpu_baseline_backward(S, name, cs)))
        log("[bench] secondary: decode_sre_4096x128")
        r = bench_decode(torch, K, S, args.decode_steps, 2)
        if cpu_on:
            log("[bench] cpu baseline (oracle): decode_sre_4096x128")
            r["cpu_baseline"] = cpu_baseline_decode(S, args.cpu_seconds * 0.5)
        secondary.append(r)
        torch.cuda.empty_cache()
        log("[bench] secondary: decode_sre_4096x128 with deferred folds")
        r2 = bench_decode(torch, K, S, args.decode_steps, 2, deferred=True)
        if cpu_on:
            # the same outputs as the line above: the same oracle chain
            r2["cpu_baseline"] = r.get("cpu_baseline")
        secondary.append(r2)
        torch.cuda.empty_cache()
        log("[bench] secondary: hybrid_2x16x16384")
        r = bench_hybrid(torch, K, S, 3, 1)
        if cpu_on:
            log("[bench] cpu baseline (oracle): hybrid_2x16x16384")
            r["cpu_baseline"] = cpu_baseline_hybrid(S, args.cpu_seconds * 0.5)
        secondary.append(r)
        torch.cuda.empty_cache()
        log("[bench] secondary: hybrid_decode_4096")
        secondary.append(bench_hybrid_decode(torch, K, S, cpu_on=cpu_on))
    cpu = None
    if cpu_on:
        log("[bench] cpu baseline (oracle): prefill_4x8x4096")
        cpu = cpu_baseline(S, name, args.cpu_seconds)

    cfg = S.CONFIGS[name]
    line = {
        "metric": "prefill tokens/sec and % bf16 MFMA peak; decode steps/sec and % HBM peak",
        "value": main_r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_r["arith"],
        "data": "synthetic",
        "config": {"workload": name, "B": cfg["B"], "H": cfg["H"], "T": cfg["T"],
                   "d_qk": cfg["d_qk"], "d_v": cfg["d_v"], "chunk": cfg["chunk"],
                   "inputs": "bf16, q/k rows L2-normalised Gaussian, v ~ N(0,1)",
                   "parallelism": "single GPU"},
        "roofline": main_r["roofline"],
        "cpu_baseline": cpu,
        "head_tokens_per_s": main_r["head_tokens_per_s"],
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
