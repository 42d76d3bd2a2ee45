"""Benchmark: LORE-KV scoring + top-B + compaction, one MI355X.

A step is one eviction pass over every layer of the Llama-3.1-8B-shaped 128K
workload: for each of the 32 resident layers (n = 131072 tokens, 32 query /
8 KV heads, d = 128, d_model = 4096, bf16), kvscore_probs -> kvscore_deletion
-> kvscore_topb_select -> kv_compact.  Inputs are seeded synthetic data
generated on the device before timing (kvsynth recipe 'facts').

Prints one JSON line.  value = KV tokens scored and compacted per second,
counting n * H_kv tokens per layer, over K plain steps.  The same K steps
then run again with the library's per-launch HIP events (kvs_timing_*),
which give each kernel's average duration: the roofline object covers the
kernel with the largest share of that instrumented region.  cpu_baseline times the fp64 oracle on a
bounded sample of the same workload on the host cores.  The H2O OPT-30B decode
workload is measured after the main timed region and reported under "h2o".

Usage: python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--layers 32]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (the tiny fp32 workload's matrix ops)


def kernel_work(cfg):
    """Algorithmic work per launch, per kernel, for one layer of cfg.

    Flops count the Gram-form contractions the method needs (QK^T and AV of
    pass 1, V.G_h for N, V.y for the cross term, W_h^T W_h); the logit
    recompute of pass 2 and the lo half of y are extra work and not counted.
    Bytes count one read of the operands and one write of the results.
    """
    b, n, hq, hk, d, D, nq = cfg.batch, cfg.n, cfg.h_q, cfg.h_kv, cfg.d, cfg.d_model, cfg.n_q
    s = 4 if cfg.dtype == "f32" else 2  # bytes per element
    kv_bytes = 2 * b * hk * n * d * s
    n_keep = cfg.n_keep
    return {
        "attn_partial": {"flops": 2 * (2 * nq * n * d) * hq * b, "bytes": kv_bytes, "bound": "mfma"},
        "vnorm": {"flops": 2 * n * d * d * hq * b, "bytes": kv_bytes // 2, "bound": "mfma"},
        "score_lore": {"flops": 2 * nq * n * d * hq * b, "bytes": kv_bytes + 4 * b * hk * n,
                       "bound": "mfma"},
        "gram": {"flops": 2 * D * d * d * hq, "bytes": D * hq * d * s, "bound": "mfma"},
        "compact": {"flops": 0, "bytes": 2 * 2 * b * hk * n_keep * d * s, "bound": "hbm"},
        # the whole selection (topb_local + topb_select): S read, kept written
        "topb": {"flops": 0, "bytes": 4 * b * hk * n + 4 * b * hk * n_keep, "bound": "hbm",
                 "parts": ("topb_local", "topb_select")},
    }


def _csrc_digest():
    """sha256 over the library sources (csrc/ and include/): HBM byte counts
    taken with rocprofv3 are reported only while this matches the digest
    recorded with them."""
    import hashlib
    h = hashlib.sha256()
    for sub in ("kv_cache_eviction_amd/csrc", "include"):
        d = os.path.join(ROOT, sub)
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/pmc_traffic.json (two
    rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE in KiB per dispatch,
    each scaled by what the counter reads for a plain copy of known size), or
    None when the record is missing or the sources changed since."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != _csrc_digest():
        return None
    parts = {"topb": ("topb_local", "topb_select")}.get(kernel, (kernel,))
    ks = [rec.get("kernels", {}).get(p) for p in parts]
    if any(k is None for k in ks):
        return None
    return int(round(sum((k["fetch_kib"] * rec["fetch_scale"] + k["write_kib"] * rec["write_scale"]) * 1024
                         for k in ks)))


# measured ceilings (kvs_measure_peaks), filled in by main(): reported beside
# the published peaks, which stay the roofline denominators
MEASURED = {}


def with_measured(roof):
    """Add the achieved rate's fraction of the measured ceiling of the same
    resource (dense bf16 MFMA loop, or streaming HBM read)."""
    if roof is None:
        return None
    key = "mfma_bf16_tflops" if roof["bound"] == "mfma" else "hbm_read_gbs"
    if key in MEASURED:
        roof["measured_peak"] = MEASURED[key]
        roof["frac_of_measured"] = round(roof["achieved"] / MEASURED[key], 4)
    return roof


def roofline_of(name, work, avg_ms):
    w = work.get(name)
    if w is None:
        return None
    if w["bound"] == "mfma":
        achieved = w["flops"] / (avg_ms * 1e-3) / 1e12
        return with_measured({"kernel": name, "bound": "mfma", "achieved": round(achieved, 2),
                              "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                              "traffic": measured_traffic(name),
                              "algorithmic_per_launch": w["flops"], "avg_launch_ms": round(avg_ms, 4)})
    achieved = w["bytes"] / (avg_ms * 1e-3) / 1e9
    return with_measured({"kernel": name, "bound": "hbm", "achieved": round(achieved, 2),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(name),
                          "algorithmic_per_launch": w["bytes"], "avg_launch_ms": round(avg_ms, 4)})


def measure_peaks(kv, torch, dev):
    """Dense bf16 MFMA and streaming HBM read ceilings on this GPU (1 GiB
    buffer, so the read exceeds the 256 MB last-level cache)."""
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    tf, gb = kv.kvs_measure_peaks(buf)
    del buf
    torch.cuda.empty_cache()
    MEASURED["mfma_bf16_tflops"] = round(tf, 1)
    MEASURED["hbm_read_gbs"] = round(gb, 1)
    return {"mfma_bf16_tflops": round(tf, 1), "mfma_frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4),
            "hbm_read_gbs": round(gb, 1), "hbm_frac_of_spec": round(gb / PEAK_HBM_GBS, 4),
            "method": "kvs_measure_peaks: back-to-back v_mfma_f32_16x16x32_bf16 on four "
                      "accumulators per wave (2048 x 4 waves); waves streaming 64 KiB each "
                      "with eight 16-byte-per-lane loads in flight over 1 GiB; best of 3"}


def cpu_baseline(cfg, layers_data, min_seconds=10.0, max_layers=4):
    """fp64 oracle over whole layers of sequence 0 (every KV head: all n tokens
    and its G query heads, then selection and compaction), layer after layer
    until at least min_seconds of host work are timed (at most max_layers)."""
    import oracle
    G, d = cfg.group, cfg.d
    threads = len(os.sched_getaffinity(0))
    heads = cfg.h_kv
    dt = 0.0
    done = 0
    for inp in layers_data[:max_layers]:
        dt += _cpu_layer(oracle, cfg, inp, G, d, heads, threads)
        done += 1
        if dt >= min_seconds:
            break
    tokens = cfg.n * heads * done
    return {"value": round(tokens / dt, 1), "unit": "KV tokens/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "%d layer(s) of sequence 0, all %d KV heads each: %d tokens x %d query "
                      "heads per KV head, fp64 scores + top-B + compaction (the Cholesky factor "
                      "of W_h^T W_h is prepared outside the timer)" % (done, heads, cfg.n, G)}


def _cpu_layer(oracle, cfg, inp, G, d, heads, threads):
    dt = 0.0
    for g in range(heads):
        Q = inp["Q"][:1, g * G:(g + 1) * G].double().cpu().numpy()
        K = inp["K"][:1, g:g + 1].double().cpu().numpy()
        V = inp["V"][:1, g:g + 1].double().cpu().numpy()
        W = inp["W_O"][:, g * G * d:(g + 1) * G * d].double().cpu().numpy()
        om = inp["omega"][:1].double().cpu().numpy()
        R = oracle.projection_factors(W, G, d)
        t0 = time.perf_counter()
        r = oracle.lore_scores(Q, K, V, W, om, w=cfg.w, m=cfg.m, t=cfg.t, eps=cfg.eps,
                               lambda_l=cfg.lambda_l, nthreads=threads, R=R)
        kept, _ = oracle.topb_select(r["S"], n_sink=cfg.n_sink, w=cfg.w, chunk=cfg.chunk,
                                     budget=cfg.budget)
        oracle.compact(K, V, kept)
        dt += time.perf_counter() - t0
    return dt


def bench_config_row(kv, torch, dev, cfg, reps=10, copies=4):
    """One whole LORE-KV eviction (probs -> deletion -> top-B -> compaction)
    on another workload shape, timed on the device (config_row_cpu times the
    fp64 oracle on the same inputs).  `copies` input sets are cycled so a
    layer that fits the 256 MB MALL (the Mistral 16K layer, 67 MB of K/V) is
    not re-read from it between reps."""
    from kvsynth import lore_inputs, TORCH_DTYPES
    dt = TORCH_DTYPES[cfg.dtype]
    sets = []
    for c in range(copies):
        inp = lore_inputs(cfg, layer=0, device=dev)
        sets.append({k: inp[k].contiguous() for k in ("Q", "K", "V", "W_O", "omega")})
    desc = kv.lore_desc(batch=cfg.batch, n=cfg.n, h_q=cfg.h_q, h_kv=cfg.h_kv, d=cfg.d,
                        d_model=cfg.d_model, w=cfg.w, m=cfg.m, t=cfg.t, n_sink=cfg.n_sink,
                        chunk=cfg.chunk, budget=cfg.budget, eps=cfg.eps,
                        lambda_l=cfg.lambda_l, dtype=dt)
    ev = kv.LoreEviction(desc, dev)
    Ko = torch.empty(cfg.batch, cfg.h_kv, desc.n_keep, cfg.d, dtype=dt, device=dev)
    Vo = torch.empty_like(Ko)

    def once(i):
        x = sets[i % copies]
        ev.run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], Ko, Vo)

    for i in range(copies):
        once(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(reps):
        once(i)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    kv.kvs_timing_reset()
    kv.kvs_timing_enable(True)
    for i in range(copies):
        once(i)
    torch.cuda.synchronize()
    per = {}
    for nm, t in kv.kvs_timing_records():
        per.setdefault(nm, []).append(t)
    kv.kvs_timing_enable(False)
    kv.kvs_timing_reset()
    work = kernel_work(cfg)
    credited = sum(w["flops"] for w in work.values())
    tokens = cfg.batch * cfg.n * cfg.h_kv
    # per launch averages (head-subset launches of one call are summed per call)
    kms = {nm: sum(v) / copies for nm, v in per.items()}
    roofs = {nm: roofline_of(nm, work, kms[nm]) for nm in kms if nm in work}
    peak = PEAK_FP32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS
    row = {"workload": cfg.name, "dtype": cfg.dtype, "batch": cfg.batch, "n": cfg.n,
           "h_q": cfg.h_q, "h_kv": cfg.h_kv, "budget": cfg.budget, "ms_per_call": round(ms, 4),
           "value": round(tokens / (ms * 1e-3), 1), "unit": "KV tokens/s",
           "mfma_frac": round(credited / (ms * 1e-3) / 1e12 / peak, 4), "mfma_peak_tflops": peak,
           "credited_gflop": round(credited / 1e9, 1),
           "kernels_ms_per_call": {k: round(v, 4) for k, v in kms.items()},
           "score_roofline": roofs.get("score_lore"),
           "timing": "%d calls cycling %d input sets, between one event pair" % (reps, copies)}
    del sets, ev
    torch.cuda.empty_cache()
    return row


def config_row_cpu(cfg, oracle_threads):
    """The fp64 oracle on the whole of a workload (the device rows' first input
    set), its inputs widened to fp64 outside the timer; once per thread count
    (0 = every host core)."""
    import oracle
    from kvsynth import lore_inputs
    tokens = cfg.batch * cfg.n * cfg.h_kv
    inp = lore_inputs(cfg, layer=0)
    x64 = {k: inp[k].double().numpy() for k in ("Q", "K", "V", "W_O", "omega")}
    cpu = []
    for nt in oracle_threads:
        t0 = time.perf_counter()
        r = oracle.lore_scores(x64["Q"], x64["K"], x64["V"], x64["W_O"], x64["omega"], w=cfg.w,
                               m=cfg.m, t=cfg.t, eps=cfg.eps, lambda_l=cfg.lambda_l, nthreads=nt)
        kept, _ = oracle.topb_select(r["S"], n_sink=cfg.n_sink, w=cfg.w, chunk=cfg.chunk,
                                     budget=cfg.budget)
        oracle.compact(x64["K"], x64["V"], kept)
        dt_s = time.perf_counter() - t0
        cores = len(os.sched_getaffinity(0)) if nt == 0 else nt
        cpu.append({"value": round(tokens / dt_s, 1), "unit": "KV tokens/s", "cores": cores,
                    "kind": "oracle", "seconds": round(dt_s, 3),
                    "sample": "the whole workload: scores (fp64, incl. the Cholesky factors), "
                              "top-B and compaction"})
    return cpu


def bench_h2o(kv, torch, dev, layers=4):
    """H2O on OPT-30B-shaped layers: prefill + 512 decode steps.  The slot
    caches of `layers` layers (565 MB each) are stepped in turn, as a model's
    layers would be, so a step never finds the previous step's slots in the
    256 MB MALL."""
    from kvsynth import OPT30B_H2O, h2o_inputs
    cfg = OPT30B_H2O
    inp = h2o_inputs(cfg, device=dev)
    caches = [kv.H2OCache(cfg.batch, cfg.heads, cfg.d, cfg.cap, torch.float16, cfg.heavy_frac,
                          cfg.recent_frac, dev) for _ in range(layers)]
    cache = caches[0]
    st = torch.cuda.current_stream()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    # the other layers' prefills first (untimed), so the timed one runs warm
    for other in caches[1:]:
        other.prefill(inp["Qp"], inp["Kp"], inp["Vp"])
    torch.cuda.synchronize()
    kv.kvs_timing_reset()
    kv.kvs_timing_enable(True)
    e0.record(st)
    cache.prefill(inp["Qp"], inp["Kp"], inp["Vp"])
    e1.record(st)
    kv.kvs_timing_enable(False)
    torch.cuda.synchronize()
    kv.kvs_timing_enable(True)
    slots = 0
    e1b = torch.cuda.Event(enable_timing=True)
    e1b.record(st)
    for s in range(cfg.steps):
        for c in caches:
            c.step(inp["q"][s], inp["k"][s], inp["v"][s])
        k_h, k_r = cache.budget(cache.cur_len)
        slots += min(k_h + k_r + 1, cache.cur_len)
    e2.record(st)
    torch.cuda.synchronize()
    recs = kv.kvs_timing_records()
    kv.kvs_timing_enable(False)
    kv.kvs_timing_reset()
    dec = [ms for nm, ms in recs if nm == "h2o_decode"]
    # the prefill's kernels (recorded before the decode steps): the causal
    # attention statistics and column sums (the accumulate), then the top-B
    # reduction and the load into slots
    pre = {}
    for nm, ms in recs:
        if nm == "h2o_decode":
            break
        pre[nm] = pre.get(nm, 0.0) + ms
    # (16-bit prompts run prefill_rows + prefill_colsum; fp32 prompts the
    # general attention pass, its row combine and the column-sum score pass)
    acc_ms = sum(pre.get(k, 0.0) for k in ("prefill_rows", "prefill_colsum", "attn_partial",
                                           "attn_combine_rows", "score_h2o_colsum"))
    # causal QK^T counted once (the statistics and the column sums each form it)
    P = cfg.prompt
    pre_flops = 2 * cfg.d * (P * (P + 1) // 2) * cfg.batch * cfg.heads
    pre_bytes = 2 * cfg.batch * cfg.heads * P * cfg.d * 2  # Q and K of the prompt, read once
    # the prefill's reduction ends with one compact of the kept prompt rows
    pc = [ms for nm, ms in recs if nm == "compact"]
    k_h, k_r = cache.budget(cfg.prompt)
    pc_bytes = 2 * 2 * cfg.batch * cfg.heads * (k_h + k_r) * cfg.d * 2
    rows = cfg.batch * cfg.heads
    # bytes per step: K and V of the retained slots, acc read+write, slot map, q/k/v/O
    avg_slots = slots / cfg.steps
    step_bytes = rows * (avg_slots * (2 * cfg.d * 2 + 8) + cfg.cap * 4 + 4 * cfg.d * 2)
    dec_ms = sum(dec) / len(dec)
    hbm = step_bytes / (dec_ms * 1e-3) / 1e9
    total = e1b.elapsed_time(e2)
    pre_tf = pre_flops / (acc_ms * 1e-3) / 1e12 if acc_ms > 0 else 0.0
    pre_gb = pre_bytes / (acc_ms * 1e-3) / 1e9 if acc_ms > 0 else 0.0
    return {"workload": cfg.name, "prefill_ms": round(e0.elapsed_time(e1), 3),
            "prefill_kernels_ms": {k: round(v, 4) for k, v in pre.items()},
            "prefill_roofline": with_measured({
                "kernel": "prefill_rows + prefill_colsum (causal prompt accumulate)",
                "bound": "mfma", "achieved": round(pre_tf, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(pre_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "algorithmic_per_launch": pre_flops, "avg_launch_ms": round(acc_ms, 4),
                "hbm_gbs_on_q_and_k": round(pre_gb, 1),
                "note": "the causal QK^T is formed twice (row statistics, then column sums) "
                        "and credited once"}),
            "decode_layers": layers,
            "decode_ms_total": round(total, 3),
            "decode_step_kernel_ms": round(dec_ms, 4),
            "slots_attended_per_s": round(layers * rows * slots / (total * 1e-3), 1),
            "roofline": with_measured({"kernel": "h2o_decode", "bound": "hbm",
                                       "achieved": round(hbm, 1), "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": round(hbm / PEAK_HBM_GBS, 4),
                                       "traffic": measured_traffic("h2o_decode")}),
            "prefill_compact": {"kernel_ms": round(pc[0], 4), "bytes": pc_bytes,
                                "achieved_gbs": round(pc_bytes / (pc[0] * 1e-3) / 1e9, 1),
                                "frac": round(pc_bytes / (pc[0] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            if pc else None}


def bench_compact_qwen(kv, torch, dev, reps=20):
    """kv_compact on the Qwen2.5-14B batch shape (8 sequences x 8 KV heads of
    32K tokens, bf16, keep 1 + 512 + 32 per head): the HBM-bound gather at a
    size where it is not launch-bound.  The kept sets have the selector's
    structure: the sink, the window, and B/chunk = 128 whole aligned chunks
    of 4 candidates (chunk pooling ranks whole chunks), drawn at random per
    row.  Each of the reps gathers a different set into its own output, so
    the rows read (K/V 1.07 GB) do not stay in the 256 MB MALL between reps;
    the launches run back to back between one event pair (per-launch events
    would add about 2 us to a few-us kernel)."""
    from kvsynth import QWEN_14B_BATCH as cfg
    b, hk, n, d = cfg.batch, cfg.h_kv, cfg.n, cfg.d
    n_keep = cfg.n_sink + cfg.budget + cfg.w
    g = torch.Generator(device=dev)
    g.manual_seed(4040)
    K = torch.randn(b, hk, n, d, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    V = torch.randn(b, hk, n, d, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rows = b * hk
    ch = cfg.chunk
    # whole chunks inside the candidates [n_sink, n - w)
    c_lo = (cfg.n_sink + ch - 1) // ch
    c_hi = (n - cfg.w) // ch
    per = cfg.budget // ch
    tail = torch.arange(n - cfg.w, n, device=dev).expand(rows, cfg.w)
    sink = torch.arange(cfg.n_sink, device=dev).expand(rows, cfg.n_sink)
    sets = []
    for _ in range(reps):
        chunks = torch.rand(rows, c_hi - c_lo, generator=g, device=dev).argsort(dim=1)[:, :per] + c_lo
        mid = (chunks[:, :, None] * ch + torch.arange(ch, device=dev)).reshape(rows, per * ch)
        kept = torch.cat([sink, mid, tail], dim=1)
        kept = kept.sort(dim=1).values.to(torch.int32).reshape(b, hk, n_keep).contiguous()
        Ko = torch.empty(b, hk, n_keep, d, dtype=torch.bfloat16, device=dev)
        sets.append((kept, Ko, torch.empty_like(Ko)))
    for kept, Ko, Vo in sets[:3]:
        kv.kv_compact(K, V, kept, Ko, Vo)
    torch.cuda.synchronize()
    # flush the rows the warm-up touched out of the MALL
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    scrub.fill_(1)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for kept, Ko, Vo in sets:
        kv.kv_compact(K, V, kept, Ko, Vo)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * 2 * rows * n_keep * d * 2  # read + write of the kept K and V rows
    gbs = nbytes / (ms * 1e-3) / 1e9
    del K, V, sets
    # The same bytes moved by a plain contiguous device copy, timed the same
    # way (reps back-to-back launches, a different source slice each, after
    # the scrub): what one launch of this size reaches on this machine without
    # the kept-index indirection.
    half = nbytes // 4  # bf16 elements read (= written) per rep
    src = torch.empty(reps * half, dtype=torch.bfloat16, device=dev)
    src.fill_(1.5)
    dst = torch.empty_like(src)
    scrub.fill_(2)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(reps):
        dst[i * half:(i + 1) * half].copy_(src[i * half:(i + 1) * half])
    e1.record(st)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    copy_gbs = nbytes / (copy_ms * 1e-3) / 1e9
    del src, dst, scrub
    torch.cuda.empty_cache()
    return {"workload": cfg.name + "-compact", "kernel_ms": round(ms, 4), "bytes": nbytes,
            "kept_sets": "sink + %d random whole chunks of %d + window, a different set per rep"
                         % (per, ch),
            "timing": "%d back-to-back launches, distinct kept sets and outputs" % reps,
            "contiguous_copy_same_bytes": {"ms": round(copy_ms, 4), "achieved_gbs": round(copy_gbs, 1),
                                           "compact_frac_of_copy": round(copy_ms / ms, 4)},
            "roofline": with_measured({"kernel": "compact", "bound": "hbm", "achieved": round(gbs, 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None})}


def bench_refresh(kv, torch, dev, reps=10):
    """Counter-causal memory refresh on a Qwen2.5-7B-shaped layer (J = 4096,
    h = J/4, n = 5120): the reversed-mask attention of every cached position
    (MFMA-bound: 2*d*n*(n-1) flops per query head over the upper triangle),
    then the token-level keep-J selection and the K, V, id gather."""
    from kvsynth import QWEN7B_REFRESH as cfg, refresh_inputs
    x = refresh_inputs(cfg, device=dev)
    b, n = cfg.batch, cfg.n
    desc = kv.lore_desc(batch=b, n=n, h_q=cfg.h_q, h_kv=cfg.h_kv, d=cfg.d, d_model=cfg.h_q * cfg.d,
                        w=0, m=1, t=1, n_sink=0, dtype=torch.bfloat16)
    m = torch.empty(b, cfg.h_q, n, device=dev)
    l = torch.empty_like(m)
    O = torch.empty(b, cfg.h_q, n, cfg.d, device=dev)
    ws = torch.empty(kv.kvs_refresh_workspace_bytes(b, n), dtype=torch.uint8, device=dev)
    kept = torch.empty(b, cfg.J, dtype=torch.int32, device=dev)
    Ko = torch.empty(b, cfg.h_kv, cfg.J, cfg.d, dtype=torch.bfloat16, device=dev)
    Vo = torch.empty_like(Ko)
    ido = torch.empty(b, cfg.J, dtype=torch.int32, device=dev)

    def once():
        kv.kvscore_counter_causal(desc, x["Q"], x["K"], x["V"], m, l, O)
        kv.kvscore_refresh(x["surprise"], x["K"], x["V"], kept, Ko, Vo, n_sys=cfg.n_sys, J=cfg.J,
                           ids=x["ids"], ids_out=ido, ws=ws)

    for _ in range(3):
        once()
    torch.cuda.synchronize()
    kv.kvs_timing_reset()
    kv.kvs_timing_enable(True)
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    per = {}
    for nm, ms in kv.kvs_timing_records():
        per.setdefault(nm, []).append(ms)
    kv.kvs_timing_enable(False)
    kv.kvs_timing_reset()
    avg = {nm: sum(v) / len(v) for nm, v in per.items()}
    total = sum(sum(v) for v in per.values()) / reps
    flops = 2 * cfg.d * n * (n - 1) * cfg.h_q * b
    tf = flops / (avg["attn_partial"] * 1e-3) / 1e12
    return {"workload": cfg.name, "n": n, "J": cfg.J, "h": cfg.h, "n_sys": cfg.n_sys,
            "kernels_ms": round(total, 4), "per_kernel_ms": {k: round(v, 4) for k, v in avg.items()},
            "roofline": {"kernel": "attn_partial (counter-causal)", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--config", default="llama3.1-8b-128k-32layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-h2o", action="store_true")
    ap.add_argument("--no-config-rows", action="store_true",
                    help="skip the Mistral 16K / Qwen batch / tiny workload rows")
    ap.add_argument("--streams", type=int, default=1,
                    help="spread the layers of a plain timed step over this many streams")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of one step instead of eager launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (3 launches), the "
                         "known-size kernel that scales HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the scoring path runs on a single MI355X and "
              "needs no collectives. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_eviction_amd as kv
    from kvsynth import (LORE_CONFIGS, lore_inputs, trajectory_token_stats, future_queries,
                         TORCH_DTYPES)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    print("[bench] measured peaks", file=sys.stderr, flush=True)
    peaks = measure_peaks(kv, torch, dev)
    cfg = LORE_CONFIGS[args.config]
    layers = args.layers or cfg.layers
    dt = TORCH_DTYPES[cfg.dtype]
    print("[bench] generating %d layers of %s on the device" % (layers, cfg.name),
          file=sys.stderr, flush=True)
    data = []
    for l in range(layers):
        inp = lore_inputs(cfg, layer=l, device=dev)
        data.append({k: inp[k].contiguous() for k in ("Q", "K", "V", "W_O", "omega", "marks")})
    desc = kv.lore_desc(batch=cfg.batch, n=cfg.n, h_q=cfg.h_q, h_kv=cfg.h_kv, d=cfg.d,
                        d_model=cfg.d_model, w=cfg.w, m=cfg.m, t=cfg.t, n_sink=cfg.n_sink,
                        chunk=cfg.chunk, budget=cfg.budget, eps=cfg.eps,
                        lambda_l=cfg.lambda_l, dtype=dt)
    ev = kv.LoreEviction(desc, dev)
    outs = [(torch.empty(cfg.batch, cfg.h_kv, desc.n_keep, cfg.d, dtype=dt, device=dev),
             torch.empty(cfg.batch, cfg.h_kv, desc.n_keep, cfg.d, dtype=dt, device=dev))
            for _ in range(layers)]

    def step():
        for l in range(layers):
            x = data[l]
            ev.run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], outs[l][0], outs[l][1])

    # layers are independent once every layer's K/V is resident, so a plain
    # step may run layer l on stream l % S, each stream with its own buffers
    # and workspace (default priority); the main stream joins them at the end
    n_str = max(1, args.streams)
    evs = [ev] + [kv.LoreEviction(desc, dev) for _ in range(n_str - 1)]
    side_streams = [torch.cuda.Stream() for _ in range(n_str - 1)]

    def step_streams():
        main = torch.cuda.current_stream()
        for sst in side_streams:
            sst.wait_stream(main)
        for l in range(layers):
            x = data[l]
            i = l % n_str
            with torch.cuda.stream(main if i == 0 else side_streams[i - 1]):
                evs[i].run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], outs[l][0], outs[l][1])
        for sst in side_streams:
            main.wait_stream(sst)

    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
        if n_str > 1:
            step_streams()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()

    # with --graph the plain timed steps replay one HIP graph of a whole step
    # (the library enqueues only kernels on the caller's stream, so a step
    # captures as is).  It measured no faster than eager launches: the GPU
    # already runs ahead of the host, so eager is the default
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            step()
        st.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    def timed(instrumented):
        """K steps between two stream events (graph replays unless
        instrumented); with instrumented, the library also brackets every
        launch with its own event pair."""
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        kv.kvs_timing_reset()
        kv.kvs_timing_enable(instrumented)
        torch.cuda.synchronize()
        start.record(st)
        for _ in range(args.steps):
            if graph is not None and not instrumented:
                graph.replay()
            elif n_str > 1 and not instrumented:
                step_streams()
            else:
                step()
        stop.record(st)
        torch.cuda.synchronize()
        recs = kv.kvs_timing_records()
        kv.kvs_timing_enable(False)
        kv.kvs_timing_reset()
        return start.elapsed_time(stop), recs

    # value comes from the plain run; the per-launch event pairs (about 70 us
    # of extra gaps per layer) are kept out of it and taken in a second run
    # of the same steps, which gives the per-kernel durations
    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    total_ms, _ = timed(False)
    print("[bench] timing %d steps with per-launch events" % args.steps, file=sys.stderr, flush=True)
    total_ms_inst, recs = timed(True)

    per = {}
    for nm, ms in recs:
        p = per.setdefault(nm, [0, 0.0])
        p[0] += 1
        p[1] += ms
    ms_per_step = total_ms / args.steps
    tokens = cfg.batch * cfg.n * cfg.h_kv * layers * args.steps
    value = tokens / (total_ms * 1e-3)
    work = kernel_work(cfg)
    kernels = {nm: {"launches": c, "avg_ms": round(t / c, 4),
                    "share": round(t / total_ms_inst, 4)} for nm, (c, t) in per.items()}
    dominant = max(per, key=lambda k: per[k][1])
    roof = roofline_of(dominant, work, per[dominant][1] / per[dominant][0])
    others = {nm: roofline_of(nm, work, per[nm][1] / per[nm][0]) for nm in per if nm in work}
    for nm, w in work.items():  # rooflines of steps that run as several kernels
        if "parts" in w and all(p in per for p in w["parts"]):
            others[nm] = roofline_of(nm, work, sum(per[p][1] / per[p][0] for p in w["parts"]))
    credited = sum(w["flops"] for w in work.values())
    layer_ms = ms_per_step / layers

    out = {
        "metric": "KV tokens scored+compacted/sec per layer (n*H_kv)",
        "value": round(value, 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_instrumented": round(total_ms_inst / args.steps, 3),
        "launch": ("hip-graph replay of one step" if graph is not None else
                   "eager, layers over %d streams" % n_str if n_str > 1 else "eager"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, generated on device)",
        "config": {"workload": cfg.name, "layers": layers, "batch": cfg.batch, "n": cfg.n,
                   "h_q": cfg.h_q, "h_kv": cfg.h_kv, "d": cfg.d, "d_model": cfg.d_model,
                   "w": cfg.w, "m": cfg.m, "t": cfg.t, "budget": cfg.budget, "chunk": cfg.chunk},
        "roofline": roof,
        "measured_peaks": peaks,
        "layer_ms": round(layer_ms, 4),
        "layer_mfma_frac": round(credited / (layer_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels": kernels,
        "kernel_rooflines": others,
    }
    # the prompt-side baseline scorer on the same layer: the window rows'
    # attention summed per token (K read once; HBM-bound: 34 GFLOP of credited
    # QK^T against 268 MB)
    print("[bench] prompt-side window score", file=sys.stderr, flush=True)
    x = data[0]
    ev.baseline(kv.KVS_BASELINE_WINDOW, x["Q"], x["K"], x["V"])
    torch.cuda.synchronize()
    kv.kvs_timing_reset()
    kv.kvs_timing_enable(True)
    for _ in range(5):
        kv.kvscore_baseline_scores(desc, kv.KVS_BASELINE_WINDOW, x["Q"], x["K"], ev.row_max,
                                   ev.row_sum, ev.S, ev.ws)
    torch.cuda.synchronize()
    brec = kv.kvs_timing_records()
    kv.kvs_timing_enable(False)
    kv.kvs_timing_reset()
    bms = sum(ms for _, ms in brec) / 5
    srec = [ms for nm, ms in brec if nm == "score_h2o_colsum"]
    sms = sum(srec) / len(srec)
    kbytes = cfg.batch * cfg.h_kv * cfg.n * cfg.d * 2 + 4 * cfg.batch * cfg.h_kv * cfg.n
    out["baseline_window"] = {
        "kernels_ms": round(bms, 4), "launches_per_call": len(brec) // 5,
        "score_kernel_ms": round(sms, 4),
        "roofline": {"kernel": "score_h2o_colsum", "bound": "hbm",
                     "achieved": round(kbytes / (sms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kbytes / (sms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("score_baseline")}}
    # the trajectory reliability weights that feed the lookahead term (Eq. 10):
    # a few microseconds of fp64 cosines over the M*T lookahead queries, so
    # launch latency bounds it; the HBM rate is over the lookahead rows read
    print("[bench] reliability weights", file=sys.stderr, flush=True)
    logp, ent = trajectory_token_stats(cfg, 0, device=dev)
    ev.weights(x["Q"], logp, ent)
    torch.cuda.synchronize()
    kv.kvs_timing_reset()
    kv.kvs_timing_enable(True)
    for _ in range(5):
        ev.weights(x["Q"], logp, ent)
    torch.cuda.synchronize()
    rrec = kv.kvs_timing_records()
    kv.kvs_timing_enable(False)
    kv.kvs_timing_reset()
    rms = sum(ms for _, ms in rrec) / 5
    cms = [ms for nm, ms in rrec if nm == "traj_cosine"]
    cms = sum(cms) / len(cms)
    qbytes = cfg.batch * cfg.h_q * cfg.m * cfg.t * cfg.d * 2
    out["reliability_weights"] = {
        "kernels_ms": round(rms, 4), "launches_per_call": len(rrec) // 5,
        "roofline": {"kernel": "traj_cosine", "bound": "hbm",
                     "achieved": round(qbytes / (cms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(qbytes / (cms * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
                     "traffic": None}}
    # attention-output fidelity of layer 0's retained cache under 64 held-out
    # queries per head aimed at the planted facts, for the LORE-KV selection
    # and for the window baseline's; timed on the LORE-KV cache (its cost is
    # the full-cache attention pass, MFMA-bound like pass 1)
    print("[bench] output fidelity", file=sys.stderr, flush=True)
    Qf = future_queries(cfg, x, 64, device=dev)
    _, fid_lore = ev.fidelity(Qf, x["K"], x["V"], outs[0][0], outs[0][1])
    ev.baseline(kv.KVS_BASELINE_WINDOW, x["Q"], x["K"], x["V"])
    ev.select()
    Kw, Vw = torch.empty_like(outs[0][0]), torch.empty_like(outs[0][1])
    ev.compact(x["K"], x["V"], Kw, Vw)
    _, fid_win = ev.fidelity(Qf, x["K"], x["V"], Kw, Vw)
    torch.cuda.synchronize()
    kv.kvs_timing_reset()
    kv.kvs_timing_enable(True)
    for _ in range(5):
        ev.fidelity(Qf, x["K"], x["V"], outs[0][0], outs[0][1])
    torch.cuda.synchronize()
    frec = kv.kvs_timing_records()
    kv.kvs_timing_enable(False)
    kv.kvs_timing_reset()
    fms = sum(ms for _, ms in frec) / 5
    aff = [ms for nm, ms in frec if nm == "attn_partial"][0::2]  # the full-cache launch of each call
    aff = sum(aff) / len(aff)
    fper = {}
    for nm, ms in frec:
        fper.setdefault(nm, []).append(ms)
    fflops = 2 * 2 * 64 * cfg.n * cfg.d * cfg.h_q * cfg.batch
    out["output_fidelity"] = {
        "held_out_queries_per_head": 64, "lore": round(float(fid_lore.mean()), 4),
        "window_baseline": round(float(fid_win.mean()), 4),
        "kernels_ms": round(fms, 4), "launches_per_call": len(frec) // 5,
        "per_kernel_ms": {nm: [round(v, 4) for v in vs[:4]] for nm, vs in fper.items()},
        "roofline": {"kernel": "attn_partial", "bound": "mfma",
                     "achieved": round(fflops / (aff * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": round(fflops / (aff * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None}}
    print("[bench] counter-causal refresh", file=sys.stderr, flush=True)
    out["refresh"] = bench_refresh(kv, torch, dev)
    # diagnostic, not timed: recall of layer 0's planted facts in the kept
    # sets of LORE-KV, of its window-only form (lambda_L = 0) and of the two
    # prompt-side baselines (the synthetic lookahead queries target the
    # facts, the window queries do not)
    print("[bench] planted-fact recall", file=sys.stderr, flush=True)
    facts = x["marks"].long()  # [b][n_facts] positions, shared by the KV heads

    def recall(kept):
        hit = (kept.long()[:, :, :, None] == facts[:, None, None, :]).any(dim=2)
        return round(float(hit.float().mean()), 4)

    Kd = torch.empty_like(outs[0][0])
    Vd = torch.empty_like(outs[0][1])
    ev.run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], Kd, Vd)
    rec = {"lore_kv": recall(ev.kept)}
    desc0 = kv.lore_desc(batch=cfg.batch, n=cfg.n, h_q=cfg.h_q, h_kv=cfg.h_kv, d=cfg.d,
                         d_model=cfg.d_model, w=cfg.w, m=cfg.m, t=cfg.t, n_sink=cfg.n_sink,
                         chunk=cfg.chunk, budget=cfg.budget, eps=cfg.eps, lambda_l=0.0, dtype=dt)
    ev0 = kv.LoreEviction(desc0, dev)
    ev0.run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], Kd, Vd)
    rec["lore_kv_window_only"] = recall(ev0.kept)
    for name, kind in (("window_baseline", kv.KVS_BASELINE_WINDOW), ("tova", kv.KVS_BASELINE_TOVA)):
        ev0.baseline(kind, x["Q"], x["K"], x["V"])
        ev0.select()
        rec[name] = recall(ev0.kept)
    # retention-order shift (LORE-KV page, "More analyses"): the share of
    # LORE-KV's kept candidates that its window-only form, and the window
    # baseline, do not keep (mean over KV heads; layer 0, B = 128)
    sh = torch.empty(cfg.batch, cfg.h_kv, device=dev)
    kept_lore = ev.kept.clone()
    ev0.run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], Kd, Vd)
    kv.kvscore_retention_shift(kept_lore, ev0.kept, sh, n=cfg.n, n_sink=cfg.n_sink, w=cfg.w)
    shift = {"budget": cfg.budget, "lore_vs_window_only": round(float(sh.mean()), 4)}
    ev0.baseline(kv.KVS_BASELINE_WINDOW, x["Q"], x["K"], x["V"])
    ev0.select()
    kv.kvscore_retention_shift(kept_lore, ev0.kept, sh, n=cfg.n, n_sink=cfg.n_sink, w=cfg.w)
    shift["lore_vs_window_baseline"] = round(float(sh.mean()), 4)
    del ev0
    out["planted_fact_recall"] = rec
    out["retention_shift"] = shift
    # every device measurement first, then the host-side oracle timings, so the
    # GPU never sits idle (and clocks down) between two device measurements
    from kvsynth import MISTRAL_16K, QWEN_14B_BATCH, TINY
    plan = ((MISTRAL_16K, 4, (0, 1)), (QWEN_14B_BATCH, 4, (0,)), (TINY, 1, (0, 1)))
    rows = {}
    if not args.no_config_rows:
        # the other LORE-KV workloads: the Mistral-7B 16K layer, the Qwen2.5-14B
        # batch and the tiny fp32 layer (launch-bound), each beside the oracle
        for c, copies, _ in plan:
            print("[bench] workload row %s" % c.name, file=sys.stderr, flush=True)
            rows[c.name] = bench_config_row(kv, torch, dev, c, copies=copies)
        out["workload_rows"] = rows
    if not args.no_h2o:
        print("[bench] H2O decode", file=sys.stderr, flush=True)
        out["h2o"] = bench_h2o(kv, torch, dev)
        print("[bench] compact on the Qwen batch shape", file=sys.stderr, flush=True)
        out["compact_qwen"] = bench_compact_qwen(kv, torch, dev)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, data)
        for c, _, threads in plan:
            if c.name in rows:
                print("[bench] workload row %s: oracle" % c.name, file=sys.stderr, flush=True)
                rows[c.name]["cpu_baseline"] = config_row_cpu(c, threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
