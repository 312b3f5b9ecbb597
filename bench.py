"""Benchmark of the MoT joint-attention hot path on one MI355X.

One step = one pass of the whole path over the workload's packed sequence,
with every input resident in HBM: region-split QKV projection -> mRoPE of K
(Q is rotated on load) -> masked flash attention -> region-split output
projection -> flow-matching Euler update of the noisy latent.

Prints ONE JSON line.  ``value`` is masked-attention TFLOP/s counting only
allowed (query, key, head) triples (4*D flops each) divided by the wall time
of the whole step, so it is a lower bound on the attention kernel's own rate;
``roofline`` reports that kernel alone (HIP events on its stream), against
the MI355X dense bf16 MFMA peak.  ``cpu_baseline`` times the CPU fp64 oracle
on a bounded sample of the same attention.
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

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
ATTN_KERNEL = "attn_fwd_mfma"
LIB_PATH = os.path.join(ROOT, "multimodal_diffusion_transformer_amd", "libmotattn.so")


def _elf_sections(elf):
    """Section headers of a little-endian ELF64 image: dicts with name,
    type, addr, off, size and link."""
    import struct

    if elf[:4] != b"\x7fELF" or elf[4] != 2 or elf[5] != 1:
        raise ValueError("not a little-endian ELF64 image")
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    secs = []
    for i in range(shnum):
        name, typ, _, addr, off, size, link, _, _, _ = struct.unpack_from(
            "<IIQQQQIIQQ", elf, shoff + i * shentsize)
        secs.append({"name": name, "type": typ, "addr": addr, "off": off, "size": size, "link": link})
    names = secs[shstrndx]["off"]
    for sec in secs:
        end = elf.index(b"\0", names + sec["name"])
        sec["name"] = elf[names + sec["name"]:end].decode()
    return secs


def attention_kernel_spans(so):
    """(name, file offset, size) of every gfx950 attention kernel and kernel
    descriptor inside the image `so` of the built library.

    The library's .hip_fatbin section holds one clang offload bundle per
    translation unit (magic, entry count, then offset / size / target
    triple per entry); each gfx950 entry is an ELF code object whose symbol
    table locates every kernel and its descriptor."""
    import struct

    fb = next(x for x in _elf_sections(so) if x["name"] == ".hip_fatbin")
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    spans = []
    pos = so.find(magic, fb["off"], fb["off"] + fb["size"])
    while pos >= 0:
        n, = struct.unpack_from("<Q", so, pos + len(magic))
        p = pos + len(magic) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", so, p)
            triple = so[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            co_off = pos + off
            co = so[co_off:co_off + size]
            if not triple.endswith("gfx950") or co[:4] != b"\x7fELF":
                continue
            secs = _elf_sections(co)
            symtab = next(x for x in secs if x["type"] == 2)  # SHT_SYMTAB
            strs = secs[symtab["link"]]["off"]
            for i in range(symtab["size"] // 24):
                st_name, _, _, shndx, value, size_ = struct.unpack_from(
                    "<IBBHQQ", co, symtab["off"] + 24 * i)
                name = co[strs + st_name:co.index(b"\0", strs + st_name)]
                if ATTN_KERNEL.encode() not in name or size_ == 0 or shndx >= len(secs):
                    continue
                sec = secs[shndx]
                spans.append((name, co_off + sec["off"] + value - sec["addr"], size_))
        pos = so.find(magic, pos + len(magic), fb["off"] + fb["size"])
    return spans


def attention_kernel_hash(lib_path=LIB_PATH):
    """First 16 hex digits of a sha256 over the gfx950 machine code and
    kernel descriptors of the attention kernels in the built library, or
    None if the library cannot be read.  It changes exactly when those
    kernels do, and not with comments, host code or where the kernels sit in
    their code object (a descriptor's bytes 16..23 hold the offset of its
    kernel's code from the descriptor, which is masked)."""
    import hashlib
    import struct

    try:
        with open(lib_path, "rb") as f:
            so = f.read()
        spans = attention_kernel_spans(so)
    except (OSError, ValueError, StopIteration, struct.error, IndexError, UnicodeDecodeError):
        return None
    if not spans:
        return None
    h = hashlib.sha256()
    for name, off, size in sorted(spans):
        body = bytearray(so[off:off + size])
        if name.endswith(b".kd") and size >= 24:
            body[16:24] = bytes(8)
        h.update(name + b"\0" + struct.pack("<Q", size) + bytes(body))
    return h.hexdigest()[:16]


def traffic_from_profile(workload):
    """HBM bytes per attention launch as recorded in profiles/ by the two
    counter runs (FETCH_SIZE, WRITE_SIZE) and their copy calibration, or None
    when the attention kernels changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.txt" % (ATTN_KERNEL, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    h = attention_kernel_hash()
    if h is None or kv.get("attention_kernel_hash") != h:
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def attention_pairs(n, n_ar):
    """Allowed pairs of the AR-causal / DM-full mask over n tokens: the AR
    rows see a causal prefix, every DM row sees all n keys."""
    return n_ar * (n_ar + 1) // 2 + (n - n_ar) * n


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(wl, budget_s=15.0):
    """Time the fp64 oracle attention on a bounded sample: blocks of 256 DM
    query rows (each reading all keys) of one head after another, until about
    budget_s of timed work.  Only the oracle calls are timed (the inputs of
    each head are drawn outside the timed intervals).  Reports the BLAS
    threads the oracle actually used and the host CPU model."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import workloads as W
    from oracle import attention as oattn

    n = wl.n_tokens
    n_ar = W.region_counts(wl.segments)[0]
    d = wl.head_dim
    avail = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    rows_done = heads = 0
    flops = 0.0
    dt = 0.0
    with threadpool_limits(limits=avail):
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        while dt < budget_s and heads < wl.n_heads:
            q, k, v = (rng.standard_normal((n, 1, d)).astype(np.float32) for _ in range(3))
            heads += 1
            r0 = n_ar
            while r0 < n and dt < budget_s:
                r1 = min(n, r0 + 256)
                t0 = time.perf_counter()
                oattn.attention(q[r0:r1], k, v, r0, W.AR_CAUSAL_DM_FULL, n_ar=n_ar)
                dt += time.perf_counter() - t0
                flops += oattn.flops((r1 - r0) * n, 1, d)
                rows_done += r1 - r0
                r0 = r1
    # and one block of 256 DM rows of a fresh head on a single thread
    q, k, v = (rng.standard_normal((n, 1, d)).astype(np.float32) for _ in range(3))
    with threadpool_limits(limits=1):
        r1 = min(n, n_ar + 256)
        t1 = time.perf_counter()
        oattn.attention(q[n_ar:r1], k, v, n_ar, W.AR_CAUSAL_DM_FULL, n_ar=n_ar)
        dt1 = time.perf_counter() - t1
        one_core = oattn.flops((r1 - n_ar) * n, 1, d) / max(dt1, 1e-9) / 1e12
    rate = flops / max(dt, 1e-9) / 1e12
    full = 4.0 * d * wl.n_heads * attention_pairs(n, n_ar) / 1e12  # the workload's attention, TFLOP
    return {"value": rate, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "single_core_value": one_core,
            "projected_full_workload_s": round(full / max(rate, 1e-12), 1),
            "sample": "fp64 oracle attention over %d DM query rows x %d keys (%d of %d heads "
                      "started, one head at a time), %.1f s of oracle time on %s, %d BLAS threads; "
                      "single_core_value: one block of %d DM rows on 1 thread, %.2f s"
                      % (rows_done, n, heads, wl.n_heads, dt, _cpu_model(), cores, r1 - n_ar, dt1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="t2v480p_bf16")
    ap.add_argument("--mode", default="step", choices=["step", "guided", "block"],
                    help="step: one sampler step of the one-layer chain (the default line); guided: "
                         "a classifier-free-guided step (both predictions in one attention launch, "
                         "fused guided Euler); block: the whole MoT layer forward (LayerNorms, "
                         "projections, attention, GELU MLP, residuals; needs a workload with an MLP "
                         "width)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", type=int, default=1, choices=[1, 2],
                    help="streaming workload: split each call's keys in two halves over a batch of "
                         "two launches and merge them through their LSE")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the auxiliary long-480p attention figure of the default line")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (10 times), the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="only summarise rocprofv3 CSV output under DIR (no GPU use)")
    ap.add_argument("--write-profiles", metavar="DIR",
                    help="only write the profiles/ summaries from the rocprofv3 runs under DIR "
                         "(prof_bench, pmc_fetch, pmc_write, pmc_copy_fetch, pmc_copy_write, "
                         "pmc_sq; see the commands in the files written), no GPU use")
    args = ap.parse_args()
    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary))
        return
    if args.write_profiles:
        write_profiles(args.write_profiles, args.workload)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the multi-GPU path (head-sharded attention "
              "behind an all-to-all) is a design, not built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 10}), flush=True)
        return

    import workloads as W
    from multimodal_diffusion_transformer_amd import pipeline

    wl = W.BY_NAME[args.workload]
    if wl.mask == W.CHUNK_CAUSAL_KV:
        return bench_stream(args, wl)
    dev = torch.device("cuda:0")
    n, hid, h, d = wl.n_tokens, wl.hidden, wl.n_heads, wl.head_dim
    hk = wl.kv_heads
    n_ar, n_clean, n_noisy = W.region_counts(wl.segments)
    X = W.make(wl.wid, W.T_X, (n, hid), wl.dtype)
    sig = tuple(wl.sigmas[:2])  # the workload's first sampler step
    if args.mode == "block":
        if not wl.ffn:
            raise SystemExit("--mode block needs a workload with an MLP width (e.g. nano_t2v480p_bf16)")
        params = W.block_params(wl)
        tp = {k: (tuple(W.to_torch(t) for t in v) if k.startswith("ln") else W.to_torch(v))
              for k, v in params.items()}
        blk = pipeline.BlockStep(wl, W.to_torch(X), tp, device=dev)
        del X, params, tp
        stages = ["ln1", "qkv", "rope_k", "attention", "o_proj_residual", "ln2", "mlp_up_gelu",
                  "mlp_down_residual"]
        fns = [blk.ln1, blk.project_qkv, blk.rope_k, blk.attention, blk.project_o, blk.ln2,
               blk.mlp_up, blk.mlp_down]
    else:
        width = (h + 2 * hk) * d
        ws = [W.make(wl.wid, W.T_WQKV_AR, (hid, width), wl.dtype, 0.02),
              W.make(wl.wid, W.T_WQKV_DM, (hid, width), wl.dtype, 0.02),
              W.make(wl.wid, W.T_WO_AR, (h * d, hid), wl.dtype, 0.02),
              W.make(wl.wid, W.T_WO_DM, (h * d, hid), wl.dtype, 0.02)]
        x = W.make(wl.wid, W.T_LATENT, (n_noisy, hid), "fp32")
        if args.mode == "guided":
            Xb = W.make(wl.wid, W.T_X_BASE, (n_ar, hid), wl.dtype)
            Xt = W.to_torch(X)
            den = pipeline.GuidedDenoiserStep(wl, Xt[:n_ar], W.to_torch(Xb), Xt[n_ar:n_ar + n_clean],
                                              *(W.to_torch(w) for w in ws), torch.from_numpy(x.f32),
                                              wl.guidance or 6.0, device=dev)
            stages = ["qkv_dm", "rope_k_dm", "attention_pair", "o_proj_pair", "cfg_euler"]
            del Xb, Xt
        else:
            den = pipeline.DenoiserStep(wl, W.to_torch(X), *(W.to_torch(w) for w in ws),
                                        torch.from_numpy(x.f32), device=dev)
            stages = ["qkv", "rope_k", "attention", "o_proj", "euler"]
        del X, ws, x
        fns = [den.project_qkv, den.rope_k, den.attention, den.project_o,
               lambda: den.euler(*sig)]

    def step(ev=None):
        for i, f in enumerate(fns):
            if ev is not None:
                ev[i][0].record()
            f()
            if ev is not None:
                ev[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in stages] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {name: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1])
                                for s in range(args.steps)]))
           for i, name in enumerate(stages)}
    ms_step = wall * 1e3 / args.steps

    attn_stage = [k for k in stages if k.startswith("attention")][0]
    if args.mode == "guided":
        # DM queries only, two predictions, every key allowed
        pairs = 2 * (n - n_ar) * n
        rows_proj = n - n_ar
        proj_flops = 2.0 * rows_proj * hid * (h + 2 * hk) * d + 2.0 * 2 * rows_proj * h * d * hid
    else:
        pairs = attention_pairs(n, n_ar)
        proj_flops = 2.0 * n * hid * (h + 2 * hk) * d + 2.0 * n * h * d * hid
        if args.mode == "block":
            proj_flops += 2.0 * 2 * n * hid * wl.ffn
    attn_flops = 4.0 * d * h * pairs
    attn_tflops = attn_flops / (per[attn_stage] * 1e-3) / 1e12
    value = attn_flops / (ms_step * 1e-3) / 1e12
    line = {
        "metric": "MoT masked-attention TFLOP/s (unmasked pairs) + % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, random init)",
        "config": {"workload": "%s: T2V 480p-shaped packed sequence, %d AR (512 text + EOS + BOG)"
                               " + %d DM-noisy (16 latent frames x 30x52), %d heads x %d, hidden %d"
                               % (wl.name, n_ar, n_noisy, h, d, hid)
                               if wl.name == "t2v480p_bf16" and args.mode == "step" else wl.name,
                   "tokens": n, "n_ar": n_ar, "n_clean": n_clean, "n_noisy": n_noisy,
                   "heads": h, "kv_heads": hk, "head_dim": d, "hidden": hid, "mask": "AR_CAUSAL_DM_FULL",
                   "step": {"step": "qkv_proj + mrope(K; Q on load) + attention + o_proj + euler",
                            "guided": "DM rows: qkv_proj + mrope(K) + attention of both predictions "
                                      "in one launch + o_proj of both + guided euler (w=%g)"
                                      % (wl.guidance or 6.0),
                            "block": "ln1 + qkv_proj + mrope(K) + attention + o_proj(+residual) + "
                                     "ln2 + mlp_up(gelu) + mlp_down(+residual), FFN %d" % wl.ffn}[args.mode]},
        "pct_of_peak_step": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "attention_kernel_tflops": round(attn_tflops, 2),
        "step_tflops_all_contractions": round((attn_flops + proj_flops) / (ms_step * 1e-3) / 1e12, 2),
        "breakdown_ms": {k: round(v, 4) for k, v in per.items()},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(wl.name) if args.mode == "step" else None},
    }
    if args.mode == "step" and wl.name == "t2v480p_bf16" and not args.no_long:
        del den, fns
        torch.cuda.empty_cache()
        try:
            line["t2v480p_long_attention"] = long_480p_attention(dev)
        except Exception as e:  # an auxiliary figure: report, do not lose the line
            line["t2v480p_long_attention"] = {"error": repr(e)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(line), flush=True)


def long_480p_attention(dev, reps=3):
    """The attention launch of the long 480p workload (76,954 tokens: 514
    AR, 1,560 clean, 74,880 noisy; 24 heads of 128), as the step runs it: Q,
    K, V strided views of one packed [N, 3, H, D] buffer, Q rotated on load.
    Inputs are random bf16 already on the device; HIP events on the launch
    stream time `reps` launches after one warm-up."""
    import numpy as np
    import torch

    import workloads as W
    from multimodal_diffusion_transformer_amd import _binding as B

    wl = W.BY_NAME["t2v480p_long_bf16"]
    pos, reg, n_ar = B.mot_build_layout(wl.segments)
    n, h, d = pos.shape[0], wl.n_heads, wl.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(wl.wid)
    Y = torch.randn((n, 3, h, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    O = torch.empty((n, h, d), dtype=torch.bfloat16, device=dev)
    P = torch.from_numpy(pos).to(dev)
    a = B.attn_args(Y[:, 0], Y[:, 1], Y[:, 2], O, mask=B.MOT_AR_CAUSAL_DM_FULL, n_ar=n_ar, q_pos=P,
                    sections=wl.sections, theta=wl.theta)
    B.mot_attention_fwd_args(a)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        B.mot_attention_fwd_args(a)
        e1.record()
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    flops = 4.0 * d * h * attention_pairs(n, n_ar)
    med = float(np.median(ms))
    tf = flops / (med * 1e-3) / 1e12
    del Y, O
    torch.cuda.empty_cache()
    return {"tokens": n, "tflop_per_launch": round(flops / 1e12, 3), "ms_median": round(med, 3),
            "ms_min": round(float(np.min(ms)), 3), "tflops": round(tf, 2),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def rocprof_summary(d):
    """Per-kernel summary of rocprofv3 CSV output: the --stats table, and the
    per-dispatch mean of every collected counter (each counter's values are
    summed over its dimension instances within a dispatch first)."""
    import csv
    import glob
    from collections import defaultdict

    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        out.append("kernel stats (%s):" % os.path.relpath(f, d))
        out.append("  %-48s %6s %14s %12s %7s" % ("kernel", "calls", "total_ns", "avg_ns", "pct"))
        with open(f) as fh:
            for row in csv.DictReader(fh):
                out.append("  %-48s %6s %14s %12.0f %7.2f" % (
                    row["Name"][:48], row["Calls"], row["TotalDurationNs"],
                    float(row["AverageNs"]), float(row["Percentage"])))
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        per = defaultdict(lambda: defaultdict(float))  # (kernel, counter) -> dispatch -> value
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row["Kernel_Name"].split("(")[0][-48:]
                per[(name, row["Counter_Name"])][row["Dispatch_Id"]] += float(row["Counter_Value"])
        out.append("counters (%s), mean per dispatch:" % os.path.relpath(f, d))
        for (name, cname), disp in sorted(per.items()):
            vals = list(disp.values())
            out.append("  %-48s %-14s dispatches %4d  mean %.6g" % (name, cname, len(vals),
                                                                  sum(vals) / len(vals)))
    return "\n".join(out)


def bench_stream(args, wl):
    """Streaming rollout: per chunk, `stream_steps` denoising steps of
    chunk-causal attention against the rolling cache (the chunk's keys are
    rotated into the cache tail, Q is rotated on load), then the chunk moves
    into its ring slot.  One timed step = one whole rollout of
    `stream_chunks` chunks; inputs are synthetic and already on the device."""
    import numpy as np
    import torch

    import workloads as W
    from multimodal_diffusion_transformer_amd import pipeline

    dev = torch.device("cuda:0")
    h, d = wl.n_heads, wl.head_dim
    ft = wl.stream_views * wl.stream_gh * wl.stream_gw
    slots = wl.stream_history_frames
    n_prefix = wl.stream_text + 2
    pos, _, n_ar = W_layout(wl)
    nhist = n_prefix + slots * ft
    g = torch.Generator(device=dev)
    g.manual_seed(wl.wid)

    def randn(*shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    st = pipeline.StreamState(h, d, n_prefix, ft, slots, wl.sections, wl.theta, device=dev, split=args.split)
    st.fill(randn(nhist, h, d), randn(nhist, h, d), torch.from_numpy(pos[:nhist]).to(dev))
    n_calls = wl.stream_chunks * wl.stream_steps
    qs = [randn(ft, h, d) for _ in range(n_calls)]
    ks = [randn(ft, h, d) for _ in range(n_calls)]
    vs = [randn(ft, h, d) for _ in range(n_calls)]
    t0 = n_ar + 15000.0
    cps = []
    for c in range(wl.stream_chunks):
        cp = pos[nhist:nhist + ft].copy()
        cp[:, 0] = np.float32(t0 + slots + c)
        cps.append(torch.from_numpy(cp).to(dev))
    O = torch.empty((ft, h, d), dtype=torch.bfloat16, device=dev)

    def rollout(ev=None):
        i = 0
        for c in range(wl.stream_chunks):
            for s in range(wl.stream_steps):
                if ev is not None:
                    ev[i][0].record()
                st.attend(qs[i], ks[i], vs[i], cps[c], O)
                if ev is not None:
                    ev[i][1].record()
                i += 1
            st.append(c)

    for _ in range(args.warmup):
        rollout()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(n_calls)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        rollout(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_call = [evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps) for i in range(n_calls)]
    pairs = ft * (nhist + ft)  # the chunk is the newest: every row sees the whole cache
    call_flops = 4.0 * d * h * pairs
    ms_step = wall * 1e3 / args.steps
    value = call_flops * n_calls / (ms_step * 1e-3) / 1e12
    med = float(np.median(per_call))
    line = {
        "metric": "MoT masked-attention TFLOP/s (unmasked pairs) + % of MI355X bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) queries, keys and values)",
        "config": {"workload": "%s: chunk-causal streaming, %d-token chunks (one latent frame, %d views "
                               "x %dx%d) against a %d-key cache (%d prefix + %d history frames), "
                               "%d chunks x %d steps per rollout"
                               % (wl.name, ft, wl.stream_views, wl.stream_gh, wl.stream_gw, nhist + ft,
                                  n_prefix, slots, wl.stream_chunks, wl.stream_steps),
                   "heads": h, "head_dim": d, "mask": "CHUNK_CAUSAL_KV",
                   "step": "per call: K/V chunk into the cache + mRoPE(K chunk) + attention (Q on load)"
                           + (" over two key halves in one launch + merge" if args.split == 2 else "")},
        "attention_call_ms": {"median": round(med, 4), "min": round(float(np.min(per_call)), 4)},
        "attention_call_tflops_median": round(call_flops / (med * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "kernel": ATTN_KERNEL,
                     "achieved": round(call_flops / (med * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(call_flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(line), flush=True)


def W_layout(wl):
    from multimodal_diffusion_transformer_amd import _binding as B
    return B.mot_build_layout(wl.segments)


def _counter_mean(d, kernel, counter):
    """Mean over dispatches of `kernel` of one counter (summed over its
    instances within a dispatch), from rocprofv3 CSV output under d."""
    import csv
    import glob
    from collections import defaultdict

    per = defaultdict(float)
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if kernel in row["Kernel_Name"] and row["Counter_Name"] == counter:
                    per[row["Dispatch_Id"]] += float(row["Counter_Value"])
    if not per:
        raise SystemExit("no %s samples of %s under %s" % (counter, kernel, d))
    return sum(per.values()) / len(per), len(per)


def attention_work_text(workload):
    """The algorithmic work of one attention launch of `workload`, as text:
    the allowed (query, key) pairs x heads x 4 D flop (the streaming chunk
    is the newest, so each of its rows sees every cached key)."""
    import workloads as W
    wl = W.BY_NAME[workload]
    n, h, d = wl.n_tokens, wl.n_heads, wl.head_dim
    if wl.mask == W.CHUNK_CAUSAL_KV:
        ft = wl.stream_views * wl.stream_gh * wl.stream_gw
        pairs = ft * n
    else:
        pairs = attention_pairs(n, W.region_counts(wl.segments)[0])
    return "%.3f TFLOP per launch (%s allowed pairs x %d heads x %d flop)" % (
        4.0 * d * h * pairs / 1e12, format(pairs, ","), h, 4 * d)


def write_profiles(d, workload):
    """Write profiles/<kernel>_<workload>_{kernel_stats,hbm_traffic,sq_counters}.txt
    from the rocprofv3 CSV runs under d (the commands are recorded in each)."""
    pre = os.path.join(ROOT, "profiles", "%s_%s" % (ATTN_KERNEL, workload))
    cmd_head = ("commands (run on an MI355X from the repository root; <repo> is its absolute path,\n"
                "<out> the output folder):\n  cd /tmp && export TMPDIR=/tmp\n")
    bench = "python3 <repo>/bench.py --workload %s" % workload
    h = attention_kernel_hash()
    flops = attention_work_text(workload)
    # 1. kernel durations
    txt = ("Kernel durations of one benchmark run of %s; one step = QKV projection, mRoPE of K,\n"
           "attention (Q rotated on load), O projection, Euler update.\n\n" % workload + cmd_head +
           "  rocprofv3 --kernel-trace --stats --output-format csv -d <out>/prof_bench -o bench -- "
           "%s --steps 5 --warmup 2 --no-cpu-baseline\n" % bench +
           "  python3 bench.py --write-profiles <out>\n\n"
           "attention_kernel_hash: %s\nattention: %s\n\n" % (h, flops) +
           rocprof_summary(os.path.join(d, "prof_bench")) + "\n")
    with open(pre + "_kernel_stats.txt", "w") as f:
        f.write(txt)
    # 2. HBM traffic, scaled by a copy of known size
    kib = 1024 * 1024
    cf, _ = _counter_mean(os.path.join(d, "pmc_copy_fetch"), "copyBuffer", "FETCH_SIZE")
    cw, _ = _counter_mean(os.path.join(d, "pmc_copy_write"), "copyBuffer", "WRITE_SIZE")
    ff, fw = kib / cf, kib / cw
    af, na = _counter_mean(os.path.join(d, "pmc_fetch"), ATTN_KERNEL, "FETCH_SIZE")
    aw, _ = _counter_mean(os.path.join(d, "pmc_write"), ATTN_KERNEL, "WRITE_SIZE")
    fb, wb = af * ff * 1024, aw * fw * 1024
    txt = ("%s on %s: HBM traffic per launch from rocprofv3 counters, each scaled by what the same\n"
           "counter reads for a device copy of known size.\n\n" % (ATTN_KERNEL, workload) + cmd_head +
           "".join("  rocprofv3 --pmc %s --output-format csv -d <out>/%s -o %s -- %s\n" % (c, o, n, a)
                   for c, o, n, a in [
                       ("FETCH_SIZE", "pmc_fetch", "bench", bench + " --steps 2 --warmup 1 --no-cpu-baseline"),
                       ("WRITE_SIZE", "pmc_write", "bench", bench + " --steps 2 --warmup 1 --no-cpu-baseline"),
                       ("FETCH_SIZE", "pmc_copy_fetch", "copy", bench + " --copy-calibration 1024"),
                       ("WRITE_SIZE", "pmc_copy_write", "copy", bench + " --copy-calibration 1024")]) +
           "  python3 bench.py --write-profiles <out>\n\n"
           "calibration: a 1 GiB device copy (__amd_rocclr_copyBuffer, 1,048,576 KiB read and written)\n"
           "  FETCH_SIZE reads %.1f KiB per dispatch -> fetch factor %.5f\n"
           "  WRITE_SIZE reads %.1f KiB per dispatch -> write factor %.5f\n\n" % (cf, ff, cw, fw) +
           "attention, mean per dispatch (%d dispatches each):\n" % na +
           "  FETCH_SIZE %.1f KiB x %.5f = %.4f GB\n  WRITE_SIZE %.1f KiB x %.5f = %.4f GB\n"
           % (af, ff, fb / 1e9, aw, fw, wb / 1e9) +
           "  algorithmic bytes: Q + K + V read once, O written once = 4 x N x H x D x 2 B\n\n"
           "attention_kernel_hash: %s\nfetch_bytes_per_launch: %.0f\nwrite_bytes_per_launch: %.0f\n"
           "traffic_bytes_per_launch: %.0f\n\nraw summaries:\n" % (h, fb, wb, fb + wb) +
           "\n".join(rocprof_summary(os.path.join(d, x))
                     for x in ("pmc_fetch", "pmc_write", "pmc_copy_fetch", "pmc_copy_write")) + "\n")
    with open(pre + "_hbm_traffic.txt", "w") as f:
        f.write(txt)
    # 3. shader counters of the attention kernel
    sq = os.path.join(d, "pmc_sq")
    if os.path.isdir(sq):
        names = ["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU",
                 "SQ_LDS_BANK_CONFLICT"]
        vals = {n: _counter_mean(sq, ATTN_KERNEL, n)[0] for n in names}
        txt = ("%s on %s: shader counters, mean per dispatch.\n\n" % (ATTN_KERNEL, workload) + cmd_head +
               "  rocprofv3 --pmc %s --output-format csv -d <out>/pmc_sq -o bench -- %s --steps 2 --warmup 1"
               " --no-cpu-baseline\n  python3 bench.py --write-profiles <out>\n\n" % (" ".join(names), bench) +
               "attention_kernel_hash: %s\n\n" % h +
               "".join("  %-26s %.6g\n" % (n, vals[n]) for n in names) +
               "\nderived:\n"
               "  MFMA busy cycles per MFMA instruction: %.2f (a 32x32x16 bf16 MFMA occupies the unit 32 cycles)\n"
               "  non-MFMA VALU instructions per MFMA: %.2f\n"
               "  LDS instructions per MFMA: %.2f\n" % (
                   vals["SQ_VALU_MFMA_BUSY_CYCLES"] / vals["SQ_INSTS_MFMA"],
                   (vals["SQ_INSTS_VALU"] - vals["SQ_INSTS_MFMA"]) / vals["SQ_INSTS_MFMA"],
                   vals["SQ_INSTS_LDS"] / vals["SQ_INSTS_MFMA"]))
        with open(pre + "_sq_counters.txt", "w") as f:
            f.write(txt)


if __name__ == "__main__":
    main()
