#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one spec_verify_attn call (paged GQA attention of the K+1 verify
rows over the whole KV cache of one layer) followed by one spec_verify_sample
call (the rejection sampler over the K+1 target rows), on seeded synthetic
inputs already resident in HBM.  Several copies of the inputs are rotated so
that every step reads cold data (the 256 MiB Infinity Cache cannot hold them).

Two timed passes of --steps steps each: an eager pass with HIP events
around every call on the launch stream (per-kernel times, from which the
roofline figure of the main attention kernel comes), then a pass that
replays each step from a captured HIP graph (one graph per input copy; the
headline steps/s, since a serving loop would replay the step the same way).

Prints one JSON line.  Default workload: the LLaMA-3-8B-style layer (B=8,
Hq=32, Hkv=8, d=128, context 4096, 16-token pages, K=5, bf16 KV, V=128256).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
ATTN_SRC = os.path.join(ROOT, "speculative_decoding_verify_attn_amd", "csrc", "attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "verify steps/sec and achieved HBM GB/s (% of MI355X peak) per config"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="rotating input copies (0: enough to defeat the MALL)")
    ap.add_argument("--algo", type=int, default=0, help="0 auto, 1 vector ALU, 2 matrix cores")
    ap.add_argument("--bps", type=int, default=0, help="context pages per split (0: planner)")
    ap.add_argument("--no-graph", action="store_true", help="headline from the eager pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tree", action="store_true", help="skip the tree-verification measurement")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the oracle sample")
    ap.add_argument("--probe", choices=["none", "copy"], default="none",
                    help="copy: run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


class HipEvents:
    """Raw HIP events (the runtime library via ctypes), so that an event can
    also be recorded by libspecverify between its kernels."""

    def __init__(self):
        import ctypes
        self.c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self):
        ev = self.c.c_void_p()
        if self.hip.hipEventCreate(self.c.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(ev)
        return ev

    def record(self, ev, stream_handle):
        if self.hip.hipEventRecord(ev, self.c.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        f = self.c.c_float()
        if self.hip.hipEventElapsedTime(self.c.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(f.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def attn_source_hash():
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def probe_copy():
    import torch
    n = 1 << 28  # 256 MiB per direction
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr, flush=True)
        sys.exit(2)
    if args.probe == "copy":
        probe_copy()
        return

    import torch
    import speculative_decoding_verify_attn_amd as sv
    import workloads as W

    cfg = W.CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    t_gen = time.time()
    a = W.make_attn(args.config, seed=args.seed)
    s = W.make_sample(args.config, seed=args.seed)
    print("# generated %s in %.1f s" % (args.config, time.time() - t_gen), file=sys.stderr, flush=True)

    attn_bytes = W.attn_algorithmic_bytes(a)
    step_in_bytes = a.k_cache.nbytes + a.v_cache.nbytes + s.target_logits.nbytes + s.draft_probs.nbytes
    copies = args.copies or max(2, int(np.ceil(3 * MALL_BYTES / step_in_bytes)) + 1)
    copies = min(copies, 16)

    def up(x, view=None):
        t = torch.from_numpy(x).to(dev)
        return t.view(view) if view is not None else t

    sets = []
    for _ in range(copies):
        st = {"q": up(a.q), "table": up(a.block_table), "lens": up(a.context_lens)}
        if a.kv_dtype == W.KV_BF16:
            st["k"] = up(a.k_cache.view(np.int16), torch.bfloat16)
            st["v"] = up(a.v_cache.view(np.int16), torch.bfloat16)
        else:
            st["k"] = up(a.k_cache)
            st["v"] = up(a.v_cache)
        if a.kv_dtype == W.KV_FP8_E4M3:
            st["ks"] = up(a.k_scale)
            st["vs"] = up(a.v_scale)
        st["logits"] = up(s.target_logits)
        st["probs"] = up(s.draft_probs)
        st["tokens"] = up(s.draft_tokens)
        st["u"] = up(s.uniforms)
        sets.append(st)
    out = torch.empty((a.B, a.T, a.Hq, a.d), dtype=torch.float32, device=dev)
    ws_a = sv.alloc_workspace(sv.attn_workspace_size(a.B, a.T, a.Hq, a.Hkv, a.d, a.max_blocks, args.bps), dev)
    ws_s = sv.alloc_workspace(sv.sample_workspace_size(s.B, s.K, s.V), dev)
    n_acc = torch.empty(s.B, dtype=torch.int32, device=dev)
    toks = torch.empty((s.B, s.K + 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    hev = HipEvents()

    def step(st, ev=None):
        if ev is not None:
            hev.record(ev[0], sh)
        sv.spec_verify_attn(st["q"], st["k"], st["v"], st["table"], st["lens"], out, ws_a,
                            k_scale=st.get("ks"), v_scale=st.get("vs"), kv_dtype=a.kv_dtype,
                            stream=stream, algo=args.algo, blocks_per_split=args.bps,
                            main_done_event=None if ev is None else ev[1])
        if ev is not None:
            hev.record(ev[2], sh)
        sv.spec_verify_sample(st["logits"], st["probs"], st["tokens"], st["u"], n_acc, toks, ws_s, stream=stream)
        if ev is not None:
            hev.record(ev[3], sh)

    def step_on(st, strm):
        sv.spec_verify_attn(st["q"], st["k"], st["v"], st["table"], st["lens"], out, ws_a,
                            k_scale=st.get("ks"), v_scale=st.get("vs"), kv_dtype=a.kv_dtype,
                            stream=strm, algo=args.algo, blocks_per_split=args.bps)
        sv.spec_verify_sample(st["logits"], st["probs"], st["tokens"], st["u"], n_acc, toks, ws_s, stream=strm)

    for i in range(args.warmup):
        step(sets[i % copies])
    torch.cuda.synchronize()
    print("# warmup done (%d copies of %.1f MB)" % (copies, step_in_bytes / 1e6), file=sys.stderr, flush=True)

    # A spin kernel holds the stream while the host enqueues the timed steps,
    # so the GPU then runs them back to back and the events bracket GPU work,
    # not host launch latency.
    c0, c1 = hev.create(), hev.create()
    hev.record(c0, sh)
    torch.cuda._sleep(1 << 20)
    hev.record(c1, sh)
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(hev.ms(c0, c1), 1e-3)

    def gate(n_steps):
        torch.cuda._sleep(int(cycles_per_ms * (2.0 + 0.25 * n_steps)))

    evs = [[hev.create() for _ in range(4)] for _ in range(args.steps)]
    t0, t1 = hev.create(), hev.create()
    torch.cuda.synchronize()
    gate(args.steps)
    hev.record(t0, sh)
    for i in range(args.steps):
        step(sets[i % copies], evs[i])
    hev.record(t1, sh)
    torch.cuda.synchronize()
    eager_ms_step = hev.ms(t0, t1) / args.steps
    main_ev_ms = np.array([hev.ms(e[0], e[1]) for e in evs])  # main attention kernel, per-step events
    attn_ms = np.array([hev.ms(e[0], e[2]) for e in evs])   # attention call (main + split merge)
    samp_ms = np.array([hev.ms(e[2], e[3]) for e in evs])   # sampler call
    print("# eager pass: %.1f us/step" % (eager_ms_step * 1e3), file=sys.stderr, flush=True)

    # The main attention kernel alone: --steps back-to-back launches between
    # two events on the launch stream (no event between launches, so the
    # average is the kernel's own duration, as a kernel trace reports it).
    k0, k1 = hev.create(), hev.create()
    torch.cuda.synchronize()
    gate(args.steps)
    hev.record(k0, sh)
    for i in range(args.steps):
        st = sets[i % copies]
        sv.spec_verify_attn(st["q"], st["k"], st["v"], st["table"], st["lens"], out, ws_a,
                            k_scale=st.get("ks"), v_scale=st.get("vs"), kv_dtype=a.kv_dtype,
                            stream=stream, algo=args.algo | sv.SV_ATTN_MAIN_ONLY, blocks_per_split=args.bps)
    hev.record(k1, sh)
    torch.cuda.synchronize()
    main_ms = hev.ms(k0, k1) / args.steps
    print("# main attention kernel: %.1f us per launch" % (main_ms * 1e3), file=sys.stderr, flush=True)

    graph_ms_step = None
    if not args.no_graph:
        graphs = []
        side = torch.cuda.Stream(dev)  # default priority
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for st in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step_on(st, side)
                graphs.append(g)
        stream.wait_stream(side)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        g0, g1 = hev.create(), hev.create()
        gate(args.steps)
        hev.record(g0, sh)
        for i in range(args.steps):
            graphs[i % copies].replay()
        hev.record(g1, sh)
        torch.cuda.synchronize()
        graph_ms_step = hev.ms(g0, g1) / args.steps
        # the last replayed copy must reproduce the eager result of that copy
        last = (args.steps - 1) % copies
        step(sets[last])
        torch.cuda.synchronize()
        ref = (n_acc.clone(), toks.clone())
        graphs[last].replay()
        torch.cuda.synchronize()
        if not (torch.equal(ref[0], n_acc) and torch.equal(ref[1], toks)):
            raise RuntimeError("graph replay disagrees with the eager step")
        del graphs
        print("# graph pass: %.1f us/step" % (graph_ms_step * 1e3), file=sys.stderr, flush=True)
    ms_step = graph_ms_step if graph_ms_step is not None else eager_ms_step

    # The paged-cache steps on either side of the verify step (reported beside
    # it): appending the T verify positions of one layer, and the rollback.
    def timed_launches(fn, n):
        e0, e1 = hev.create(), hev.create()
        torch.cuda.synchronize()
        gate(n)
        hev.record(e0, sh)
        for i in range(n):
            fn(i)
        hev.record(e1, sh)
        torch.cuda.synchronize()
        return hev.ms(e0, e1) / n

    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    k_new = torch.randn((a.B, a.T, a.Hkv, a.d), generator=gen, device=dev)
    v_new = torch.randn((a.B, a.T, a.Hkv, a.d), generator=gen, device=dev)
    if a.kv_dtype == W.KV_FP8_E4M3:
        k_new *= 4.0
        v_new *= 4.0
    st0 = sets[0]
    append_ms = timed_launches(lambda i: sv.spec_verify_kv_append(
        k_new, v_new, st0["k"], st0["v"], st0["table"], st0["lens"], k_scale=st0.get("ks"), v_scale=st0.get("vs"),
        kv_dtype=a.kv_dtype, stream=stream), args.steps)
    lens_scratch = st0["lens"].clone()
    pages_scratch = torch.empty_like(lens_scratch)
    rollback_ms = timed_launches(lambda i: sv.spec_verify_rollback(n_acc, lens_scratch, s.K, pages_in_use=pages_scratch,
                                                                   stream=stream), args.steps)
    n_plain = n_acc.clone()  # accepted counts of the plain sampler (for its algorithmic bytes)
    # The sampler alone, back to back: plain, and with a target temperature
    # and top-p cut per sequence (0.7 and 0.9, the draft rows as given).
    samp_b2b_ms = timed_launches(lambda i: sv.spec_verify_sample(
        sets[i % copies]["logits"], sets[i % copies]["probs"], sets[i % copies]["tokens"], sets[i % copies]["u"],
        n_acc, toks, ws_s, stream=stream), args.steps)
    temp_t = torch.full((s.B,), 0.7, dtype=torch.float32, device=dev)
    cut_t = torch.full((s.B,), 0.9, dtype=torch.float32, device=dev)
    samp_tp_ms = timed_launches(lambda i: sv.spec_verify_sample(
        sets[i % copies]["logits"], sets[i % copies]["probs"], sets[i % copies]["tokens"], sets[i % copies]["u"],
        n_acc, toks, ws_s, stream=stream, temperature=temp_t, top_p=cut_t), args.steps)
    samp_ty_ms = timed_launches(lambda i: sv.spec_verify_sample_typical(
        sets[i % copies]["logits"], sets[i % copies]["tokens"], sets[i % copies]["u"], n_acc, toks, ws_s,
        0.09, 0.3, stream=stream), args.steps)
    print("# sampler %.1f us, with temperature + top-p %.1f us, typical acceptance %.1f us" % (
        samp_b2b_ms * 1e3, samp_tp_ms * 1e3, samp_ty_ms * 1e3), file=sys.stderr, flush=True)
    # Tree verification at the same geometry: the widest tree shape whose
    # nodes fit the row tiles (N * Hq/Hkv <= 64), attention over the same
    # cache with N verify rows, and the tree sampler over N target rows.
    tree = None
    if not args.no_tree:
        G = a.Hq // a.Hkv
        shapes = sorted(W.TREE_SHAPES.items(), key=lambda kv: -len(W.tree_parents(kv[1])))
        fit = [(nm, sh) for nm, sh in shapes if len(W.tree_parents(sh)) * G <= 64]
        if fit:
            tname, tshape = fit[0]
            par = W.tree_parents(tshape)
            N = par.shape[0]
            masks = np.zeros((a.B, N), np.uint32)
            for c in range(N):
                m, u = 0, c
                while u >= 0:
                    m |= 1 << u
                    u = par[u]
                masks[:, c] = m
            gq = torch.Generator(device=dev)
            gq.manual_seed(args.seed + 1)
            q_tree = torch.randn((a.B, N, a.Hq, a.d), generator=gq, device=dev)
            tm = torch.from_numpy(masks.view(np.int32)).to(dev)
            out_tree = torch.empty((a.B, N, a.Hq, a.d), dtype=torch.float32, device=dev)
            ws_ta = sv.alloc_workspace(sv.attn_workspace_size(a.B, N, a.Hq, a.Hkv, a.d, a.max_blocks, 0), dev)
            tree_attn_ms = timed_launches(lambda i: sv.spec_verify_attn_tree(
                q_tree, sets[i % copies]["k"], sets[i % copies]["v"], sets[i % copies]["table"],
                sets[i % copies]["lens"], tm, out_tree, ws_ta, k_scale=sets[i % copies].get("ks"),
                v_scale=sets[i % copies].get("vs"), kv_dtype=a.kv_dtype, stream=stream), args.steps)
            t_gen = time.time()
            ti = W.make_tree(args.seed, s.B, par, s.V, cfg["target_sigma"],
                             cfg["noise"] if not isinstance(cfg["noise"], tuple) else 1.0)
            tl = up(ti.target_logits)
            tsets = [{"logits": tl if j == 0 else tl.clone(), "probs": up(ti.draft_probs) if j == 0 else None}
                     for j in range(max(2, int(np.ceil(3 * MALL_BYTES / (2 * tl.numel() * 4))) + 1))]
            for j in range(1, len(tsets)):
                tsets[j]["probs"] = tsets[0]["probs"].clone()
            ttok, tpar, tu = up(ti.tokens), up(ti.parents), up(ti.uniforms)
            tn = torch.empty(s.B, dtype=torch.int32, device=dev)
            tot = torch.empty((s.B, N), dtype=torch.int32, device=dev)
            tpath = torch.empty((s.B, N), dtype=torch.int32, device=dev)
            ws_ts = sv.alloc_workspace(sv.sample_tree_workspace_size(s.B, N, s.V), dev)
            tree_samp_ms = timed_launches(lambda i: sv.spec_verify_sample_tree(
                tsets[i % len(tsets)]["logits"], tsets[i % len(tsets)]["probs"], ttok, tpar, tu, tn, tot, tpath,
                ws_ts, max(tshape), stream=stream), args.steps)
            # committing the accepted paths (moves K/V within the cache of copy 0;
            # the lengths shrink from call to call and are clamped at N, which
            # only moves the work to other pages)
            path_np = tpath.cpu().numpy()
            tn_np = tn.cpu().numpy()
            cpath = torch.from_numpy(np.ascontiguousarray(path_np[:a.B] if path_np.shape[0] >= a.B else
                                                          np.resize(path_np, (a.B, N)))).to(dev)
            cn = torch.from_numpy(np.ascontiguousarray(np.resize(tn_np, a.B).astype(np.int32))).to(dev)
            clens = sets[0]["lens"].clone()
            tree_commit_ms = timed_launches(lambda i: sv.spec_verify_tree_commit(
                cpath, cn, sets[0]["k"], sets[0]["v"], sets[0]["table"], clens,
                k_scale=sets[0].get("ks"), v_scale=sets[0].get("vs"), kv_dtype=a.kv_dtype, stream=stream), args.steps)
            tree_bytes = attn_bytes + 2 * a.B * (N - a.T) * a.Hq * a.d * 4
            tree = {"shape": tname, "nodes": N, "attn_us": tree_attn_ms * 1e3,
                    "attn_gbs": tree_bytes / (tree_attn_ms * 1e-3) / 1e9, "sample_us": tree_samp_ms * 1e3,
                    "commit_us": tree_commit_ms * 1e3,
                    "mean_accepted": float(tn.float().mean().item())}
            print("# tree %s (N=%d): attention %.1f us, sampler %.1f us, commit %.1f us (inputs %.1f s)" % (
                tname, N, tree_attn_ms * 1e3, tree_samp_ms * 1e3, tree_commit_ms * 1e3, time.time() - t_gen),
                file=sys.stderr, flush=True)
            del tsets, tl
    ap_bytes = 2 * k_new.numel() * (4 + {W.KV_F32: 4, W.KV_BF16: 2, W.KV_FP8_E4M3: 1}[a.kv_dtype]) + 4 * a.B * (a.T + 1)
    print("# append %.1f us, rollback %.1f us" % (append_ms * 1e3, rollback_ms * 1e3), file=sys.stderr, flush=True)
    hev.close()
    n_rej = int((n_plain.cpu().numpy() < s.K).sum())
    samp_bytes = W.sample_algorithmic_bytes(s, n_rej)

    attn_gbs = attn_bytes / (main_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get(args.config)
        if ent and ent.get("attn_src_sha") == attn_source_hash() and args.algo == 0 and args.bps == 0:
            traffic = ent.get("bytes_per_launch")

    res = {
        "metric": METRIC,
        "value": 1000.0 / ms_step,
        "unit": "verify steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "timing": "HIP graph replay per step" if graph_ms_step is not None else "eager launches",
        "eager_ms_per_step": eager_ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {W.KV_F32: "f32", W.KV_BF16: "bf16", W.KV_FP8_E4M3: "fp8e4m3"}[a.kv_dtype],
        "data": "synthetic",
        "config": {
            "workload": "%s: %s (B=%d, Hq=%d, Hkv=%d, d=%d, ctx=%s, page 16, K=%d, %s KV, V=%d)" % (
                args.config, cfg["desc"], a.B, a.Hq, a.Hkv, a.d, cfg["ctx"], s.K, cfg["kv"], s.V),
            "B": a.B, "K": s.K, "V": s.V, "context": int(a.context_lens.max()),
            "rotating_copies": copies,
        },
        "attn_main_kernel_us": float(main_ms * 1e3),
        "attn_main_kernel_us_step_events": float(main_ev_ms.mean() * 1e3),
        "attn_us": float(attn_ms.mean() * 1e3),
        "attn_us_p10_p90": [float(np.percentile(attn_ms, 10) * 1e3), float(np.percentile(attn_ms, 90) * 1e3)],
        "sample_us": float(samp_ms.mean() * 1e3),
        "sample_us_back_to_back": float(samp_b2b_ms * 1e3),
        "sample_temp_topp_us_back_to_back": float(samp_tp_ms * 1e3),
        "sample_typical_us_back_to_back": float(samp_ty_ms * 1e3),
        "kv_append_us_per_layer": float(append_ms * 1e3),
        "kv_append_bytes_per_layer": int(ap_bytes),
        "rollback_us": float(rollback_ms * 1e3),
        "tree_verify": tree,
        "attn_bytes": attn_bytes,
        "sample_bytes": samp_bytes,
        "step_gbs": (attn_bytes + samp_bytes) / (ms_step * 1e-3) / 1e9,
        "roofline": {
            "kernel": "sv_attn_mfma_kernel (main attention kernel; algorithmic bytes: KV of every visible "
                      "position once, Q in, out, used block-table entries)",
            "bound": "hbm",
            "achieved": attn_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": attn_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": attn_bytes,
        },
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(a, s, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_baseline(a, s, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same step:
    a subset of attention output rows and a subset of sequences through the
    sampler, each timed and scaled to a whole step."""
    import oracle
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)
    total_rows = a.B * a.T * a.Hq
    # calibrate on a few rows, then take as many as fit the budget
    probe = rng.choice(total_rows, size=min(total_rows, 2 * threads), replace=False).astype(np.int64)
    t = time.time()
    oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                k_scale=a.k_scale, v_scale=a.v_scale, rows=probe, nthreads=threads)
    per_row = max(1e-6, (time.time() - t) / len(probe))
    n_rows = int(min(total_rows, max(len(probe), 0.7 * budget_s / per_row)))
    rows = rng.choice(total_rows, size=n_rows, replace=False).astype(np.int64)
    t = time.time()
    oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                k_scale=a.k_scale, v_scale=a.v_scale, rows=rows, nthreads=threads)
    t_attn = (time.time() - t) * total_rows / n_rows
    n_seq = max(1, min(s.B, threads))
    t = time.time()
    oracle.sample(s.target_logits[:n_seq], s.draft_probs[:n_seq], s.draft_tokens[:n_seq], s.uniforms[:n_seq],
                  nthreads=threads)
    t_samp = (time.time() - t) * s.B / n_seq
    return {
        "value": 1.0 / (t_attn + t_samp),
        "unit": "verify steps/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d of %d attention rows and %d of %d sampler sequences, scaled to one step "
                  "(attention %.3f s, sampler %.3f s per step)" % (n_rows, total_rows, n_seq, s.B, t_attn, t_samp),
    }


if __name__ == "__main__":
    main()
