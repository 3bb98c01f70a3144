#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one spec_verify_attn call (paged GQA attention of the K+1 verify
rows over the whole KV cache of one layer) followed by one spec_verify_sample
call (the rejection sampler over the K+1 target rows), on seeded synthetic
inputs already resident in HBM.  Several copies of the inputs are rotated so
that every step reads cold data (the 256 MiB Infinity Cache cannot hold them).

With no --config every configuration is measured in one process (c1 tiny
fp32, c2 LLaMA-3-8B-style layer, c3 70B-style layer, c4 ragged batch, c5a/c5b
131k-token context with bf16 / E4M3 KV) and one JSON line is printed: the
headline is c4, the largest single-GPU configuration, and "per_config" holds
every configuration's figures.  --config <name> measures one configuration
and makes it the headline.

Per configuration:
  * eager pass: HIP events around every call on the launch stream;
  * main attention kernel alone: back-to-back launches between two events
    (spec_verify_attn_timing_main_only) -- the roofline figure;
  * HIP-graph pass: each step replayed from a captured graph (one graph per
    input copy) -- the headline steps/s;
  * the practical read ceiling: a plain streaming read of the same number of
    bytes as the attention must move (spec_verify_probe_read);
  * parity: the timed path's outputs of one input copy against the CPU
    oracle -- attention rows covering every (sequence, KV head) unit, the
    sampler's accepted counts and tokens of every sequence (bit-exact except
    at positions the oracle decided within 1e-6 of a threshold, which are
    counted);
  * the rows around the step (append, rollback, the sampler with temperature
    + top-p and with typical acceptance) and, for the configurations named by
    --tree-configs, tree verification;
  * cpu_baseline: the oracle on a bounded sample of the same step.
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
SAMPLE_SRC = os.path.join(ROOT, "speculative_decoding_verify_attn_amd", "csrc", "sample.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "verify steps/sec and achieved HBM GB/s (% of MI355X peak) per config"
ALL_CONFIGS = ["c1", "c2", "c3", "c4", "c5a", "c5b"]
HEADLINE = "c4"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None, help="one configuration (default: all, headline c4)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="rotating input copies (0: enough to defeat the MALL)")
    ap.add_argument("--algo", type=int, default=0, help="0 auto, 1 vector ALU, 2 matrix cores")
    ap.add_argument("--bps", type=int, default=0, help="context pages per split (0: planner, -1: balanced)")
    ap.add_argument("--no-graph", action="store_true", help="headline from the eager pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip append/rollback/temperature/typical/tree timings (profiling runs)")
    ap.add_argument("--tree-configs", default="c2,c3", help="configurations that also time tree verification")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU work for the headline's oracle sample (a quarter for the others)")
    ap.add_argument("--probe", choices=["none", "copy"], default="none",
                    help="copy: run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


class HipEvents:
    """Raw HIP events (the runtime library via ctypes), recorded on the
    launch stream itself."""

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


def source_hash(path):
    with open(path, "rb") as f:
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


def log(msg):
    print("# " + msg, file=sys.stderr, flush=True)


def unit_rows(a, seed=1, per_unit=1):
    """Flat output-row indices (b*T + t)*Hq + h with per_unit rows of every
    (sequence, KV head) unit (random verify row and head of the group), plus
    the last verify row of the first and last head of every unit's group."""
    rng = np.random.default_rng(seed)
    G = a.Hq // a.Hkv
    rows = []
    for b in range(a.B):
        for g in range(a.Hkv):
            for _ in range(per_unit):
                t = int(rng.integers(0, a.T))
                h = g * G + int(rng.integers(0, G))
                rows.append((b * a.T + t) * a.Hq + h)
            rows.append((b * a.T + a.T - 1) * a.Hq + g * G)
            rows.append((b * a.T + a.T - 1) * a.Hq + g * G + G - 1)
    return np.unique(np.array(rows, dtype=np.int64))


class Bench:
    def __init__(self, args):
        import torch
        import speculative_decoding_verify_attn_amd as sv
        self.torch, self.sv = torch, sv
        self.args = args
        self.dev = torch.device("cuda", 0)
        self.stream = torch.cuda.current_stream(self.dev)
        self.sh = self.stream.cuda_stream
        self.hev = HipEvents()
        c0, c1 = self.hev.create(), self.hev.create()
        torch.cuda.synchronize()
        self.hev.record(c0, self.sh)
        torch.cuda._sleep(1 << 20)
        self.hev.record(c1, self.sh)
        torch.cuda.synchronize()
        self.cycles_per_ms = (1 << 20) / max(self.hev.ms(c0, c1), 1e-3)
        self.sink = sv.probe_read_sink(self.dev)

    def gate(self, n_steps, per_step_ms=0.25):
        """A spin kernel that holds the stream while the host enqueues the
        timed launches, so the GPU then runs them back to back and the events
        bracket GPU work, not host launch latency."""
        self.torch.cuda._sleep(int(self.cycles_per_ms * (2.0 + per_step_ms * n_steps)))

    def timed(self, fn, n, per_step_ms=0.25):
        e0, e1 = self.hev.create(), self.hev.create()
        self.torch.cuda.synchronize()
        self.gate(n, per_step_ms)
        self.hev.record(e0, self.sh)
        for i in range(n):
            fn(i)
        self.hev.record(e1, self.sh)
        self.torch.cuda.synchronize()
        return self.hev.ms(e0, e1) / n

    def read_ceiling(self, nbytes, n):
        """Streaming-read time of nbytes over rotating windows of one arena
        (three windows: a window is never in the Infinity Cache when read)."""
        torch, sv = self.torch, self.sv
        nbytes = (int(nbytes) + 15) // 16 * 16
        arena = torch.empty(3 * nbytes, dtype=torch.uint8, device=self.dev)
        views = [arena[i * nbytes:(i + 1) * nbytes] for i in range(3)]
        for i in range(3):
            sv.spec_verify_probe_read(views[i], nbytes, self.sink, stream=self.stream)
        ms = self.timed(lambda i: sv.spec_verify_probe_read(views[i % 3], nbytes, self.sink, stream=self.stream),
                        n, per_step_ms=nbytes / 5e9)
        del views, arena
        return ms

    def run(self, name, cpu_seconds, tree):
        torch, sv = self.torch, self.sv
        import workloads as W
        args = self.args
        cfg = W.CONFIGS[name]
        dev, stream, sh, hev = self.dev, self.stream, self.sh, self.hev
        t_gen = time.time()
        a = W.make_attn(name, seed=args.seed)
        s = W.make_sample(name, seed=args.seed)
        log("%s: generated in %.1f s" % (name, time.time() - t_gen))
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

        def attn(st, strm=stream, ev=None):
            sv.spec_verify_attn(st["q"], st["k"], st["v"], st["table"], st["lens"], out, ws_a,
                                k_scale=st.get("ks"), v_scale=st.get("vs"), kv_dtype=a.kv_dtype,
                                stream=strm, algo=args.algo, blocks_per_split=args.bps, main_done_event=ev)

        def sample(st, strm=stream):
            sv.spec_verify_sample(st["logits"], st["probs"], st["tokens"], st["u"], n_acc, toks, ws_s, stream=strm)

        def step(st, ev=None):
            if ev is not None:
                hev.record(ev[0], sh)
            attn(st, ev=None if ev is None else ev[1])
            if ev is not None:
                hev.record(ev[2], sh)
            sample(st)
            if ev is not None:
                hev.record(ev[3], sh)

        for i in range(args.warmup):
            step(sets[i % copies])
        torch.cuda.synchronize()
        per_step_ms = max(0.05, 1.5 * attn_bytes / 5e9)

        # eager pass, an event around every call
        evs = [[hev.create() for _ in range(4)] for _ in range(args.steps)]
        t0, t1 = hev.create(), hev.create()
        torch.cuda.synchronize()
        self.gate(args.steps, per_step_ms)
        hev.record(t0, sh)
        for i in range(args.steps):
            step(sets[i % copies], evs[i])
        hev.record(t1, sh)
        torch.cuda.synchronize()
        eager_ms_step = hev.ms(t0, t1) / args.steps
        main_ev_ms = np.array([hev.ms(e[0], e[1]) for e in evs])
        attn_ms = np.array([hev.ms(e[0], e[2]) for e in evs])
        samp_ms = np.array([hev.ms(e[2], e[3]) for e in evs])

        # the main attention kernel alone, back to back
        def main_only(i):
            st = sets[i % copies]
            sv.spec_verify_attn_timing_main_only(st["q"], st["k"], st["v"], st["table"], st["lens"], out, ws_a,
                                                 k_scale=st.get("ks"), v_scale=st.get("vs"),
                                                 kv_dtype=a.kv_dtype, stream=stream, algo=args.algo,
                                                 blocks_per_split=args.bps)
        main_ms = self.timed(main_only, args.steps, per_step_ms)
        # the attention call (main kernel + split merge) and the sampler call, each back to back
        attn_b2b_ms = self.timed(lambda i: attn(sets[i % copies]), args.steps, per_step_ms)
        samp_b2b_ms = self.timed(lambda i: sample(sets[i % copies]), args.steps)

        graph_ms_step = None
        if not args.no_graph:
            graphs = []
            side = torch.cuda.Stream(dev)  # default priority
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for st in sets:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side):
                        attn(st, strm=side)
                        sample(st, strm=side)
                    graphs.append(g)
            stream.wait_stream(side)
            for i in range(args.warmup):
                graphs[i % copies].replay()
            torch.cuda.synchronize()
            graph_ms_step = self.timed(lambda i: graphs[i % copies].replay(), args.steps, per_step_ms)
            # the last replayed copy must reproduce the eager result of that copy
            last = (args.steps - 1) % copies
            step(sets[last])
            torch.cuda.synchronize()
            ref = (n_acc.clone(), toks.clone(), out.clone())
            graphs[last].replay()
            torch.cuda.synchronize()
            if not (torch.equal(ref[0], n_acc) and torch.equal(ref[1], toks) and torch.equal(ref[2], out)):
                raise RuntimeError("%s: graph replay disagrees with the eager step" % name)
            del graphs
        ms_step = graph_ms_step if graph_ms_step is not None else eager_ms_step
        log("%s: step %.1f us (graph), %.1f us (eager); main kernel %.1f us, attention call %.1f us, "
            "sampler %.1f us" % (name, ms_step * 1e3, eager_ms_step * 1e3, main_ms * 1e3, attn_b2b_ms * 1e3,
                                 samp_b2b_ms * 1e3))

        ceil_ms = self.read_ceiling(attn_bytes, args.steps)

        # outputs of the timed path on input copy 0, for the parity summary
        step(sets[0])
        torch.cuda.synchronize()
        out_np = out.cpu().numpy()
        n_np = n_acc.cpu().numpy()
        toks_np = toks.cpu().numpy()
        n_rej = int((n_np < s.K).sum())
        samp_bytes = W.sample_algorithmic_bytes(s, n_rej)

        extras = None
        if not args.no_extras:
            extras = self.extras(a, s, sets, ws_s, n_acc, toks, copies, tree, cfg)

        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                tr = json.load(f)
            ent = tr.get(name)
            if ent and ent.get("attn_src_sha") == source_hash(ATTN_SRC) and args.algo == 0 and args.bps == 0:
                traffic = ent.get("bytes_per_launch")

        attn_gbs = attn_bytes / (main_ms * 1e-3) / 1e9
        res = {
            "workload": "%s: %s (B=%d, Hq=%d, Hkv=%d, d=%d, ctx=%s, page 16, K=%d, %s KV, V=%d)" % (
                name, cfg["desc"], a.B, a.Hq, a.Hkv, a.d, cfg["ctx"], s.K, cfg["kv"], s.V),
            "B": a.B, "K": s.K, "V": s.V, "context": int(a.context_lens.max()),
            "dtype": {W.KV_F32: "f32", W.KV_BF16: "bf16", W.KV_FP8_E4M3: "fp8e4m3"}[a.kv_dtype],
            "rotating_copies": copies,
            "verify_steps_per_s": 1000.0 / ms_step,
            "ms_per_step": ms_step,
            "timing": "HIP graph replay per step" if graph_ms_step is not None else "eager launches",
            "eager_ms_per_step": eager_ms_step,
            "attn_main_kernel_us": main_ms * 1e3,
            "attn_main_kernel_us_step_events": float(main_ev_ms.mean() * 1e3),
            "attn_call_us": attn_b2b_ms * 1e3,
            "attn_call_us_step_events": float(attn_ms.mean() * 1e3),
            "attn_call_us_p10_p90": [float(np.percentile(attn_ms, 10) * 1e3), float(np.percentile(attn_ms, 90) * 1e3)],
            "sample_call_us": samp_b2b_ms * 1e3,
            "sample_call_us_step_events": float(samp_ms.mean() * 1e3),
            "attn_bytes": attn_bytes,
            "sample_bytes": samp_bytes,
            "frac_main_kernel": attn_gbs / HBM_PEAK_GBS,
            "frac_attn_call": attn_bytes / (attn_b2b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "frac_sample_call": samp_bytes / (samp_b2b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "frac_step": (attn_bytes + samp_bytes) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "read_ceiling": {"us": ceil_ms * 1e3, "bytes": attn_bytes,
                             "gbs": attn_bytes / (ceil_ms * 1e-3) / 1e9,
                             "frac": attn_bytes / (ceil_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "what": "plain streaming read of the attention's algorithmic bytes "
                                     "(spec_verify_probe_read, 1024 contiguous chunks)"},
            "roofline": {
                "kernel": "sv_attn_mfma_kernel" if a.kv_dtype != W.KV_F32 else "sv_attn_valu_kernel",
                "what": "main attention kernel; algorithmic bytes: KV of every visible position once, Q in, out, "
                        "used block-table entries (+ page scales for E4M3)",
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
        if extras is not None:
            res.update(extras)
        del sets, ws_a, ws_s
        torch.cuda.empty_cache()
        if not args.no_parity:
            res["parity"] = self.parity(name, a, s, out_np, n_np, toks_np)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline(a, s, cpu_seconds)
        return res

    def extras(self, a, s, sets, ws_s, n_acc, toks, copies, tree, cfg):
        """The rows around the step, back to back: append, rollback, the
        sampler with temperature + top-p and with typical acceptance, and
        tree verification."""
        torch, sv = self.torch, self.sv
        import workloads as W
        args, dev, stream = self.args, self.dev, self.stream
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        k_new = torch.randn((a.B, a.T, a.Hkv, a.d), generator=gen, device=dev)
        v_new = torch.randn((a.B, a.T, a.Hkv, a.d), generator=gen, device=dev)
        if a.kv_dtype == W.KV_FP8_E4M3:
            k_new *= 4.0
            v_new *= 4.0
        st0 = sets[0]
        append_ms = self.timed(lambda i: sv.spec_verify_kv_append(
            k_new, v_new, st0["k"], st0["v"], st0["table"], st0["lens"], k_scale=st0.get("ks"),
            v_scale=st0.get("vs"), kv_dtype=a.kv_dtype, stream=stream), args.steps)
        lens_scratch = st0["lens"].clone()
        pages_scratch = torch.empty_like(lens_scratch)
        n_keep = n_acc.clone()
        rollback_ms = self.timed(lambda i: sv.spec_verify_rollback(n_keep, lens_scratch, s.K,
                                                                    pages_in_use=pages_scratch, stream=stream),
                                 args.steps)
        temp_t = torch.full((s.B,), 0.7, dtype=torch.float32, device=dev)
        cut_t = torch.full((s.B,), 0.9, dtype=torch.float32, device=dev)
        samp_tp_ms = self.timed(lambda i: sv.spec_verify_sample(
            sets[i % copies]["logits"], sets[i % copies]["probs"], sets[i % copies]["tokens"], sets[i % copies]["u"],
            n_acc, toks, ws_s, stream=stream, temperature=temp_t, top_p=cut_t), args.steps)
        samp_ty_ms = self.timed(lambda i: sv.spec_verify_sample_typical(
            sets[i % copies]["logits"], sets[i % copies]["tokens"], sets[i % copies]["u"], n_acc, toks, ws_s,
            0.09, 0.3, stream=stream), args.steps)
        ap_bytes = 2 * k_new.numel() * (4 + W.KV_BYTES[a.kv_dtype]) + 4 * a.B * (a.T + 1)
        res = {"kv_append_us_per_layer": append_ms * 1e3, "kv_append_bytes_per_layer": int(ap_bytes),
               "rollback_us": rollback_ms * 1e3, "sample_temp_topp_us": samp_tp_ms * 1e3,
               "sample_typical_us": samp_ty_ms * 1e3, "tree_verify": None}
        if tree:
            res["tree_verify"] = self.tree(a, s, sets, copies, cfg)
        return res

    def tree(self, a, s, sets, copies, cfg):
        """Tree verification at the same geometry: the widest tree shape the
        attention accepts, attention over the same cache with N verify rows,
        the tree sampler over N target rows, and the commit of the accepted
        paths."""
        torch, sv = self.torch, self.sv
        import workloads as W
        args, dev, stream = self.args, self.dev, self.stream
        G = a.Hq // a.Hkv
        shapes = sorted(W.TREE_SHAPES.items(), key=lambda kv: -len(W.tree_parents(kv[1])))
        fit = [(nm, shp) for nm, shp in shapes
               if sv.attn_shape_supported(a.B, len(W.tree_parents(shp)), a.Hq, a.Hkv, a.d, a.max_blocks)]
        if not fit:
            return None
        t_gen = time.time()
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
        per_step_ms = max(0.05, 3 * W.attn_algorithmic_bytes(a) / 5e9)
        tree_attn_ms = self.timed(lambda i: sv.spec_verify_attn_tree(
            q_tree, sets[i % copies]["k"], sets[i % copies]["v"], sets[i % copies]["table"],
            sets[i % copies]["lens"], tm, out_tree, ws_ta, k_scale=sets[i % copies].get("ks"),
            v_scale=sets[i % copies].get("vs"), kv_dtype=a.kv_dtype, stream=stream), args.steps, per_step_ms)
        ti = W.make_tree(args.seed, s.B, par, s.V, cfg["target_sigma"],
                         cfg["noise"] if not isinstance(cfg["noise"], tuple) else 1.0)
        tl = torch.from_numpy(ti.target_logits).to(dev)
        ncopy = max(2, int(np.ceil(3 * MALL_BYTES / (2 * tl.numel() * 4))) + 1)
        tsets = [{"logits": tl if j == 0 else tl.clone()} for j in range(ncopy)]
        tsets[0]["probs"] = torch.from_numpy(ti.draft_probs).to(dev)
        for j in range(1, ncopy):
            tsets[j]["probs"] = tsets[0]["probs"].clone()
        ttok = torch.from_numpy(ti.tokens).to(dev)
        tpar = torch.from_numpy(ti.parents).to(dev)
        tu = torch.from_numpy(ti.uniforms).to(dev)
        tn = torch.empty(s.B, dtype=torch.int32, device=dev)
        tot = torch.empty((s.B, N), dtype=torch.int32, device=dev)
        tpath = torch.empty((s.B, N), dtype=torch.int32, device=dev)
        ws_ts = sv.alloc_workspace(sv.sample_tree_workspace_size(s.B, N, s.V), dev)
        tree_samp_ms = self.timed(lambda i: sv.spec_verify_sample_tree(
            tsets[i % ncopy]["logits"], tsets[i % ncopy]["probs"], ttok, tpar, tu, tn, tot, tpath,
            ws_ts, max(tshape), stream=stream), args.steps)
        # committing the accepted paths (moves K/V within the cache of copy 0;
        # the lengths shrink from call to call and are clamped at N, which
        # only moves the work to other pages)
        path_np = tpath.cpu().numpy()
        tn_np = tn.cpu().numpy()
        cpath = torch.from_numpy(np.ascontiguousarray(np.resize(path_np, (a.B, N)))).to(dev)
        cn = torch.from_numpy(np.ascontiguousarray(np.resize(tn_np, a.B).astype(np.int32))).to(dev)
        clens = sets[0]["lens"].clone()
        tree_commit_ms = self.timed(lambda i: sv.spec_verify_tree_commit(
            cpath, cn, sets[0]["k"], sets[0]["v"], sets[0]["table"], clens,
            k_scale=sets[0].get("ks"), v_scale=sets[0].get("vs"), kv_dtype=a.kv_dtype, stream=stream), args.steps)
        tree_bytes = W.attn_algorithmic_bytes(a) + 2 * a.B * (N - a.T) * a.Hq * a.d * 4
        res = {"shape": tname, "nodes": N, "rows_per_kv_head": N * G, "attn_us": tree_attn_ms * 1e3,
               "attn_gbs": tree_bytes / (tree_attn_ms * 1e-3) / 1e9, "sample_us": tree_samp_ms * 1e3,
               "commit_us": tree_commit_ms * 1e3, "mean_accepted": float(tn.float().mean().item())}
        log("tree %s (N=%d): attention %.1f us, sampler %.1f us, commit %.1f us (inputs %.1f s)" % (
            tname, N, tree_attn_ms * 1e3, tree_samp_ms * 1e3, tree_commit_ms * 1e3, time.time() - t_gen))
        return res

    def parity(self, name, a, s, out_np, n_np, toks_np):
        """The timed path's outputs of input copy 0 against the CPU oracle."""
        import oracle
        import workloads as W
        t = time.time()
        tol = {W.KV_F32: 1e-3, W.KV_BF16: 2e-2, W.KV_FP8_E4M3: 2e-2}[a.kv_dtype]
        total_rows = a.B * a.T * a.Hq
        rows = np.arange(total_rows, dtype=np.int64) if total_rows <= 1536 else unit_rows(a, seed=1)
        units = {(int(r) // (a.T * a.Hq), (int(r) % a.Hq) // (a.Hq // a.Hkv)) for r in rows}
        ref = oracle.attn(a.q, a.k_cache, a.v_cache, a.block_table, a.context_lens, kv_dtype=a.kv_dtype,
                          k_scale=a.k_scale, v_scale=a.v_scale, rows=rows)
        got = out_np.reshape(-1, a.d)[rows].astype(np.float64)
        err = np.max(np.abs(got - ref), axis=1) / np.max(np.abs(ref), axis=1)
        sref = oracle.sample(s.target_logits, s.draft_probs, s.draft_tokens, s.uniforms)
        mism, flagged = 0, 0
        for b in range(s.B):
            k = int(sref["near_pos"][b])
            if k < 0:
                if n_np[b] != sref["num_accepted"][b] or not np.array_equal(toks_np[b], sref["out_tokens"][b]):
                    mism += 1
            else:
                flagged += 1
                if not np.array_equal(toks_np[b, :k], sref["out_tokens"][b, :k]):
                    mism += 1
        res = {"attn_rows": int(len(rows)), "attn_units_covered": len(units), "attn_units": a.B * a.Hkv,
               "attn_max_row_rel_err": float(err.max()), "attn_tol": tol,
               "attn_ok": bool(err.max() <= tol and np.isfinite(got).all()),
               "sampler_sequences": int(s.B), "sampler_mismatches": mism, "sampler_near_threshold": flagged,
               "mean_accepted": float(n_np.mean()), "oracle_mean_accepted": float(sref["num_accepted"].mean())}
        log("%s parity: %d rows over %d/%d units, max row err %.2e; sampler %d mismatches, %d near-threshold "
            "(%.1f s)" % (name, len(rows), len(units), a.B * a.Hkv, err.max(), mism, flagged, time.time() - t))
        return res


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


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr, flush=True)
        sys.exit(2)
    if args.probe == "copy":
        probe_copy()
        return
    configs = [args.config] if args.config else ALL_CONFIGS
    headline = args.config or HEADLINE
    trees = set(x for x in args.tree_configs.split(",") if x)
    t_all = time.time()
    bench = Bench(args)
    per = {}
    for name in configs:
        budget = args.cpu_seconds if name == headline else args.cpu_seconds / 4
        per[name] = bench.run(name, budget, name in trees)
    bench.hev.close()
    h = per[headline]
    res = {
        "metric": METRIC,
        "value": h["verify_steps_per_s"],
        "unit": "verify steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "timing": h["timing"],
        "eager_ms_per_step": h["eager_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic",
        "config": {"workload": h["workload"], "B": h["B"], "K": h["K"], "V": h["V"], "context": h["context"],
                   "rotating_copies": h["rotating_copies"]},
        "attn_main_kernel_us": h["attn_main_kernel_us"],
        "attn_call_us": h["attn_call_us"],
        "sample_call_us": h["sample_call_us"],
        "frac_step": h["frac_step"],
        "read_ceiling": h["read_ceiling"],
        "roofline": h["roofline"],
    }
    if "cpu_baseline" in h:
        res["cpu_baseline"] = h["cpu_baseline"]
    if "parity" in h:
        res["parity"] = h["parity"]
    res["per_config"] = per
    res["sources"] = {"attn.hip": source_hash(ATTN_SRC), "sample.hip": source_hash(SAMPLE_SRC)}
    res["wall_s"] = time.time() - t_all
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
