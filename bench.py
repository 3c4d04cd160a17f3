#!/usr/bin/env python3
"""Decode benchmark of the activation-sparse FFN on one MI355X.

Workload: one OPT-6.7B-shaped ReLU FFN layer, d_model 4096, d_ffn 16384, fp16
weights with fp32 accumulate, predictor 4096 -> 1024 -> 16384, power-law
firing at ~7% active per token, batch 1, seeded N(0,1) hidden states (1000
decode tokens, cycled).  A step is one decode step of one layer: predictor,
threshold, compaction, gathered FC1 + ReLU, gathered FC2 AXPY, reduction.

Steps rotate over a ring of identical layer copies at distinct addresses, so
that the ~61 MB a step reads cannot be served from the 256 MB Infinity Cache
(a layer ring standing in for the other layers of a model).

Prints ONE JSON line: tokens/s (value: exactly --steps steps after --warmup
steps, bracketed by device synchronisations), effective HBM GB/s on
algorithmic bytes, the median of five repeats of --repeat-steps steps (HIP
events on the stream) and a cache-hot figure (one layer copy), the roofline
of the dominant kernel (the median of --trace-samples kernel durations,
timed by HIP events on the dispatch packets in a traced pass after the timed
region, so that tracing never perturbs the timed steps), the dense
comparator, the CPU oracle baseline and the per-token count of neurons
inside the 1e-3 margin.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "opt6.7b_ffn"
KERNELS = ["pred_l1", "score", "score_fc1", "fc1", "fc2", "list"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--ring", type=int, default=16, help="distinct layer copies")
    ap.add_argument("--tokens", type=int, default=1000)
    ap.add_argument("--dense-steps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle time on all host threads; the 1-thread, dense and stack-subset "
                         "legs take about half, a third and a few seconds more")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--trace-samples", type=int, default=48,
                    help="steps traced with per-kernel HIP events, in a pass of their own "
                         "after the timed region (one step in 8, from the 17th on)")
    ap.add_argument("--repeat-steps", type=int, default=1000,
                    help="steps per repeat of the median-of-5 and cache-hot measurements")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--ffn-rhos", type=float, nargs="*", default=[0.07, 0.10],
                    help="mean activations of the sparse_ffn-alone measurement (none skips it)")
    ap.add_argument("--ffn-sets", type=int, default=256)
    ap.add_argument("--gated-steps", type=int, default=1000,
                    help="decode steps of the gated Llama-7B-shaped layer (0 skips it)")
    ap.add_argument("--gated-ring", type=int, default=12)
    ap.add_argument("--shards", type=int, nargs="*", default=[2, 4, 8],
                    help="neuron-shard counts G of the per-GPU shard measurement (none skips it)")
    ap.add_argument("--shard-steps", type=int, default=1000)
    ap.add_argument("--shard-ring", type=int, default=16)
    ap.add_argument("--stack-tokens", type=int, default=256,
                    help="tokens through the 48-layer stack (0 skips the stack)")
    ap.add_argument("--stack-warmup", type=int, default=8)
    ap.add_argument("--stack-dense-tokens", type=int, default=8)
    ap.add_argument("--batches", type=int, nargs="*", default=[1, 4, 16, 32],
                    help="batch sizes of the batched-union workload (none skips it)")
    ap.add_argument("--batched-ring", type=int, default=3)
    ap.add_argument("--batched-max-steps", type=int, default=0,
                    help="cap on the steps per batch size (0: 1000 // B)")
    ap.add_argument("--layout-steps", type=int, default=1000,
                    help="decode steps per neuron-table variant (0 skips the layout ablation)")
    ap.add_argument("--layout-ring", type=int, default=8)
    ap.add_argument("--head-calls", type=int, default=1000,
                    help="calls of the attention-head predictor per batch size (0 skips it)")
    ap.add_argument("--head-ring", type=int, default=48)
    ap.add_argument("--layout-calib", type=int, default=512,
                    help="calibration tokens of the on-device activation profile")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def bytes_model(sh, k_mean, nz=None, one_launch=False):
    """Algorithmic bytes (each distinct byte the method must read or write,
    counted once) of one decode step and of each kernel.  nz: hidden units of
    the predictor that are nonzero (mean per token); predictor layer 2 reads
    the P2 entries of those units only (one token), all H of them when nz is
    None (batches).  one_launch: predictor layer 1 runs in the score/FC1
    kernel (its bytes are that kernel's)."""
    d, f, H = sh.d, sh.f, sh.H
    ws = 2 if sh.wdtype == "f16" else 4
    nmat = 3 if sh.gated else 2
    words = (f + 63) // 64
    nz = H if nz is None else nz
    l1 = H * d * ws + H * 4 + d * 4            # P1, c1, x
    l2 = nz * f * ws + f * 4                   # P2 entries of the nonzero units, c2
    rows = k_mean * (nmat * d * ws + 4)        # bundles (gate,) up, down + b1
    # single-token decode step: the score/FC1 kernel also reads the listed
    # down columns (FC2 into per-owner rows); the FC2 kernel adds the owner
    # rows (implementation traffic, not counted) with b2 into y
    per = {
        "pred_l1": l1 + H * 4,
        "score": l2 + H * 4 + words * 8,
        "score_fc1": (l1 if one_launch else H * 4 + d * 4) + l2 + words * 8 + rows,
        "fc1": k_mean * ((nmat - 1) * d * ws + 4) + d * 4,
        "fc2": d * 4 * 2,
        "list": words * 8 + k_mean * 4,
    }
    step = l1 + l2 + rows + d * 4 + d * 4
    dense = f * (nmat * d * ws + 4) + d * 4 * 3
    return step, per, dense


def hidden_nonzero(torch, p1, c1, X):
    """Mean count per token of the predictor's hidden units with
    ReLU(P1 x + c1) != 0 (fp32 on the device; the one-token predictor layer
    2 reads the P2 entries of these units only)."""
    w = p1.float().t().contiguous()
    h = torch.matmul(X.float(), w)
    if c1 is not None:
        h = h + c1.float()
    return float((torch.relu(h) != 0).sum(dim=1).double().mean())


PROFILE = os.path.join(ROOT, "profiles", "decode_step_opt6.7b_4096x16384_fp16.md")
KERNEL_SOURCES = [os.path.join(ROOT, "activation_sparse_ffn_02_amd", "csrc", n)
                  for n in ("asf_kernels.hip", "asf_internal.h")]


def kernel_source_hash():
    """SHA-256 of the kernel sources with comments and blank space removed, so
    that a comment edit keeps counters taken on the same code valid."""
    import hashlib
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"\s+", " ", text)
        h.update(text.encode("utf-8"))
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE)
    from the committed counter summary, or None when that summary is missing
    or was taken on kernel sources other than the ones built here."""
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    k = rec.get("per_launch_bytes", {}).get(kernel)
    return None if k is None else k["fetch"] + k["write"]


class HipEvents:
    """A pool of raw hipEvent_t handles (timing enabled), created through the
    HIP runtime so they exist before the library records them."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def record(self, i, stream):
        if self.hip.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def cpu_info():
    """Host CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    return model, ncpu


def cpu_baseline(args, L, x, gpu_sets):
    """The oracle as it stands, on the host cores, on bounded samples of the
    same workload:
      - predict + FFN over the oracle's own set, token by token, on every
        thread OpenMP is given (the reported value) and on one thread;
      - the dense FFN, token by token;
      - the 48-layer OPT-30B-shaped stack's layers 0, 23 and 47 (weights
        generated on the device and read back) x 16 tokens.
    Beside the timing, the oracle's scores of the first tokens give the
    per-token count of neurons inside the 1e-3 margin and how many of them
    the GPU decided the other way (``gpu_sets``: the GPU's active ids of
    those tokens)."""
    import numpy as np

    import oracle
    import workload as wl
    model, ncpu = cpu_info()
    n_thr = oracle.num_threads()

    def run(fn, seconds, n_max):
        t0 = time.perf_counter()
        done = 0
        while done < n_max:
            fn(done)
            done += 1
            if time.perf_counter() - t0 > seconds and done >= 2:
                break
        return done, time.perf_counter() - t0

    scores = {}

    def sparse_tok(t):
        xt = x[t:t + 1]
        _, s, act = oracle.predict(L.p1, L.c1, L.p2, L.c2, xt)
        if t < len(gpu_sets):
            scores[t] = s[0]
        ids = oracle.active_list(act[0], L.perm)
        oracle.ffn(L.w_up, L.w_down, xt, ids, b1=L.b1, b2=L.b2, W_gate=L.w_gate)

    def dense_tok(t):
        oracle.dense_ffn(L.w_up, L.w_down, x[t:t + 1], b1=L.b1, b2=L.b2, W_gate=L.w_gate)

    done, dt = run(sparse_tok, args.cpu_seconds, x.shape[0])
    oracle.set_num_threads(1)
    try:
        done1, dt1 = run(lambda t: sparse_tok(x.shape[0] - 1 - t), args.cpu_seconds / 2,
                         x.shape[0])
    finally:
        oracle.set_num_threads(n_thr)
    dn, ddt = run(dense_tok, args.cpu_seconds / 3, x.shape[0])
    res = {"value": done / dt, "unit": "tokens/s", "cores": int(n_thr), "kind": "oracle",
           "sample": "%d decode tokens of the same layer and token stream (fp64 predictor + "
                     "FFN over the predicted set), %.1f s on %d threads" % (done, dt, n_thr),
           "cpu_model": model, "host_cpus": ncpu,
           "one_thread": {"tokens_per_s": done1 / dt1, "tokens": done1, "seconds": dt1},
           "dense": {"tokens_per_s": dn / ddt, "tokens": dn, "seconds": ddt,
                     "threads": int(n_thr)}}
    if args.stack_tokens > 0:
        import torch
        from workload.gpu import stack_layer_device, stack_tokens
        xs = stack_tokens(16)
        t_all, n_all, ks = 0.0, 0, []
        for l in (0, 23, 47):
            SL = stack_layer_device(l, torch.device("cuda:0")).to_numpy()
            torch.cuda.empty_cache()
            t0 = time.perf_counter()
            for t in range(xs.shape[0]):
                _, _, act = oracle.predict(SL.p1, SL.c1, SL.p2, SL.c2, xs[t:t + 1])
                ids = oracle.active_list(act[0], SL.perm)
                oracle.ffn(SL.w_up, SL.w_down, xs[t:t + 1], ids, b1=SL.b1, b2=SL.b2)
                ks.append(ids.size)
            t_all += time.perf_counter() - t0
            n_all += xs.shape[0]
            del SL
        res["stack_subset"] = {
            "sample": "layers 0, 23, 47 of the 48-layer 7168x28672 stack x 16 tokens (each "
                      "layer fed the stack's input tokens), predict + FFN over the set",
            "layer_tokens": n_all, "seconds": t_all, "ms_per_layer_token": t_all * 1e3 / n_all,
            "est_ms_per_token_48_layers": t_all * 1e3 / n_all * wl.STACK_LAYERS,
            "active_mean": float(np.mean(ks))}
    # margin statistics of the oracle's scores (not timed)
    amb = None
    if scores:
        band, flips = [], []
        for t, s in sorted(scores.items()):
            inband = np.abs(s) <= 1e-3
            g = np.zeros(s.shape[0], bool)
            g[gpu_sets[t]] = True
            diff = g != (s > 0)
            band.append(int(inband.sum()))
            flips.append(int(diff.sum()))
            if np.any(diff & ~inband):
                raise AssertionError("token %d: the GPU set differs from the oracle's beyond "
                                     "the 1e-3 margin" % t)
        amb = {"tokens": len(band), "in_margin_per_token": float(np.mean(band)),
               "gpu_flips_per_token": float(np.mean(flips)), "max_in_margin": int(max(band)),
               "rule": "|s - theta| <= 1e-3: either decision is correct"}
    return res, amb


def bench_stack(args, asf, torch, np, wl, dev, stream):
    """The 48-layer OPT-30B-shaped stack (7168x28672 fp16, ~40 GB resident):
    B = 1 tokens through all layers per asf_stack_decode call."""
    from workload.gpu import stack_layer_device, stack_tokens
    t0 = time.perf_counter()
    layers, shapes, p1s = [], [], []
    for l in range(wl.STACK_LAYERS):
        DL = stack_layer_device(l, dev)
        layers.append(asf.Layer(DL.w_up, DL.w_down, DL.p1, DL.p2, b1=DL.b1, b2=DL.b2, c2=DL.c2,
                                neuron_table=DL.perm))
        shapes.append(DL.shape)
        p1s.append(DL.p1)
        del DL
        torch.cuda.synchronize()
    torch.cuda.empty_cache()
    resident = sum(l.storage.numel() for l in layers)
    log(args, "stack of %d layers, %.2f GB, built in %.1f s" % (len(layers), resident / 1e9,
                                                             time.perf_counter() - t0))
    st = asf.Stack(layers)
    n = args.stack_tokens
    X = torch.from_numpy(stack_tokens(n + args.stack_warmup)).to(dev)
    Y = torch.empty((1, wl.STACK_D), dtype=torch.float32, device=dev)
    work = torch.empty_like(Y)
    sh_ = stream.cuda_stream
    xs = [X[t].data_ptr() for t in range(X.shape[0])]
    for t in range(args.stack_warmup):
        st.decode_raw(xs[n + t], 1, Y.data_ptr(), work.data_ptr(), sh_)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(n):
        st.decode_raw(xs[t], 1, Y.data_ptr(), work.data_ptr(), sh_)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the look-ahead form (layer l+1's set from layer l's input, predicted in
    # the same launches as layer l's FC1/FC2), same tokens
    for t in range(args.stack_warmup):
        st.decode_lookahead_raw(xs[n + t], Y.data_ptr(), work.data_ptr(), sh_)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(n):
        st.decode_lookahead_raw(xs[t], Y.data_ptr(), work.data_ptr(), sh_)
    torch.cuda.synchronize()
    elapsed_la = time.perf_counter() - t0
    # per-layer active counts of the same tokens (outside the timed region)
    counts = torch.zeros((n, len(layers)), dtype=torch.int32, device=dev)
    nzs = np.zeros(len(layers))
    for t in range(n):
        cur = X[t:t + 1]
        for l, lay in enumerate(layers):
            lay.predict(cur, n_active=counts[t, l:l + 1], want_list=False)
            if t < 16:
                nzs[l] += hidden_nonzero(torch, p1s[l], None, cur) / min(n, 16)
            cur = lay.decode_step(cur)
    torch.cuda.synchronize()
    del p1s
    k = counts.double().mean(dim=0).cpu().numpy()
    tok_bytes = sum(bytes_model(shapes[l], float(k[l]), float(nzs[l]))[0]
                    for l in range(len(layers)))
    dense_bytes = sum(bytes_model(shapes[l], 0.0)[2] for l in range(len(layers)))
    # dense comparator: every layer's dense FFN, chained, a few tokens
    nd = args.stack_dense_tokens
    dense_ms = None
    if nd > 0:
        cur = X[:1]
        for l, lay in enumerate(layers):
            cur = lay.dense_ffn_ref(cur)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for t in range(nd):
            cur = X[t:t + 1]
            for lay in layers:
                cur = lay.dense_ffn_ref(cur)
        torch.cuda.synchronize()
        dense_ms = (time.perf_counter() - t1) * 1e3 / nd
    ms_tok = elapsed * 1e3 / n
    res = {
        "workload": "OPT-30B-shaped FFN stack: 48 layers 7168x28672 fp16, predictors 7168->"
                    "{512,1024,2048}->28672, activation 3%->15% by depth, batch 1",
        "tokens": n, "tokens_per_s": n / elapsed, "ms_per_token": ms_tok,
        "resident_gb": resident / 1e9,
        "algorithmic_bytes_per_token": tok_bytes,
        "effective_gbps": tok_bytes / (ms_tok * 1e-3) / 1e9,
        "effective_frac_of_peak": tok_bytes / (ms_tok * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "lookahead_tokens_per_s": n / elapsed_la,
        "lookahead_ms_per_token": elapsed_la * 1e3 / n,
        "active_frac_by_layer": [round(float(k[l]) / shapes[l].f, 4) for l in range(len(layers))],
        "pred_hidden_by_layer": [shapes[l].H for l in range(len(layers))],
        "pred_hidden_nonzero_by_layer": [round(float(nzs[l]), 1) for l in range(len(layers))],
        "launches_by_layer": [lay.step_launches(1) for lay in layers],
        "dense_ms_per_token": dense_ms,
        "dense_gbps": None if dense_ms is None else dense_bytes / (dense_ms * 1e-3) / 1e9,
        "speedup_vs_dense": None if dense_ms is None else dense_ms / ms_tok,
    }
    for lay in layers:
        lay.close()
    return res


def bench_layout(args, asf, torch, np, wl, dev, stream):
    """Neuron-table ablation on the benchmark layer: the decode step with the
    identity table, with the hot-first table profiled on the device
    (asf_profile_activations over calibration tokens, then
    asf_hot_first_table), and with the generator's own hot-first table."""
    import dataclasses
    L = wl.config_layer(WORKLOAD)
    sh = L.shape
    t0 = time.perf_counter()
    calib = torch.from_numpy(wl.config_calib_tokens(WORKLOAD, args.layout_calib)).to(dev)
    ident = asf.layer_from_numpy(L, use_table=False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    counts = ident.profile_activations(calib)
    table = asf.hot_first_table(counts)
    torch.cuda.synchronize()
    prof_ms = (time.perf_counter() - t1) * 1e3
    del ident
    tab = table.cpu().numpy().astype(L.perm.dtype)
    top = min(1000, sh.f)
    overlap = len(set(tab[:top].tolist()) & set(L.perm[:top].tolist())) / top
    X = torch.from_numpy(wl.config_tokens(WORKLOAD, args.tokens)).to(dev)
    xs = [X[t:t + 1].data_ptr() for t in range(args.tokens)]
    sh_ = stream.cuda_stream
    res = {"workload": "OPT-6.7B-shaped layer 4096x16384 fp16, batch 1, ring of %d copies per table"
                       % args.layout_ring,
           "calibration_tokens": args.layout_calib, "profile_and_table_ms": prof_ms,
           "profiled_top1000_overlap_with_generator": overlap}
    variants = [("identity", dict(use_table=False), L),
                ("profiled", {}, dataclasses.replace(L, perm=tab)),
                ("generator", {}, L)]
    for name, kw, LL in variants:
        ring = [asf.layer_from_numpy(LL, **kw) for _ in range(args.layout_ring)]
        Y = torch.empty((args.layout_ring, 1, sh.d), dtype=torch.float32, device=dev)
        ys = [Y[r].data_ptr() for r in range(args.layout_ring)]
        for i in range(50):
            ring[i % len(ring)].decode_step_raw(xs[i % args.tokens], 1, ys[i % len(ring)], sh_)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.layout_steps):
            ring[i % len(ring)].decode_step_raw(xs[i % args.tokens], 1, ys[i % len(ring)], sh_)
        e1.record()
        torch.cuda.synchronize()
        res[name + "_us_per_step"] = e0.elapsed_time(e1) * 1e3 / args.layout_steps
        del ring, Y
        torch.cuda.empty_cache()
    log(args, "layout ablation (us per step): identity %.2f, profiled %.2f, generator %.2f; %.1f s"
        % (res["identity_us_per_step"], res["profiled_us_per_step"], res["generator_us_per_step"],
           time.perf_counter() - t0))
    return res


def bench_gated(args, asf, torch, np, wl, dev, stream):
    """The Llama-7B-shaped gated ReLU layer (4096x11008, gate/up/down fp16,
    predictor 4096->1024->11008, ~10% active): batch-1 decode steps over a
    ring of layer copies, and the dense comparator on the same ring."""
    name = "llama7b_gated_relu"
    L = wl.config_layer(name)
    sh = L.shape
    X = torch.from_numpy(wl.config_tokens(name, args.tokens)).to(dev)

    def up(a):
        return None if a is None else torch.from_numpy(a).to(dev)
    orig = dict(w_up=up(L.w_up), w_down=up(L.w_down), w_gate=up(L.w_gate), p1=up(L.p1),
                p2=up(L.p2), b1=up(L.b1), b2=up(L.b2), c2=up(L.c2), neuron_table=up(L.perm))
    ring = [asf.Layer(orig["w_up"], orig["w_down"], orig["p1"], orig["p2"],
                      w_gate=orig["w_gate"], b1=orig["b1"], b2=orig["b2"], c2=orig["c2"],
                      neuron_table=orig["neuron_table"]) for _ in range(args.gated_ring)]
    torch.cuda.synchronize()
    nz = hidden_nonzero(torch, orig["p1"], None, X)
    del orig
    torch.cuda.empty_cache()
    Y = torch.empty((len(ring), 1, sh.d), dtype=torch.float32, device=dev)
    xs = [X[t].data_ptr() for t in range(X.shape[0])]
    ys = [Y[r].data_ptr() for r in range(len(ring))]
    sh_ = stream.cuda_stream
    n = args.gated_steps
    for i in range(50):
        ring[i % len(ring)].decode_step_raw(xs[i % len(xs)], 1, ys[i % len(ring)], sh_)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        ring[i % len(ring)].decode_step_raw(xs[i % len(xs)], 1, ys[i % len(ring)], sh_)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    counts = torch.zeros(n, dtype=torch.int32, device=dev)
    for i in range(n):
        ring[i % len(ring)].predict(X[i % X.shape[0]], active=None, n_active=counts[i:i + 1],
                                    want_list=False)
    torch.cuda.synchronize()
    k = float(counts.double().mean())
    step_bytes, _, dense_bytes = bytes_model(sh, k, nz)
    nd = max(5, min(args.dense_steps, n))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ring[0].dense_ffn_ref(X[:1])
    e0.record()
    for i in range(nd):
        ring[i % len(ring)].dense_ffn_ref(X[i % X.shape[0]], out=Y[i % len(ring)])
    e1.record()
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1) / nd
    ms = el * 1e3 / n
    for lay in ring:
        lay.close()
    res = {"workload": "Llama-7B-shaped gated ReLU FFN layer 4096x11008 fp16 (gate, up, down), "
                       "predictor 4096->1024->11008, ~10% active, batch 1",
           "ring_layers": len(ring), "steps": n, "tokens_per_s": n / el, "ms_per_step": ms,
           "active_frac": k / sh.f, "pred_hidden_nonzero_mean": nz,
           "algorithmic_bytes_per_step": step_bytes,
           "effective_gbps": step_bytes / (ms * 1e-3) / 1e9,
           "effective_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "dense_ms_per_step": dense_ms, "dense_gbps": dense_bytes / (dense_ms * 1e-3) / 1e9,
           "speedup_vs_dense": dense_ms / ms, "byte_ceiling_vs_dense": dense_bytes / step_bytes}
    log(args, "gated: %.1f us per step, %.1f%% active, %.2fx dense" % (ms * 1e3, 100 * k / sh.f,
                                                                      dense_ms / ms))
    return res


def shard_slices(L, G):
    """Shard 0 of layer L sharded by neurons over G GPUs: every G-th neuron by
    hotness rank (so each shard's expected active count is the same), in rank
    order, with its up rows, down columns, b1, P2 rows and c2; P1 (and c1)
    replicated; b2 added by shard 0."""
    ids = L.perm[0::G]
    return dict(w_up=L.w_up[ids], w_down=L.w_down[:, ids], p1=L.p1, p2=L.p2[ids],
                b1=L.b1[ids], b2=L.b2, c2=L.c2[ids])


def bench_shards(args, asf, torch, np, wl, dev, stream, L, X):
    """One GPU's share of a layer sharded by neurons over G GPUs (shard_slices):
    batch-1 decode steps of the OPT-6.7B-shaped layer's shard, and batch-32
    steps of the OPT-13B-shaped layer's shard, each over a ring of shard
    copies.  The all-reduce of the partial y that joins the shards is not part
    of it."""
    sh_ = stream.cuda_stream
    L13 = wl.config_layer("opt13b_batched")
    X13 = wl.config_tokens("opt13b_batched", 1000)
    out = []
    for G in args.shards:
        for B, lay, toks in ((1, L, X), (32, L13, X13)):
            sh = lay.shape
            if G < 1 or sh.f % (64 * G):
                continue
            Xd = torch.from_numpy(toks).to(dev)
            w = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
                 for k, v in shard_slices(lay, G).items()}
            nring = args.shard_ring if B == 1 else max(4, args.shard_ring // 2)
            ring = [asf.Layer(w["w_up"], w["w_down"], w["p1"], w["p2"], b1=w["b1"], b2=w["b2"],
                              c2=w["c2"], max_batch=B) for _ in range(nring)]
            torch.cuda.synchronize()
            nz = hidden_nonzero(torch, w["p1"], None, Xd) if B == 1 else None
            del w
            torch.cuda.empty_cache()
            nst = Xd.shape[0] // B
            Y = torch.empty((nring, B, sh.d), dtype=torch.float32, device=dev)
            xs = [Xd[i * B:(i + 1) * B].data_ptr() for i in range(nst)]
            ys = [Y[r].data_ptr() for r in range(nring)]
            n = args.shard_steps if B == 1 else max(10, args.shard_steps // 10)
            for i in range(min(100, n)):
                ring[i % nring].decode_step_raw(xs[i % nst], B, ys[i % nring], sh_)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(n):
                ring[i % nring].decode_step_raw(xs[i % nst], B, ys[i % nring], sh_)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            counts = torch.zeros(n, dtype=torch.int32, device=dev)
            for i in range(n):
                ring[i % nring].predict(Xd[(i % nst) * B:(i % nst + 1) * B], active=None,
                                        n_active=counts[i:i + 1], want_list=False)
            torch.cuda.synchronize()
            k = float(counts.double().mean())
            fs = sh.f // G
            step_bytes, _, _ = bytes_model(wl.scaled_shape(sh, sh.d, fs, sh.H), k, nz)
            ms = el * 1e3 / n
            rec = {"layer": "OPT-6.7B-shaped 4096x16384" if B == 1 else
                            "OPT-13B-shaped 5120x20480",
                   "batch": B, "gpus": G, "d_ffn_per_gpu": fs, "launches": ring[0].step_launches(B),
                   "ring_layers": nring, "steps": n, "us_per_step": ms * 1e3,
                   "active_per_step": k, "active_frac": k / fs,
                   "algorithmic_bytes_per_step": step_bytes,
                   "effective_gbps": step_bytes / (ms * 1e-3) / 1e9,
                   "effective_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            out.append(rec)
            log(args, "shard 1/%d, B=%d: %.1f us per step, %.0f active" % (G, B, ms * 1e3, k))
            for lay_ in ring:
                lay_.close()
            del ring, Y, Xd
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    return {"workload": "one GPU's shard of a layer sharded by neurons over G GPUs (every G-th "
                        "neuron by hotness rank, P1 replicated, fp16): the OPT-6.7B-shaped "
                        "layer at batch 1 and the OPT-13B-shaped layer at batch 32; the "
                        "all-reduce of y is not included",
            "by_gpus": out}


def bench_heads(args, asf, torch, np, wl, dev, stream):
    """The attention-head predictor of the OPT-30B-shaped attention block
    (d_model 7168, 56 heads, hidden 1024, fp16) over a ring of copies (one
    per layer of the 48-layer stack): per-token head masks, lists and
    counts, batch 1 and 32."""
    name = "opt30b_heads"
    P = wl.head_config(name)
    sh = P.shape
    X = torch.from_numpy(wl.head_config_tokens(name, 1024)).to(dev)
    ring = [asf.head_predictor_from_numpy(P, device=dev, max_batch=32)
            for _ in range(args.head_ring)]
    torch.cuda.synchronize()
    words = (sh.heads + 63) // 64
    out = []
    sh_ = stream.cuda_stream
    for B in (1, 32):
        n = args.head_calls
        masks = torch.empty((len(ring), B, words), dtype=torch.int64, device=dev)
        heads = torch.empty((len(ring), B, sh.heads), dtype=torch.int32, device=dev)
        counts = torch.zeros((len(ring), B), dtype=torch.int32, device=dev)
        xs = [X[(i * B) % (1024 - B):(i * B) % (1024 - B) + B].data_ptr() for i in range(n)]

        def call(i):
            r = i % len(ring)
            ring[r].predict_raw(xs[i], B, masks[r].data_ptr(), heads[r].data_ptr(),
                                counts[r].data_ptr(), sh_)
        for i in range(min(50, n)):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        ws = 2 if sh.wdtype == "f16" else 4
        byts = (sh.H * sh.d + sh.heads * sh.H) * ws + 4 * (sh.H + sh.heads) + 4 * B * sh.d
        out.append({"batch": B, "calls": n, "ms_per_call": ms,
                    "tokens_per_s": B / (ms * 1e-3),
                    "algorithmic_bytes_per_call": byts,
                    "effective_gbps": byts / (ms * 1e-3) / 1e9,
                    "effective_frac_of_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "selected_frac": float(counts.double().mean()) / sh.heads})
        log(args, "head predictor B=%d: %.2f us per call, %.1f%% of heads selected"
            % (B, ms * 1e3, 100 * out[-1]["selected_frac"]))
    for hp in ring:
        hp.close()
    return {"workload": "attention-head predictor of an OPT-30B-shaped layer: 7168 -> 1024 -> "
                        "56 heads fp16, ~20%% of heads selected, ring of %d copies"
                        % args.head_ring, "by_batch": out}


def bench_batched(args, asf, torch, np, wl, dev, stream):
    """Batched decode on the OPT-13B-shaped layer (5120x20480 fp16, predictor
    5120->1024->20480, ~5% active per token): B tokens per step share the
    union of their predicted sets.  1000 // B steps per batch size over a ring
    of layer copies; the dense comparators are this library's dense FFN and
    torch's fp16 GEMMs (hipBLASLt) of the same shape."""
    name = "opt13b_batched"
    L = wl.config_layer(name)
    sh = L.shape
    X = torch.from_numpy(wl.config_tokens(name, 1000)).to(dev)

    def up(a):
        return None if a is None else torch.from_numpy(a).to(dev)
    w_up, w_down = up(L.w_up), up(L.w_down)
    orig = dict(p1=up(L.p1), p2=up(L.p2), b1=up(L.b1), b2=up(L.b2), c2=up(L.c2),
                neuron_table=up(L.perm))
    ring = [asf.Layer(w_up, w_down, orig["p1"], orig["p2"], b1=orig["b1"], b2=orig["b2"],
                      c2=orig["c2"], neuron_table=orig["neuron_table"], max_batch=32)
            for _ in range(args.batched_ring)]
    torch.cuda.synchronize()
    nz1 = hidden_nonzero(torch, orig["p1"], None, X)
    del orig
    sh_ = stream.cuda_stream
    out = []
    for B in args.batches:
        steps = 1000 // B
        if args.batched_max_steps > 0:
            steps = min(steps, args.batched_max_steps)
        Y = torch.empty((args.batched_ring, B, sh.d), dtype=torch.float32, device=dev)
        xs = [X[i * B:(i + 1) * B].data_ptr() for i in range(steps)]
        ys = [Y[r].data_ptr() for r in range(args.batched_ring)]
        for i in range(min(10, steps)):
            ring[i % len(ring)].decode_step_raw(xs[i], B, ys[i % len(ring)], sh_)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ring[i % len(ring)].decode_step_raw(xs[i], B, ys[i % len(ring)], sh_)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        counts = torch.zeros(steps, dtype=torch.int32, device=dev)
        for i in range(steps):
            ring[0].predict(X[i * B:(i + 1) * B], n_active=counts[i:i + 1], want_list=False)
        torch.cuda.synchronize()
        k = float(counts.double().mean())
        step_bytes, _, dense_bytes = bytes_model(sh, k, nz1 if B == 1 else None)
        ms = el * 1e3 / steps
        rec = {
            "batch": B, "steps": steps, "tokens_per_s": B * steps / el, "ms_per_step": ms,
            "union_frac": k / sh.f, "algorithmic_bytes_per_step": step_bytes,
            "effective_gbps": step_bytes / (ms * 1e-3) / 1e9,
            "effective_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "dense_ms_per_step": None, "dense_gbps": None, "speedup_vs_dense": None,
            "torch_fp16_gemm_ms_per_step": None,
        }
        out.append(rec)
        log(args, "batched B=%d: %.1f us/step, union %.3f" % (B, ms * 1e3, k / sh.f))
        if args.dense_steps <= 0:
            continue     # comparators skipped (e.g. counter runs of the step's kernels alone)
        nd = max(5, min(50, steps))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ring[0].dense_ffn_ref(X[:B])
        e0.record()
        for i in range(nd):
            ring[i % len(ring)].dense_ffn_ref(X[i * B:(i + 1) * B], out=Y[i % len(ring)])
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / nd
        # torch fp16 GEMMs of the same shape (context)
        xh = X[:B].half()
        bh = torch.from_numpy(L.b1).to(dev).half()
        for _ in range(3):
            torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(xh, w_up, bh)), w_down)
        torch.cuda.synchronize()
        e0.record()
        for i in range(nd):
            xh = X[i * B:(i + 1) * B].half()
            torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(xh, w_up, bh)), w_down)
        e1.record()
        torch.cuda.synchronize()
        torch_ms = e0.elapsed_time(e1) / nd
        rec.update({"dense_ms_per_step": dense_ms,
                    "dense_gbps": dense_bytes / (dense_ms * 1e-3) / 1e9,
                    "speedup_vs_dense": dense_ms / ms, "torch_fp16_gemm_ms_per_step": torch_ms})
    for lay in ring:
        lay.close()
    return {"workload": "OPT-13B-shaped FFN layer 5120x20480 fp16, predictor 5120->1024->20480, "
                        "~5% active per token, batch union", "ring_layers": len(ring),
            "operand_precision": "fp16 weights, fp32 accumulation; predictor x and h and the FC2 "
                                 "activations enter the matrix cores as fp16 hi + lo (products "
                                 "exact in fp32); FC1 takes x rounded to fp16 once",
            "by_batch": out}


def bench_ffn_only(args, ring, Xd, Y, L, dense_ms, dense_bytes, torch, wl, dev, sh_):
    """asf_sparse_ffn alone (FC1 + ReLU + FC2 over a caller's id list, no
    predictor) on the benchmark ring, against the dense FFN of the same ring:
    per-token sets drawn from the layer's firing law (its hotness order) at
    each mean activation in --ffn-rhos."""
    sh = L.shape
    ws = 2 if sh.wdtype == "f16" else 4
    nmat = 3 if sh.gated else 2
    n = args.ffn_sets
    out = []
    for rho in args.ffn_rhos:
        sets = wl.sampled_sets(L.perm, rho, n, seed=4000 + int(round(rho * 1000)))
        ids = torch.zeros((n, sh.f), dtype=torch.int32)
        cnt = torch.zeros(n, dtype=torch.int32)
        for t, st in enumerate(sets):
            ids[t, :len(st)] = torch.from_numpy(st)
            cnt[t] = len(st)
        ids, cnt = ids.to(dev), cnt.to(dev)
        ap = [ids[t].data_ptr() for t in range(n)]
        cp = [cnt[t:t + 1].data_ptr() for t in range(n)]
        xs = [Xd[t % Xd.shape[0]].data_ptr() for t in range(n)]
        ys = [Y[r].data_ptr() for r in range(len(ring))]
        for i in range(20):
            ring[i % len(ring)].sparse_ffn_raw(xs[i % n], 1, ap[i % n], cp[i % n],
                                               ys[i % len(ring)], sh_)
        torch.cuda.synchronize()
        # one call is two short kernels, faster than the host issues them
        # from Python, so the calls are captured once into a HIP graph and the
        # graph is replayed (the same kernels, launched by the device queue)
        steps = n
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(steps):
                ring[i % len(ring)].sparse_ffn_raw(xs[i], 1, ap[i], cp[i], ys[i % len(ring)], cs)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.dense_steps // steps + 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * steps)
        del g
        # the same calls issued one by one from Python (host-bound)
        e0.record()
        for i in range(steps):
            ring[i % len(ring)].sparse_ffn_raw(xs[i], 1, ap[i], cp[i], ys[i % len(ring)], sh_)
        e1.record()
        torch.cuda.synchronize()
        ms_eager = e0.elapsed_time(e1) / steps
        k = float(sum(len(st) for st in sets)) / n
        # the set's rows and down columns (+ b1, ids), x, b2, y
        b = k * (nmat * sh.d * ws + 4 + 4) + sh.d * 4 * 3
        r = {"rho": rho, "active_mean": k, "active_frac": k / sh.f, "calls": steps * reps,
             "ms_per_call": ms, "ms_per_call_python_issued": ms_eager, "algorithmic_bytes_per_call": b,
             "effective_gbps": b / (ms * 1e-3) / 1e9,
             "effective_frac_of_peak": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
             "speedup_vs_dense": None if dense_ms is None else dense_ms / ms,
             "byte_ceiling_vs_dense": dense_bytes / b}
        out.append(r)
        log(args, "sparse_ffn alone at rho %.2f: %.1f us per call, %.2fx dense"
            % (rho, ms * 1e3, r["speedup_vs_dense"] or 0.0))
    return {"workload": "asf_sparse_ffn over given per-token sets (firing law of the benchmark "
                        "layer at each mean activation), batch 1, same ring as the decode step, "
                        "calls replayed from a HIP graph",
            "sets_per_rho": n, "by_rho": out}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the per-GPU kernel is the neuron-sharded design's shard); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_sparse_ffn_02_amd as asf
    import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = wl.config_layer(WORKLOAD)
    sh = L.shape
    X = wl.config_tokens(WORKLOAD, args.tokens)
    log(args, "workload generated", sh)

    def up(a):
        return None if a is None else torch.from_numpy(a).to(dev)

    orig = dict(w_up=up(L.w_up), w_down=up(L.w_down), p1=up(L.p1), p2=up(L.p2),
                w_gate=up(L.w_gate), b1=up(L.b1), b2=up(L.b2), c1=up(L.c1), c2=up(L.c2),
                neuron_table=up(L.perm))
    ring = []
    for _ in range(args.ring):
        ring.append(asf.Layer(orig["w_up"], orig["w_down"], orig["p1"], orig["p2"],
                              w_gate=orig["w_gate"], b1=orig["b1"], b2=orig["b2"],
                              c1=orig["c1"], c2=orig["c2"], neuron_table=orig["neuron_table"]))
    torch.cuda.synchronize()
    nz_mean = hidden_nonzero(torch, orig["p1"], orig["c1"], torch.from_numpy(X).to(dev))
    del orig
    torch.cuda.empty_cache()
    ring_bytes = sum(l.storage.numel() for l in ring)
    log(args, "ring of %d layers, %.2f GB" % (args.ring, ring_bytes / 1e9))

    Xd = torch.from_numpy(X).to(dev)
    Y = torch.empty((args.ring, 1, sh.d), dtype=torch.float32, device=dev)
    K, W = args.steps, args.warmup
    counts = torch.zeros(K + W, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    lib = asf.library()

    sh_ = stream.cuda_stream
    xs = [Xd[t].data_ptr() for t in range(args.tokens)]
    ys = [Y[r].data_ptr() for r in range(args.ring)]

    def step(i, ring_n=args.ring):
        ring[i % ring_n].decode_step_raw(xs[i % args.tokens], 1, ys[i % ring_n], sh_)

    # the timed region: exactly K steps after W warm-up steps, no events
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K

    # repeats: 5 x R steps each bracketed by HIP events on the stream (the
    # median of the five is the steady-state step time); then the same with
    # one layer copy (its 61 MB stay in the 256 MB Infinity Cache: cache-hot)
    R = max(1, args.repeat_steps)
    hrep = HipEvents(20)

    def repeats(ring_n, base):
        per = []
        for r in range(5):
            hrep.record(base + 2 * r, sh_)
            for i in range(R):
                step(r * R + i, ring_n)
            hrep.record(base + 2 * r + 1, sh_)
        torch.cuda.synchronize()
        return sorted(hrep.ms(base + 2 * r, base + 2 * r + 1) / R for r in range(5))

    rep = repeats(args.ring, 0)
    for i in range(50):
        step(i, 1)
    hot = repeats(1, 10)
    hrep.close()

    # per-kernel durations: a traced pass of its own (each traced step
    # launches its kernels with HIP events on the dispatch packets, so the
    # events time the kernels themselves on the stream they run on); one
    # step in 8 from the 17th on, median per kernel
    one_launch = ring[0].step_launches(1) == 2
    used = [KERNELS.index(k) for k in
            (("score_fc1", "fc2") if one_launch else ("pred_l1", "score_fc1", "fc2"))]
    NE = 2 * len(KERNELS)
    ns = max(1, args.trace_samples)
    hev = HipEvents(NE * ns)
    EvArr = ctypes.c_void_p * NE

    def ev_slots(n):
        slots = [None] * NE
        for j in used:
            slots[2 * j] = hev.ev[NE * n + 2 * j]
            slots[2 * j + 1] = hev.ev[NE * n + 2 * j + 1]
        return EvArr(*slots)

    arrs = [ev_slots(n) for n in range(ns)]
    for i in range(16 + 8 * ns):
        traced = i >= 16 and (i - 16) % 8 == 0
        lay = ring[i % args.ring]
        if traced:
            lay.set_trace(arrs[(i - 16) // 8], len(KERNELS))
        step(i)
        if traced:
            lay.set_trace(None)
    torch.cuda.synchronize()
    kt = np.zeros((ns, len(KERNELS)))
    for n in range(ns):
        for j in used:
            kt[n, j] = hev.ms(NE * n + 2 * j, NE * n + 2 * j + 1)
    kmed = np.median(kt, axis=0)        # ms
    # each traced step's span, first kernel's start to last kernel's stop:
    # the kernels run one after another on one stream, so their durations
    # must add up to at most that span (tracing itself makes a traced step
    # slower than an untraced one)
    j0, j1 = used[0], used[-1]
    span = np.array([hev.ms(NE * n + 2 * j0, NE * n + 2 * j1 + 1) for n in range(ns)])
    hev.close()

    # active counts of the timed steps, outside the timed region (the steps
    # are deterministic, so these are the sets the timed steps used)
    for i in range(W, W + K):
        ring[i % args.ring].predict(Xd[i % args.tokens], active=None, n_active=counts[i:i + 1],
                                    want_list=False)
    torch.cuda.synchronize()
    ks = counts[W:].cpu().numpy()
    k_mean = float(ks.mean())
    step_bytes, per_bytes, dense_bytes = bytes_model(sh, k_mean, nz_mean, one_launch)
    dom = int(np.argmax(kmed))
    dname = KERNELS[dom]
    achieved = per_bytes[dname] / (kmed[dom] * 1e-3) / 1e9
    # the same kernel's bytes counted with every P2 entry (predictor layer 2
    # charged as dense, although the step reads only the entries of nonzero
    # hidden units), reported beside the count of what the step reads
    _, per_dense_p2, _ = bytes_model(sh, k_mean, None, one_launch)
    kernel_sum_ms = float(kmed[used].sum())
    within = bool(np.all(kt[:, used].sum(axis=1) <= span + 1e-6))
    if not within:
        log(args, "warning: a traced step's kernel durations add up to more than its span")
    # GPU sets of the first tokens, for the margin statistics of the CPU leg
    n_amb = 0 if args.no_cpu else min(32, args.tokens)
    gpu_sets = []
    act_buf = torch.empty(sh.f, dtype=torch.int32, device=dev)
    n_buf = torch.empty(1, dtype=torch.int32, device=dev)
    for t in range(n_amb):
        ring[0].predict(Xd[t], active=act_buf, n_active=n_buf)
        gpu_sets.append(act_buf[:int(n_buf.item())].cpu().numpy())

    # dense comparator on the same ring (skipped with --dense-steps 0, e.g. for
    # counter runs that must see the sparse step's kernels only)
    dense_ms = None
    if args.dense_steps > 0:
        for i in range(20):
            ring[i % args.ring].dense_ffn_ref(Xd[i % args.tokens], out=Y[i % args.ring])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.dense_steps):
            ring[i % args.ring].dense_ffn_ref(Xd[i % args.tokens], out=Y[i % args.ring])
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_steps

    # exact-mask mode (no predictor, every pre-activation, the true set) on the
    # same ring and tokens, timed like the dense comparator
    exact = None
    if args.dense_steps > 0:
        ne = args.dense_steps
        n_true = torch.zeros(ne, dtype=torch.int32, device=dev)
        act = torch.empty(sh.f, dtype=torch.int32, device=dev)
        for i in range(ne):
            ring[i % args.ring].exact_ffn(Xd[i % args.tokens], out=Y[i % args.ring], active=act,
                                          n_active=n_true[i:i + 1])
        torch.cuda.synchronize()
        k_true = float(n_true.float().mean().item())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(ne):
            ring[i % args.ring].exact_ffn_raw(xs[i % args.tokens], ys[i % args.ring], sh_)
        e1.record()
        torch.cuda.synchronize()
        ex_ms = e0.elapsed_time(e1) / ne
        ws = 2 if sh.wdtype == "f16" else 4
        # every mask row (+ b1), the true set's down columns (and up rows when
        # gated), x, b2, y
        ex_bytes = (sh.f * (sh.d * ws + 4) + k_true * sh.d * ws * (2 if sh.gated else 1)
                    + sh.d * 4 * 3)
        exact = {"ms_per_step": ex_ms, "true_active_mean": k_true,
                 "true_active_frac": k_true / sh.f, "algorithmic_bytes_per_step": ex_bytes,
                 "effective_gbps": ex_bytes / (ex_ms * 1e-3) / 1e9,
                 "effective_frac_of_peak": ex_bytes / (ex_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "speedup_vs_dense": None if dense_ms is None else dense_ms / ex_ms,
                 "byte_ceiling_vs_dense": dense_bytes / ex_bytes}
        log(args, "exact-mask mode: %.1f us per step, true set %.1f%%" % (ex_ms * 1e3,
                                                                        100 * k_true / sh.f))

    # predictor quality on the same tokens: the predicted set against the
    # true set (every pre-activation computed by asf_exact_ffn)
    quality = None
    if args.dense_steps > 0:
        nqt = min(200, args.tokens)
        act_p = torch.empty(sh.f, dtype=torch.int32, device=dev)
        act_t = torch.empty(sh.f, dtype=torch.int32, device=dev)
        n_p = torch.empty(1, dtype=torch.int32, device=dev)
        n_t = torch.empty(1, dtype=torch.int32, device=dev)
        hit = tot_p = tot_t = 0
        for t in range(nqt):
            ring[0].predict(Xd[t], active=act_p, n_active=n_p)
            ring[0].exact_ffn(Xd[t], out=Y[0], active=act_t, n_active=n_t)
            kp, kt_ = int(n_p.item()), int(n_t.item())
            hit += int(torch.isin(act_p[:kp], act_t[:kt_]).sum().item())
            tot_p += kp
            tot_t += kt_
        quality = {"tokens": nqt, "recall": hit / max(tot_t, 1), "precision": hit / max(tot_p, 1),
                   "predicted_frac": tot_p / nqt / sh.f, "true_frac": tot_t / nqt / sh.f}
        log(args, "predictor: recall %.3f precision %.3f" % (quality["recall"],
                                                           quality["precision"]))

    # a plain device-to-device copy of 1 GiB: this box's measured stream rate
    stream_ref = None
    if args.dense_steps > 0:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / 10
        copy_gbs = 2 * src.numel() * 2 / (cms * 1e-3) / 1e9
        stream_ref = {"kind": "device-to-device copy of 1 GiB (read + write bytes)",
                  "gbps": copy_gbs, "frac_of_peak": copy_gbs / HBM_PEAK_GBS}
        del src, dst
        torch.cuda.empty_cache()

    ffn_only = None
    if args.dense_steps > 0 and args.ffn_rhos:
        ffn_only = bench_ffn_only(args, ring, Xd, Y, L, dense_ms, dense_bytes, torch, wl, dev, sh_)

    tok_s = K / elapsed
    eff_gbs = step_bytes * K / elapsed / 1e9
    out = {
        "metric": "sparse-FFN decode tokens/s + effective HBM GB/s (% peak), 4096x16384 fp16",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-weights/f32-accumulate",
        "data": "synthetic (seeded N(0,1) hidden states; random-init weights with a power-law "
                "firing law and a training-free predictor)",
        "config": {"workload": "OPT-6.7B-shaped FFN layer 4096x16384 fp16, predictor "
                               "4096->1024->16384, ~7% active, batch 1",
                   "d_model": sh.d, "d_ffn": sh.f, "pred_hidden": sh.H, "batch": 1,
                   "rho": sh.rho, "ring_layers": args.ring, "tokens": args.tokens},
        "effective_gbps": eff_gbs,
        "effective_frac_of_peak": eff_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": step_bytes,
        "active_mean": k_mean,
        "active_frac": k_mean / sh.f,
        "pred_hidden_nonzero_mean": nz_mean,
        "step_launches": 2 if one_launch else 3,
        "repeats_ms_per_step": rep,
        "median5_ms_per_step": rep[2],
        "median5_tokens_per_s": 1.0 / (rep[2] * 1e-3),
        "median5_effective_frac_of_peak": step_bytes / (rep[2] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "cache_hot": {"kind": "one layer copy, its bytes resident in the 256 MB Infinity Cache",
                      "median5_ms_per_step": hot[2],
                      "effective_gbps": step_bytes / (hot[2] * 1e-3) / 1e9},
        "kernel_ms_median": {KERNELS[j]: float(kmed[j]) for j in used},
        "kernel_ms_sum": kernel_sum_ms,
        "traced_step_span_ms_median": float(np.median(span)),
        "kernel_sum_within_traced_span": within,
        "traced_steps": ns,
        "dense_ms_per_step": dense_ms,
        "dense_gbps": None if dense_ms is None else dense_bytes / (dense_ms * 1e-3) / 1e9,
        "sparse_step_speedup_vs_dense": None if dense_ms is None else dense_ms / ms_per_step,
        "effective_frac_of_stream": None if stream_ref is None else eff_gbs / stream_ref["gbps"],
        "stream_copy": stream_ref,
        "predictor_quality": quality,
        "exact_mask": exact,
        "sparse_ffn_only": ffn_only,
        "roofline": {"bound": "hbm", "kernel": dname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dname),
                     "algorithmic_bytes": per_bytes[dname],
                     "duration_ms_median": float(kmed[dom]), "samples": ns,
                     "frac_counting_all_p2": per_dense_p2[dname] / (kmed[dom] * 1e-3) / 1e9
                                             / HBM_PEAK_GBS,
                     "algorithmic_bytes_all_p2": per_dense_p2[dname]},
    }
    if not args.no_cpu:
        out["cpu_baseline"], out["ambiguous"] = cpu_baseline(args, L, X, gpu_sets)
    del ring, Xd, Y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if args.shards:
        out["shards"] = bench_shards(args, asf, torch, np, wl, dev, stream, L, X)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.layout_steps > 0:
        out["layout"] = bench_layout(args, asf, torch, np, wl, dev, stream)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.gated_steps > 0:
        out["gated"] = bench_gated(args, asf, torch, np, wl, dev, stream)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.stack_tokens > 0:
        out["stack"] = bench_stack(args, asf, torch, np, wl, dev, stream)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.head_calls > 0:
        out["head_predictor"] = bench_heads(args, asf, torch, np, wl, dev, stream)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if args.batches:
        out["batched"] = bench_batched(args, asf, torch, np, wl, dev, stream)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
