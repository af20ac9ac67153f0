#!/usr/bin/env python
"""Benchmark of the ReaDy state-reader path on one AMD Instinct MI355X.

One step = one readyStateReader call over one batch of seeded synthetic
input already resident in HBM (all five steps: gather, state preparation,
projection, query/readout, packing + MLP + residual).

value      committed-state GB/s on the batched workload (B = 64 sequences,
           32 layer-head pairs, bf16 128 x 128 states): (state bytes read +
           gathered bytes written) per step / time per step.  Steps rotate
           over several copies of the inputs so the 256 MB last-level cache
           cannot hold them.
roofline   the dominant (and only) kernel, k_reader: its algorithmic bytes per launch /
           its average duration, timed inside the timed loop with HIP events
           that its own launch records (hipExtLaunchKernelGGL) on the launch
           stream, against 8 TB/s.
b1_latency single-block latency at the paper shape (B = 1), eager and
           graph-replayed, cache-cold and warm, next to an unfused PyTorch
           eager composition of the same five steps.
cpu_baseline  the float64 oracle on a bounded sample of the batched
           workload, on the host with its BLAS on every core this process may
           use (`cores` is the thread count the BLAS reports), with a parity
           check of the GPU outputs on that sample; plus a one-thread run of
           the paper shape (B = 1).
operators  the pages report the gather and the reader as two operators:
           the gather alone (readyGather) and the whole call, cold, at the
           paper and wide shapes, and their difference.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "state-reader µs per 7-token draft block (B=1); committed-state GB/s at B=64"
HBM_PEAK_GBS = 8000.0
# the sources k_reader is compiled from: the kernel and the headers it includes
KERNEL_SRC = [os.path.join(ROOT, "hla_recurrent_state_amd", "csrc", f)
              for f in ("ready_fast.hip", "ready_sync.h", "ready_common.h", "ready_internal.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_reader_batched_pmc.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- HIP events

class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        f = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


# ---------------------------------------------------------------- helpers

def pct(xs, p):
    xs = sorted(xs)
    k = (len(xs) - 1) * p / 100.0
    lo, hi = math.floor(k), math.ceil(k)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def esize(dt):
    return 2 if dt == "bf16" else 4


def algorithmic_bytes(cfg):
    """Bytes the method must move per call (states read at the accepted
    positions only, gathered written, h read, out written, every weight read
    once, accept indices)."""
    s, a, w = esize(cfg.state_dtype), esize(cfg.act_dtype), esize(cfg.weight_dtype)
    M, r, d, F, Hm, B, n = cfg.M, cfg.r, cfg.d, cfg.F, cfg.Hm, cfg.B, cfg.n
    mz = 1 if cfg.shared else M
    committed = 2 * B * M * 128 * 128 * s
    weights = (mz * r * d + 2 * mz * r * 128 + Hm * F + d * Hm) * w
    acts = 2 * B * n * d * a
    return {"committed_state": committed, "weights": weights, "activations": acts,
            "accept_idx": 4 * B, "total": committed + weights + acts + 4 * B}


def reader_kernel_bytes(cfg):
    """Algorithmic bytes of one launch of the bf16 path's single kernel
    (k_reader: all five steps), per unit: each (sequence, pair) tile reads its
    committed 128 x 128 state and writes the copy (2 x 32768 B at bf16); each
    draft position reads h_j and writes out_j (2 x d x 2 B); every weight
    (W_q, U, V, W1, W2) is read once; 4 B per accept index.  This equals the
    whole call's algorithmic bytes.  Intermediates passed between work items
    (z partial sums, P, ell, a) are implementation traffic, not counted."""
    return algorithmic_bytes(cfg)["total"]


def kernel_src_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per k_reader launch from the committed PMC summary, if it was
    taken on the current kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    for line in open(PMC_SUMMARY, encoding="utf-8"):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_src_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- device setup

class Prepared:
    """ctypes argument tuples built once, so the timed loop does no Python
    work beyond the call itself."""

    def __init__(self, R, reader, dev_in, outs, ws, stream):
        st = dev_in["states"].stride()
        self.keep = (dev_in, outs, ws)
        self.sd = R.readyStates(base=dev_in["states"].data_ptr(), stride_b=st[0], stride_p=st[1],
                                stride_l=st[2], stride_h=st[3])
        w = dev_in["weights"]
        self.wd = R.readyWeights(**{k: (w[k].data_ptr() if k in w else None)
                                    for k in ("wq", "u", "v", "h_gamma", "w1", "b1", "w2", "b2")})
        self.od = R.readyOutputs(gathered=outs["gathered"].data_ptr(), out=outs["out"].data_ptr(),
                                 logrms=None, delta=None, feat=None, dev_status=outs["dev_status"].data_ptr())
        self.args = (reader.plan, ctypes.byref(self.sd), dev_in["accept_idx"].data_ptr(),
                     dev_in["h"].data_ptr(), ctypes.byref(self.wd), ctypes.byref(self.od),
                     ws.data_ptr(), ws.numel(), stream)


def device_sets(inp, nsets, device, reader, stream):
    import torch
    from synth.device import to_device, torch_dtype
    import hla_recurrent_state_amd as R
    cfg = inp.cfg
    base = to_device(inp, device)
    sets = []
    for i in range(nsets):
        d = dict(base) if i == 0 else {
            "states": base["states"].clone(), "accept_idx": base["accept_idx"].clone(),
            "h": base["h"].clone(), "weights": base["weights"]}
        outs = {
            "gathered": torch.empty((cfg.B, cfg.M, 128, 128), dtype=torch_dtype(cfg.state_dtype), device=device),
            "out": torch.empty((cfg.B, cfg.n, cfg.d), dtype=torch_dtype(cfg.act_dtype), device=device),
            "dev_status": torch.zeros(1, dtype=torch.int32, device=device),
        }
        ws = reader.new_workspace(device)
        sets.append(Prepared(R, reader, d, outs, ws, stream))
    return sets


# ---------------------------------------------------------------- batched throughput

def run_batched(args, hip, torch, R, synth, seed=0):
    device = torch.device("cuda:0")
    cfg = synth.make_shape("batched")
    t0 = time.time()
    inp = synth.make(cfg, seed=seed)
    log("batched inputs generated in %.1f s" % (time.time() - t0))
    reader = R.StateReader(shape_of(R, cfg), cfg.slots)
    stream = torch.cuda.current_stream(device).cuda_stream
    foot = algorithmic_bytes(cfg)["total"]
    nsets = max(2, int(math.ceil(1.0e9 / foot)))
    sets = device_sets(inp, nsets, device, reader, stream)
    lib = R.load()
    K, W = args.steps, args.warmup
    for i in range(W):
        code = lib.readyStateReader(*sets[i % nsets].args)
        if code != 0:
            raise R.ReadyError(code, "warmup")
    torch.cuda.synchronize(device)
    # timed region: K plain launches back to back on the launch stream, with
    # one HIP event before and one after it on that stream.  The bf16 path is
    # one kernel per call, so (stop - start) / K is that kernel's average launch
    # duration (any gap between launches included).  Events recorded by every
    # launch would add about 5 us per launch, so they are kept out of it.
    start, stop = hip.event(), hip.event()
    hip.record(start, stream)
    t_host = time.perf_counter()
    for i in range(K):
        code = lib.readyStateReader(*sets[i % nsets].args)
        if code != 0:
            raise R.ReadyError(code, "timed")
    hip.record(stop, stream)
    torch.cuda.synchronize(device)
    host_s = time.perf_counter() - t_host
    total_ms = hip.ms(start, stop)
    kern_us = [1000.0 * total_ms / K]
    # per-launch kernel durations (each launch records its own start and end),
    # a separate pass: a cross-check of the average above
    stage_us = stage_breakdown(hip, lib, sets, R, stream, torch, device, reps=min(K, 50))
    for s in sets:
        if int(s.keep[1]["dev_status"].item()) != 0:
            raise RuntimeError("device status set during the batched run")
    result = {"cfg": cfg, "inp": inp, "reader": reader, "set0": sets[0], "nsets": nsets,
              "ms_per_step": total_ms / K, "host_s": host_s, "kern_us": kern_us, "stage_us": stage_us}
    return result


def stage_breakdown(hip, lib, sets, R, stream, torch, device, reps):
    """Median kernel duration of the bf16 path's single kernel (start and end
    recorded by its launch)."""
    n = 2 * R.READY_STAGES
    evs = [[hip.event() for _ in range(n)] for _ in range(reps)]
    for i in range(reps):
        arr = (ctypes.c_void_p * n)(*evs[i])
        code = lib.readyStateReaderProfiled(*sets[i % len(sets)].args, arr)
        if code != 0:
            raise R.ReadyError(code, "stages")
    torch.cuda.synchronize(device)
    out = {"k_reader": round(pct([1000.0 * hip.ms(evs[i][2], evs[i][3]) for i in range(reps)], 50), 2)}
    for row in evs:
        for e in row:
            hip.destroy(e)
    return out


def shape_of(R, cfg, B=None, path="fused"):
    return R.make_shape(B=cfg.B if B is None else B, P=cfg.P, n=cfg.n, L_tot=cfg.L_tot, L_sel=cfg.L_sel,
                        H=cfg.H, r=cfg.r, d=cfg.d, Hm=cfg.Hm, state_dtype=cfg.state_dtype,
                        act_dtype=cfg.act_dtype, weight_dtype=cfg.weight_dtype, act=cfg.act,
                        shared=cfg.shared, state_eps=cfg.state_eps, h_eps=cfg.h_eps, path=path)


# ---------------------------------------------------------------- B = 1 latency

def unfused_torch(dev_in, cfg, gathered, torch):
    """PyTorch eager composition of the five steps (index then copy into the
    execution buffer, casts, pow-mean-rsqrt, matmuls, cat, silu, add): the
    unfused comparator."""
    import torch.nn.functional as Fn
    B, n, M, r, d = cfg.B, cfg.n, cfg.M, cfg.r, cfg.d
    w = dev_in["weights"]
    slots = dev_in["_slots"]
    sel = dev_in["states"][torch.arange(B, device=gathered.device), dev_in["accept_idx"].long()]
    gathered.copy_(sel[:, slots].reshape(B, M, 128, 128))
    Sf = gathered.float()
    rms = (Sf.pow(2).mean(dim=(2, 3), keepdim=True) + cfg.state_eps).sqrt()
    T = torch.matmul(dev_in["_Vt"], Sf / rms)                          # [B][M][r][128]
    hf = dev_in["h"].float()
    hh = hf * torch.rsqrt(hf.pow(2).mean(-1, keepdim=True) + cfg.h_eps)
    z = Fn.linear(hh, dev_in["_Wq2"])                                  # [B][n][M r]
    q = torch.matmul(z.view(B, n, M, 1, r), dev_in["_U"]).squeeze(3)  # [B][n][M][128]
    qt = q.permute(0, 2, 3, 1).contiguous()                           # [B][M][128][n]
    u = torch.matmul(T, qt).permute(0, 3, 1, 2) / math.sqrt(128.0)    # [B][n][M][r]
    ell = torch.log(rms.view(B, 1, M, 1)).expand(B, n, M, 1)
    f = torch.cat([u, ell], dim=-1).reshape(B, n, M * (r + 1))
    a = Fn.silu(Fn.linear(f, dev_in["_W1"]))
    dh = Fn.linear(a, dev_in["_W2"])
    return (hf + dh).to(dev_in["h"].dtype)


def run_b1(args, hip, torch, R, synth, seed=0):
    device = torch.device("cuda:0")
    cfg = synth.make_shape("paper")
    inp = synth.make(cfg, seed=seed)
    reader = R.StateReader(shape_of(R, cfg), cfg.slots)
    stream = torch.cuda.current_stream(device).cuda_stream
    sets = device_sets(inp, 1, device, reader, stream)
    s0 = sets[0]
    lib = R.load()
    K = args.b1_steps
    flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=device)  # 512 MB

    def call():
        code = lib.readyStateReader(*s0.args)
        if code != 0:
            raise R.ReadyError(code, "b1")

    def timed(fn, cold, reps):
        starts = [hip.event() for _ in range(reps)]
        ends = [hip.event() for _ in range(reps)]
        for i in range(reps):
            if cold:
                flush.add_(1.0)
            hip.record(starts[i], stream)
            fn()
            hip.record(ends[i], stream)
        torch.cuda.synchronize(device)
        vals = [1000.0 * hip.ms(starts[i], ends[i]) for i in range(reps)]
        for e in starts + ends:
            hip.destroy(e)
        return vals

    def back_to_back(fn, reps):
        a, b = hip.event(), hip.event()
        for _ in range(5):
            fn()
        torch.cuda.synchronize(device)
        hip.record(a, stream)
        for _ in range(reps):
            fn()
        hip.record(b, stream)
        torch.cuda.synchronize(device)
        return 1000.0 * hip.ms(a, b) / reps

    for _ in range(10):
        call()
    torch.cuda.synchronize(device)
    res = {"stage_us": stage_breakdown(hip, lib, sets, R, stream, torch, device, reps=50)}
    res["fused_eager_cold_us"] = timed(call, True, K)
    res["fused_eager_warm_us"] = back_to_back(call, K)

    # the same call captured into a HIP graph
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device)
    cap.wait_stream(torch.cuda.current_stream(device))
    with torch.cuda.stream(cap):
        gargs = list(s0.args)
        gargs[-1] = cap.cuda_stream
        lib.readyStateReader(*gargs)  # warm the capture stream
        torch.cuda.synchronize(device)
        with torch.cuda.graph(g, stream=cap):
            code = lib.readyStateReader(*gargs)
    if code != 0:
        raise R.ReadyError(code, "capture")
    torch.cuda.current_stream(device).wait_stream(cap)
    torch.cuda.synchronize(device)
    res["fused_graph_cold_us"] = timed(g.replay, True, K)
    res["fused_graph_warm_us"] = back_to_back(g.replay, K)

    # what a graph launch costs by itself on this runtime: a one-element
    # kernel, eager and as a one-node graph, cold like the reader
    tiny = torch.zeros(1, device=device)
    gt = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        tiny.add_(1.0)
        torch.cuda.synchronize(device)
        with torch.cuda.graph(gt, stream=cap):
            tiny.add_(1.0)
    torch.cuda.current_stream(device).wait_stream(cap)
    torch.cuda.synchronize(device)
    res["tiny_kernel_eager_cold_us"] = timed(lambda: tiny.add_(1.0), True, K)
    res["tiny_kernel_graph_cold_us"] = timed(gt.replay, True, K)
    # ten reader calls captured in one graph (as a drafter step would hold
    # them): the per-call cost with the launch overhead paid once
    g10 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g10, stream=cap):
            for _ in range(10):
                code = lib.readyStateReader(*gargs)
                if code != 0:
                    break
    if code != 0:
        raise R.ReadyError(code, "capture of ten calls")
    torch.cuda.current_stream(device).wait_stream(cap)
    torch.cuda.synchronize(device)
    res["fused_graph10_warm_us_per_call"] = [v / 10.0 for v in timed(g10.replay, False, max(K // 10, 10))]

    # the library's unfused path on the same inputs: four launches (query sums;
    # gather, RMS, log-RMS, readout; MLP layer 1; MLP layer 2 and residual)
    ureader = R.StateReader(shape_of(R, cfg, path="unfused"), cfg.slots)
    uouts = {"gathered": torch.empty_like(s0.keep[1]["gathered"]), "out": torch.empty_like(s0.keep[1]["out"]),
             "dev_status": torch.zeros(1, dtype=torch.int32, device=device)}
    uprep = Prepared(R, ureader, s0.keep[0], uouts, ureader.new_workspace(device), stream)

    def ucall():
        code = lib.readyStateReader(*uprep.args)
        if code != 0:
            raise R.ReadyError(code, "b1 unfused")

    for _ in range(10):
        ucall()
    torch.cuda.synchronize(device)
    res["library_unfused_cold_us"] = timed(ucall, True, K)
    res["library_unfused_warm_us"] = back_to_back(ucall, K)

    # unfused PyTorch comparator
    dev_in = dict(s0.keep[0])
    w = dev_in["weights"]
    dev_in["_slots"] = torch.tensor(list(cfg.slots), device=device)
    dev_in["_Vt"] = w["v"].float().transpose(1, 2).contiguous()
    dev_in["_Wq2"] = w["wq"].float().reshape(cfg.M * cfg.r, cfg.d).contiguous()
    dev_in["_U"] = w["u"].float().contiguous()
    dev_in["_W1"] = w["w1"].float().contiguous()
    dev_in["_W2"] = w["w2"].float().contiguous()
    gath2 = torch.empty_like(s0.keep[1]["gathered"])
    ref_out = unfused_torch(dev_in, cfg, gath2, torch)
    torch.cuda.synchronize(device)
    res["unfused_torch_cold_us"] = timed(lambda: unfused_torch(dev_in, cfg, gath2, torch), True, K)
    res["unfused_torch_warm_us"] = back_to_back(lambda: unfused_torch(dev_in, cfg, gath2, torch), K)
    # sanity: the two paths agree
    call()
    torch.cuda.synchronize(device)
    ours = s0.keep[1]["out"].float()
    diff = (ours - ref_out.float()).abs().max().item()
    res["unfused_vs_fused_max_abs_diff"] = diff
    res["gathered_equal"] = bool(torch.equal(gath2.view(torch.int16), s0.keep[1]["gathered"].view(torch.int16)))
    res["library_unfused_vs_fused_max_abs_diff"] = (uouts["out"].float() - ours).abs().max().item()
    res["library_unfused_gathered_equal"] = bool(torch.equal(uouts["gathered"].view(torch.int16),
                                                             s0.keep[1]["gathered"].view(torch.int16)))
    if int(uouts["dev_status"].item()) != 0:
        raise RuntimeError("device status set during the unfused B = 1 run")
    ureader.close()
    res["cfg"] = cfg
    return res


# ---------------------------------------------------------------- step 1 alone

def run_gather(args, hip, torch, R, synth, seed=0):
    """readyGather (step 1 alone: the committed states into the caller's
    buffer) at the paper shape (B = 1, 32 pairs, bf16: 1 MiB read + 1 MiB
    written), the wide shape (B = 1, 96 pairs, fp32: 6 MiB + 6 MiB) and the
    batched shape (B = 64: 64 MiB + 64 MiB), cold (after a 512 MB update) and
    back to back, with the states drawn on the device.  The pages time the
    same operator on their hardware as context."""
    from synth.device import torch_dtype
    device = torch.device("cuda:0")
    stream = torch.cuda.current_stream(device).cuda_stream
    lib = R.load()
    flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=device)
    K = args.config_steps
    res = {}
    for name in ("paper", "wide", "batched"):
        cfg = synth.make_shape(name)
        sdt = torch_dtype(cfg.state_dtype)
        states = torch.empty((cfg.B, cfg.P, cfg.L_tot, cfg.H, 128, 128), dtype=sdt, device=device)
        _fill_states_random(states, seed, torch)
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        acc = torch.randint(0, cfg.P, (cfg.B,), generator=g, device=device, dtype=torch.int32)
        gathered = torch.empty((cfg.B, cfg.M, 128, 128), dtype=sdt, device=device)
        status = torch.zeros(1, dtype=torch.int32, device=device)
        reader = R.StateReader(shape_of(R, cfg), cfg.slots)
        st = states.stride()
        sd = R.readyStates(base=states.data_ptr(), stride_b=st[0], stride_p=st[1], stride_l=st[2], stride_h=st[3])
        gargs = (reader.plan, ctypes.byref(sd), acc.data_ptr(), gathered.data_ptr(), status.data_ptr(), stream)

        def call():
            code = lib.readyGather(*gargs)
            if code != 0:
                raise R.ReadyError(code, "gather")

        for _ in range(5):
            call()
        torch.cuda.synchronize(device)
        cold = []
        for _ in range(K):
            flush.add_(1.0)
            a, b = hip.event(), hip.event()
            hip.record(a, stream)
            call()
            hip.record(b, stream)
            torch.cuda.synchronize(device)
            cold.append(1000.0 * hip.ms(a, b))
            hip.destroy(a)
            hip.destroy(b)
        a, b = hip.event(), hip.event()
        hip.record(a, stream)
        for _ in range(K):
            call()
        hip.record(b, stream)
        torch.cuda.synchronize(device)
        warm = 1000.0 * hip.ms(a, b) / K
        hip.destroy(a)
        hip.destroy(b)
        if int(status.item()) != 0:
            raise RuntimeError("device status set during the gather run")
        nbytes = 2 * cfg.B * cfg.M * 128 * 128 * esize(cfg.state_dtype)
        res[name] = {"B": cfg.B, "M": cfg.M, "state_dtype": cfg.state_dtype, "bytes_read_plus_written": nbytes,
                     "cold_us": {"p10": round(pct(cold, 10), 2), "p50": round(pct(cold, 50), 2),
                                 "p90": round(pct(cold, 90), 2)},
                     "warm_mean_us": round(warm, 2),
                     "warm_GBps": round(nbytes / (warm * 1e-6) / 1e9, 1),
                     "warm_frac_of_hbm_peak": round(nbytes / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        reader.close()
        del states, gathered
    del flush
    torch.cuda.empty_cache()
    res["kernel"] = "k_gather"
    return res


# ---------------------------------------------------------------- other configurations

def _fill_states_random(buf, seed, torch):
    """Seeded standard-normal states scaled by 1/128 (the size of a decayed
    delta-rule state entry), drawn on the device.  Used only to time the
    rank configuration, whose delta-rule generation takes about a minute on
    the host; the kernels' work does not depend on the values."""
    g = torch.Generator(device=buf.device)
    g.manual_seed(seed)
    flat = buf.view(-1)
    step = 1 << 26
    for i in range(0, flat.numel(), step):
        blk = flat[i:i + step]
        blk.copy_(torch.randn(blk.numel(), generator=g, device=buf.device, dtype=torch.float32) / 128.0)


def footprint(cfg):
    """Element counts of the state-access footprint: the committed states,
    M d_v d_k, which do not grow with the prefix, against the key-value cache
    a softmax-attention reader would read at the same prefix length t,
    M t (d_k + d_v) (arXiv text, section 3.2 "State-access footprint")."""
    st = cfg.M * cfg.d_v * cfg.d_k
    kv = cfg.M * cfg.t * (cfg.d_k + cfg.d_v)
    return {"t": cfg.t, "state_elements": st, "kv_cache_elements": kv, "ratio": "1 : %g" % (kv / st)}


def run_config(name, args, hip, torch, R, synth, seed=0, cfg=None, random_states=None, copy_ref=True):
    """Cold (after a 512 MB flush) and back-to-back latency of one call of a
    configuration, its per-stage kernel medians, and a plain device copy that
    moves the same number of bytes (half read, half written)."""
    from synth.device import to_device, torch_dtype
    device = torch.device("cuda:0")
    if cfg is None:
        cfg = synth.make_shape(name)
    if random_states is None:
        random_states = name == "rank"
    t0 = time.time()
    inp = synth.make(cfg, seed=seed, states=not random_states)
    dev_in = to_device(inp, device)
    if random_states:
        shape = (cfg.B, cfg.P, cfg.L_tot, cfg.H, 128, 128)
        dev_in["states"] = torch.empty(shape, dtype=torch_dtype(cfg.state_dtype), device=device)
        _fill_states_random(dev_in["states"], seed, torch)
    log("%s inputs in %.1f s" % (name, time.time() - t0))
    reader = R.StateReader(shape_of(R, cfg), cfg.slots)
    stream = torch.cuda.current_stream(device).cuda_stream
    outs = {
        "gathered": torch.empty((cfg.B, cfg.M, 128, 128), dtype=torch_dtype(cfg.state_dtype), device=device),
        "out": torch.empty((cfg.B, cfg.n, cfg.d), dtype=torch_dtype(cfg.act_dtype), device=device),
        "dev_status": torch.zeros(1, dtype=torch.int32, device=device),
    }
    prep = Prepared(R, reader, dev_in, outs, reader.new_workspace(device), stream)
    lib = R.load()
    K = args.config_steps
    flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=device)

    def call():
        code = lib.readyStateReader(*prep.args)
        if code != 0:
            raise R.ReadyError(code, name)

    def timed(fn, reps):
        starts = [hip.event() for _ in range(reps)]
        ends = [hip.event() for _ in range(reps)]
        for i in range(reps):
            flush.add_(1.0)
            hip.record(starts[i], stream)
            fn()
            hip.record(ends[i], stream)
        torch.cuda.synchronize(device)
        vals = [1000.0 * hip.ms(starts[i], ends[i]) for i in range(reps)]
        for e in starts + ends:
            hip.destroy(e)
        return vals

    def back_to_back(fn, reps):
        a, b = hip.event(), hip.event()
        for _ in range(3):
            fn()
        torch.cuda.synchronize(device)
        hip.record(a, stream)
        for _ in range(reps):
            fn()
        hip.record(b, stream)
        torch.cuda.synchronize(device)
        us = 1000.0 * hip.ms(a, b) / reps
        hip.destroy(a)
        hip.destroy(b)
        return us

    for _ in range(3):
        call()
    torch.cuda.synchronize(device)
    cold = timed(call, K)
    warm = back_to_back(call, K)
    # per-stage kernel durations (events recorded by the launches themselves)
    n = 2 * R.READY_STAGES
    evs = [[hip.event() for _ in range(n)] for _ in range(K)]
    for i in range(K):
        code = lib.readyStateReaderProfiled(*prep.args, (ctypes.c_void_p * n)(*evs[i]))
        if code != 0:
            raise R.ReadyError(code, name + " stages")
    torch.cuda.synchronize(device)
    med = [pct([1000.0 * hip.ms(evs[i][2 * k], evs[i][2 * k + 1]) for i in range(K)], 50)
           for k in range(R.READY_STAGES)]
    # the single-kernel path records the events of stages 0, 2 and 3 after its one
    # kernel (stage 1), so stage 0 "starts" after stage 1 ends; the general path
    # runs stage 0 first
    fast = hip.ms(evs[0][3], evs[0][0]) >= 0.0
    kname = "k_reader_f32" if cfg.state_dtype == "f32" else "k_reader"
    stage_names = (kname,) if fast else ("query_gemm", "state_kernel", "mlp1", "mlp2_residual")
    stage_idx = (1,) if fast else (0, 1, 2, 3)
    stages = {nm: round(med[k], 2) for nm, k in zip(stage_names, stage_idx)}
    for row in evs:
        for e in row:
            hip.destroy(e)
    if int(outs["dev_status"].item()) != 0:
        raise RuntimeError("device status set during the %s run" % name)
    alg = algorithmic_bytes(cfg)["total"]
    if copy_ref:
        # plain copy of the same bytes
        half = alg // 2
        src = torch.empty(half, dtype=torch.uint8, device=device).fill_(1)
        dst = torch.empty_like(src)
        copy_cold = timed(lambda: dst.copy_(src), K)
        copy_warm = back_to_back(lambda: dst.copy_(src), K)
        del src, dst
    del flush
    p50 = pct(cold, 50)
    res = {
        "path": kname + " (single persistent kernel)" if fast else "general (4 kernels)",
        "states": "seeded normal / 128, drawn on the device" if random_states else "fp32 gated delta rule",
        "B": cfg.B, "M": cfg.M, "r": cfg.r, "d": cfg.d, "state_dtype": cfg.state_dtype,
        "algorithmic_bytes": alg,
        "cold_us": {"p10": round(pct(cold, 10), 2), "p50": round(p50, 2), "p90": round(pct(cold, 90), 2)},
        "warm_mean_us": round(warm, 2),
        "cold_GBps": round(alg / (p50 * 1e-6) / 1e9, 1),
        "warm_GBps": round(alg / (warm * 1e-6) / 1e9, 1),
        "cold_frac_of_hbm_peak": round(alg / (p50 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "warm_frac_of_hbm_peak": round(alg / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "stage_median_us": stages,
        "state_vs_kv": footprint(cfg),
    }
    if copy_ref:
        res["same_bytes_copy"] = {"cold_p50_us": round(pct(copy_cold, 50), 2), "warm_mean_us": round(copy_warm, 2),
                                  "warm_GBps": round(2 * half / (copy_warm * 1e-6) / 1e9, 1)}
    del prep, dev_in, outs
    torch.cuda.empty_cache()
    return res


def run_sweeps(args, hip, torch, R, synth):
    """The batched workload's shape with one parameter changed: the reader
    rank (8 .. 128; r <= 32 takes the single-kernel path, larger ranks the
    general path with the matrix-core readout V^T (S_bar q)), and a single
    selected layer (2, 30 or 62: 16 layer-head pairs).  Timing only: the
    states are drawn on the device."""
    out = {"rank": {}, "single_layer": {}}
    for r in (8, 16, 32, 64, 128):
        cfg = synth.make_shape("batched", r=r)
        out["rank"][str(r)] = run_config("batched_r%d" % r, args, hip, torch, R, synth, cfg=cfg,
                                         random_states=True, copy_ref=False)
    for layer in (2, 30, 62):
        cfg = synth.make_shape("batched", layer_ids=(layer,))
        out["single_layer"][str(layer)] = run_config("batched_layer%d" % layer, args, hip, torch, R, synth,
                                                     cfg=cfg, random_states=True, copy_ref=False)
    return out


def run_multi(args, hip, torch, R, synth, seed=0):
    """Several readers sharing one gather at the batched shape (B = 64, 32
    layer-head pairs, r = 8, bf16): readers in draft layers (0, 2, 4) and in
    all five (3 and 5 readers, each with its own weights and h).  Times one
    readyStatePrepare plus one readyStateApply per reader against one
    readyStateReader call per reader (each re-reading the states), cold (after
    a 512 MB flush) and back to back.  Timing only: states, weights and h are
    drawn on the device; parity is in tests/test_gpu_multi.py."""
    device = torch.device("cuda:0")
    cfg = synth.make_shape("batched")
    B, P, n, d, r, Hm, M, F = cfg.B, cfg.P, cfg.n, cfg.d, cfg.r, cfg.Hm, cfg.M, cfg.F
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    bf = torch.bfloat16

    def normal(shape, scale):
        return (torch.randn(shape, generator=g, device=device) * scale).to(bf)

    states = normal((B, P, cfg.L_tot, cfg.H, 128, 128), 1.0 / 128)
    acc = torch.randint(0, P, (B,), generator=g, device=device, dtype=torch.int32)
    reader = R.StateReader(shape_of(R, cfg), cfg.slots)
    stream = torch.cuda.current_stream(device).cuda_stream
    lib = R.load()
    ws = reader.new_workspace(device)
    st = states.stride()
    sd = R.readyStates(base=states.data_ptr(), stride_b=st[0], stride_p=st[1], stride_l=st[2], stride_h=st[3])
    gathered = torch.empty((B, M, 128, 128), dtype=bf, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=device)
    K = args.config_steps
    out = {"workload": "batched shape (B=64, 32 layer-head pairs, r=8, bf16), readers at several draft layers",
           "readers": {}}
    for n_inj in (3, 5):
        keep = []
        wlist, hs, outs = [], [], []
        for i in range(n_inj):
            w = {"wq": normal((M, r, d), d ** -0.5), "u": normal((M, r, 128), r ** -0.5),
                 "v": normal((M, 128, r), 128 ** -0.5), "w1": normal((Hm, F), F ** -0.5),
                 "w2": normal((d, Hm), Hm ** -0.5)}
            wlist.append(w)
            hs.append(normal((B, n, d), 1.0))
            outs.append(torch.empty((B, n, d), dtype=bf, device=device))
        keep += [wlist, hs, outs]
        wd = [R.readyWeights(**{k: (w[k].data_ptr() if k in w else None)
                                for k in ("wq", "u", "v", "h_gamma", "w1", "b1", "w2", "b2")}) for w in wlist]
        od = [R.readyOutputs(gathered=gathered.data_ptr(), out=o.data_ptr(), logrms=None, delta=None, feat=None,
                             dev_status=status.data_ptr()) for o in outs]
        oa = [R.readyOutputs(gathered=None, out=o.data_ptr(), logrms=None, delta=None, feat=None,
                             dev_status=status.data_ptr()) for o in outs]
        warr = (R.readyWeights * n_inj)(*wd)
        prep = reader.new_prep(n_inj, device)
        keep.append(prep)
        single_args = [(reader.plan, ctypes.byref(sd), acc.data_ptr(), hs[i].data_ptr(), ctypes.byref(wd[i]),
                        ctypes.byref(od[i]), ws.data_ptr(), ws.numel(), stream) for i in range(n_inj)]
        prep_args = (reader.plan, ctypes.byref(sd), acc.data_ptr(), n_inj, warr, gathered.data_ptr(), None,
                     status.data_ptr(), prep.data_ptr(), prep.numel(), ws.data_ptr(), ws.numel(), stream)
        apply_args = [(reader.plan, prep.data_ptr(), prep.numel(), n_inj, i, hs[i].data_ptr(), ctypes.byref(wd[i]),
                       ctypes.byref(oa[i]), ws.data_ptr(), ws.numel(), stream) for i in range(n_inj)]

        def check(code, what):
            if code != 0:
                raise R.ReadyError(code, what)

        def singles():
            for a in single_args:
                check(lib.readyStateReader(*a), "single")

        def prepare():
            check(lib.readyStatePrepare(*prep_args), "prepare")

        def applies():
            for a in apply_args:
                check(lib.readyStateApply(*a), "apply")

        def shared():
            prepare()
            applies()

        def timed(fn, cold):
            for _ in range(3):
                fn()
            torch.cuda.synchronize(device)
            if cold:
                vals = []
                for _ in range(K):
                    flush.add_(1.0)
                    a, b = hip.event(), hip.event()
                    hip.record(a, stream)
                    fn()
                    hip.record(b, stream)
                    torch.cuda.synchronize(device)
                    vals.append(1000.0 * hip.ms(a, b))
                    hip.destroy(a)
                    hip.destroy(b)
                return pct(vals, 50)
            a, b = hip.event(), hip.event()
            hip.record(a, stream)
            for _ in range(K):
                fn()
            hip.record(b, stream)
            torch.cuda.synchronize(device)
            us = 1000.0 * hip.ms(a, b) / K
            hip.destroy(a)
            hip.destroy(b)
            return us

        res = {
            "separate_calls_cold_p50_us": round(timed(singles, True), 2),
            "separate_calls_warm_us": round(timed(singles, False), 2),
            "shared_gather_cold_p50_us": round(timed(shared, True), 2),
            "shared_gather_warm_us": round(timed(shared, False), 2),
            "prepare_warm_us": round(timed(prepare, False), 2),
            "apply_warm_us_each": round(timed(applies, False) / n_inj, 2),
        }
        res["speedup_warm"] = round(res["separate_calls_warm_us"] / res["shared_gather_warm_us"], 3)
        if int(status.item()) != 0:
            raise RuntimeError("device status set during the multi-reader run")
        out["readers"][str(n_inj)] = res
        log("multi-reader n=%d: %s" % (n_inj, res))
        del keep
    reader.close()
    del flush
    torch.cuda.empty_cache()
    return out


def run_producer(args, hip, torch, R, synth, seed=0):
    """The verify-state producer at the batched shape (B = 64 sequences,
    32 layer-head pairs, P = 8 positions, bf16 states, keys and values):
    cold and back-to-back time of one call, against its algorithmic bytes
    (S_t, k, v, alpha, beta read once; the P states written once) and a plain
    copy of the same byte count."""
    from synth.device import tensor
    device = torch.device("cuda:0")
    B, P, L, H = 64, 8, 2, 16
    M, steps = L * H, P - 1
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    # timing inputs drawn on the device (the producer's work does not depend on
    # the values); parity is in tests/test_gpu_verify.py
    st = (torch.randn((B, M, 128, 128), generator=g, device=device) / 128).to(torch.bfloat16)
    k = torch.nn.functional.normalize(torch.randn((B, steps, M, 128), generator=g, device=device), dim=-1)
    k = k.to(torch.bfloat16)
    v = torch.randn((B, steps, M, 128), generator=g, device=device).to(torch.bfloat16)
    al = 0.9 + 0.1 * torch.rand((B, steps, M), generator=g, device=device)
    be = torch.rand((B, steps, M), generator=g, device=device)
    out = torch.empty((B, P, L, H, 128, 128), dtype=torch.bfloat16, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    lib = R.load()
    buf = R.readyVerifyBuffer(base=out.data_ptr(), stride_b=out.stride(0), stride_p=out.stride(1),
                              stride_l=out.stride(2), stride_h=out.stride(3))
    cargs = (B, P, L, H, R.READY_BF16, R.READY_BF16, st.data_ptr(), k.data_ptr(), v.data_ptr(), al.data_ptr(),
             be.data_ptr(), ctypes.byref(buf), stream)

    def call():
        code = lib.readyVerifyStates(*cargs)
        if code != 0:
            raise R.ReadyError(code, "producer")

    K = args.config_steps
    flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=device)
    for _ in range(3):
        call()
    torch.cuda.synchronize(device)
    starts = [hip.event() for _ in range(K)]
    ends = [hip.event() for _ in range(K)]
    for i in range(K):
        flush.add_(1.0)
        hip.record(starts[i], stream)
        call()
        hip.record(ends[i], stream)
    torch.cuda.synchronize(device)
    cold = [1000.0 * hip.ms(starts[i], ends[i]) for i in range(K)]
    a, b = hip.event(), hip.event()
    hip.record(a, stream)
    for _ in range(K):
        call()
    hip.record(b, stream)
    torch.cuda.synchronize(device)
    warm = 1000.0 * hip.ms(a, b) / K
    alg = B * M * 128 * 128 * 2 + 2 * B * steps * M * 128 * 2 + 2 * B * steps * M * 4 + B * P * M * 128 * 128 * 2
    half = alg // 2
    src = torch.empty(half, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize(device)
    hip.record(a, stream)
    for _ in range(K):
        dst.copy_(src)
    hip.record(b, stream)
    torch.cuda.synchronize(device)
    copy_warm = 1000.0 * hip.ms(a, b) / K
    for e in starts + ends + [a, b]:
        hip.destroy(e)
    p50 = pct(cold, 50)
    return {
        "workload": "verify-state producer: B=64, 32 layer-head pairs, P=8 positions (7 gated delta rule "
                    "steps), bf16 states, keys and values, fp32 gates",
        "kernel": "k_verify_states",
        "algorithmic_bytes": alg,
        "cold_us": {"p10": round(pct(cold, 10), 2), "p50": round(p50, 2), "p90": round(pct(cold, 90), 2)},
        "warm_mean_us": round(warm, 2),
        "warm_GBps": round(alg / (warm * 1e-6) / 1e9, 1),
        "warm_frac_of_hbm_peak": round(alg / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "same_bytes_copy_warm_us": round(copy_warm, 2),
        "same_bytes_copy_warm_GBps": round(2 * half / (copy_warm * 1e-6) / 1e9, 1),
    }


# ---------------------------------------------------------------- CPU oracle baseline

def _blas_threads():
    """Threads the BLAS under numpy will use, as it reports them (None if
    threadpoolctl cannot tell)."""
    try:
        from threadpoolctl import threadpool_info
    except ImportError:
        return None
    n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    return max(n) if n else None


def _time_oracle(inp, nseq_max, budget_s):
    """Mean time of the oracle over the first nseq sequences, nseq sized so a
    pass takes about budget_s, repeated until budget_s is spent."""
    from tests.gpu_util import oracle_reference
    t0 = time.perf_counter()
    oracle_reference(inp, [0])
    one = time.perf_counter() - t0
    nseq = int(max(1, min(nseq_max, budget_s / max(one, 1e-3))))
    seqs = list(range(nseq))
    t0 = time.perf_counter()
    ref = oracle_reference(inp, seqs)
    el = time.perf_counter() - t0
    reps = 1
    while el < budget_s and reps < 1000:
        t0 = time.perf_counter()
        oracle_reference(inp, seqs)
        el += time.perf_counter() - t0
        reps += 1
    return ref, nseq, reps, el / reps


def cpu_baseline(bat, budget_s, synth):
    """Time the float64 oracle on a bounded sample of the batched workload,
    with the BLAS on every core this process may use, and check the GPU
    outputs of the same sequences against it; then one thread on the paper
    shape (B = 1)."""
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    from tests.gpu_util import compare
    from synth.device import to_numpy_bits
    inp, cfg = bat["inp"], bat["cfg"]
    avail = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=avail) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        threads = _blas_threads()
        ref, nseq, reps, el = _time_oracle(inp, cfg.B, budget_s)
    committed = 2 * nseq * cfg.M * 128 * 128 * esize(cfg.state_dtype)
    # one thread, paper shape
    pinp = synth.make("paper", seed=0)
    ctx1 = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    with ctx1:
        threads1 = _blas_threads()
        _, _, reps1, el1 = _time_oracle(pinp, 1, budget_s / 2)
    # parity of the GPU outputs (set 0) on the sampled sequences
    s0 = bat["set0"]
    outs = s0.keep[1]
    import torch
    dev = outs["out"].device
    extra = {"logrms": torch.empty((cfg.B, cfg.M), dtype=torch.float32, device=dev),
             "delta": torch.empty((cfg.B, cfg.n, cfg.d), dtype=torch.float32, device=dev),
             "feat": torch.empty((cfg.B, cfg.n, cfg.F), dtype=torch.float32, device=dev)}
    d = s0.keep[0]
    bat["reader"](d["states"], d["accept_idx"], d["h"], d["weights"], outs["gathered"], outs["out"],
                  logrms=extra["logrms"], delta=extra["delta"], feat=extra["feat"],
                  dev_status=outs["dev_status"], workspace=s0.keep[2])
    torch.cuda.synchronize(dev)
    res = {"gathered": to_numpy_bits(outs["gathered"], cfg.state_dtype),
           "out": to_numpy_bits(outs["out"], cfg.act_dtype),
           "logrms": extra["logrms"].cpu().numpy(), "delta": extra["delta"].cpu().numpy(),
           "feat": extra["feat"].cpu().numpy(), "dev_status": int(outs["dev_status"].item())}
    rep = compare(inp, res, ref)
    model = ""
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    base = {"value": round(committed / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_cores_available": avail,
            "sample": "float64 numpy oracle, steps 1-5, on %d of the %d sequences of the batched "
                      "workload, BLAS limited to the %d cores of this process's affinity (it reports %s "
                      "threads), %d timed passes of %.2f s each (committed-state bytes of the sample / "
                      "mean time)" % (nseq, cfg.B, avail, threads, reps, el),
            "paper_one_thread": {"us_per_block": round(1e6 * el1, 1), "cores": threads1,
                                 "sample": "the paper shape (B = 1, 32 pairs), one thread, %d timed passes"
                                           % reps1}}
    return base, rep


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--b1-steps", type=int, default=200)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work on the batched sample (half that again at the paper shape)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-b1", action="store_true")
    ap.add_argument("--configs", default="tiny,wide,rank",
                    help="other configurations timed after the headline (comma list, or 'none')")
    ap.add_argument("--config-steps", type=int, default=50)
    ap.add_argument("--no-sweeps", action="store_true", help="skip the rank and single-layer sweeps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (the reference for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the state reader shards by sequence with no "
              "communication, so a multi-GPU figure is not part of this benchmark "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "copies": 10}))
        return
    if not os.path.exists(os.path.join(ROOT, "hla_recurrent_state_amd", "libready.so")):
        import __graft_entry__
        __graft_entry__.build()
    import hla_recurrent_state_amd as R
    import synth
    R.load()
    hip = Hip()

    bat = run_batched(args, hip, torch, R, synth)
    cfg = bat["cfg"]
    alg = algorithmic_bytes(cfg)
    ms = bat["ms_per_step"]
    value = alg["committed_state"] / (ms * 1e-3) / 1e9
    kern_avg_us = sum(bat["kern_us"]) / len(bat["kern_us"])
    kb = reader_kernel_bytes(cfg)
    achieved = kb / (kern_avg_us * 1e-6) / 1e9
    traffic = read_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "batched: B=64 sequences, M=32 layer-head pairs (layers 30, 62 x 16 heads), "
                        "bf16 128x128 states from the fp32 gated delta rule at t=4096, verify buffer of 8 "
                        "positions, block n=7, d=5120, r=8, MLP 288->256->5120 SiLU, bf16 storage with fp32 "
                        "arithmetic",
            "B": cfg.B, "M": cfg.M, "n": cfg.n, "r": cfg.r, "d": cfg.d, "Hm": cfg.Hm,
            "storage": "bf16", "accumulation": "fp32", "input_sets_rotated": bat["nsets"],
            "algorithmic_bytes_per_step": alg["total"],
            "committed_state_bytes_per_step": alg["committed_state"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_reader",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kb,
            "avg_launch_us": round(kern_avg_us, 3),
            "avg_launch_from": "HIP events before and after the timed region of K back-to-back launches",
        },
        "whole_step": {
            "algorithmic_GBps": round(alg["total"] / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_median_us_per_launch_events": bat["stage_us"],
            "host_wall_us_per_step": round(1e6 * bat["host_s"] / args.steps, 2),   # enqueue loop + final sync
        },
    }
    if not args.no_b1:
        b1 = run_b1(args, hip, torch, R, synth)
        pcfg = b1["cfg"]
        pbytes = algorithmic_bytes(pcfg)["total"]
        roof_us = pbytes / (HBM_PEAK_GBS * 1e9) * 1e6

        def summ(v):
            return {"p10": round(pct(v, 10), 2), "p50": round(pct(v, 50), 2), "p90": round(pct(v, 90), 2)}
        best = min(pct(b1["fused_graph_cold_us"], 50), pct(b1["fused_eager_cold_us"], 50))
        out["b1_latency"] = {
            "workload": "paper shape: B=1, M=32 (layers 30, 62 x 16 heads), bf16 states at t=4096, n=7, "
                        "d=5120, r=8, MLP 288->256->5120",
            "unit": "us per 7-token draft block",
            "fused_graph_cold": summ(b1["fused_graph_cold_us"]),
            "fused_eager_cold": summ(b1["fused_eager_cold_us"]),
            "fused_graph_warm_mean": round(b1["fused_graph_warm_us"], 2),
            "fused_eager_warm_mean": round(b1["fused_eager_warm_us"], 2),
            # the graph penalty is the runtime's per-launch cost: the same for a
            # one-element kernel, and paid once for a graph of many calls
            "graph_launch_overhead": {
                "tiny_kernel_eager_cold_p50": round(pct(b1["tiny_kernel_eager_cold_us"], 50), 2),
                "tiny_kernel_graph_cold_p50": round(pct(b1["tiny_kernel_graph_cold_us"], 50), 2),
                "per_graph_launch_us": round(pct(b1["tiny_kernel_graph_cold_us"], 50)
                                             - pct(b1["tiny_kernel_eager_cold_us"], 50), 2),
                "fused_graph_cold_p50_minus_it": round(pct(b1["fused_graph_cold_us"], 50)
                                                       - (pct(b1["tiny_kernel_graph_cold_us"], 50)
                                                          - pct(b1["tiny_kernel_eager_cold_us"], 50)), 2),
            },
            "fused_graph10_warm_per_call": summ(b1["fused_graph10_warm_us_per_call"]),
            "library_unfused_cold": summ(b1["library_unfused_cold_us"]),
            "library_unfused_warm_mean": round(b1["library_unfused_warm_us"], 2),
            "unfused_torch_cold": summ(b1["unfused_torch_cold_us"]),
            "unfused_torch_warm_mean": round(b1["unfused_torch_warm_us"], 2),
            "algorithmic_bytes": pbytes,
            "hbm_roofline_us": round(roof_us, 3),
            "frac_of_hbm_roofline": round(roof_us / best, 4),   # against the faster cold path
            "stage_median_us": b1["stage_us"],
            "unfused_vs_fused_max_abs_diff": b1["unfused_vs_fused_max_abs_diff"],
            "unfused_gathered_equal": b1["gathered_equal"],
            "library_unfused_vs_fused_max_abs_diff": b1["library_unfused_vs_fused_max_abs_diff"],
            "library_unfused_gathered_equal": b1["library_unfused_gathered_equal"],
        }
    if not args.no_b1:
        out["gather_only"] = run_gather(args, hip, torch, R, synth)
    if args.configs and args.configs != "none":
        out["configs"] = {}
        for name in args.configs.split(","):
            out["configs"][name] = run_config(name, args, hip, torch, R, synth)
    # the pages' two operators (arXiv text, section 3.2, Fig. 4): the gather
    # alone and the reader; the fused call has no separate gather, so the
    # reader's own share is reported as the difference of the two cold medians
    if "gather_only" in out:
        ops = {}
        whole = {}
        if "b1_latency" in out:
            whole["paper"] = out["b1_latency"]["fused_eager_cold"]["p50"]
        if "configs" in out and "wide" in out["configs"]:
            whole["wide"] = out["configs"]["wide"]["cold_us"]["p50"]
        for name, w in whole.items():
            g = out["gather_only"][name]["cold_us"]["p50"]
            ops[name] = {"gather_cold_p50_us": g, "reader_call_cold_p50_us": w,
                         "reader_minus_gather_cold_p50_us": round(w - g, 2)}
        out["operators"] = ops
    if not args.no_sweeps:
        out["sweeps"] = run_sweeps(args, hip, torch, R, synth)
        out["producer"] = run_producer(args, hip, torch, R, synth)
        out["multi_reader"] = run_multi(args, hip, torch, R, synth)
    ok = True
    if not args.no_cpu:
        base, rep = cpu_baseline(bat, args.cpu_budget, synth)
        out["cpu_baseline"] = base
        out["parity"] = {k: rep[k] for k in ("gather_bitexact", "dh_rel", "logrms_err", "feat_rel", "ok")}
        ok = rep["ok"]
    print(json.dumps(out))
    sys.stdout.flush()
    if not ok:
        print("PARITY FAILED", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
