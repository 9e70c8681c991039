"""Benchmark of the layer-streamed training step on one MI355X.

Workload: a 7B-shaped decoder (28 layers, d_model 3584, 28 query / 4 KV heads
of 128, SwiGLU ffn 18944, vocab 152064, untied embeddings), batch 8 x seq
1024 of seeded uniform token ids, weights N(0, 0.02^2) in bf16 from seed 1234,
host store of 16 bytes per parameter.  One step = streamed forward of every
layer, the fused LM head, recompute + backward of every layer with gradient
offload, and the host Adam over all 7.6B parameters.  Defaults: cross-step
pipelining (the next forward overlaps this step's host Adam; the timed region
ends with a sync, so every step's update is timed), the weight regions in one
page-locked block, layer-sized LM-head chunks, two weight slots, 16 gradient
slabs.

Prints ONE JSON line on stdout (progress goes to stderr):
  value            whole-step training tokens/s (inputs resident on the host
                   store and in pinned memory, as the step consumes them)
  roofline         the dominant kernel (fused gate|up GEMM, bf16 MFMA):
                   algorithmic FLOPs per launch / mean launch time, timed live
                   with HIP events on the compute stream over the timed steps
  cpu_baseline     the CPU oracle on the host cores, on a bounded sample of the
                   same workload, extrapolated to a full step
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "training tokens/sec + MFMA util & PCIe H2D/D2H GB/s overlap, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PCIE_GEN5_X16_GBS = 64.0

SHAPES = {
    "7b": dict(n_layers=28, d_model=3584, n_heads=28, n_kv_heads=4, head_dim=128, ffn_dim=18944, vocab=152064,
               batch=8, seq=1024,
               workload="7B-shaped decoder, 28 layers, d_model 3584, 28q/4kv heads x 128, ffn 18944, "
                        "vocab 152064, batch 8 x seq 1024, layer-streamed train step with host Adam"),
    "tiny": dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=688, vocab=1024,
                 batch=2, seq=128,
                 workload="tiny decoder, 2 layers, d_model 256, 4 heads x 64, ffn 688, vocab 1024, "
                          "batch 2 x seq 128"),
    "long": dict(n_layers=8, d_model=3584, n_heads=28, n_kv_heads=4, head_dim=128, ffn_dim=18944, vocab=152064,
                 batch=1, seq=131072,
                 workload="long-context step: 8 layers of the 7B-shaped layer, batch 1 x seq 131072, causal, "
                          "layer-streamed with host Adam"),
    "14b": dict(n_layers=48, d_model=5120, n_heads=40, n_kv_heads=8, head_dim=128, ffn_dim=13824, vocab=152064,
                batch=4, seq=2048,
                workload="14B-shaped decoder, 48 layers, d_model 5120, 40q/8kv heads x 128, ffn 13824, "
                         "vocab 152064, batch 4 x seq 2048, layer-streamed train step with host Adam"),
    "70b": dict(n_layers=4, d_model=8192, n_heads=64, n_kv_heads=8, head_dim=128, ffn_dim=28672, vocab=128256,
                batch=4, seq=2048,
                workload="70B-layer-shaped decoder, {L} layers, d_model 8192, 64q/8kv heads x 128, ffn 28672, "
                         "vocab 128256, batch 4 x seq 2048, layer-streamed train step with host Adam"),
}
SHAPES["70b_x4"] = SHAPES["70b"]


# HBM bytes per launch of the dominant kernel (the gate|up GEMM at the 7B
# shape) from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE), each scaled
# by the same counter's reading for a 1 GiB device copy; see
# profiles/gemm_gateup_traffic_7b.md.  Valid only for the kernel sources it was
# taken on (sha256 over the files in order): reported as null once they change.
TRAFFIC = {"sources": ["layer_streaming_amd/csrc/gemm_nt.hip", "layer_streaming_amd/csrc/kcommon.h"],
           "sha256": "7c18c8380f7c45fd6c1f40a83faf45f0015b07065f770a66f9d42c36614b6017",
           "fetch_bytes": 3317900536, "write_bytes": 620756992}


def traffic_bytes(config):
    """Measured HBM bytes per gate|up launch: only for the shape and the
    kernel sources the counters were taken on."""
    import hashlib
    if config != "7b":
        return None
    h = hashlib.sha256()
    try:
        for src in TRAFFIC["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    if h.hexdigest() != TRAFFIC["sha256"]:
        return None
    return TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(cfg, T):
    """Algorithmic FLOPs of every GEMM site per launch (2*M*N*K)."""
    d, F, V = cfg["d_model"], cfg["ffn_dim"], cfg["vocab"]
    nq = cfg["n_heads"] * cfg["head_dim"]
    nqkv = (cfg["n_heads"] + 2 * cfg["n_kv_heads"]) * cfg["head_dim"]
    f = {
        "gemm_qkv": 2 * T * nqkv * d, "gemm_o": 2 * T * d * nq, "gemm_gateup": 2 * T * 2 * F * d,
        "gemm_down": 2 * T * d * F,
        "gemm_down_dx": 2 * T * F * d, "gemm_down_dw": 2 * d * F * T,
        "gemm_gateup_dx": 2 * T * d * 2 * F, "gemm_gateup_dw": 2 * 2 * F * d * T,
        "gemm_o_dx": 2 * T * nq * d, "gemm_o_dw": 2 * d * nq * T,
        "gemm_qkv_dx": 2 * T * d * nqkv, "gemm_qkv_dw": 2 * nqkv * d * T,
    }
    return f


def head_gemm_flops(cfg, T):
    """The LM head's three products over all token chunks (one launch each per chunk)."""
    return 2 * T * cfg["vocab"] * cfg["d_model"]


def hbm_bytes(cfg, T):
    """Algorithmic HBM bytes per launch of the bandwidth-bound kernel sites."""
    d, F = cfg["d_model"], cfg["ffn_dim"]
    nqkv = (cfg["n_heads"] + 2 * cfg["n_kv_heads"]) * cfg["head_dim"]
    return {
        "rms1_fwd": T * d * 2 + 2 * T * d * 2 + T * 4,     # x in; n (bf16) and n (fp16) out; rstd
        "rms2_fwd": T * d * 4 + T * d * 2 + T * 4,         # fp32 h1 in; n2 out; rstd
        "rope_fwd": T * nqkv * 4 + T * nqkv * 2,           # fp32 projection in; q, k, v fp16 out
        "swiglu_fwd": T * 2 * F * 2 + T * F * 2,           # gate|up in; m out
        "swiglu_bwd": T * F * 2 + T * 2 * F * 2 + T * 2 * F * 2,  # dm, gate|up in; dgate|dup out
        "rms1_bwd": 4 * T * d * 2 + T * 4,                # dn, x, residual in; dx out; rstd
        "rms2_bwd": T * d * 2 + T * d * 4 + 2 * T * d * 2 + T * 4,  # dn, fp32 h1, residual in; dh1 out
    }


def host_bytes_per_step(cfg, T, n_micro=1, pinned=False, keep_grads=True):
    """Host DRAM bytes one step moves.  Per micro-batch: for the forward and
    the backward visit of every streamed unit, the DMA read of its weights,
    preceded, unless the W regions are pinned (pin_weights), by the pack (read
    W, streaming write to staging); the DMA write of every streamed unit's
    gradient, the checkpoint ring out and back in, and the embedding rows.
    Per optimizer step and parameter: Adam's 30 B with one micro-batch (read
    the slab, master, m, v; write master, m, v, W and the copy into G), 28 B
    when the store does not keep gradients (keep_grads = 0: no G copy); with
    n > 1 the first stores the slab into G (4 B), each middle one adds into G
    (6 B), the last adds and runs Adam (34 B)."""
    L, d, F, V = cfg["n_layers"], cfg["d_model"], cfg["ffn_dim"], cfg["vocab"]
    hq, hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    p_layer = d * hq * hd + 2 * d * hkv * hd + hq * hd * d + 3 * d * F + 2 * d
    streamed = L * p_layer + V * d + d
    p_embed = V * d
    per_param = (30 if keep_grads else 28) if n_micro == 1 else 4 + 6 * (n_micro - 2) + 34
    visit = 2 if pinned else 4 + 2
    per_micro = 2 * visit * streamed + 2 * streamed + 2 * L * T * d * 2 + 2 * T * d * 2
    return per_param * (streamed + p_embed) + n_micro * per_micro


def model_flops_per_step(cfg, T, S):
    """6 * params * tokens for the matmuls plus causal attention (fwd 2 matmuls
    of 2*S/2*hd per query-head on average, x3 for fwd+bwd); recompute excluded."""
    L, d, F, V = cfg["n_layers"], cfg["d_model"], cfg["ffn_dim"], cfg["vocab"]
    hq, hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    p_lin = d * hq * hd + 2 * d * hkv * hd + hq * hd * d + 3 * d * F
    attn_fwd = 2 * 2 * T * hq * hd * (S + 1) / 2
    return 6 * p_lin * L * T + 6 * T * d * V + 3 * attn_fwd * L


def pages_flops_per_step(cfg, T, S):
    """The pages' throughput convention, for comparability only: 6 N T over
    all N parameters (embeddings included) plus 12 L Hq hd S T for the
    attention scores and values (non-causal, forward and backward)."""
    L, d, F, V = cfg["n_layers"], cfg["d_model"], cfg["ffn_dim"], cfg["vocab"]
    hq, hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    n_total = L * (d * hq * hd + 2 * d * hkv * hd + hq * hd * d + 3 * d * F + 2 * d) + 2 * V * d + d
    return 6 * n_total * T + 12 * L * hq * hd * S * T


def host_mem_available():
    """MemAvailable of /proc/meminfo in bytes (None when unreadable)."""
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return None


def host_info():
    """CPU model, sockets, cores, threads and NUMA layout (lscpu), and the
    CPUs this process may run on."""
    import subprocess
    info = {"cpus_usable": len(os.sched_getaffinity(0))}
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        keys = {"Model name": "model", "Socket(s)": "sockets", "Core(s) per socket": "cores_per_socket",
                "Thread(s) per core": "threads_per_core", "NUMA node(s)": "numa_nodes", "CPU(s)": "cpus"}
        for line in r.stdout.splitlines():
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k in keys:
                info[keys[k]] = int(v) if v.isdigit() else v
            elif k.startswith("NUMA node") and k.endswith("CPU(s)"):
                info.setdefault("numa_cpus", {})[k.split()[1]] = v
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def traffic_probe(torch, mt, cfg):
    """The dominant GEMM (gate|up, NT, bf16, random operands) three times,
    then a 1 GiB fill and three 1 GiB device copies as the counters'
    yardstick of known size."""
    M, N, K = cfg["batch"] * cfg["seq"], 2 * cfg["ffn_dim"], cfg["d_model"]
    g = torch.Generator(device="cpu").manual_seed(0)
    A = torch.randn(M, K, generator=g).to("cuda", torch.bfloat16)
    B = torch.randn(N, K, generator=g).to("cuda", torch.bfloat16)
    C = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        mt.check(mt.lib.mt_k_gemm(0, 0, A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N, None, 0, None, 0,
                                  M, N, K, s), "gemm")
    x = torch.ones(1 << 29, device="cuda", dtype=torch.int16)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    log("traffic probe done")


def attention_probe(torch, mt, cfg, S, B=1, dq_form=0):
    """The attention kernels alone at B sequences of length S with the
    workload's heads: forward and backward three times each on seeded
    synthetic q, k, v (fp16) and dO (bf16); HIP-event times and TFLOP/s
    (causal: 4 B Hq hd S(S+1)/2 for the
    forward, 2.5 times that for the backward)."""
    Hq, Hkv, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    ld, nq = (Hq + 2 * Hkv) * hd, Hq * hd
    T = B * S
    g = torch.Generator(device="cpu").manual_seed(0)
    qkv = torch.randn(T, ld, generator=g).to(torch.float16).cuda().view(torch.int16)
    do = torch.randn(T, nq, generator=g).to(torch.bfloat16).cuda().view(torch.int16)
    o = torch.zeros(T, nq, dtype=torch.int16, device="cuda")
    lse = torch.zeros(Hq * T, device="cuda")
    work = torch.zeros(int(mt.lib.mt_k_attn_bwd_work_bytes(B, S, Hq, Hkv, hd)), dtype=torch.uint8, device="cuda")
    dqkv = torch.zeros(T, ld, dtype=torch.int16, device="cuda")
    tab = torch.zeros(S * hd, dtype=torch.float32, device="cuda")
    base = [10000.0]   # the first call computes the RoPE table, later ones reuse it
    st = torch.cuda.current_stream()
    s = st.cuda_stream

    def fwd():
        mt.check(mt.lib.mt_k_attn_fwd(qkv.data_ptr(), ld, o.data_ptr(), nq, lse.data_ptr(), B, S, Hq, Hkv, hd, None, s),
                 "attn_fwd")

    def bwd():
        # as the step runs it: dQ and dK rotated back where they are finished
        # (bf16 out), and, after the first (untimed) call, the maxima of |dO|
        # and |v| already in the scratch, as the step's O dX product and
        # rotation leave them (no maxima pass)
        mt.check(mt.lib.mt_k_attn_bwd_rope(qkv.data_ptr(), ld, o.data_ptr(), do.data_ptr(), nq, lse.data_ptr(),
                                           work.data_ptr(), dqkv.data_ptr(), ld, B, S, Hq, Hkv, hd, None, 0, 0,
                                           dq_form, None, tab.data_ptr(), base[0], 0 if base[0] else 1, s),
                 "attn_bwd")
        base[0] = 0.0
    fl = 4.0 * B * Hq * hd * S * (S + 1) / 2
    out = {}
    for name, fn, f in (("fwd", fwd, fl), ("bwd", bwd, 2.5 * fl)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(3):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        out[name] = {"ms": round(ms, 3), "tflops": round(f / (ms / 1e3) / 1e12, 1)}
        log(f"attention {name} B={B} S={S}: {ms:.2f} ms, {f / ms / 1e9:.0f} TFLOP/s")
    print(json.dumps({"attention_probe": {"B": B, "S": S, "heads": [Hq, Hkv, hd], **out}}), flush=True)


def ablations(torch, mt, shape, cfg, args, tokens, labels, base_value):
    """The cheap ablations: the same workload with one weight slot (no
    prefetch), one gradient slab, and W and G sharing combined slots."""
    from layer_streaming_amd import synth
    B, S = cfg["batch"], cfg["seq"]
    res = {}
    for name, kw in (("one_weight_slot", dict(n_weight_slots=1)), ("one_grad_slab", dict(n_grad_slabs=1)),
                     ("combined_slots", dict(slot_mode=1))):
        base = dict(host_threads=args.host_threads, seed=synth.SEED_WEIGHTS, cross_step=args.cross_step,
                    pin_weights=args.pin_weights, head_vocab_chunk=args.head_vocab_chunk, n_grad_slabs=args.slabs)
        base.update(kw)
        opt = mt.default_options(max_batch=B, max_seq=S, **base)
        arena_bytes, _, _ = mt.workspace_bytes(shape, opt)
        arena = torch.empty(arena_bytes, dtype=torch.uint8, device="cuda")
        ctx = mt.Context(shape, opt, arena.data_ptr(), arena_bytes, [st.cuda_stream for st in bench_streams(torch)])
        ctx.train_step(tokens, labels)
        ctx.sync()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(2):
            ctx.train_step(tokens, labels)
        ctx.sync()
        torch.cuda.synchronize()
        v = 2 * B * S / (time.perf_counter() - t0)
        res[name] = {"value": round(v, 1), "vs_default": round(v / base_value, 3)}
        log(f"ablation {name}: {v:.0f} tokens/s ({v / base_value:.3f} of the default)")
        ctx.close()
        del arena
        torch.cuda.empty_cache()
    return res


def host_adam_probe(mt, n=256 << 20):
    """Host DRAM rate the library's Adam reaches on its own (all threads,
    30 B/param), the yardstick for the step's host traffic."""
    w = np.zeros(n, np.uint16)
    g = np.zeros(n, np.uint16)
    gs = np.full(n, 0x3A83, np.uint16)
    ms, m, v = np.ones(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    best = 1e9
    for _ in range(3):
        t0 = time.perf_counter()
        mt.check(mt.lib.mt_host_adam(w.ctypes.data, g.ctypes.data, ms.ctypes.data, m.ctypes.data, v.ctypes.data,
                                     gs.ctypes.data, n, 1, 1e-4, 0.9, 0.999, 1e-8, min(16, os.cpu_count() or 1)),
                 "mt_host_adam")
        best = min(best, time.perf_counter() - t0)
    return round(30 * n / best / 1e9, 1)


def pcie_probe(torch, nbytes=512 << 20):
    """Pinned host <-> device copy rates on their own (best of 5, HIP events
    on a side stream): the yardstick for the step's H2D and D2H rates."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()
    out = {}
    for name, fn in (("h2d", lambda: d.copy_(h, non_blocking=True)), ("d2h", lambda: h.copy_(d, non_blocking=True))):
        best = 1e9
        with torch.cuda.stream(st):
            fn()
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                fn()
                e1.record(st)
                e1.synchronize()
                best = min(best, e0.elapsed_time(e1))
        out[name] = round(nbytes / (best / 1e3) / 1e9, 1)
    del h, d
    return out


def host_probe(mt):
    """The host's DRAM against the host Adam: the library's Adam alone at 8,
    12 and 16 threads (30 B/param), and a parallel copy and a parallel read
    of 8 GB at 8 and 16 threads, as one JSON line."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor
    out = {"cpus": len(os.sched_getaffinity(0)), "adam_GBps": {}, "copy_GBps": {}, "read_GBps": {}}
    n = 512 << 20
    w, g = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    gs = np.full(n, 0x3A83, np.uint16)
    ms, m, v = np.ones(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for th in (8, 12, 16):
        best = 1e9
        for _ in range(3):
            t0 = time.perf_counter()
            mt.check(mt.lib.mt_host_adam(w.ctypes.data, g.ctypes.data, ms.ctypes.data, m.ctypes.data,
                                         v.ctypes.data, gs.ctypes.data, n, 1, 1e-4, 0.9, 0.999, 1e-8, th),
                     "mt_host_adam")
            best = min(best, time.perf_counter() - t0)
        out["adam_GBps"][th] = round(30 * n / best / 1e9, 1)
        log(f"host Adam, {th} threads: {out['adam_GBps'][th]} GB/s")
    del w, g, gs, ms, m, v
    nb = 8 << 30
    src, dst = np.ones(nb, np.uint8), np.zeros(nb, np.uint8)
    for th in (8, 16):
        ch = nb // th

        def cp(i):
            ctypes.memmove(dst.ctypes.data + i * ch, src.ctypes.data + i * ch, ch)

        def rd(i):
            return int(src[i * ch:(i + 1) * ch].view(np.uint64).sum())
        with ThreadPoolExecutor(th) as ex:
            list(ex.map(cp, range(th)))
            for name, fn, mult in (("copy_GBps", cp, 2), ("read_GBps", rd, 1)):
                best = 1e9
                for _ in range(3):
                    t0 = time.perf_counter()
                    list(ex.map(fn, range(th)))
                    best = min(best, time.perf_counter() - t0)
                out[name][th] = round(mult * nb / best / 1e9, 1)
        log(f"copy (read + write) and read, {th} threads: {out['copy_GBps'][th]}, {out['read_GBps'][th]} GB/s")
    print(json.dumps({"host_probe": out}), flush=True)


def cpu_baseline(ctx, cfg, mt):
    """Time the oracle (float64 numpy, all host cores) on a bounded sample:
    one decoder layer (forward, recompute, backward) and the LM head at
    B=1 x S=1024 tokens of the workload's shapes, and Adam over a 16M-element
    slice; extrapolate to the full step (L layers, head, Adam over all
    parameters) in the metric's unit.  For sequences longer than 4096 the
    layer's attention terms grow with S^2: the layer is timed at S = 1024 and
    2048 and t(S) = a S + b S^2 is fitted through the two points and
    evaluated at the workload's length."""
    from oracle import step as ostep
    from layer_streaming_amd import synth
    sh = ostep.Shape(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                     cfg["ffn_dim"], cfg["vocab"])
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = {n: widen(ctx.get_tensor(0, j, mt.MT_W)) for j, n in enumerate(ostep.LAYER_TENSORS)}
    L = cfg["n_layers"]
    hw = {n: widen(ctx.get_tensor(L, j, mt.MT_W)) for j, n in enumerate(ostep.HEAD_TENSORS)}
    rng = np.random.default_rng(0)

    def time_layer(Ss):
        x = rng.standard_normal((Ss, sh.d_model)) * 0.02
        dy = rng.standard_normal((Ss, sh.d_model)) * 1e-4
        t0 = time.perf_counter()
        ostep.layer_fwd(x, w, sh, 1, Ss)                     # forward
        _, c = ostep.layer_fwd(x, w, sh, 1, Ss)              # recompute
        ostep.layer_bwd(dy, c, w, sh, 1, Ss)                 # backward
        t = time.perf_counter() - t0
        log(f"cpu oracle: layer fwd+recompute+bwd at 1x{Ss}: {t:.2f} s")
        return t

    B, S = cfg["batch"], cfg["seq"]
    T = B * S
    cores = len(os.sched_getaffinity(0))
    if sh.n_params() < 100_000_000:
        # a small model: the oracle's whole streamed step (gradients, BF16
        # rounding, Adam over every tensor) on the workload's batch, median of 3
        def unit(u, names):
            return {n: {"w": widen(ctx.get_tensor(u, j, mt.MT_W)).astype(np.float32),
                        "master": ctx.get_tensor(u, j, mt.MT_MASTER).copy(),
                        "m": ctx.get_tensor(u, j, mt.MT_M).copy(), "v": ctx.get_tensor(u, j, mt.MT_V).copy()}
                    for j, n in enumerate(names)}
        store = {"layers": [unit(i, ostep.LAYER_TENSORS) for i in range(L)], "head": unit(L, ostep.HEAD_TENSORS),
                 "e_in": unit(L + 1, ("e_in",))}
        tokens, labels = synth.tokens_labels(synth.SEED_TOKENS, B, S, sh.vocab)
        ts = []
        for k in range(3):
            t0 = time.perf_counter()
            ostep.train_step(store, tokens, labels, sh, k + 1)
            ts.append(time.perf_counter() - t0)
        t_step = sorted(ts)[1]
        log(f"cpu oracle: full step at {B}x{S}: {t_step:.3f} s (median of 3)")
        return {"value": T / t_step, "unit": "tokens/s", "cores": cores, "kind": "oracle", "host": host_info(),
                "sample": f"float64 numpy oracle: the whole streamed step at {B}x{S} (gradients, BF16 rounding, "
                          f"Adam over every tensor), measured, median of 3 ({t_step:.3f} s per step)"}
    Sh = min(1024, S)
    if S > 4096:
        (S1, t1), (S2, t2) = [(s_, time_layer(s_)) for s_ in (1024, 2048)]
        b = (t2 / S2 - t1 / S1) / (S2 - S1)
        a = t1 / S1 - b * S1
        t_layers = L * B * (a * S + b * S * S)
        how = (f"one decoder layer (fwd, recompute, bwd) at 1x1024 and 1x2048 tokens, fitted as a*S + b*S^2 "
               f"(a = {a:.3e} s, b = {b:.3e} s) and evaluated at S = {S}; the LM head at 1x{Sh} tokens scaled to "
               f"{T}")
    else:
        t_layers = L * time_layer(Sh) * (T / Sh)
        how = f"one decoder layer (fwd, recompute, bwd) and the LM head at 1x{Sh} tokens, scaled to {T} tokens"
    x = rng.standard_normal((Sh, sh.d_model)) * 0.02
    _, labels = synth.tokens_labels(synth.SEED_TOKENS, 1, Sh, sh.vocab)
    t0 = time.perf_counter()
    ostep.head_fwd_bwd(x, hw, labels.reshape(-1), sh)
    t_head = time.perf_counter() - t0
    log(f"cpu oracle: head fwd+bwd at T={Sh}: {t_head:.2f} s")
    n = 1 << 24
    st = [rng.standard_normal(n).astype(np.float32) for _ in range(4)]
    t0 = time.perf_counter()
    ostep.adam_update(st[0], st[1], np.abs(st[2]), st[3], 1, 1e-4, 0.9, 0.999, 1e-8)
    t_adam = (time.perf_counter() - t0) * sh.n_params() / n
    log(f"cpu oracle: Adam over {sh.n_params() / 1e9:.2f}B params (from a {n} sample): {t_adam:.2f} s")
    t_step = t_layers + t_head * (T / Sh) + t_adam
    return {"value": T / t_step, "unit": "tokens/s", "cores": cores, "kind": "oracle", "host": host_info(),
            "sample": f"float64 numpy oracle: {how}; Adam over a 16M-element slice scaled to all parameters; "
                      f"step extrapolated as L layers + head + Adam ({t_step:.1f} s per step)"}


def step_batches(cfg, n_micro, k):
    """Seeded token ids of timed or warm-up step k: a fresh batch every step
    (the attention forward's rescaling depends on the data)."""
    from layer_streaming_amd import synth
    B, S = cfg["batch"], cfg["seq"]
    tl = [synth.tokens_labels(synth.SEED_TOKENS + 1000 * k + j, B, S, cfg["vocab"]) for j in range(n_micro)]
    if n_micro == 1:
        return tl[0]
    return np.stack([t for t, _ in tl]), np.stack([lb for _, lb in tl])


_STREAMS = []


def bench_streams(torch):
    """The three streams (compute, weight H2D, gradient D2H) every context of
    this process runs on, created once: the runtime maps streams onto a few
    hardware queues in creation order, and two of the three sharing a queue
    would serialize compute and copies (seen as an overlap ratio near zero on
    the second context of a process that created fresh streams for it)."""
    if not _STREAMS:
        _STREAMS.extend(torch.cuda.Stream() for _ in range(3))
    return _STREAMS


def run_workload(torch, mt, cfg, args, opt_kw, steps, warmup, keep=False):
    """One context on the workload: init, warm-up steps, timed steps (fresh
    tokens each), closing sync inside the timed region.  Refuses, before
    allocating anything, when the host store and pinned memory would not fit
    the host's available memory.  Returns (result dict, ctx, arena); the
    context is closed unless keep."""
    from layer_streaming_amd import synth
    B, S = cfg["batch"], cfg["seq"]
    T = B * S
    nm = args.micro
    shape = mt.make_shape(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                          cfg["ffn_dim"], cfg["vocab"])
    opt = mt.default_options(max_batch=B, max_seq=S, seed=synth.SEED_WEIGHTS, **opt_kw)
    arena_bytes, pinned_bytes, store_bytes = mt.workspace_bytes(shape, opt)
    # resident host bytes: the store (its W regions stay untouched when they
    # live in the pinned block), the pinned memory, the fp32 embedding
    # scatter accumulator, 8 GB for the process itself
    w_bytes = 2 * (store_bytes // 16)
    need = store_bytes - (w_bytes if opt_kw.get("pin_weights") else 0) + pinned_bytes + \
        4 * cfg["vocab"] * cfg["d_model"] + (8 << 30)
    avail = host_mem_available()
    log(f"[{cfg['n_layers']} layers] arena {arena_bytes / 1e9:.2f} GB, pinned {pinned_bytes / 1e9:.2f} GB, "
        f"store {store_bytes / 1e9:.2f} GB; host needs ~{need / 1e9:.1f} GB, available "
        f"{avail / 1e9 if avail else float('nan'):.1f} GB")
    if avail is not None and need > avail:
        return {"refused": "host memory", "need_bytes": int(need), "available_bytes": int(avail)}, None, None
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    arena = torch.empty(arena_bytes, dtype=torch.uint8, device="cuda")
    streams = bench_streams(torch)
    t0 = time.time()
    ctx = mt.Context(shape, opt, arena.data_ptr(), arena_bytes,
                     (None, None, None) if args.own_streams else [s.cuda_stream for s in streams])
    torch.cuda.synchronize()
    mem_delta = int(free0 - torch.cuda.mem_get_info()[0])
    log(f"init (host store + seeded weights) {time.time() - t0:.1f} s; device memory taken {mem_delta / 1e9:.3f} GB")

    def one_step(k):
        t, lb = step_batches(cfg, nm, k)
        return ctx.train_step(t, lb) if nm == 1 else ctx.train_step_accum(t, lb)

    for i in range(warmup):
        loss, st = one_step(i)
        log(f"warmup {i}: loss {loss:.4f} step {st.step_ms:.0f} ms")
    ctx.sync()  # queued host updates (cross_step) land before the clock starts
    torch.cuda.synchronize()
    stats = []
    t0 = time.perf_counter()
    for i in range(steps):
        loss, st = one_step(warmup + i)
        stats.append(mt.stats_dict(st))
        log(f"step {i}: loss {loss:.4f} step {st.step_ms:.0f} ms (fwd {st.fwd_ms:.0f} head {st.head_ms:.0f} "
            f"bwd {st.bwd_ms:.0f} adam tail {st.adam_tail_ms:.0f}; adam busy {st.adam_ms:.0f}, "
            f"pack {st.pack_ms:.0f}; waited for adam {st.adam_wait_ms:.0f}; overlap {st.overlap_ratio:.2f})")
    ctx.sync()  # every step's host Adam is inside the timed region
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    res = {"value": nm * T * steps / elapsed, "ms_per_step": elapsed * 1e3 / steps, "stats": stats,
           "mem_delta": mem_delta, "loss": float(loss), "opt": dict(opt_kw)}
    if not keep:
        ctx.close()
        ctx = None
        del arena
        arena = None
        torch.cuda.empty_cache()
    return res, ctx, arena


def pcie_block(stats):
    """Transfer and overlap figures (device clock, averaged over timed steps)."""
    def mean(k, i=None):
        return float(np.mean([s[k] if i is None else s[k][i] for s in stats]))
    h2d_b, h2d_ms, d2h_b, d2h_ms = mean("h2d_bytes"), mean("h2d_busy_ms"), mean("d2h_bytes"), mean("d2h_busy_ms")
    phases = ("fwd", "head", "bwd")
    x_ms, ov_ms = mean("copy_union_ms"), mean("overlap_ms")
    return {"h2d_GBps": round(h2d_b / (h2d_ms / 1e3) / 1e9, 2) if h2d_ms else None,
            "d2h_GBps": round(d2h_b / (d2h_ms / 1e3) / 1e9, 2) if d2h_ms else None,
            "h2d_GB_per_step": round(h2d_b / 1e9, 3), "d2h_GB_per_step": round(d2h_b / 1e9, 3),
            "peak_GBps": PCIE_GEN5_X16_GBS,
            "h2d_frac_of_peak_while_busy": round(h2d_b / (h2d_ms / 1e3) / 1e9 / PCIE_GEN5_X16_GBS, 3) if h2d_ms else None,
            "h2d_busy_frac_of_step": round(mean("pcie_busy_frac"), 3),
            "overlap_ratio": round(mean("overlap_ratio"), 3),
            "transfer_hidden_frac": round(ov_ms / x_ms, 3) if x_ms else None,
            "compute_union_ms": round(mean("compute_union_ms"), 1), "copy_union_ms": round(x_ms, 1),
            "overlap_by_phase": {ph: round(mean("overlap_phase", i), 3) for i, ph in enumerate(phases)},
            "exposed_transfer_ms_by_phase": {ph: round(mean("exposed_transfer_ms", i), 1)
                                             for i, ph in enumerate(phases)},
            "switch_gap_ms_median_by_phase": {ph: round(mean("switch_gap_ms", i), 3) for i, ph in enumerate(phases)},
            "device_idle_ms_by_phase": {ph: round(mean("device_idle_ms", i), 1) for i, ph in enumerate(phases)},
            # link idle before each weight-stream copy by what it waited for: its slot (the earliest any
            # schedule over the same slots could issue it), the host (the weights' update or pack), other
            # copies (checkpoint restores, labels, inputs)
            "h2d_link_idle_ms_by_phase": {ph: {c: round(mean("h2d_idle_ms", 3 * i + j), 1)
                                               for j, c in enumerate(("slot", "host", "other"))}
                                          for i, ph in enumerate(phases)},
            # visits whose inputs were ready before the previous visit ended: start minus that end
            "switch_latency_ready_visits_ms": {"median": round(mean("ready_switch_ms", 0), 4),
                                               "p90": round(mean("ready_switch_ms", 1), 4),
                                               "ready_visits": round(mean("ready_switches"), 1),
                                               "visits": round(mean("switches"), 1)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)  # ~8 s timed: the closing sync drains one step's host Adam once
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="7b", choices=sorted(SHAPES))
    ap.add_argument("--layers", type=int, default=0, help="override the workload's depth")
    ap.add_argument("--depths", default="",
                    help="comma-separated depths: run the workload at each depth in a fresh context, one after "
                         "the other, and report tokens/s and the device memory taken per depth (70b: 4,8)")
    ap.add_argument("--no-profile", action="store_true", help="skip per-kernel HIP event timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pages-config", action="store_true",
                    help="skip the second timed run on the pages' pinned footprint (pageable W packed into two "
                         "pinned staging buffers, 12 gradient slabs)")
    ap.add_argument("--host-threads", type=int, default=0)
    ap.add_argument("--slots", type=int, default=2)
    # 16 gradient slabs: with the pages' 12 the host Adam (slower than the
    # backward on this host) holds every slab near the end of the backward and
    # the gradient copies stall (measured 9.72K against 10.28K tokens/s,
    # alternating runs on one box); --slabs 12 runs the pages' pool
    ap.add_argument("--slabs", type=int, default=16)
    ap.add_argument("--slot-mode", type=int, default=0)
    ap.add_argument("--resident", type=int, default=0)
    ap.add_argument("--pin-store", type=int, default=0)
    ap.add_argument("--pin-weights", type=int, default=1,
                    help="1 (default): W regions in one page-locked block, streamed with no pack copy")
    ap.add_argument("--ablations", action="store_true",
                    help="after the timed run, time 2 steps each with one weight slot, one gradient slab and "
                         "combined W/G slots (the pages' ablations), reported as tokens/s and ratio")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only launch the gate|up GEMM three times and a 1 GiB device copy three times (run "
                         "under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to measure the GEMM's HBM traffic)")
    ap.add_argument("--head-vocab-chunk", type=int, default=-1,
                    help="stream the LM head in E_out row chunks; -1 (default): chunks sized to the largest "
                         "decoder layer, so every slot is layer-sized; 0: the head as one unit")
    ap.add_argument("--own-streams", action="store_true",
                    help="let the library create its three streams instead of passing torch's")
    ap.add_argument("--attn-probe", type=int, default=0, metavar="S",
                    help="only time the attention kernels at sequences of length S with the workload's heads")
    ap.add_argument("--attn-batch", type=int, default=1, metavar="B", help="sequences in the attention probe")
    ap.add_argument("--attn-dq-form", type=int, default=0, choices=(0, 1, 2),
                    help="attention probe's dQ: 0 as the step takes it, 1 recomputed, 2 from the stored dS")
    ap.add_argument("--host-probe", action="store_true",
                    help="only measure host DRAM: the host Adam alone at 8/12/16 threads, a parallel copy and read")
    ap.add_argument("--micro", type=int, default=1,
                    help="micro-batches of batch x seq per optimizer step (gradient accumulation on the host)")
    ap.add_argument("--ckpt-attn", type=int, default=-1,
                    help="1: checkpoint each layer's attention output and log-sum-exp with its input, so the "
                         "backward's recompute skips the attention forward (same results); 0: recompute it; "
                         "-1 (default): 1 for sequences of 8192 and longer, where that forward dominates")
    ap.add_argument("--keep-grads", type=int, default=0,
                    help="0 (default): with one micro-batch Adam reads each gradient slab without copying it into "
                         "the store's G (2 B/param less host traffic; same weights and optimizer state); 1: the "
                         "slab is copied into G as the pages' unpack step does")
    ap.add_argument("--cross-step", type=int, default=1,
                    help="1 (default): the next step's forward overlaps this step's Adam tail (same results); "
                         "0: every step synchronous")
    args = ap.parse_args()
    if args.micro < 1 or (args.micro > 1 and (args.ablations or args.traffic_probe)):
        ap.error("--micro must be >= 1, and 1 with --ablations or --traffic-probe")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build streams one model through one MI355X; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from layer_streaming_amd import mt
    cfg = dict(SHAPES[args.config])
    if args.layers:
        cfg["n_layers"] = args.layers
    cfg["workload"] = cfg["workload"].format(L=cfg["n_layers"])
    if args.host_probe:
        host_probe(mt)
        return
    if args.traffic_probe:
        traffic_probe(torch, mt, cfg)
        return
    if args.attn_probe:
        attention_probe(torch, mt, cfg, args.attn_probe, args.attn_batch, args.attn_dq_form)
        return
    torch.cuda.init()
    ckpt_attn = args.ckpt_attn if args.ckpt_attn >= 0 else int(cfg["seq"] >= 8192)
    opt_kw = dict(profile_kernels=0 if args.no_profile else 1, host_threads=args.host_threads,
                  n_weight_slots=args.slots, n_grad_slabs=args.slabs, slot_mode=args.slot_mode,
                  resident=args.resident, pin_store=args.pin_store, cross_step=args.cross_step,
                  pin_weights=args.pin_weights, head_vocab_chunk=args.head_vocab_chunk,
                  keep_grads=args.keep_grads, ckpt_attn=ckpt_attn)
    if args.depths:
        depth_sweep(torch, mt, cfg, args, opt_kw)
        return
    B, S = cfg["batch"], cfg["seq"]
    T = B * S
    nm = args.micro
    res, ctx, arena = run_workload(torch, mt, cfg, args, opt_kw, args.steps, args.warmup, keep=True)
    if ctx is None:
        print(json.dumps({"metric": METRIC, "value": None, "refused": res}), flush=True)
        sys.exit(3)
    stats, value, ms_per_step = res["stats"], res["value"], res["ms_per_step"]
    sat = int(sum(s["fp16_saturated"] for s in stats))

    out = {"metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 2), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "precision": {"storage": "bf16 weights, gradients and activations; fp32 master, m, v; fp32 accumulation",
                         "attention": "fp16 operands (n1, Wqkv, q, k, v, P, o, Wo) and fp16 MFMA in the forward, "
                                      "range-guarded", "fp16_saturated_in_timed_steps": sat},
           "data": "synthetic: seeded uniform token ids, a fresh batch every step",
           "config": {"workload": cfg["workload"], "global_batch": nm * B, "micro_batches": nm, "seq_len": S,
                      "layers": cfg["n_layers"],
                      "parallelism": "single GPU, layer-streamed", "weight_slots": args.slots,
                      "grad_slabs": args.slabs, "slot_mode": args.slot_mode, "resident": args.resident,
                      "cross_step": args.cross_step, "pin_weights": args.pin_weights,
                      "head_vocab_chunk": args.head_vocab_chunk, "keep_grads": args.keep_grads,
                      "ckpt_attn": ckpt_attn}}
    mf = nm * model_flops_per_step(cfg, T, S)
    out["model_tflops_per_s"] = round(mf / (ms_per_step / 1e3) / 1e12, 2)
    out["pages_convention_tflops_per_s"] = round(nm * pages_flops_per_step(cfg, T, S) / (ms_per_step / 1e3) / 1e12, 2)
    # hardware FLOPs add the recomputed forward of every layer (the down GEMM
    # is not recomputed: backward needs its input, not its output; nor is the
    # attention forward when its output is checkpointed)
    fl0 = gemm_flops(cfg, T)
    recompute = cfg["n_layers"] * (fl0["gemm_qkv"] + fl0["gemm_o"] + fl0["gemm_gateup"] +
                                   (0 if ckpt_attn else 2 * 2 * T * cfg["n_heads"] * cfg["head_dim"] * (S + 1) / 2))
    # a vocabulary-chunked head (head_vocab_chunk != 0) computes the logits
    # twice: its backward recomputes each chunk's logits
    logit_passes = 2 if args.head_vocab_chunk != 0 else 1
    recompute += (logit_passes - 1) * head_gemm_flops(cfg, T)
    out["hw_tflops_per_s"] = round((mf + nm * recompute) / (ms_per_step / 1e3) / 1e12, 2)
    hb_step = host_bytes_per_step(cfg, T, nm, pinned=bool(args.pin_weights), keep_grads=bool(args.keep_grads))
    if ckpt_attn:  # the attention checkpoint ring, written in forward and read in backward
        hb_step += nm * 2 * cfg["n_layers"] * T * cfg["n_heads"] * (2 * cfg["head_dim"] + 4)
    out["host_memory"] = {"bytes_per_step": int(hb_step), "achieved_GBps": round(hb_step / (ms_per_step / 1e3) / 1e9, 1),
                          "adam_alone_GBps": host_adam_probe(mt)}
    out["pcie"] = pcie_block(stats)
    probe = pcie_probe(torch)
    out["pcie"]["probe_GBps"] = probe
    if out["pcie"]["h2d_GBps"]:
        out["pcie"]["h2d_frac_of_probe_while_busy"] = round(out["pcie"]["h2d_GBps"] / probe["h2d"], 3)
    out["phases_ms"] = {k: round(float(np.mean([s[k] for s in stats])), 1)
                        for k in ("fwd_ms", "head_ms", "bwd_ms", "adam_tail_ms", "compute_busy_ms",
                                  "adam_ms", "adam_wait_ms", "pack_ms")}
    out["memory"] = {"gpu_arena_bytes": int(stats[0]["gpu_arena_bytes"]),
                     "gpu_mem_used_delta_bytes": res["mem_delta"],
                     "pinned_bytes": int(stats[0]["pinned_bytes"]),
                     "host_store_bytes": int(stats[0]["host_store_bytes"])}
    if not args.no_profile:
        sites = {}
        for s in stats:
            for k, v in s["sites"].items():
                a = sites.setdefault(k, [0.0, 0])
                a[0] += v["ms"]
                a[1] += v["launches"]
        fl = gemm_flops(cfg, T)
        g_ms = sum(sites[k][0] for k in fl if k in sites)
        g_fl = sum(fl[k] * sites[k][1] for k in fl if k in sites)
        out["mfma_util_block_gemms"] = round(g_fl / (g_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4) if g_ms else None
        out["kernel_ms_per_step"] = {k: round(v[0] / len(stats), 3) for k, v in sorted(sites.items())}
        out["gemm_tflops"] = {k: round(fl[k] * sites[k][1] / (sites[k][0] / 1e3) / 1e12, 1)
                              for k in fl if k in sites and sites[k][0] > 0}
        hf = head_gemm_flops(cfg, T)
        for k in ("head_logits", "head_dx", "head_dw"):
            if k in sites and sites[k][0] > 0:
                passes = logit_passes if k == "head_logits" else 1
                out["gemm_tflops"][k] = round(hf * passes * nm * len(stats) / (sites[k][0] / 1e3) / 1e12, 1)
        hb = hbm_bytes(cfg, T)
        out["hbm_kernels_GBps"] = {k: round(hb[k] * sites[k][1] / (sites[k][0] / 1e3) / 1e9, 1)
                                   for k in hb if k in sites and sites[k][0] > 0}
        if sites.get("head_ce", [0.0])[0] > 0:
            # fp32 logits read by the forward (logsumexp) pass, read again and bf16 dlogits written by the
            # backward pass of the chunked head; read once and dlogits written by the single-unit head
            ce_b = T * cfg["vocab"] * (10 if args.head_vocab_chunk != 0 else 6) * nm * len(stats)
            out["hbm_kernels_GBps"]["head_ce"] = round(ce_b / (sites["head_ce"][0] / 1e3) / 1e9, 1)
        af = 4.0 * cfg["batch"] * cfg["n_heads"] * cfg["head_dim"] * cfg["seq"] * (cfg["seq"] + 1) / 2
        out["attention_tflops"] = {k: round(f * sites[k][1] / (sites[k][0] / 1e3) / 1e12, 1)
                                   for k, f in (("attn_fwd", af), ("attn_bwd", 2.5 * af))
                                   if k in sites and sites[k][0] > 0}
        dom = "gemm_gateup"
        ms, n = sites[dom]
        avg_ms = ms / n
        achieved = fl[dom] / (avg_ms / 1e3) / 1e12
        out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic_bytes(args.config), "avg_launch_ms": round(avg_ms, 4),
                           "launches": n,
                           "flops_per_launch": fl[dom]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ctx, cfg, mt)
    ctx.close()
    del arena
    torch.cuda.empty_cache()
    if not args.no_pages_config and args.pin_weights and nm == 1:
        # The pages' pinned footprint: pageable W packed into two pinned
        # staging buffers sized to the largest streamed block, 12 slabs, and
        # every gradient slab unpacked into the store's G before Adam.
        pk = dict(opt_kw, pin_weights=0, n_grad_slabs=12, keep_grads=1)
        ps = max(2, min(args.steps, 5))
        log(f"pages configuration: pin_weights=0, 12 slabs, keep_grads=1, {ps} timed steps")
        pres, _, _ = run_workload(torch, mt, cfg, args, pk, ps, 1)
        if "refused" in pres:
            out["pages_config"] = pres
        else:
            pst = pres["stats"]
            out["pages_config"] = {
                "value": round(pres["value"], 2), "unit": "tokens/s", "steps": ps,
                "ms_per_step": round(pres["ms_per_step"], 2), "pin_weights": 0, "grad_slabs": 12, "keep_grads": 1,
                "pinned_bytes": int(pst[0]["pinned_bytes"]), "gpu_arena_bytes": int(pst[0]["gpu_arena_bytes"]),
                "phases_ms": {k: round(float(np.mean([s[k] for s in pst])), 1)
                              for k in ("fwd_ms", "head_ms", "bwd_ms", "adam_ms", "adam_wait_ms", "pack_ms")},
                "pcie": pcie_block(pst)}
    if args.ablations:
        out["ablations"] = ablations(torch, mt, mt.make_shape(
            cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn_dim"],
            cfg["vocab"]), cfg, args, *step_batches(cfg, 1, 0), T / (ms_per_step / 1e3))
    print(json.dumps(out), flush=True)


def depth_sweep(torch, mt, cfg, args, opt_kw):
    """The workload at several depths, each in a fresh context one after the
    other: tokens/s, layer-tokens/s (tokens/s times depth: constant when the
    step time grows linearly with depth), and the device memory each context
    took (the arena does not depend on the depth)."""
    depths = [int(x) for x in args.depths.split(",") if x]
    # One untimed step of a one-layer context first: the runtime's one-time
    # device allocations (code objects, the library's static buffers) then
    # fall outside every measured context.
    run_workload(torch, mt, dict(cfg, n_layers=1), args, dict(opt_kw, profile_kernels=0), 1, 0)
    rows = []
    for L in depths:
        c = dict(cfg, n_layers=L)
        res, _, _ = run_workload(torch, mt, c, args, opt_kw, args.steps, args.warmup)
        if "refused" in res:
            rows.append({"layers": L, **res})
            continue
        st = res["stats"]
        rows.append({"layers": L, "tokens_per_s": round(res["value"], 1),
                     "layer_tokens_per_s": round(res["value"] * L, 1), "ms_per_step": round(res["ms_per_step"], 1),
                     "gpu_arena_bytes": int(st[0]["gpu_arena_bytes"]), "gpu_mem_used_delta_bytes": res["mem_delta"],
                     "pinned_bytes": int(st[0]["pinned_bytes"]), "host_store_bytes": int(st[0]["host_store_bytes"]),
                     "pcie": pcie_block(st)})
        log(f"depth {L}: {res['value']:.0f} tokens/s, device memory taken {res['mem_delta'] / 1e9:.3f} GB")
    ok = [r for r in rows if "refused" not in r]
    print(json.dumps({"metric": METRIC, "depth_sweep": rows, "workload": cfg["workload"].replace(
        f"{cfg['n_layers']} layers", "L layers"), "steps": args.steps, "warmup": args.warmup,
        "gpu_arena_constant_across_depths": len({r["gpu_arena_bytes"] for r in ok}) == 1 if ok else None,
        "gpu_mem_used_delta_spread_bytes": (max(r["gpu_mem_used_delta_bytes"] for r in ok) -
                                            min(r["gpu_mem_used_delta_bytes"] for r in ok)) if ok else None}),
        flush=True)


if __name__ == "__main__":
    main()
