"""Benchmark of the block-wise attention hot path on one MI355X.

One step = one pass of the whole hot path over the 8 queued blocks that one
GPU holds (each block: 24 heads x 64, 5400 queries = 4 latent frames of 30x45
tokens, keys = 5400 cached neighbouring-block + 5400 own + 226 text, its own
ring slots in a 16-slot ring):
  1. ba_cache_append_batched  the blocks' K/V into their ring slots
  2. ba_block_attention       one launch: every block's queries over
                              [cached neighbour | own block | text]
  3. ba_block_update          every block's latents, DDIM step at its own
                              timestep (1, 143, ..., 1000)
`--workload N` runs the step on another bf16 workload instead.  Inputs are
seeded synthetic tensors (N(0,1)*0.5 bf16 for Q/K/V, N(0,1) for latents and
noise) already resident in HBM when the timed region starts.

Prints one JSON line.  `value` is block-attention TFLOP/s over the whole
step (algorithmic FLOPs 4*Lq*Lk*D*H*n_blocks over valid keys / step time).
The `roofline` object rates the attention kernel alone against the bf16
dense MFMA peak, from HIP events around each of its launches on the launch
stream.  `other_configs` times the attention of the other target workloads
(the 480p and 720p blocks) alone, after the timed region.  `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
PEAK_HBM_GBS = 8000.0
CLOCK_GHZ, N_CU = 2.4, 256
EXP_PER_CLK_PER_CU = 16        # v_exp_f32: a wave64 every 16 clocks on each of 4 SIMDs
ATTN_SRC = os.path.join(ROOT, "block_wise_long_amd", "csrc", "attention.hip")


# the producer's tile shape lives in internal.h: both files key its counters
PROJ_SRC = (os.path.join(ROOT, "block_wise_long_amd", "csrc", "project.hip"),
            os.path.join(ROOT, "block_wise_long_amd", "csrc", "internal.h"))
PROJ_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "project_d64_qkv480p_traffic.md")


def attention_kernel_name(B, D, max_keys):
    """The bf16 attention kernel a launch takes for a one-segment key set: its
    launch shape (0 wide, 1 narrow, 2 resident) follows from the query tile
    the library reports for the key set."""
    tile = B.ba_attention_query_tile(D, B.BA_BF16, max_keys)
    if tile == 32:
        return "attention_resident_kernel<2>"
    wide = B.ba_attention_query_tile(D, B.BA_BF16, 1 << 30)
    return f"attention_bf16_kernel<{D}, {0 if tile == wide else 1}>"


def kernel_hash(src=ATTN_SRC):
    h = hashlib.sha256()
    for path in ((src,) if isinstance(src, str) else src):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload_name, traffic_file, src=ATTN_SRC):
    """HBM bytes per launch from a committed counter summary, or None when it
    is missing or was taken on another version of the kernel's source."""
    if not os.path.exists(traffic_file):
        return None
    text = open(traffic_file).read()
    m = re.search(r"kernel_sha256_16:\s*([0-9a-f]+)", text)
    w = re.search(r"workload:\s*(\S+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m and b and w) or m.group(1) != kernel_hash(src) or w.group(1) != workload_name:
        return None
    return float(b.group(1))


def _oracle_block(cfg, inputs, b):
    """The oracle's ring model of block b's key set (one ring slot per
    segment, in key order), its text ring and its meta."""
    from oracle import ring as R
    H, D = cfg.heads, cfg.head_dim
    if cfg.full_sequence:
        n = len(cfg.segs[0])
        seg = cfg.segs[0][0][1]
        ks = [inputs["k_cur"][0][i * seg:(i + 1) * seg] for i in range(n)]
        vs = [inputs["v_cur"][0][i * seg:(i + 1) * seg] for i in range(n)]
    else:
        ks = [inputs["k_ctx"][b], inputs["k_cur"][b]]
        vs = [inputs["v_ctx"][b], inputs["v_cur"][b]]
    ring = R.RingModel(len(ks), max(k.shape[0] for k in ks), H, D, cfg.dtype)
    for k, v in zip(ks, vs):
        ring.append(k, v, k.shape[0])
    text = R.RingModel(1, cfg.text_len, H, D, cfg.dtype)
    text.append(inputs["k_text"], inputs["v_text"], cfg.text_len)
    meta = {"q_len": cfg.q_len, "segs": [(i, k.shape[0]) for i, k in enumerate(ks)],
            "text_slot": 0, "text_len": cfg.text_len}
    return ring, text, meta


def cpu_baseline(cfg, inputs, budget_s):
    """The oracle, as it stands, on the workload's own inputs: units of
    (block, head, a quarter of the block's queries over all its keys), taken
    in order until the time budget is used (at least one unit)."""
    from oracle import attention as A
    from oracle import numerics as N
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    chunk = -(-cfg.q_len // 4)
    units = [(b, h, r0) for b in range(cfg.n_blocks) for h in range(cfg.heads)
             for r0 in range(0, cfg.q_len, chunk)]
    done, rows_done, setup_s, t_run = 0, 0, 0.0, 0.0
    cur_b, ring, text, meta, q = None, None, None, None, None
    for b, h, r0 in units:
        if b != cur_b:
            t_s = time.perf_counter()
            ring, text, meta = _oracle_block(cfg, inputs, b)
            q = N.decode(inputs["q"][b:b + 1], cfg.dtype)
            cur_b = b
            setup_s += time.perf_counter() - t_s
        rows = list(range(r0, min(r0 + chunk, cfg.q_len)))
        t0 = time.perf_counter()
        A.block_attention_ref(q, ring, text, [meta], heads=[h], rows=rows)
        t_run += time.perf_counter() - t0
        done += 1
        rows_done += len(rows)
        if t_run >= budget_s:
            break
    flops = 4.0 * rows_done * cfg.key_len * cfg.head_dim
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:  # noqa: BLE001
        affinity = None
    return {"value": flops / t_run / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(units)} (block, head, {chunk}-query chunk) units of {cfg.name} "
                      f"({rows_done} query rows, each over all {cfg.key_len} keys), fp64 numpy "
                      f"(BLAS dgemm), {t_run:.1f} s wall in the oracle call",
            "gflops_fp64": round(flops / t_run / 1e9, 2), "os_cpu_count": os.cpu_count(),
            "sched_affinity": affinity, "blas_threads": threads}


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE readings give the counters' scale (bytes moved
    per KiB reported)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def update_size_sweep(B, torch, sizes_mb=(16, 64, 256, 1024, 2048), reps=5):
    """ba_block_update alone at growing sizes (bytes moved = 3 x 2 B per
    element), with a 512 MB write between calls so that no call finds its
    operands in the 256 MB Infinity Cache: shows where the kernel reaches the
    HBM plateau (the per-block updates of the workloads are a few MB)."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = []
    for mb in sizes_mb:
        n = (mb << 20) // 6 // 8 * 8
        x = torch.randn(n, device="cuda").to(torch.bfloat16).view(1, n)
        eps = torch.randn(n, device="cuda").to(torch.bfloat16).view(1, n)
        times = []
        for _ in range(reps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.ba_block_update(x, eps, [143])
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        out.append({"MB": round(6.0 * n / 1e6, 1), "ms": round(ms, 4), "GBs": round(6.0 * n / (ms * 1e-3) / 1e9, 1)})
        del x, eps
    del flush
    return out


def traffic_file(cfg):
    """Committed counter summary of the attention kernel on this workload."""
    return os.path.join(ROOT, "profiles", f"attention_bf16_d{cfg.head_dim}_{cfg.name}_traffic.md")


def warm_up(torch, fn, n_min, min_s):
    """Untimed warm-up: at least n_min calls, continued until min_s seconds of
    load have passed (the shader clock ramps up over tens of milliseconds of
    sustained work).  Returns (calls run, seconds)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < n_min or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n, time.perf_counter() - t0


class Workload:
    """A workload's inputs on the device: the ring with every block's cached
    context (written by the previous step), the text ring, q, out, the metas,
    the blocks' own K/V to append each step, and (optionally) the latents."""

    def __init__(self, B, torch, cfg, with_update=False):
        from workloads import make_attention_inputs, make_update_inputs
        self.B, self.cfg = B, cfg
        inputs = make_attention_inputs(cfg)
        self.inputs = inputs

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

        H, D = cfg.heads, cfg.head_dim
        self.ring = B.ba_ring_init(cfg.n_slots, cfg.slot_tokens, H, D, B.BA_BF16)
        self.text = B.ba_ring_init(1, cfg.text_len, H, D, B.BA_BF16)
        B.ba_cache_append(self.text, dev(inputs["k_text"]), dev(inputs["v_text"]), cfg.text_len)
        if cfg.full_sequence:
            # the whole prefix is the block's own keys, one ring slot per 4-frame block
            nseg = len(cfg.segs[0])
            seg_len = cfg.segs[0][0][1]
            self.k_cur = dev(inputs["k_cur"]).view(nseg, seg_len, H, D)
            self.v_cur = dev(inputs["v_cur"]).view(nseg, seg_len, H, D)
            self.cur_slots = [sl for sl, _ in cfg.segs[0]]
        else:
            B.ba_cache_append_batched(self.ring, dev(inputs["k_ctx"]), dev(inputs["v_ctx"]),
                                      [sg[0][0] for sg in cfg.segs])
            self.k_cur = dev(inputs["k_cur"])      # [n_blocks][L][H][D]
            self.v_cur = dev(inputs["v_cur"])
            self.cur_slots = [sg[1][0] for sg in cfg.segs]
        self.q = dev(inputs["q"])
        self.out = torch.empty_like(self.q)
        self.metas = [B.make_meta(cfg.q_len, list(cfg.segs[b]), 0, cfg.text_len) for b in range(cfg.n_blocks)]
        self.appended_tokens = self.k_cur.shape[0] * self.k_cur.shape[1]
        # the cached context is in place: from here on a step appends the blocks' own K/V
        B.ba_cache_append_batched(self.ring, self.k_cur, self.v_cur, self.cur_slots)
        if with_update:
            upd = make_update_inputs(cfg, inputs["_rng"])
            self.x = dev(upd["x"])
            self.eps = dev(upd["eps"])
            self.ts = [int(t) for t in upd["t"]]
        torch.cuda.synchronize()

    def append(self):
        self.B.ba_cache_append_batched(self.ring, self.k_cur, self.v_cur, self.cur_slots)

    def attention(self):
        self.B.ba_block_attention(self.q, self.ring, self.text, self.metas, out=self.out)

    def release(self):
        """Free the device buffers (the host inputs stay for the oracle)."""
        for name in ("ring", "text", "k_cur", "v_cur", "q", "out", "x", "eps"):
            if hasattr(self, name):
                delattr(self, name)


def attention_alone(B, torch, cfg, steps, warmup, min_s):
    """ba_block_attention alone on a workload: mean/median/p10/p90 of `steps`
    calls, HIP events on the launch stream around each call."""
    w = Workload(B, torch, cfg)
    stream = torch.cuda.current_stream()
    n_warm, s_warm = warm_up(torch, w.attention, warmup, min_s)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        w.attention()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    w.release()
    del w
    torch.cuda.empty_cache()
    mean = float(np.mean(ms))
    tf = cfg.flops() / (mean * 1e-3) / 1e12
    return {"n_blocks": cfg.n_blocks, "heads": cfg.heads, "head_dim": cfg.head_dim, "queries": cfg.q_len,
            "keys": cfg.key_len, "calls": steps, "warmup_calls_run": n_warm, "warmup_s": round(s_warm, 3),
            "attention_ms": round(mean, 5), "attention_median": round(float(np.median(ms)), 5),
            "attention_p10": round(float(np.percentile(ms, 10)), 5),
            "attention_p90": round(float(np.percentile(ms, 90)), 5),
            "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "latent_frames_per_s": round(cfg.latent_frames / (mean * 1e-3), 1),
            "kernel": attention_kernel_name(B, cfg.head_dim, cfg.key_len)}


def append_size_sweep(B, torch, sizes_mb=(16, 64, 256, 1024, 2048), reps=5):
    """ba_cache_append alone at growing sizes (bytes moved = K and V read
    plus K and V written, 24 heads x 64), with a 512 MB write between calls
    so that no call finds its source in the 256 MB Infinity Cache."""
    H, D = 24, 64
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = []
    for mb in sizes_mb:
        n = max((mb << 20) // (4 * H * D * 2) // 64 * 64, 64)   # tokens: 2 tensors x (read + write)
        k = torch.randn((n, H, D), device="cuda").to(torch.bfloat16)
        v = torch.randn((n, H, D), device="cuda").to(torch.bfloat16)
        ring = B.ba_ring_init(1, n, H, D, B.BA_BF16)
        times = []
        for _ in range(reps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.ba_cache_append_batched(ring, k.view(1, n, H, D), v.view(1, n, H, D), [0])
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        moved = 4.0 * n * H * D * 2
        out.append({"MB": round(moved / 1e6, 1), "ms": round(ms, 4), "GBs": round(moved / (ms * 1e-3) / 1e9, 1)})
        del k, v, ring
    del flush
    torch.cuda.empty_cache()
    return out


def queue_bench(args):
    """One JSON line for the single-GPU FIFO queue step at the shape of the
    8-block workload: 8 queued blocks of 5400 tokens (4 latent frames) x 24
    heads x 64, 226 text keys, T = 1000 (stride 125); every step appends the
    blocks' K/V, runs one attention launch over all 8 blocks (each over its
    neighbour's K/V of the previous step, its own and the text: 11026 keys),
    updates every block at its own timestep, pops the clean head and takes a
    new noise block at the tail."""
    import torch
    from block_wise_long_amd.fifo import FifoQueue
    torch.cuda.set_device(0)
    n, L, H, D, TXT, T = 8, 5400, 24, 64, 226, 1000
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20254)
    lat = (torch.randn((n, L, H, D), device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    tk = (torch.randn((TXT, H, D), device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    tv = (torch.randn((TXT, H, D), device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    noise = (torch.randn((L, H, D), device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    layer = None
    if args.layer:
        # the layer through the fused K/V producer: random W, the usual
        # rotation frequencies at positions 0..L-1 (pair-major table)
        dim = H * D
        w = (torch.randn((3 * dim, dim), device="cuda", generator=gen) * dim ** -0.5).to(torch.bfloat16)
        pos = torch.arange(L, device="cuda", dtype=torch.float32)[:, None]
        freq = 10000.0 ** (-torch.arange(D // 2, device="cuda", dtype=torch.float32) * 2 / D)[None, :]
        ang = (pos * freq).t()
        layer = {"w": w, "rope": torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).contiguous()}
    fq = FifoQueue(lat, tk, tv, T=T, layer=layer)
    # from step 1 on every block has its neighbour's context; the warm-up
    # also lasts long enough for the shader clock to ramp up
    warm_up(torch, lambda: fq.step(noise), max(args.warmup, 1), args.warmup_min_s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        fq.step(noise)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 4.0 * n * L * (2 * L + TXT) * D * H
    res = {"metric": "FIFO queue step: latent frames/s and attention-equivalent TFLOP/s at 1 GPU",
           "value": round(4 / (ms * 1e-3), 1), "unit": "latent frames/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "fifo-queue-8x480p" + ("-qkv-layer" if args.layer else ""), "n_queue": n,
                      "block_tokens": L, "heads": H, "head_dim": D, "text": TXT, "T": T, "stride": T // n,
                      "layer": "qkv-projection (fused K/V producer)" if args.layer else "latents as q, k, v"},
           "tflops_step": round(flops / (ms * 1e-3) / 1e12, 2),
           "pct_bf16_peak_step": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    print(json.dumps(res), flush=True)


def project_bench(args):
    """One JSON line for the fused K/V producer at the 480p block's shape:
    5400 tokens x 1536 (24 heads x 64) projected to q, k, v (4608 rows),
    rotation on, K/V straight into a ring slot.  Compared with the plain
    append of the same K/V."""
    import torch
    import block_wise_long_amd as B
    torch.cuda.set_device(0)
    L, H, D = 5400, 24, 64
    dim = H * D
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20255)
    x = torch.randn((L, dim), device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn((3 * H * D, dim), device="cuda", generator=gen) * dim ** -0.5).to(torch.bfloat16)
    pos = torch.arange(L, device="cuda", dtype=torch.float32)[:, None]
    freq = 10000.0 ** (-torch.arange(D // 2, device="cuda", dtype=torch.float32) * 2 / D)[None, :]
    ang = (pos * freq).t()                                    # pair-major: [D/2][L]
    rope = torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).contiguous()
    ring = B.ba_ring_init(2, L, H, D, B.BA_BF16)
    q = torch.empty((L, H, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, L, H, D), dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        warm_up(torch, fn, max(args.warmup, 1), args.warmup_min_s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_proj = timed(lambda: B.ba_qkv_project(x, w, ring, 1, q=q, rope=rope))
    # the 8 queued blocks of a FIFO step in one launch (43200 tokens)
    nb = 8
    xb = torch.randn((nb, L, dim), device="cuda", generator=gen).to(torch.bfloat16)
    ringb = B.ba_ring_init(nb, L, H, D, B.BA_BF16)
    qb = torch.empty((nb, L, H, D), dtype=torch.bfloat16, device="cuda")
    ms_batch = timed(lambda: B.ba_qkv_project_batched(xb, w, ringb, list(range(nb)), q=qb, rope=rope))
    del xb, ringb, qb
    ms_append = timed(lambda: B.ba_cache_append_batched(ring, k, k, [0]))
    # context only: the vendor library's linear layer on the same operands
    # (plain [tokens][rows] output, no rotation, no ring layout)
    y = torch.empty((L, 3 * H * D), dtype=torch.bfloat16, device="cuda")
    ms_lib = timed(lambda: torch.mm(x, w.t(), out=y))
    flops = 2.0 * L * dim * 3 * H * D
    tf = flops / (ms_proj * 1e-3) / 1e12
    res = {"metric": "fused K/V producer TFLOP/s (QKV projection + rotation + ring layout) at 1 GPU",
           "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_proj, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "qkv-producer-480p-block", "tokens": L, "dim": dim, "rows": 3 * H * D,
                      "heads": H, "head_dim": D, "rotation": True},
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_from_profile("qkv-producer-480p-block", PROJ_TRAFFIC_FILE, PROJ_SRC),
                        "kernel": f"project_kernel<{D}>", "flop_per_launch": flops},
           "batched_8_blocks_ms": round(ms_batch, 5),
           "batched_8_blocks_tflops": round(8 * flops / (ms_batch * 1e-3) / 1e12, 2),
           "append_ms_same_kv": round(ms_append, 5),
           "library_mm_ms": round(ms_lib, 5),
           "library_mm_tflops": round(flops / (ms_lib * 1e-3) / 1e12, 2)}
    print(json.dumps(res), flush=True)


def noise_bench(args):
    """One JSON line for the coordinated noise initialisation: a new 480p
    block's latents (16 channels x 4 frames of a 60 x 90 plane, bf16) gathered
    from a 21-frame pool (last 3 excluded); beside it the queue's stand-in
    block (5400 x 24 x 64) and a size sweep with the Infinity Cache flushed
    between calls."""
    import torch
    import block_wise_long_amd as B
    torch.cuda.set_device(0)

    def timed(pool, frames, out, flush=None, reps=None):
        """Median over single calls, each between two events on the launch
        stream (launch latency included: a block's gather is a few
        microseconds of kernel time); with a flush, the Infinity Cache is
        overwritten before each call."""
        reps = args.steps if reps is None else reps
        warm_up(torch, lambda: B.ba_noise_block(pool, frames, out), max(args.warmup, 1), args.warmup_min_s)
        ts = []
        for _ in range(reps):
            if flush is not None:
                flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            B.ba_noise_block(pool, frames, out)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    C, F, E, excl, bf = 16, 21, 60 * 90, 3, 4
    pool = torch.randn((C, F, E), device="cuda").to(torch.bfloat16)
    out = torch.empty((C, bf, E), dtype=torch.bfloat16, device="cuda")
    frames = B.ba_noise_assign(20257, 5, F, excl, bf)
    ms = timed(pool, frames, out)
    nbytes = 2.0 * out.numel() * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the queue's stand-in block: 8.3 M elements as 16 x 4 frames of 129600
    E2 = 5400 * 24 * 64 // (C * bf)
    pool2 = torch.randn((C, F, E2), device="cuda").to(torch.bfloat16)
    out2 = torch.empty((C, bf, E2), dtype=torch.bfloat16, device="cuda")
    ms2 = timed(pool2, frames, out2)
    del pool2, out2
    sweep = []
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for mb in (16, 64, 256, 1024):
        e = (mb << 20) // (2 * 2 * C * bf) // 8 * 8          # read + write = mb
        p = torch.empty((C, F, e), dtype=torch.bfloat16, device="cuda").normal_()
        o = torch.empty((C, bf, e), dtype=torch.bfloat16, device="cuda")
        t = timed(p, frames, o, flush=flush, reps=5)
        sweep.append({"MB": round(4.0 * o.numel() / 1e6, 1), "ms": round(t, 4),
                      "GBs": round(4.0 * o.numel() / (t * 1e-3) / 1e9, 1)})
        del p, o
    del flush
    res = {"metric": "noise-block gather GB/s (coordinated noise initialisation) at 1 GPU",
           "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "noise-block-480p", "channels": C, "pool_frames": F, "n_exclude": excl,
                      "block_frames": bf, "frame_elems": E},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                        "frac": round(gbs / 8000.0, 4), "traffic": None, "kernel": "noise_gather_kernel",
                        "bytes_per_launch": nbytes},
           "standin_block_ms": round(ms2, 5),
           "standin_block_GBs": round(4.0 * C * bf * E2 / (ms2 * 1e-3) / 1e9, 1),
           "sweep": sweep}
    print(json.dumps(res), flush=True)


def cross_bench(args):
    """One JSON line for the separate text cross-attention at the 480p
    block's shape: 5400 queries, 24 heads x 64, a 512-token text (a padded
    prompt), no cache segments; beside it the self part alone (cache
    [5400 | 5400], no text), the joint call over [cache | text], and the
    text-only call of the 8 queued blocks of a step in one launch."""
    import torch
    import block_wise_long_amd as B
    torch.cuda.set_device(0)
    L, H, D, TXT, NQ = 5400, 24, 64, 512, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20256)

    def rnd(*shape):
        return (torch.randn(shape, device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    ring = B.ba_ring_init(2, L, H, D, B.BA_BF16)
    B.ba_cache_append_batched(ring, rnd(2, L, H, D), rnd(2, L, H, D), [0, 1])
    text = B.ba_ring_init(1, TXT, H, D, B.BA_BF16)
    B.ba_cache_append(text, rnd(TXT, H, D), rnd(TXT, H, D), TXT)
    q = rnd(NQ, L, H, D)
    out = torch.empty_like(q)
    segs = [(0, L), (1, L)]
    m_cross = [B.make_meta(L, [], 0, TXT)]
    m_self = [B.make_meta(L, segs, 0, 0)]
    m_joint = [B.make_meta(L, segs, 0, TXT)]
    m_queue = [B.make_meta(L, [], 0, TXT) for _ in range(NQ)]
    stream = torch.cuda.current_stream()

    def timed(metas):
        nb = len(metas)

        def call():
            B.ba_block_attention(q[:nb], ring, text, metas, out=out[:nb])
        warm_up(torch, call, max(args.warmup, 1), args.warmup_min_s)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))

    ms_cross = timed(m_cross)
    ms_self = timed(m_self)
    ms_joint = timed(m_joint)
    ms_queue = timed(m_queue)
    flops = 4.0 * L * TXT * D * H
    tf = flops / (ms_cross * 1e-3) / 1e12
    tf_q = NQ * flops / (ms_queue * 1e-3) / 1e12
    res = {"metric": "separate text cross-attention TFLOP/s at 1 GPU",
           "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_cross, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "text-cross-attention-480p-block", "queries": L, "heads": H, "head_dim": D,
                      "text_keys": TXT},
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "kernel": attention_kernel_name(B, D, TXT), "flop_per_launch": flops},
           # q and out cross HBM once each; text K/V are 3 MB
           "hbm_bytes_per_launch": 2 * L * H * D * 2 + 2 * TXT * H * D * 2,
           "self_only_ms": round(ms_self, 5),
           "split_ms": round(ms_self + ms_cross, 5),
           "joint_ms": round(ms_joint, 5),
           # the queue step's text-only call: its 8 blocks in one launch
           "queued_8_blocks": {"ms": round(ms_queue, 5), "tflops": round(tf_q, 2),
                               "frac": round(tf_q / PEAK_BF16_TFLOPS, 4)}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    # the shader clock ramps up over the first tens of milliseconds of
    # sustained load: the warm-up runs at least this long, whatever --warmup says
    ap.add_argument("--warmup-min-s", type=float, default=0.3)
    ap.add_argument("--workload", type=int, default=3,
                    help="config index of the step (3, the 8 queued blocks, is the default bench line)")
    ap.add_argument("--also", type=lambda t: [int(x) for x in t.split(",") if x], default=[1, 2],
                    help="config indices whose attention is also timed alone (comma list, empty: none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--no-sweeps", action="store_true",
                    help="skip the append and update size sweeps (for profiler runs of the step)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--queue", action="store_true",
                    help="time the single-GPU FIFO queue step (8 blocks of the 480p shape) instead")
    ap.add_argument("--layer", action="store_true",
                    help="with --queue: the layer's q, k, v come from the fused K/V producer")
    ap.add_argument("--noise", action="store_true",
                    help="time the noise-block gather (coordinated noise initialisation) instead")
    ap.add_argument("--cross", action="store_true",
                    help="time the separate text cross-attention (480p block, 512 text keys) instead")
    ap.add_argument("--project", action="store_true",
                    help="time the fused K/V producer (QKV projection of the 480p block) instead")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.noise:
        if args.gpus != 1:
            print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}))
            sys.exit(2)
        noise_bench(args)
        return
    if args.cross:
        if args.gpus != 1:
            print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}))
            sys.exit(2)
        cross_bench(args)
        return
    if args.project:
        if args.gpus != 1:
            print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}))
            sys.exit(2)
        project_bench(args)
        return
    if args.queue:
        if args.gpus != 1:
            print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}))
            sys.exit(2)
        queue_bench(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import block_wise_long_amd as B
    from workloads import CONFIGS

    cfg = CONFIGS[args.workload]
    if cfg.dtype != "bf16":
        print(json.dumps({"error": "bench steps cover the bf16 workloads (1-4)"}))
        sys.exit(2)
    torch.cuda.set_device(0)
    w = Workload(B, torch, cfg, with_update=True)
    H, D = cfg.heads, cfg.head_dim
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        w.append()
        if ev is not None:
            ev[1].record(stream)
        w.attention()
        if ev is not None:
            ev[2].record(stream)
        B.ba_block_update(w.x, w.eps, w.ts)
        if ev is not None:
            ev[3].record(stream)

    warm_steps, warm_s = warm_up(torch, step, args.warmup, args.warmup_min_s)

    # timed region: exactly `steps` whole steps, bracketed by synchronisation
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    ms_append = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_attn_all = [e[1].elapsed_time(e[2]) for e in evs]
    ms_attn = float(np.mean(ms_attn_all))
    ms_update = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    w.release()

    # the other target configurations, attention alone, after the timed region
    others = {}
    for i in args.also:
        if i == args.workload or CONFIGS[i].dtype != "bf16":
            continue
        others[CONFIGS[i].name] = attention_alone(B, torch, CONFIGS[i], args.steps, args.warmup, args.warmup_min_s)

    update_sweep = None if args.no_sweeps else update_size_sweep(B, torch)
    append_sweep = None if args.no_sweeps else append_size_sweep(B, torch)

    flops = float(cfg.flops())
    tflops_step = flops / (ms_step * 1e-3) / 1e12
    tflops_attn = flops / (ms_attn * 1e-3) / 1e12
    append_bytes = 2.0 * 2 * w.appended_tokens * H * D * 2    # read K,V + write K,V (valid tokens)
    update_bytes = 3.0 * cfg.update_elems * cfg.n_blocks * 2
    exps = float(cfg.n_blocks) * H * cfg.q_len * cfg.key_len

    res = {
        "metric": "block-attention TFLOP/s + % bf16 MFMA peak; latent frames/s at 1 GPU",
        "value": round(tflops_step, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "n_blocks": cfg.n_blocks, "heads": H, "head_dim": D,
                   "queries": cfg.q_len, "keys": cfg.key_len,
                   "key_segments": [cfg.ctx_len, cfg.cur_len, cfg.text_len],
                   "latent_frames_per_step": cfg.latent_frames},
        # untimed warm-up actually run: the steps asked for, continued until
        # the shader clock has had warmup_min_s of load to ramp up
        "warmup_steps_run": warm_steps,
        "warmup_s": round(warm_s, 3),
        "pct_bf16_peak_step": round(100 * tflops_step / PEAK_BF16_TFLOPS, 2),
        "latent_frames_per_s": round(cfg.latent_frames / (ms_step * 1e-3), 1),
        "kernel_ms": {"append": round(ms_append, 5), "attention": round(ms_attn, 5),
                      "attention_median": round(float(np.median(ms_attn_all)), 5),
                      "attention_p10": round(float(np.percentile(ms_attn_all, 10)), 5),
                      "attention_p90": round(float(np.percentile(ms_attn_all, 90)), 5),
                      "update": round(ms_update, 5)},
        "latent_frames_per_s_24_heads": round(cfg.latent_frames / (ms_step * 1e-3) * H / 24, 1),
        "other_configs": others,
        # in the step the same blocks are appended every time, so the append
        # reads from the 256 MB Infinity Cache; append_sweep is the HBM figure
        "append_GBs_in_step": round(append_bytes / (ms_append * 1e-3) / 1e9, 1),
        "append_sweep": append_sweep,
        "update_GBs": round(update_bytes / (ms_update * 1e-3) / 1e9, 1),
        "update_sweep": update_sweep,
        # the softmax's second bound: one exponential per (query, valid key,
        # head) against v_exp_f32's issue rate
        "exp_rate": {"exps_per_launch": exps,
                     "per_clk_per_cu": round(exps / (ms_attn * 1e-3) / (CLOCK_GHZ * 1e9) / N_CU, 3),
                     "peak_per_clk_per_cu": EXP_PER_CLK_PER_CU},
        "roofline": {"bound": "mfma", "achieved": round(tflops_attn, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops_attn / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(cfg.name, traffic_file(cfg)),
                     "kernel": attention_kernel_name(B, D, cfg.key_len),
                     "flop_per_launch": flops},
    }
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(cfg, w.inputs, args.cpu_budget)
        res["cpu_baseline"]["gpu_over_oracle"] = round(tflops_attn / res["cpu_baseline"]["value"], 1)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
