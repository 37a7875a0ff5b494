#!/usr/bin/env python3
"""Benchmark of the block-sparse video attention hot path on one MI355X.

One step = the whole path over one batch already resident in HBM:
  build_mask(q, k)  (block pooling, screened reduced map kept on chip, CDF cut + window, CSR)
  prepare_v(v)      (V to fractal block order, per-block transposed)
  attend(q, k, v')  (block-sparse attention over the kept 64 x 64 tiles)
The fractal permutation of Q, K and O is fused into the loads/stores of these
kernels (inputs and outputs stay in original (t, h, w) order).

Prints ONE JSON line.  `value` is dense-equivalent TFLOP/s of a whole step
(4*B*heads*L^2*D / step time); `roofline` covers the attention kernel
(executed FLOPs / its own event-timed duration vs the bf16 MFMA peak);
`cpu_baseline` times the float64 CPU oracle on a bounded sample of the same
workload and extrapolates it to one full call.  The default invocation (no
--config) also times the Wan2.1-scale workload (config 2, short rows) and
reports it under `short_rows`.
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

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_hunyuan_hybrid_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_fractal_amd", "csrc", "attn_bf16.hip")
MASK_SRCS = [os.path.join(ROOT, "block_sparse_attention_fractal_amd", "csrc", f)
             for f in ("pool.hip", "mask_screen.hip", "mask.hip", "mask_util.h")]
MASK_TRAFFIC = {4: os.path.join(ROOT, "profiles", "mask_hunyuan_hybrid_traffic.json"),
                2: os.path.join(ROOT, "profiles", "mask_wan21_traffic.json")}


def kernel_sha() -> str:
    """Fingerprint of the attention kernel: its source plus the flags it is built with."""
    from block_sparse_attention_fractal_amd import build as _b
    h = hashlib.sha256()
    with open(ATTN_SRC, "rb") as f:
        h.update(f.read())
    h.update(repr(_b._flags()[:-4] + _b.EXTRA.get("attn_bf16.hip", [])).encode())
    return h.hexdigest()[:16]


def traffic_for_current_kernel(cfg_idx: int):
    """HBM bytes per attention launch from the committed PMC summary, or None when the
    kernel (source or flags) changed since the counters were taken, or the counters
    were taken on another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha() or t.get("config") != cfg_idx:
        return None
    return t.get("bytes_per_launch")


def mask_sha() -> str:
    """Fingerprint of the mask-stage kernels: their sources plus their build flags."""
    from block_sparse_attention_fractal_amd import build as _b
    h = hashlib.sha256()
    for p in MASK_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(repr(_b._flags()[:-4] + _b.EXTRA.get("mask_screen.hip", [])).encode())
    return h.hexdigest()[:16]


def mask_traffic(cfg_idx: int):
    """HBM bytes of one build_mask call from the committed PMC summary (scaled
    FETCH_SIZE + WRITE_SIZE over every kernel of the stage), or None when the mask
    kernels changed since the counters were taken or none were taken here."""
    try:
        with open(MASK_TRAFFIC[cfg_idx]) as f:
            t = json.load(f)
    except (KeyError, OSError, ValueError):
        return None
    if t.get("mask_sha") != mask_sha() or t.get("config") != cfg_idx:
        return None
    return t.get("bytes_per_call")


def density_by_class(cfg, mask):
    """Kept-block density of the local heads (positional term) and of the diffuse
    (pure N(0,1)) heads, from the GPU CSR."""
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    per_head = np.diff(rp[::cfg.S]).reshape(cfg.batch, cfg.heads) / float(cfg.S * cfg.S)
    nl = cfg.n_local_heads()
    out = {"local": round(float(per_head[:, :nl].mean()), 5)}
    if nl < cfg.heads:
        out["diffuse"] = round(float(per_head[:, nl:].mean()), 5)
    out["heads"] = f"local {nl}, diffuse {cfg.heads - nl} per batch item"
    return out


def cpu_baseline(cfg, inputs, row_ptr, col_idx, exec_flops, budget_s):
    """Time the oracle on a bounded sample and extrapolate to one full call.  The
    whole-head masks the sample builds are also compared with the GPU's CSR:
    returns (baseline, mask_check) where mask_check counts the blocks whose oracle
    exclusive cumulative mass lies within 1e-4 of 1 - thr (the band) and the
    blocks on which the two masks differ (all of which must lie in the band)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = 1
    S, N = cfg.S, cfg.block
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    wmask = None
    if cfg.window is not None:
        wmask = oracle.sta_window(cfg.T, cfg.H // cfg.patch, cfg.W // cfg.patch, cfg.window)
    # mask: whole heads
    t0 = time.perf_counter()
    t_check = 0.0
    n_heads = 0
    band = mism = out_of_band = 0
    while True:
        b, h = divmod(n_heads, cfg.heads)
        m = oracle.head_mask(inputs["q"][b, h][src], inputs["k"][b, h][src], N, cfg.thr, wmask)
        tc = time.perf_counter()
        r0 = n_heads * S
        got = np.zeros((S, S), dtype=bool)
        lo = int(row_ptr[r0])
        got[np.repeat(np.arange(S), np.diff(row_ptr[r0:r0 + S + 1])), col_idx[lo:int(row_ptr[r0 + S])]] = True
        in_band = np.abs(m["cexcl"] - (1.0 - cfg.thr)) <= 1e-4 if cfg.thr > 0 else np.zeros((S, S), dtype=bool)
        diff = got != m["keep"]
        band += int(in_band.sum())
        mism += int(diff.sum())
        out_of_band += int((diff & ~in_band).sum())
        t_check += time.perf_counter() - tc
        n_heads += 1
        if time.perf_counter() - t0 - t_check > budget_s / 3 or n_heads >= cfg.batch * cfg.heads:
            break
    t_mask = (time.perf_counter() - t0 - t_check) / n_heads * cfg.batch * cfg.heads
    # attention: random CSR rows until the budget is used
    rng = np.random.default_rng(cfg.seed)
    order = rng.permutation(cfg.rows)
    t0 = time.perf_counter()
    flops = 0.0
    n_rows = 0
    for r in order:
        bh, i = divmod(int(r), S)
        b, h = divmod(bh, cfg.heads)
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]].astype(np.int64)
        ktok = src[(cols[:, None] * N + np.arange(N)).reshape(-1)]
        qf = inputs["q"][b, h][src[i * N:(i + 1) * N]][None, None].astype(np.float64)
        kf = inputs["k"][b, h][ktok][None, None].astype(np.float64)
        vf = inputs["v"][b, h][ktok][None, None].astype(np.float64)
        nb = len(cols)
        qpad = np.zeros((1, 1, N * nb, cfg.head_dim))
        qpad[:, :, :N] = qf
        oracle.block_sparse_attention(qpad, kf, vf, np.array([0, nb]), np.arange(nb, dtype=np.int32), N, rows=[0])
        flops += 4.0 * N * N * cfg.head_dim * nb
        n_rows += 1
        if time.perf_counter() - t0 > 2 * budget_s / 3:
            break
    t_attn = (time.perf_counter() - t0) / flops * exec_flops
    total = t_mask + t_attn
    check = {"heads": n_heads, "band_blocks": band, "mismatches": mism, "mismatches_outside_band": out_of_band,
             "what": "GPU CSR vs the oracle's whole-head masks built for the baseline sample"}
    return {
        "value": cfg.dense_flops / total / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: mask of {n_heads} of {cfg.batch * cfg.heads} heads and attention of "
                   f"{n_rows} of {cfg.rows} CSR rows ({flops / 1e9:.1f} GFLOP), extrapolated to one full call "
                   f"by head count and executed-FLOP share = {total:.1f} s per call"),
    }, check


def time_groups(bsa, cfg, q, k, v, g, steps, warmup, stream):
    """Event-timed key-group path: build_group_mask, prepare_v_groups and
    attend_groups on the same inputs.  A problem whose group CSR would need more
    than int32 offsets (batch*heads*S*L/4 >= 2^31) runs one call per batch item,
    all within the timed region.  Executed FLOPs: 4*64*64*D per gathered 64-key
    tile (ceil(groups/16) tiles per row)."""
    import torch
    D = q.shape[-1]
    parts = [slice(None)] if cfg.batch * cfg.heads * cfg.S * (cfg.L // 4) < 2 ** 31 else \
        [slice(b, b + 1) for b in range(cfg.batch)]
    qs, ks, vs = ([x[p] for p in parts] for x in (q, k, v))
    prob = bsa.make_problem(qs[0], g)
    gs = bsa.query_group_sizes(prob)
    mws = torch.empty(gs["mask_ws"], dtype=torch.uint8, device=q.device)
    fws = torch.empty(bsa.attend_groups_workspace_bytes(prob), dtype=torch.uint8, device=q.device)
    vg = torch.empty(qs[0].numel(), dtype=q.dtype, device=q.device)
    outs = [torch.empty_like(x) for x in qs]
    masks = [None] * len(parts)

    def one(ev=None):
        t = [0.0, 0.0, 0.0]
        for x in range(len(parts)):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            masks[x] = bsa.build_group_mask(qs[x], ks[x], g, cfg.thr, cfg.window, workspace=mws)
            e[1].record(stream)
            bsa.prepare_v_groups(vs[x], g, out=vg)
            e[2].record(stream)
            bsa.attend_groups(qs[x], ks[x], vg, masks[x], g, workspace=fws, out=outs[x])
            e[3].record(stream)
            if ev is not None:
                ev.append(e)

    for _ in range(max(1, warmup)):
        one()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        one(evs)
    torch.cuda.synchronize()
    per = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(3)]
    ms = [float(np.sum(x)) / steps for x in per]
    nnz = sum(m.nnz() for m in masks)
    tiles = sum(int(((m.row_ptr[1:] - m.row_ptr[:-1] + 15) // 16).sum()) for m in masks)
    flops = 4.0 * 64 * 64 * D * tiles
    tf = flops / (ms[2] * 1e-3) / 1e12
    total_groups = cfg.rows * (cfg.L // 4)
    return {"calls_per_step": len(parts), "ms_mask": round(ms[0], 4), "ms_prepare_v": round(ms[1], 4),
            "ms_attend": round(ms[2], 4), "ms_total": round(sum(ms), 4), "nnz_groups": nnz,
            "density": round(nnz / total_groups, 5), "tiles": tiles, "executed_tflop": round(flops / 1e12, 3),
            "attend_tflops": round(tf, 2), "attend_mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def time_backward(bsa, q, k, v, mask, g, fwd_ws, steps, warmup, stream):
    """Event-timed bsa_backward calls (one call = lse prep, transposed mask, operand
    transposes, the Delta walk, the dQ kernel and the dK/dV kernel) on the bench's mask,
    with a seeded N(0,1) dout.  Executed FLOPs count the 7 tile products of 64 x 64 x D
    (dQ: S, dP, dQ; dK/dV: S, dP, dV, dK) per kept tile; the Delta walk's two products
    (S, dP again) and the dQ kernel's second (low-part) dZ product are extra work on top.
    For bf16 head_dim 128 the training pair is timed as well (attend_train, then
    backward_train without the Delta walk)."""
    import torch
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    vt = bsa.prepare_v(v, g)
    o, lse = bsa.attend(q, k, vt, mask, g, workspace=fwd_ws, out=o, return_lse=True)
    del vt
    gen = torch.Generator(device=q.device)
    gen.manual_seed(1234)
    dout = torch.randn(q.shape, generator=gen, device=q.device, dtype=torch.float32).to(q.dtype)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    prob = bsa.make_problem(q, g)
    ws = torch.empty(max(bsa.backward_workspace_bytes(prob), 256), dtype=torch.uint8, device=q.device)
    for _ in range(max(1, warmup)):
        bsa.backward(q, k, v, mask, g, lse, dout, workspace=ws, out=grads)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        bsa.backward(q, k, v, mask, g, lse, dout, workspace=ws, out=grads)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    D = q.shape[-1]
    flops = 7.0 * 2 * g.block * g.block * D * mask.nnz()
    tf = flops / (ms * 1e-3) / 1e12
    res = {"ms_per_call": round(ms, 4), "executed_tflop": round(flops / 1e12, 3),
           "executed_tflops": round(tf, 2), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
           "dout": "seeded N(0,1), bf16"}
    if q.dtype == torch.bfloat16 and D == 128:
        # the training pair: attend_train (P as a bf16 pair in the PV product, o + o_lo)
        # and backward_train (row term from o + o_lo, no walk over the kept tiles)
        vt = bsa.prepare_v(v, g)
        pair = (torch.empty_like(q), torch.empty_like(q))
        for _ in range(max(1, warmup)):
            o_t, olo_t, lse_t = bsa.attend_train(q, k, vt, mask, g, workspace=fwd_ws, out=pair)
            bsa.backward_train(q, k, v, mask, g, o_t, olo_t, lse_t, dout, workspace=ws, out=grads)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for _ in range(steps):
            o_t, olo_t, lse_t = bsa.attend_train(q, k, vt, mask, g, workspace=fwd_ws, out=pair)
        ev[1].record(stream)
        for _ in range(steps):
            bsa.backward_train(q, k, v, mask, g, o_t, olo_t, lse_t, dout, workspace=ws, out=grads)
        ev[2].record(stream)
        torch.cuda.synchronize()
        fms = ev[0].elapsed_time(ev[1]) / steps
        bms = ev[1].elapsed_time(ev[2]) / steps
        btf = flops / (bms * 1e-3) / 1e12
        res["train_pair"] = {"attend_train_ms": round(fms, 4), "backward_train_ms": round(bms, 4),
                             "backward_train_tflops": round(btf, 2),
                             "backward_train_mfma_frac": round(btf / MFMA_BF16_PEAK_TFLOPS, 4),
                             "what": "attend_train (o, o_lo, lse) then backward_train (row term dO.(o+o_lo)); "
                                     "FLOPs as above (7 tile products), the forward's lo PV product on top"}
        del vt, pair
    return res


def time_short_rows(bsa, steps, warmup, stream, scratch):
    """The Wan2.1-scale workload (config 2: 2.8 % of the tiles kept, ~14 per row): the
    short-row regime, timed like the main line (events per stage, scratch written
    between steps) and reported beside it."""
    import torch
    from workloads import get_config, make_inputs
    cfg = get_config(2)
    dev = torch.device("cuda:0")
    inputs = make_inputs(cfg)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(inputs[n + "_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
               for n in "qkv")
    del inputs
    g = bsa.VideoGrid(cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block)
    sz = bsa.query_sizes(bsa.make_problem(q, g))
    mask_ws = torch.empty(sz["mask_ws"], dtype=torch.uint8, device=dev)
    fwd_ws = torch.empty(max(sz["fwd_ws"], 256), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for s in range(warmup + steps):
        if scratch.numel():
            scratch.fill_(s & 0xFF)
        ev = events[s - warmup] if s >= warmup else None
        if ev is not None:
            ev[0].record(stream)
        mask = bsa.build_mask(q, k, g, cfg.thr, cfg.window, workspace=mask_ws)
        if ev is not None:
            ev[1].record(stream)
        vt = bsa.prepare_v(v, g)
        if ev is not None:
            ev[2].record(stream)
        bsa.attend(q, k, vt, mask, g, workspace=fwd_ws, out=o)
        if ev is not None:
            ev[3].record(stream)
    torch.cuda.synchronize()
    st = [np.array([e[i].elapsed_time(e[i + 1]) for e in events]) for i in range(3)]
    nnz = mask.nnz()
    flops = 4.0 * cfg.block * cfg.block * cfg.head_dim * nnz
    att = float(np.median(st[2]))
    return {"workload": f"config 2 {cfg.name}: B={cfg.batch}, heads={cfg.heads}, T x H x W = {cfg.T}x{cfg.H}x{cfg.W}, "
                        f"thr={cfg.thr}",
            "build_mask_ms": {"median": round(float(np.median(st[0])), 4), "min": round(float(st[0].min()), 4)},
            "prepare_v_ms": {"median": round(float(np.median(st[1])), 4), "min": round(float(st[1].min()), 4)},
            "attend_ms": {"median": round(att, 4), "min": round(float(st[2].min()), 4)},
            "density": round(nnz / float(mask.rows * mask.S), 5),
            "attend_tflops": round(flops / (att * 1e-3) / 1e12, 2),
            "attend_frac": round(flops / (att * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "dense_equiv_tflops": round(cfg.dense_flops / (float(np.median(st[0] + st[1] + st[2])) * 1e-3) / 1e12, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--scratch-mb", type=int, default=512,
                    help="MB of scratch written between timed steps so that the 256 MB MALL holds none of the "
                         "inputs when a step starts (0 disables)")
    ap.add_argument("--config", type=int, default=None,
                    help="workload index (default 4: HunyuanVideo-scale hybrid; the default run also reports the "
                         "Wan2.1-scale config 2 figures under short_rows)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="CPU budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra", action="store_true", help="also print per-stage details on stderr")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward pass (dq, dk, dv) on the same mask after the forward steps")
    ap.add_argument("--groups", action="store_true",
                    help="also time the 4-token key-group path (group mask, V preparation, gathered attention)")
    ap.add_argument("--sip-seed", type=int, default=None,
                    help="build the mask by SIP sampling with this Philox seed instead of the CDF cut")
    args = ap.parse_args()
    short_rows = args.config is None and args.sip_seed is None
    if args.config is None:
        args.config = 4
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the hot path shards by (batch, head) "
                                   "without communication, so a multi-GPU figure is N independent copies of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import block_sparse_attention_fractal_amd as bsa
    from workloads import get_config, make_inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    bsa.lib()
    dev = torch.device("cuda:0")
    cfg = get_config(args.config)
    if cfg.dtype != "bf16":
        print(json.dumps({"error": "the benchmark times the bf16 MFMA path; pick a bf16 config (1-4)"}))
        sys.exit(2)

    t_gen = time.perf_counter()
    inputs = make_inputs(cfg)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(inputs[n + "_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
               for n in "qkv")
    for n in ("q_bits", "k_bits", "v_bits"):
        inputs.pop(n)
    t_gen = time.perf_counter() - t_gen
    g = bsa.VideoGrid(cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block)
    prob = bsa.make_problem(q, g)
    sz = bsa.query_sizes(prob)
    mask_ws = torch.empty(sz["mask_ws"], dtype=torch.uint8, device=dev)
    fwd_ws = torch.empty(max(sz["fwd_ws"], 256), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        mask = bsa.build_mask(q, k, g, cfg.thr, cfg.window, workspace=mask_ws, sip_seed=args.sip_seed)
        if ev is not None:
            ev[1].record(stream)
        vt = bsa.prepare_v(v, g)
        if ev is not None:
            ev[2].record(stream)
        bsa.attend(q, k, vt, mask, g, workspace=fwd_ws, out=o)
        if ev is not None:
            ev[3].record(stream)
        return mask

    scratch = torch.empty(max(args.scratch_mb, 0) << 20, dtype=torch.uint8, device=dev)

    def flush(i):
        if scratch.numel():
            scratch.fill_(i & 0xFF)   # a plain write kernel on the same stream, outside the step's events

    for i in range(args.warmup):
        flush(i)
        mask = step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        flush(s)
        mask = step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    per_stage = [np.array([e[i].elapsed_time(e[i + 1]) for e in events]) for i in range(3)]
    per_step = np.array([e[0].elapsed_time(e[3]) for e in events])
    attn_ms = float(per_stage[2].mean())                            # the roofline uses the average launch
    mask_ms, prep_ms = (float(np.median(x)) for x in per_stage[:2])  # HBM figures from the median

    def stats(x):
        return {"median": round(float(np.median(x)), 4), "min": round(float(x.min()), 4),
                "mean": round(float(x.mean()), 4)}

    nnz = mask.nnz()
    rows, S = mask.rows, mask.S
    density = nnz / float(rows * S)
    exec_flops = 4.0 * cfg.block * cfg.block * cfg.head_dim * nnz
    achieved = exec_flops / (attn_ms * 1e-3) / 1e12
    elt = 2
    mask_bytes = 2.0 * cfg.batch * cfg.heads * cfg.L * cfg.head_dim * elt + 4.0 * (rows + 1) + 4.0 * nnz
    mask_gbs = mask_bytes / (mask_ms * 1e-3) / 1e9
    mask_tr = mask_traffic(cfg.idx)       # counter-based HBM bytes per call (committed profile), or None
    prep_bytes = 2.0 * cfg.batch * cfg.heads * cfg.L * cfg.head_dim * elt
    prep_gbs = prep_bytes / (prep_ms * 1e-3) / 1e9
    value = cfg.dense_flops / (ms_step * 1e-3) / 1e12

    win = "none" if cfg.window is None else "+-%d,%d,%d tiles" % cfg.window
    line = {
        "metric": "block-sparse attn ms/call + dense-equiv TFLOP/s; % MFMA peak on executed FLOPs",
        "value": round(value, 3),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + positional term, bf16)",
        "config": {
            "workload": f"config {cfg.idx} {cfg.name}: B={cfg.batch}, heads={cfg.heads}, T x H x W = "
                        f"{cfg.T}x{cfg.H}x{cfg.W} (L={cfg.L}), D={cfg.head_dim}, P={cfg.patch}, N={cfg.block}, "
                        f"thr={cfg.thr}, window={win}",
            "global_batch": cfg.batch,
            "seq_len": cfg.L,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_for_current_kernel(cfg.idx),
            "kernel": "attn_bf16_kernel",
            "flops_per_launch": exec_flops,
            "avg_launch_ms": round(attn_ms, 4),
        },
        "stages_ms": {"build_mask": stats(per_stage[0]), "prepare_v": stats(per_stage[1]),
                      "attend": stats(per_stage[2]), "step_events": stats(per_step),
                      "timing": f"HIP events over {args.steps} steps, {args.scratch_mb} MB scratch written "
                                f"between steps (outside the events, inside ms_per_step)"},
        "mask_stage": {"algorithmic_bytes": mask_bytes, "gbs": round(mask_gbs, 1),
                       "hbm_frac": round(mask_gbs / HBM_PEAK_GBS, 4), "from": "median build_mask time",
                       "traffic": mask_tr,
                       "counter_gbs": None if mask_tr is None else round(mask_tr / (mask_ms * 1e-3) / 1e9, 1)},
        "prepare_v": {"gbs": round(prep_gbs, 1), "hbm_frac": round(prep_gbs / HBM_PEAK_GBS, 4)},
        "mask_mode": "cdf" if args.sip_seed is None else f"sip(seed={args.sip_seed})",
        "density": round(density, 5),
        "density_by_head_class": density_by_class(cfg, mask),
        "nnz": nnz,
        "executed_tflop": round(exec_flops / 1e12, 3),
        "input_gen_s": round(t_gen, 1),
    }
    if args.groups:
        line["groups"] = time_groups(bsa, cfg, q, k, v, g, args.steps, args.warmup, stream)
    if args.backward:
        line["backward"] = time_backward(bsa, q, k, v, mask, g, fwd_ws, args.steps, args.warmup, stream)
    if not args.no_cpu_baseline:
        rp = mask.row_ptr.cpu().numpy().astype(np.int64)
        ci = mask.col_idx[:nnz].cpu().numpy()
        line["cpu_baseline"], line["mask_check"] = cpu_baseline(cfg, inputs, rp, ci, exec_flops, args.cpu_seconds)
    if short_rows:
        del inputs, q, k, v, o, mask_ws, fwd_ws, mask
        torch.cuda.empty_cache()
        line["short_rows"] = time_short_rows(bsa, args.steps, args.warmup, stream, scratch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
