"""Benchmark of the persistent decode step on one MI355X.

Workload (synthetic, seeded): a 64-layer stack with hidden 5120, projections
5120 -> 10240 -> 5120 and a 5120 -> 17408 -> 5120 SiLU FFN per layer in
Q4_K-style blocks (13.40 GB), an fp16 lm_head of 151,936 x 5120, and a Gated
DeltaNet mixer (32 heads of 128 x 128 fp32 state) in 48 of the 64 layers, one
state per agent.  A step is one mk_decode_step call: one persistent launch
over all layers, lm_head, argmax and verification, plus the readback of the
accepted tokens.  The primary line is T = 12 rows (4 agents x [token + 2
drafts]); T = 1 and T = 5 (one sequence, 4 drafts) are measured too.

Each agent replays the largest possible number of ring rows every step
(T_agent - 1), which makes the Gated DeltaNet part of the step its most
expensive; drafts are uniform random ids.

Prints ONE JSON line.  --gpus N > 1 exits: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
HIDDEN, PROJ, FFN, VOCAB, LAYERS = 5120, 10240, 17408, 151936, 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_step_T12.json")
KERNEL_SOURCES = ["bit_weight_streaming_q4_amd/csrc/mk_step.hip", "bit_weight_streaming_q4_amd/csrc/mk_device.h",
                  "bit_weight_streaming_q4_amd/csrc/mk_gdn.h", "bit_weight_streaming_q4_amd/csrc/mk_lm.h",
                  "bit_weight_streaming_q4_amd/csrc/mk_attn.h"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stack_bytes(layers=LAYERS, hidden=HIDDEN, proj=PROJ, ffn=FFN) -> int:
    per = (proj * hidden + hidden * proj + 2 * ffn * hidden + hidden * ffn) // 256 * 144
    return per * layers


def step_bytes(T, n_agents, layers=LAYERS, vocab=VOCAB, hidden=HIDDEN, replay=True):
    """Algorithmic HBM bytes of one step: every weight block once, the lm_head
    once, each agent's GDN state read and written once, and the GDN step's
    inputs, outputs and ring traffic."""
    from synth.recipes import gdn_layers
    w = stack_bytes(layers)
    lm = vocab * hidden * 2
    nh = len(gdn_layers(layers)) * 32
    state = 2 * n_agents * nh * 128 * 128 * 4
    t_a = T // n_agents
    io = T * nh * (3 * 128 * 4 + 2 * 4) + T * nh * 128 * 4  # q, k, v, g, beta in; o out
    ring = n_agents * nh * 258 * 4 * (t_a - 1) * (2 if replay else 1)
    return {"weights": w, "lm_head": lm, "gdn": state + io + ring, "total": w + lm + state + io + ring}


# ------------------------------------------------------------------ setup
def build_stack(device="cuda", layers=LAYERS, progress=True):
    """Generates and uploads the 64-layer synthetic stack and the lm_head."""
    import torch

    import bit_weight_streaming_q4_amd as mk
    from synth import recipes

    t0 = time.time()
    Ls = []
    bufs = {}  # field arrays reused across layers (fresh arrays cost page faults)
    host = np.empty(mk.mk_q4k_bytes(FFN, HIDDEN), np.uint8)
    for l in range(layers):
        Ls.append({})
        for m in recipes.STACK_MATS:
            bufs[m] = recipes.stack_weight(l, m, out=bufs.get(m))
            Ls[-1][m] = mk.pack_to_device(bufs[m], device, host_buf=host)
        if progress and (l % 8 == 7 or l == layers - 1):
            log(f"layers generated {l + 1}/{layers} ({time.time() - t0:.1f}s)")
    lm = torch.from_numpy(recipes.stack_lm_head()).to(device)
    torch.cuda.synchronize()
    log(f"lm_head uploaded ({time.time() - t0:.1f}s)")
    return Ls, lm


def make_agents(n_agents, n_gdn_layers, T_max, device="cuda"):
    import torch

    import bit_weight_streaming_q4_amd as mk
    from synth import recipes

    out = []
    for a in range(n_agents):
        S0 = torch.from_numpy(recipes.stack_gdn_state(a, n_gdn_layers)).to(device)
        out.append(mk.DeltaNetState(n_gdn_layers * 32, T_max, device=device, S=S0.view(-1, 128, 128)))
    return out


def step_inputs(T, steps, n_gdn_layers, device="cuda"):
    """Seeded inputs of `steps` distinct steps: the T input rows and the
    Gated DeltaNet rows of every GDN layer (one set per step)."""
    import torch

    from synth import recipes
    xs = [torch.from_numpy(recipes.stack_step_input(s, T)).to(device) for s in range(steps)]
    gins = []
    for s in range(steps):
        g = recipes.stack_gdn_inputs(s, T, n_gdn_layers)
        gins.append({k: torch.from_numpy(v).to(device) for k, v in g.items()})
    return xs, gins


# ------------------------------------------------------------------ timing
def time_steps(stack, T, gs, n_agents, xs, gins, steps, warmup, attn=None):
    import torch

    import bit_weight_streaming_q4_amd as mk
    from synth import recipes
    dev = xs[0].device
    G = len(gs) - 1
    drafts = torch.from_numpy(np.ascontiguousarray(
        recipes.uniform_i32(2, 50000 + T, 0, max(T - G, 1), 0, VOCAB - 1))).to(dev)
    nh = gins[0]["q"].shape[1]
    go = torch.empty(T, nh, 128, dtype=torch.float32, device=dev)
    if attn is None:
        ws = stack.workspace(T, dev)
    else:
        gsa = np.asarray(gs, np.int32)
        ws = mk.workspace(int(mk.lib().mk_decode_step_attn_workspace(stack.h, T, gsa.ctypes.data, G,
                                                                       ctypes.byref(attn))), dev)
    xbuf = torch.empty_like(xs[0])
    # Each input's drafts are its own rows' argmax, so every draft is accepted
    # and every step replays the most ring rows possible (rows - 1 per agent)
    # from the accept lengths the previous step wrote; the argmax depends on
    # the input rows alone (the mixer outputs are not fed back).
    am = torch.empty(T, dtype=torch.int32, device=dev)
    drafts_of = []
    for i in range(len(xs)):
        xbuf.copy_(xs[i])
        mk.mk_decode_step(stack, xbuf, gs, drafts, gdn=gins[i % len(gins)], gdn_o=go, ws=ws, attn=attn, argmax=am)
        a = am.cpu().numpy()
        d = np.concatenate([a[gs[g]:gs[g + 1] - 1] for g in range(G)]).astype(np.int32)
        drafts_of.append(torch.from_numpy(d).to(dev) if d.size else drafts)
    accepted_all = []

    def one(i):
        xbuf.copy_(xs[i % len(xs)])
        tok, na = mk.mk_decode_step(stack, xbuf, gs, drafts_of[i % len(xs)], gdn=gins[i % len(gins)], gdn_o=go,
                                    ws=ws, attn=attn)
        accepted_all.append(bool(np.all(na == np.diff(gs) - 1)))
        return tok, na

    one(0)  # the accept lengths the first timed step replays
    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kernel_ms, wall_ms = [], []
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        t1 = time.perf_counter()
        one(warmup + i)  # returns after the step's one synchronisation
        wall_ms.append((time.perf_counter() - t1) * 1e3)
        kernel_ms.append(mk.mk_decode_step_last_ms(stack))
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_event = ev0.elapsed_time(ev1) / steps
    r = {"ms_per_step": wall * 1e3 / steps, "ms_event": ms_event, "kernel_ms": float(np.mean(kernel_ms)),
         "all_drafts_accepted": all(accepted_all),
         "kernel_ms_median": float(np.median(kernel_ms)),
         "kernel_ms_p10_p90": [float(np.percentile(kernel_ms, 10)), float(np.percentile(kernel_ms, 90))],
         "step_ms_median": float(np.median(wall_ms)),
         "step_ms_p10_p90": [float(np.percentile(wall_ms, 10)), float(np.percentile(wall_ms, 90))]}
    if os.environ.get("MK_BENCH_PHASES"):
        st = mk.mk_decode_step_stamps(stack, T, ws)
        L = (len(st) - 8) // 4  # stamps: start, prep, 4 per layer, lm_prep, ..., end
        n_layers = stack.d_layers
        d = np.diff(st[: 2 + 4 * n_layers + 1])
        per = d[1:1 + 4 * n_layers].reshape(n_layers, 4) * 1e6
        log(f"T={T} phases (us): prep {d[0] * 1e6:.1f}, per-layer mean P_in {per[:, 0].mean():.1f} "
            f"P_out {per[:, 1].mean():.1f} gate/up {per[:, 2].mean():.1f} down {per[:, 3].mean():.1f}, "
            f"lm_prep {d[-1] * 1e6:.1f}, lm+verify {(st[-1] - st[2 + 4 * n_layers]) * 1e6:.1f}, "
            f"total {st[-1] * 1e6:.1f}")
        log(f"T={T} P_out with GDN {per[[l for l in range(n_layers) if l % 4 != 3], 1].mean():.1f} us, "
            f"without {per[[l for l in range(n_layers) if l % 4 == 3], 1].mean():.1f} us")
    return r


def attention_step(layers, lm, gl, steps, warmup, q8=False, n_attn=16, ctx=32768):
    """The T = 12 step with its 16 full-attention layers' attention in the
    launch: 4 agents of 3 rows, each with `ctx` cached positions per layer
    (fp16 or q8_0 cache, 32 query / 8 KV heads of 128, gated).  Every layer's
    caches hold the same seeded values (the bytes read per layer are what
    matters here)."""
    import torch

    import bit_weight_streaming_q4_amd as mk
    from synth import recipes
    T, gs, G = 12, [0, 3, 6, 9, 12], 4
    sizes = [3] * G
    cap = recipes.attn_cap([ctx] * G, sizes)
    t0 = time.time()
    a = recipes.step_attn_inputs(n_attn, [ctx] * G, sizes, cap=cap, q8=q8)
    caches = []
    for key in (("k8", "ks", "v8", "vs") if q8 else ("k", "v")):
        one = torch.from_numpy(a[key]).to("cuda")
        c = torch.empty((n_attn,) + tuple(one.shape), dtype=one.dtype, device="cuda")
        for i in range(n_attn):
            c[i].copy_(one)
        caches.append(c)
        del one
    q, gate = torch.from_numpy(a["q"]).to("cuda"), torch.from_numpy(a["gate"]).to("cuda")
    o = torch.empty_like(q)
    fmt = "q8_0" if q8 else "fp16"
    log(f"attention inputs ({fmt}): {n_attn} layers x {G} agents x {ctx} positions ({time.time() - t0:.1f}s)")
    at = (mk.step_attn_q8 if q8 else mk.step_attn)(q, *caches, o, a["ctx"], gate=gate)
    agents = make_agents(G, len(gl), 5)
    stack = mk.Stack(layers, lm, gdn_layers=gl, agents=agents)
    xs, gins = step_inputs(T, min(steps + warmup, 8), len(gl))
    log(f"timing T=12 with attention ({fmt})")
    r = time_steps(stack, T, gs, G, xs, gins, steps, warmup, attn=at)
    b = step_bytes(T, G, len(layers))
    # bytes per cached position and KV head: fp16 K and V rows, or q8_0 codes
    # (2 x 128) and scales (K: 4 per position, V: 128 per 32 positions)
    per_pos = 2 * 128 * 2 if not q8 else 2 * 128 + 4 * 2 + 128 * 2 // 32
    kv = n_attn * sum(ctx + n for n in sizes) * recipes.ATTN_KV_HEADS * per_pos
    io = n_attn * T * recipes.ATTN_Q_HEADS * 128 * 4 * 3
    total = b["total"] + kv + io
    out = {"cache": fmt, "attention_layers": n_attn, "agents": G, "positions_per_agent": ctx, "rows": T,
           "ms_per_step": round(r["ms_per_step"], 4), "kernel_ms": round(r["kernel_ms"], 4),
           "kernel_ms_median": round(r["kernel_ms_median"], 4),
           "attention_bytes": int(kv + io), "total_bytes": int(total),
           "total_gb_s_kernel": round(total / (r["kernel_ms"] * 1e-3) / 1e9, 1),
           "frac_of_8TBs": round(total / (r["kernel_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    log(f"T=12 with attention ({fmt}): kernel {r['kernel_ms']:.3f} ms, {out['total_gb_s_kernel']:.0f} GB/s over "
        f"{total / 1e9:.2f} GB")
    stack.close()
    del stack, agents, caches, q, gate, o, at, xs, gins
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ standalone entry points
def _time_calls(fn, n, warm=3):
    """Mean ms per call of fn(i) over n calls, from events on the current stream."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(warm + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _time_graph(fn, n, out, state=(), reps=3):
    """Mean ms per call of fn(i), i < n, captured once in a HIP graph and
    replayed, so that no host launch cost is in the figure.  Every checked
    replay starts from the same device state (the tensors in state are
    restored) and its output out() must equal that of the same n calls made
    eagerly, with eager calls in between; returns (ms, same)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    snap = [t.clone() for t in state]

    def restore():
        for t, v in zip(state, snap):
            t.copy_(v)

    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    ref = out().clone()
    restore()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    same = True
    for _ in range(2):
        restore()
        g.replay()
        torch.cuda.synchronize()
        same = same and bool(torch.equal(out(), ref))
        fn(0)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n)
    del g
    restore()
    return ms, same


def kernel_bench(lm, device="cuda"):
    """The standalone entry points at the pages' single-kernel workloads, each
    on rotating device copies of its weights (more bytes than the 256 MB
    Infinity Cache, so every call streams from HBM): the T-row GEMV (5120 x
    5120), the FFN block (5120 -> 17408 -> 5120, T = 5), lm_head + verify
    (151936 x 5120 and the 32768-row draft prefix, T = 5), the Gated
    DeltaNet step + commit (48 x 32 heads of 128 x 128, T = 5) and
    full-attention decode over fp16 and q8_0 KV caches."""
    import torch

    import bit_weight_streaming_q4_amd as mk
    from synth import recipes
    out = {}

    def rec(name, fn, n, res, nbytes, state=()):
        """fn(i) timed eagerly (host launches included) and replayed from a
        HIP graph of n calls; res() is the output the graph check compares."""
        ms_eager = _time_calls(fn, n)
        ms, same = _time_graph(fn, n, res, state)
        if not same:
            log(f"kernel {name}: graph replay differs from eager calls; reporting the eager time")
            ms = ms_eager
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 2), "gb_s": round(gbs, 1), "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4),
                     "bytes": int(nbytes), "us_eager_calls": round(ms_eager * 1e3, 2),
                     "timing": "hip graph replay" if same else "eager calls"}
        log(f"kernel {name}: {ms * 1e3:.2f} us ({out[name]['timing']}; eager {ms_eager * 1e3:.2f} us), "
            f"{gbs:.0f} GB/s")

    # T-row GEMV, 64 copies (944 MB)
    W = mk.pack_to_device(recipes.gemv_weight(), device)
    copies = [W] + [mk.Q4K(W.blocks.clone(), W.n_out, W.n_in) for _ in range(63)]
    for T in (1, 5, 12):
        x = torch.from_numpy(recipes.rows_f32(T, HIDDEN)).to(device)
        y = torch.empty(T, HIDDEN, dtype=torch.float32, device=device)
        ws = mk.workspace(mk.mk_qgemv_rows_workspace(T, HIDDEN, HIDDEN), device)
        rec(f"qgemv_5120x5120_T{T}", lambda i: mk.mk_qgemv_rows(copies[i % 64], x, y, ws=ws), 128, lambda: y,
            HIDDEN * HIDDEN // 256 * 144 + T * 2 * HIDDEN * 4)
    del copies, W
    # FFN block, 4 copies (602 MB)
    fw = recipes.ffn_weights()
    g0, u0, d0 = (mk.pack_to_device(fw[m], device) for m in ("gate", "up", "down"))
    del fw
    sets = [(g0, u0, d0)] + [tuple(mk.Q4K(w.blocks.clone(), w.n_out, w.n_in) for w in (g0, u0, d0)) for _ in range(3)]
    for T in (1, 5, 12):
        x = torch.from_numpy(recipes.rows_f32(T, HIDDEN)).to(device)
        y = torch.empty(T, HIDDEN, dtype=torch.float32, device=device)
        ws = mk.workspace(mk.mk_ffn_rows_workspace(T, HIDDEN, FFN), device)
        rec(f"ffn_5120_17408_T{T}", lambda i: mk.mk_ffn_rows(*sets[i % 4], x, y, ws=ws), 32, lambda: y,
            3 * HIDDEN * FFN // 256 * 144 + T * 2 * HIDDEN * 4)
    del sets, g0, u0, d0
    torch.cuda.empty_cache()
    # lm_head + verify, T = 5 (one group, 4 drafts); full vocabulary and draft prefix
    T = 5
    hid = torch.from_numpy(recipes.lm_hidden(T)).to(device)
    drafts = torch.from_numpy(recipes.uniform_i32(3, 50, 0, T - 1, 0, VOCAB - 1)).to(device)
    am = torch.empty(T, dtype=torch.int32, device=device)
    na = torch.empty(1, dtype=torch.int32, device=device)
    tok = torch.empty(T, dtype=torch.int32, device=device)
    for V in (VOCAB, recipes.DRAFT_VOCAB):
        ws = mk.workspace(mk.mk_lmhead_verify_workspace(V, HIDDEN, T), device)
        rec(f"lmhead_verify_V{V}_T{T}", lambda i: mk.mk_lmhead_verify(lm, hid, None, drafts, am, na, tok, ws=ws, V=V),
            20, lambda: torch.cat([am, na, tok]), V * HIDDEN * 2 + T * HIDDEN * 4)
    # sampling-mode verification: 4 agents x 3 rows, top_k 32, temperature 0.6
    T12, gs12 = 12, [0, 3, 6, 9, 12]
    hid12 = torch.from_numpy(recipes.lm_hidden(T12, trial=1)).to(device)
    dr12 = torch.from_numpy(recipes.uniform_i32(3, 51, 0, 8, 0, VOCAB - 1)).to(device)
    ua = torch.from_numpy(recipes.uniform_f64(3, 52, 0, T12).astype(np.float32)).to(device)
    us = torch.from_numpy(recipes.uniform_f64(3, 53, 0, T12).astype(np.float32)).to(device)
    na4 = torch.empty(4, dtype=torch.int32, device=device)
    tok12 = torch.empty(T12, dtype=torch.int32, device=device)
    ws = mk.workspace(mk.mk_lmhead_sample_workspace(VOCAB, HIDDEN, T12), device)
    rec(f"lmhead_sample_V{VOCAB}_T{T12}_k32",
        lambda i: mk.mk_lmhead_sample(lm, hid12, gs12, dr12, 32, 0.6, ua, us, na4, tok12, ws=ws), 10,
        lambda: torch.cat([na4, tok12]), VOCAB * HIDDEN * 2 + T12 * HIDDEN * 4)
    del ws
    # the on-device MTP draft loop: 4 agents x 3 rows with 2 drafts each, and
    # one sequence of 5 rows with 4 drafts (passes x (fc + FFN + draft prefix))
    head = mk.MtpHead.from_fields(recipes.mtp_weights(), device)
    head_bytes = (2 * HIDDEN * HIDDEN + 3 * HIDDEN * FFN) // 256 * 144 + recipes.DRAFT_VOCAB * HIDDEN * 2
    for T, gs, nd, n_acc in ((12, [0, 3, 6, 9, 12], 2, [2, 0, 1, 2]), (5, [0, 5], 4, [3])):
        hidm = torch.from_numpy(recipes.stack_step_input(60, T)).to(device)
        toks = torch.from_numpy(recipes.uniform_i32(3, 54, T, T, 0, VOCAB - 1)).to(device)
        nacc = torch.tensor(n_acc, dtype=torch.int32, device=device)
        dr = torch.empty(nd, len(gs) - 1, dtype=torch.int32, device=device)
        ws = mk.workspace(mk.mk_mtp_draft_workspace(head, recipes.DRAFT_VOCAB, T, len(gs) - 1), device)
        rec(f"mtp_draft_T{T}_G{len(gs) - 1}_n{nd}",
            lambda i: mk.mk_mtp_draft(head, lm, recipes.DRAFT_VOCAB, hidm, gs, toks, nacc, nd, dr, ws=ws), 8,
            lambda: dr.flatten(), nd * head_bytes)
        del ws
    del head
    torch.cuda.empty_cache()
    # Gated DeltaNet step + commit, 48 x 32 heads, T = 5, seeded accept lengths
    nh = 48 * 32
    st = mk.DeltaNetState(nh, T, device=device,
                          S=torch.from_numpy(recipes.gdn_initial_state().reshape(nh, 128, 128)).to(device))
    g = recipes.gdn_step(0, T)
    gin = [torch.from_numpy(g[k]).to(device) for k in ("q", "k", "v", "g", "beta")]
    o = torch.empty(T, nh, 128, dtype=torch.float32, device=device)
    acc = recipes.gdn_accept_lengths(64, T)

    def gdn(i):
        st.n_acc[0:1].fill_(int(acc[i % 64]))
        mk.mk_deltanet_step(st, *gin, o)
    io = T * nh * (3 * 128 + 2) * 4 + T * nh * 128 * 4
    gdn_bytes = 2 * nh * 128 * 128 * 4 + io + nh * 258 * 4 * (T - 1) * 2
    rec(f"deltanet_step_48x32_T{T}", gdn, 32, lambda: torch.cat([o.flatten(), st.S.flatten()]), gdn_bytes,
        state=(st.S, st.ring, st.n_acc))
    # The 100 MB state fits the 256 MB Infinity Cache, so successive calls may
    # find it there.  Each call again after an untimed 1 GiB write that
    # evicts it: only the call is inside the events.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(16):
        flush.fill_(float(i))
        torch.cuda.synchronize()
        e0.record()
        gdn(i)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    gbs = gdn_bytes / (ms * 1e-3) / 1e9
    out[f"deltanet_step_48x32_T{T}_cache_flushed"] = {
        "us": round(ms * 1e3, 2), "gb_s": round(gbs, 1), "frac_of_8TBs": round(gbs / PEAK_HBM_GBS, 4),
        "bytes": int(gdn_bytes), "timing": "eager call after an untimed 1 GiB write, median of 16"}
    log(f"kernel deltanet_step_48x32_T{T}_cache_flushed: {ms * 1e3:.2f} us, {gbs:.0f} GB/s")
    del flush
    del st
    torch.cuda.empty_cache()
    # Full-attention decode (32 query / 8 KV heads of 128, gated, fp16 cache):
    # 4 agents x 32768 cached positions with 3 rows each (T = 12), and one
    # agent at 81920 positions (the long end of the fp16 cache) with T = 5.
    # Two caches alternate, so successive calls stream from HBM.
    for ctx, sizes in (([32768] * 4, [3] * 4), ([81920], [5])):
        a = recipes.attn_inputs(ctx, sizes)
        q = torch.from_numpy(a["q"]).to(device)
        gt = torch.from_numpy(a["gate"]).to(device)
        kc = torch.from_numpy(a["k"].view(np.int16)).to(device)
        vc = torch.from_numpy(a["v"].view(np.int16)).to(device)
        del a
        caches = [(kc, vc), (kc.clone(), vc.clone())]
        o = torch.empty_like(q)
        T = int(sum(sizes))
        gs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        ws = mk.workspace(mk.mk_attn_decode_workspace(T, q.shape[1], kc.shape[1], ctx, gs), device)
        nbytes = attn_bytes(ctx, sizes)
        rec(f"attn_decode_{len(ctx)}x{ctx[0]}_T{T}",
            lambda i: mk.mk_attn_decode(q, gt, *caches[i % 2], ctx, gs, o, ws=ws), 16, lambda: o, nbytes)
        del caches, kc, vc
        torch.cuda.empty_cache()
    # The same over a q8_0 cache: 4 x 32768 at T = 12, and one agent at 131072
    # positions (the pages' long-context setting, where the cache is q8_0).
    for ctx, sizes in (([32768] * 4, [3] * 4), ([131072], [5])):
        a = recipes.attn_inputs_q8(ctx, sizes)
        q = torch.from_numpy(a["q"]).to(device)
        gt = torch.from_numpy(a["gate"]).to(device)
        t = [torch.from_numpy(a["k8"]).to(device), torch.from_numpy(a["ks"].view(np.int16)).to(device),
             torch.from_numpy(a["v8"]).to(device), torch.from_numpy(a["vs"].view(np.int16)).to(device)]
        del a
        sets = [t, [x.clone() for x in t]]
        o = torch.empty_like(q)
        T = int(sum(sizes))
        gs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        ws = mk.workspace(mk.mk_attn_decode_workspace(T, q.shape[1], t[0].shape[1], ctx, gs), device)
        rec(f"attn_decode_q8_{len(ctx)}x{ctx[0]}_T{T}",
            lambda i: mk.mk_attn_decode_q8(q, gt, *sets[i % 2], ctx, gs, o, ws=ws), 16, lambda: o,
            attn_bytes_q8(ctx, sizes))
        del sets, t
        torch.cuda.empty_cache()
    return out


def attn_bytes_q8(ctx, sizes, Hq=32, Hkv=8, d=128) -> int:
    """Algorithmic bytes of one q8_0 attention call: every visible K and V
    code once, the K scales of visible positions, the V scales of the 32-
    position blocks holding them, plus q, gate and o (fp32)."""
    L = [int(c) + int(n) for c, n in zip(ctx, sizes)]
    codes = sum(L) * Hkv * d * 2
    scales = sum(L) * Hkv * (d // 32) * 2 + sum((x + 31) // 32 for x in L) * Hkv * d * 2
    return codes + scales + int(sum(sizes)) * Hq * d * 4 * 3


def attn_bytes(ctx, sizes, Hq=32, Hkv=8, d=128) -> int:
    """Algorithmic bytes of one attention decode call: every visible K and V
    row once (fp16) plus q, gate and o (fp32)."""
    kv = sum(int(c) + int(n) for c, n in zip(ctx, sizes)) * Hkv * d * 2 * 2
    return kv + int(sum(sizes)) * Hq * d * 4 * 3


def read_probe(device="cuda", gib=4, reps=5):
    """Read bandwidth the device attains: mk_read_probe over a 4 GiB buffer
    (16 x the Infinity Cache), timed with events over `reps` calls."""
    import torch

    import bit_weight_streaming_q4_amd as mk
    buf = torch.ones(gib << 28, dtype=torch.float32, device=device)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    mk.mk_read_probe(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mk.mk_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = buf.numel() * 4 / (ms * 1e-3) / 1e9
    log(f"read probe: {gib} GiB in {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    del buf
    torch.cuda.empty_cache()
    return round(gbs, 1)


# ------------------------------------------------------------------ lm_head workload: accept lengths
def accept_histogram(lm, trials=200, device="cuda"):
    """The lm_head + verify workload over `trials` seeded trials: T = 5 rows,
    4 drafts, draft i the argmax of row i with probability 0.7 (the argmax
    from a first call), else a uniform id.  Returns the n_acc histogram, its
    mean against 0.7 + 0.49 + 0.343 + 0.2401 = 1.7731 and the chi-square
    against P(k) = 0.7^k 0.3 (k < 4), 0.7^4."""
    import torch

    import bit_weight_streaming_q4_amd as mk
    from synth import recipes
    T = 5
    am = torch.empty(T, dtype=torch.int32, device=device)
    na = torch.empty(1, dtype=torch.int32, device=device)
    tok = torch.empty(T, dtype=torch.int32, device=device)
    zero = torch.zeros(T - 1, dtype=torch.int32, device=device)
    ws = mk.workspace(mk.mk_lmhead_verify_workspace(VOCAB, HIDDEN, T), device)
    hist = np.zeros(5, np.int64)
    for tr in range(trials):
        hid = torch.from_numpy(recipes.lm_hidden(T, trial=tr)).to(device)
        mk.mk_lmhead_verify(lm, hid, None, zero, am, na, tok, ws=ws)
        top = am.cpu().numpy()
        dr = torch.from_numpy(recipes.drafts_from_argmax(top[:T - 1], VOCAB, trial=tr)).to(device)
        mk.mk_lmhead_verify(lm, hid, None, dr, am, na, tok, ws=ws)
        hist[int(na.item())] += 1
    p = np.array([0.3, 0.21, 0.147, 0.1029, 0.2401])
    chi2 = float((((hist - trials * p) ** 2) / (trials * p)).sum())
    mean = float((hist * np.arange(5)).sum() / trials)
    log(f"accept lengths over {trials} trials: {hist.tolist()}, mean {mean:.4f} (expected 1.7731), chi2 {chi2:.2f}")
    return {"trials": trials, "histogram": hist.tolist(), "mean": round(mean, 4), "expected_mean": 1.7731,
            "chi2_4dof": round(chi2, 2), "chi2_crit_p001": 18.47}


def manifest(seeds):
    """What the numbers were measured on: device, software versions, clocks,
    a hash of the sources, the seeds and the host cores."""
    import platform

    import torch
    h = hashlib.sha256()
    for root in ("bit_weight_streaming_q4_amd/csrc", "include", "oracle", "synth"):
        for f in sorted(os.listdir(os.path.join(ROOT, root))):
            if f.endswith((".hip", ".h", ".c", ".py")):
                with open(os.path.join(ROOT, root, f), "rb") as fh:
                    h.update(fh.read())
    with open(os.path.join(ROOT, "bench.py"), "rb") as fh:
        h.update(fh.read())
    prop = torch.cuda.get_device_properties(0)
    m = {"gpu": torch.cuda.get_device_name(0) or HOST_FACTS.get("product") or "",
         "arch": getattr(prop, "gcnArchName", ""),
         "compute_units": prop.multi_processor_count, "hbm_bytes": prop.total_memory,
         "torch": torch.__version__, "hip": torch.version.hip, "python": platform.python_version(),
         "host_cores": len(os.sched_getaffinity(0)), "source_sha256_16": h.hexdigest()[:16], "seeds": seeds}
    try:
        with open("/sys/module/amdgpu/version") as f:
            m["amdgpu_driver"] = f.read().strip()
    except OSError:
        m["amdgpu_driver"] = None
    m.update(HOST_FACTS)
    return m


# Facts that come from other programs (clocks, git), gathered by host_facts()
# before this process touches the GPU: a child process started from a process
# that has initialised the GPU must not exec another program.
HOST_FACTS = {"clocks": None, "git_sha": None, "product": None}


def host_facts():
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        clk = json.loads(r.stdout) if r.returncode == 0 and r.stdout.strip().startswith("{") else {}
        card = next(iter(clk.values()), {}) if clk else {}
        HOST_FACTS["clocks"] = {k: v for k, v in card.items() if "clk" in k.lower()} or None
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showproductname", "--json"], capture_output=True, text=True, timeout=20)
        prod = json.loads(r.stdout) if r.returncode == 0 and r.stdout.strip().startswith("{") else {}
        card = next(iter(prod.values()), {}) if prod else {}
        name = card.get("Card Series") or card.get("Card series") or card.get("Card Model") or card.get("Card model")
        HOST_FACTS["product"] = str(name).strip() if name and str(name).strip() not in ("N/A", "") else None
    except (OSError, ValueError, subprocess.SubprocessError, AttributeError):
        pass
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True, text=True,
                           timeout=10)
        HOST_FACTS["git_sha"] = r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        pass


def cpu_baseline_one_core(T=12):
    """The oracle on one core (OMP_NUM_THREADS=1, in a child process that
    touches no GPU, started before this process touches the GPU): the first
    layer's P_in GEMV (5120 -> 10240) at T = 12, reported as weight GB/s."""
    import subprocess
    code = ("import json, time, sys; sys.path.insert(0, %r)\n"
            "import oracle\nfrom synth import recipes\n"
            "W = recipes.stack_weight(0, 'p_in'); x = recipes.stack_step_input(0, %d)\n"
            "oracle.qgemv(W, x[:1])\n"
            "t0 = time.perf_counter(); oracle.qgemv(W, x); dt = time.perf_counter() - t0\n"
            "print(json.dumps({'s': dt}))\n") % (ROOT, T)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    if r.returncode != 0:
        log(f"one-core oracle run failed: {r.stderr[-300:]}")
        return None
    dt = json.loads(r.stdout.strip().splitlines()[-1])["s"]
    nbytes = PROJ * HIDDEN // 256 * 144
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 P_in ({PROJ} x {HIDDEN}) at T={T}, {dt:.2f} s"}


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(T=12, budget_s=20.0):
    """The oracle (as it stands) on a bounded sample of the same step at
    T = 12: the stack's layers in order (each layer's weights generated
    outside the timed region, then P_in, P_out, gate, up, down through the
    oracle), until about budget_s seconds of oracle time, then 1/4 of the
    lm_head rows on the final hidden rows; timed on this host's cores and
    reported as weight GB/s."""
    import oracle
    from synth import recipes
    cores = len(os.sched_getaffinity(0))
    x = recipes.stack_step_input(0, T)
    dt, layers = 0.0, 0
    for l in range(LAYERS):
        Wl = {m: recipes.stack_weight(l, m) for m in recipes.STACK_MATS}
        t0 = time.perf_counter()
        x = oracle.layer(x, Wl)
        dt += time.perf_counter() - t0
        layers += 1
        del Wl
        if dt > budget_s:
            break
    lmrows = VOCAB // 4
    W16 = recipes.stack_lm_head(r1=lmrows)
    t0 = time.perf_counter()
    oracle.lmhead(W16, oracle.rmsnorm(x))
    dt += time.perf_counter() - t0
    nbytes = stack_bytes(layers) + lmrows * HIDDEN * 2
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{layers} of {LAYERS} layers + {lmrows} of {VOCAB} lm_head rows at T={T}, {dt:.1f} s of oracle time"}


def cpu_entry_points():
    """The oracle (as it stands) beside each standalone call that bench times
    on the GPU (same names as config.standalone_kernels): one bounded sample
    of the call's workload, timed on this host's cores and scaled by the
    sample's share of the call.  us is the oracle's time for one whole call
    at that scale, gb_s the call's algorithmic bytes over that time."""
    import oracle
    from synth import recipes
    out = {}

    def put(name, dt, scale, nbytes, sample):
        us = dt * scale * 1e6
        out[name] = {"us": round(us, 1), "gb_s": round(nbytes / (us * 1e-6) / 1e9, 4), "sample": sample,
                     "oracle_s_per_sample": round(dt, 4)}

    def timed(fn, min_s=0.25):
        """Mean time of fn over as many calls as fill min_s (at least one)."""
        n, t0 = 0, time.perf_counter()
        while True:
            r = fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return dt / n, r

    W = recipes.gemv_weight()
    for T in (1, 5, 12):
        x = recipes.rows_f32(T, HIDDEN)
        dt, _ = timed(lambda: oracle.qgemv(W, x))
        put(f"qgemv_5120x5120_T{T}", dt, 1, HIDDEN * HIDDEN // 256 * 144 + T * 2 * HIDDEN * 4, "the whole call")
    del W
    fw = recipes.ffn_weights()
    x = recipes.rows_f32(5, HIDDEN)
    dt, _ = timed(lambda: oracle.ffn(fw["gate"], fw["up"], fw["down"], x))
    put("ffn_5120_17408_T5", dt, 1, 3 * HIDDEN * FFN // 256 * 144 + 5 * 2 * HIDDEN * 4, "the whole call")
    del fw
    # lm_head + verify and the sampling verify: 1/16 of the vocabulary
    part = 16
    rows = VOCAB // part
    W16 = recipes.stack_lm_head(r1=rows)
    hid = recipes.lm_hidden(5)
    drafts = recipes.uniform_i32(3, 50, 0, 4, 0, rows - 1)
    dt, _ = timed(lambda: oracle.verify(oracle.lmhead(W16, hid)["top1"], [0, 5], drafts))
    put(f"lmhead_verify_V{VOCAB}_T5", dt, part, VOCAB * HIDDEN * 2 + 5 * HIDDEN * 4,
        f"{rows} of {VOCAB} vocabulary rows, x {part}")
    hid12 = recipes.lm_hidden(12, trial=1)
    gs12 = [0, 3, 6, 9, 12]
    dr12 = recipes.uniform_i32(3, 51, 0, 8, 0, rows - 1)
    ua, us = recipes.uniform_f64(3, 52, 0, 12), recipes.uniform_f64(3, 53, 0, 12)

    def sample_call():
        lg = oracle.lmhead(W16, hid12, return_logits=True)["logits"]
        ti, tv = oracle.topk_rows(lg, 32)
        return oracle.sample_verify(ti, tv, gs12, dr12, 0.6, ua, us)
    dt, _ = timed(sample_call)
    put(f"lmhead_sample_V{VOCAB}_T12_k32", dt, part, VOCAB * HIDDEN * 2 + 12 * HIDDEN * 4,
        f"{rows} of {VOCAB} vocabulary rows, x {part}")
    del W16
    # Gated DeltaNet step: 384 of the 1536 heads, T = 5, committed through row 4
    nh, sh = 48 * 32, 384
    S = recipes.gdn_initial_state().reshape(nh, 128, 128)[:sh].copy()
    g = recipes.gdn_step(0, 5)
    gi = [np.ascontiguousarray(g[k].reshape(5, nh, -1)[:, :sh]) for k in ("q", "k", "v")]
    gb = [np.ascontiguousarray(g[k].reshape(5, nh)[:, :sh]) for k in ("g", "beta")]
    dt, _ = timed(lambda: oracle.gdn_step(S, *gi, *gb, 4))
    io = 5 * nh * (3 * 128 + 2) * 4 + 5 * nh * 128 * 4
    put("deltanet_step_48x32_T5", dt, nh / sh, 2 * nh * 128 * 128 * 4 + io + nh * 258 * 4 * 4 * 2,
        f"{sh} of {nh} heads, x {nh // sh}")
    del S
    # attention: one of the four agents at 32768 positions (3 rows), x 4
    a = recipes.attn_inputs([32768], [3])
    dt, _ = timed(lambda: oracle.attn_decode(a["q"], a["gate"], a["k"], a["v"], a["ctx"], a["group_start"]))
    put("attn_decode_4x32768_T12", dt, 4, attn_bytes([32768] * 4, [3] * 4), "1 of 4 agents, x 4")
    del a
    a = recipes.attn_inputs_q8([32768], [3])
    dt, _ = timed(lambda: oracle.attn_decode_q8(a["q"], a["gate"], a["k8"], a["ks"], a["v8"], a["vs"], a["ctx"],
                                                a["group_start"]))
    put("attn_decode_q8_4x32768_T12", dt, 4, attn_bytes_q8([32768] * 4, [3] * 4), "1 of 4 agents, x 4")
    del a
    # MTP draft loop, 4 agents x 3 rows, 2 drafts: the catch-up pass over the
    # accepted rows (2 + 0 + 1 + 2, plus one each) and the second pass over
    # one row per agent, each pass with its draft lm_head over 1/16 of the
    # 32768-row draft vocabulary (x 16 for that part)
    mtp = recipes.mtp_weights()
    dv = recipes.DRAFT_VOCAB // part
    Wd = recipes.stack_lm_head(r1=dv)
    hidm = recipes.stack_step_input(60, 12)
    toks = recipes.uniform_i32(3, 54, 12, 12, 0, dv - 1)
    rows0 = [0, 1, 2, 3, 6, 7, 9, 10, 11]
    dt0, x0 = timed(lambda: oracle.mtp_block(mtp, Wd, toks[rows0], hidm[rows0]))
    dl0, _ = timed(lambda: oracle.lmhead(Wd, oracle.rmsnorm(x0[[2, 3, 5, 8]])))
    dt1, x1 = timed(lambda: oracle.mtp_block(mtp, Wd, toks[:4], x0[[2, 3, 5, 8]]))
    dl1, _ = timed(lambda: oracle.lmhead(Wd, oracle.rmsnorm(x1)))
    head_bytes = (2 * HIDDEN * HIDDEN + 3 * HIDDEN * FFN) // 256 * 144 + recipes.DRAFT_VOCAB * HIDDEN * 2
    put("mtp_draft_T12_G4_n2", dt0 + dt1 + part * (dl0 + dl1), 1, 2 * head_bytes,
        f"both passes; their draft lm_head over {dv} of {recipes.DRAFT_VOCAB} rows, x {part}")
    out["mtp_draft_T12_G4_n2"]["oracle_s_per_sample"] = round(dt0 + dt1 + dl0 + dl1, 4)
    return out


# ------------------------------------------------------------------ HBM traffic record
def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_per_dispatch(d, counter, kernel_sub):
    """Mean over the matching dispatches of the counter's value (summed over
    its instances within a dispatch)."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if kernel_sub in r.get("Kernel_Name", "") and r.get("Counter_Name") == counter:
            k = r.get("Dispatch_Id") or r.get("Correlation_Id")
            per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for {kernel_sub} under {d}")
    return float(np.mean(list(per.values()))), len(per)


def traffic_record(root):
    """The traffic record of k_decode_step<12, false> (the step without
    attention items) from rocprofv3 output under
    root: trace/ (--kernel-trace --stats), fetch/ and write/ (--pmc FETCH_SIZE,
    WRITE_SIZE on the bench), copy_fetch/ and copy_write/ (the same counters on
    --copy-probe).  Counter values are KiB per dispatch; each is scaled by what
    the same counter reads for the plain 1 GiB copy."""
    kern = "k_decode_step<12, false>"
    stats = [r for r in _csv_rows(os.path.join(root, "trace"), "kernel_stats.csv") if kern in r.get("Name", "")]
    avg_ns, calls = float(stats[0]["AverageNs"]), int(stats[0]["Calls"])
    fetch, nf = _counter_per_dispatch(os.path.join(root, "fetch"), "FETCH_SIZE", kern)
    write, nw = _counter_per_dispatch(os.path.join(root, "write"), "WRITE_SIZE", kern)
    # the copy probe's device-to-device copies (its first dispatch is the fill of the source)
    cf, _ = _counter_per_dispatch(os.path.join(root, "copy_fetch"), "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_per_dispatch(os.path.join(root, "copy_write"), "WRITE_SIZE", "copyBuffer")
    copy_bytes = 1 << 30
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    rd, wr = fetch * 1024 * fs, write * 1024 * ws
    return {"kernel": kern, "kernel_source_hash": kernel_source_hash(), "fetch_size_kib_per_dispatch": fetch,
            "write_size_kib_per_dispatch": write, "dispatches_fetch": nf, "dispatches_write": nw,
            "copy_probe_bytes": copy_bytes, "copy_probe_fetch_kib": cf, "copy_probe_write_kib": cw,
            "fetch_scale": fs, "write_scale": ws, "bytes_per_launch": int(rd + wr), "read_bytes_per_launch": int(rd),
            "write_bytes_per_launch": int(wr), "algorithmic_bytes_per_launch": step_bytes(12, 4)["total"],
            "kernel_avg_ns": avg_ns, "kernel_calls": calls}


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only-primary", action="store_true", help="measure T = 12 only")
    ap.add_argument("--rows", metavar="T,T,...", help="measure only these row counts (one verify group each, except "
                                                      "T = 12 and 24: 4 and 8 agents of 3 rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the standalone entry-point timings")
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--sweep", action="store_true", help="also time the step at every T in 1..16")
    ap.add_argument("--series", type=int, default=100,
                    help="also time this many seeded T = 12 steps, each with its own inputs (0: skip)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="write the traffic record from rocprofv3 output under DIR (no GPU work) and exit")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the HBM byte counters)")
    ap.add_argument("--ffn-calls", type=int, metavar="T", default=0,
                    help="only make 24 eager mk_ffn_rows calls at T rows on rotating weight copies (for a kernel "
                         "trace of the FFN's launches)")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the T = 12 step with the attention layers in the launch")
    ap.add_argument("--no-children", action="store_true",
                    help="start no child process (no clocks, git SHA or one-core oracle run): for runs under a "
                         "profiler that initialises the GPU in this process before it starts")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        rec = traffic_record(args.traffic_from)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec), flush=True)
        return
    # every child process starts here, before this process touches the GPU
    one_core = None
    if not args.copy_probe and not args.ffn_calls and not args.no_children:
        host_facts()
        if not args.no_cpu_baseline:
            one_core = cpu_baseline_one_core()
    import torch

    import __graft_entry__
    import bit_weight_streaming_q4_amd as mk
    from synth import recipes
    if not os.path.exists(mk.LIB_PATH):
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mk.mk_init(0)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": src.numel() * 4, "copy_probe_bytes_written": dst.numel() * 4,
                          "launches": 3}), flush=True)
        return
    if args.ffn_calls:
        T = args.ffn_calls
        fw = recipes.ffn_weights()
        g0, u0, d0 = (mk.pack_to_device(fw[m], "cuda") for m in ("gate", "up", "down"))
        del fw
        sets = [(g0, u0, d0)] + [tuple(mk.Q4K(w.blocks.clone(), w.n_out, w.n_in) for w in (g0, u0, d0))
                                 for _ in range(3)]
        x = torch.from_numpy(recipes.rows_f32(T, HIDDEN)).to("cuda")
        y = torch.empty(T, HIDDEN, dtype=torch.float32, device="cuda")
        ws = mk.workspace(mk.mk_ffn_rows_workspace(T, HIDDEN, FFN), "cuda")
        for i in range(24):
            mk.mk_ffn_rows(*sets[i % 4], x, y, ws=ws)
        torch.cuda.synchronize()
        print(json.dumps({"ffn_calls": 24, "rows": T}), flush=True)
        return
    L = args.layers
    gl = recipes.gdn_layers(L)
    layers, lm = build_stack(layers=L)
    results = {}
    series = None
    # the metric's rows (T = 12, 5, 1), then eight agents of three rows (T = 24)
    configs = [(12, [0, 3, 6, 9, 12], 4), (5, [0, 5], 1), (1, [0, 1], 1), (24, list(range(0, 25, 3)), 8)]
    if args.sweep:  # one verify group of T rows, one agent
        configs += [(T, [0, T], 1) for T in (2, 3, 4, 6, 7, 8, 9, 10, 11, 13, 14, 15, 16)]
    for T, gs, n_agents in configs:
        if args.only_primary and T != 12:
            continue
        if args.rows and T not in [int(t) for t in args.rows.split(",")]:
            continue
        agents = make_agents(n_agents, len(gl), max(5, gs[1] - gs[0]))  # ring rows for the longest group
        stack = mk.Stack(layers, lm, gdn_layers=gl, agents=agents)
        xs, gins = step_inputs(T, min(args.steps + args.warmup, 8), len(gl))
        log(f"timing T={T}")
        r = time_steps(stack, T, gs, n_agents, xs, gins, args.steps, args.warmup)
        b = step_bytes(T, n_agents, L)
        r["bytes"] = b
        r["weight_gb_s"] = (b["weights"] + b["lm_head"]) / (r["ms_event"] * 1e-3) / 1e9
        r["total_gb_s"] = b["total"] / (r["ms_event"] * 1e-3) / 1e9
        r["kernel_gb_s"] = b["total"] / (r["kernel_ms"] * 1e-3) / 1e9
        r["steps_per_s"] = 1e3 / r["ms_per_step"]
        r["agents"] = n_agents
        results[T] = r
        log(f"T={T}: {r['ms_per_step']:.3f} ms/step (events {r['ms_event']:.3f}, kernel {r['kernel_ms']:.3f}), "
            f"weights {r['weight_gb_s']:.0f} GB/s, total {r['total_gb_s']:.0f} GB/s, kernel {r['kernel_gb_s']:.0f} GB/s")
        if T == 12 and not args.only_primary and args.series:
            # the stack workload as defined: 100 seeded steps, each with its own input rows and GDN rows
            del xs, gins
            torch.cuda.empty_cache()
            xs, gins = step_inputs(T, args.series, len(gl))
            log(f"timing T=12 over {args.series} seeded steps")
            rs = time_steps(stack, T, gs, n_agents, xs, gins, args.series, 0)
            series = {"steps": args.series, "all_drafts_accepted": rs["all_drafts_accepted"],
                      "kernel_ms_mean": round(rs["kernel_ms"], 4),
                      "kernel_ms_median": round(rs["kernel_ms_median"], 4),
                      "kernel_ms_p10_p90": [round(v, 4) for v in rs["kernel_ms_p10_p90"]],
                      "step_ms_median": round(rs["step_ms_median"], 4),
                      "step_ms_p10_p90": [round(v, 4) for v in rs["step_ms_p10_p90"]],
                      "weight_gb_s_median_kernel": round((b["weights"] + b["lm_head"]) / (rs["kernel_ms_median"] * 1e-3)
                                                         / 1e9, 1)}
        stack.close()
        del stack, agents
        del xs, gins
        torch.cuda.empty_cache()
    p = results[12]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tj = json.load(open(TRAFFIC_FILE))
        if tj.get("kernel_source_hash") == kernel_source_hash():
            traffic = tj.get("bytes_per_launch")
    attention = attention_q8 = None
    if not (args.no_attention or args.only_primary):
        attention = attention_step(layers, lm, gl, args.steps, args.warmup)
        attention_q8 = attention_step(layers, lm, gl, args.steps, args.warmup, q8=True)
    kernels = None if args.no_kernels else kernel_bench(lm)
    accepts = None if args.no_kernels else accept_histogram(lm)
    attainable = read_probe()
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    if cpu is not None:
        cpu["one_core"] = one_core
        if not args.no_kernels:
            cpu["entry_points"] = cpu_entry_points()
    seeds = {"stack": recipes.STACK_SEED, "lm_head": recipes.LM_SEED, "gdn": recipes.GDN_SEED,
             "mtp": recipes.STACK_SEED, "step_inputs": "stack seed, tensors 10000 + step and 20000 + step"}
    out = {
        "metric": "weight-stream GB/s (% of 8 TB/s) and decode steps/s at T=1,5,12 rows",
        "value": round(p["weight_gb_s"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(p["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4k-int8",
        "data": "synthetic (seeded Q4_K-style weights, fp16 lm_head, fp32 Gated DeltaNet states)",
        "config": {"workload": "64-layer Q4_K-style stack (hidden 5120, proj 10240, ffn 17408) + fp16 lm_head "
                               "151936x5120 + 48 GDN layers x 4 agents, T=12 (4 agents x 3 rows), one "
                               "persistent launch per step",
                   "rows": 12, "layers": L, "weight_bytes_per_step": p["bytes"]["weights"] + p["bytes"]["lm_head"],
                   "pct_of_8TBs": round(100 * p["weight_gb_s"] / PEAK_HBM_GBS, 2),
                   "per_T": {str(T): {"agents": r["agents"], "lm_head_streams": (T + 15) // 16,
                                      "ms_per_step": round(r["ms_per_step"], 4),
                                      "steps_per_s": round(r["steps_per_s"], 2),
                                      "rows_steps_per_s": round(r["steps_per_s"] * T, 1),
                                      "weight_gb_s": round(r["weight_gb_s"], 1),
                                      "total_gb_s": round(r["total_gb_s"], 1),
                                      "kernel_ms": round(r["kernel_ms"], 4),
                                      "kernel_ms_median": round(r["kernel_ms_median"], 4),
                                      "kernel_ms_p10_p90": [round(v, 4) for v in r["kernel_ms_p10_p90"]],
                                      "step_ms_median": round(r["step_ms_median"], 4),
                                      "step_ms_p10_p90": [round(v, 4) for v in r["step_ms_p10_p90"]],
                                      "all_drafts_accepted": r["all_drafts_accepted"]}
                             for T, r in sorted(results.items())},
                   "seeded_series_T12": series,
                   "with_attention_T12": attention,
                   "with_attention_q8_T12": attention_q8,
                   "lm_head_accept_lengths": accepts,
                   "standalone_kernels": kernels},
        "manifest": manifest(seeds),
        "roofline": {"bound": "hbm", "achieved": round(p["kernel_gb_s"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(p["kernel_gb_s"] / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "k_decode_step<12, false>", "kernel_ms": round(p["kernel_ms"], 4),
                     "algorithmic_bytes_per_launch": p["bytes"]["total"],
                     "attainable_read_gb_s": attainable},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    # explicit teardown: every device object of the run is released here, with
    # the device idle, not in finalizers at interpreter exit
    del layers, lm
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
