"""CPU oracle of the multi-row speculative-decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product library
(``bit_weight_streaming_q4_amd``) never imports, links or calls it, and shares
no code with it; the two meet only through the seeded inputs of :mod:`synth`.

The arithmetic lives in ``oracle.c`` (plain C, double accumulation, no FMA
contraction); this module marshals numpy arrays and composes the C steps in
the order the pages give them.  Each function names the step it follows:

  C1 dequant        Q4_K-style superblock -> fp32 weights
  C2 quantize_rows  per-32 int8 activation quantization
  C3 qgemv          T-row GEMV (dequantize, accumulate in double)
  C4 ffn            SiLU(gate) * up, then down
  C5 layer          pre-RMSNorm, projections, FFN, fp32 residual (synthetic glue)
  C6 lmhead/verify  logits, argmax, accepted-prefix length, emitted tokens
  C7 gdn_step       gated delta rule with commit through the accepted row
  C8 decode_step    composition of one whole step
  M1 mtp_block      one pass of the synthetic MTP draft head
  M2 mtp_draft      catch-up rows, then the draft steps (draft vocabulary prefix)
  F1 topk_rows      the k largest logits of each row (sampling mode)
  F2 sample_weights target weights softmax(top-k / temperature)
  F3 sample_verify  sampling-mode verification that keeps the target distribution
  A1 attn_decode    full-attention decode of T rows over an fp16 KV cache
  A2 attn_decode_q8 the same over a q8_0 KV cache

Pages: richland.au "Fusing the whole speculative-decoding cycle into one CUDA
kernel" (section "What shipped"), richland.au "OpenJet's CUDA megakernel runs
4 coding agents" (section "Why it matters"), pulse-3k2 "UPDATE: ... KL
divergence" (section "Decode accuracy").

Parity status: every function is pinned in tests/test_oracle_pins.py against
something other than itself: C1-C4, C6, C7, A1 and A2 against brute force,
closed forms and library routines; C5 (the layer glue, a reading of the pages:
pre-RMSNorm, identity mixer, fp32 residual) against an identity case and an
independent float64 numpy evaluation of the same definition; C8 against
planted drafts, a float64 numpy argmax and a full-matrix delta-rule recompute
of the committed state.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liborc.so")
_lib = None
RMS_EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile ``liborc.so`` with gcc: -O2, OpenMP, no FMA contraction, no fast-math."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-D_GNU_SOURCE",
               "-shared", "-fPIC", os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f32.restype = ctypes.c_float
    lib.orc_dequant.argtypes = [P, P, P, P, P, i32, i32, P]
    lib.orc_quantize_rows.argtypes = [P, i32, i32, P, P, P]
    lib.orc_qgemv_q8.argtypes = [P, P, P, P, P, i32, i32, P, P, i32, P]
    lib.orc_qgemv.argtypes = [P, P, P, P, P, i32, i32, P, i32, P]
    lib.orc_q4k_partials.argtypes = [P, i32, i32, P, i32, P]
    lib.orc_silu_mul.argtypes = [P, P, i64, P]
    lib.orc_ffn.argtypes = [P] * 15 + [i32, i32, P, i32, P, P]
    lib.orc_rmsnorm.argtypes = [P, i32, i32, dbl, P]
    lib.orc_residual_add.argtypes = [P, P, i64]
    lib.orc_lmhead.argtypes = [P, i32, i32, P, i32, P, P, P, P, P, P, P]
    lib.orc_verify.argtypes = [P, P, i32, P, P, P]
    lib.orc_gdn_rows.argtypes = [P, i32, i32, P, P, P, P, P, i32, i64, i64, i64, P, i64, ctypes.c_int]
    lib.orc_gdn_step.argtypes = [P, i32, i32, i32, P, P, P, P, P, i32, i32, P]
    lib.orc_attn_decode.argtypes = [P, P, i32, i32, P, P, i32, i32, i32, P, P, i32, P]
    lib.orc_attn_decode_q8.argtypes = [P, P, i32, i32, P, P, P, P, i32, i32, i32, P, P, i32, P]
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data if a is not None else None


def _fields(W):
    d = _c(W["d"], np.uint16)
    dmin = _c(W["dmin"], np.uint16)
    sc = _c(W["sc"], np.uint8)
    m = _c(W["m"], np.uint8)
    q = _c(W["q"], np.uint8)
    return d, dmin, sc, m, q


def f16_to_f32(bits: int) -> float:
    return float(_load().orc_f16_to_f32(int(bits)))


def dequant(W) -> np.ndarray:
    """C1: fp32 weights [N][K] of a field-array matrix."""
    d, dmin, sc, m, q = _fields(W)
    N, K = q.shape
    w = np.empty((N, K), np.float32)
    _load().orc_dequant(_p(d), _p(dmin), _p(sc), _p(m), _p(q), N, K, _p(w))
    return w


def quantize_rows(x):
    """C2: (a8 int8 [T][K], s fp32 [T][K/32], gsum int32 [T][K/32])."""
    x = _c(np.atleast_2d(x), np.float32)
    T, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    a8 = np.empty((T, K), np.int8)
    s = np.empty((T, K // 32), np.float32)
    gs = np.empty((T, K // 32), np.int32)
    _load().orc_quantize_rows(_p(x), T, K, _p(a8), _p(s), _p(gs))
    return a8, s, gs


def qgemv_q8(W, a8, s) -> np.ndarray:
    """C3 on quantized rows: y fp32 [T][N]."""
    d, dmin, sc, m, q = _fields(W)
    N, K = q.shape
    a8 = _c(a8, np.int8)
    s = _c(s, np.float32)
    T = a8.shape[0]
    y = np.empty((T, N), np.float32)
    _load().orc_qgemv_q8(_p(d), _p(dmin), _p(sc), _p(m), _p(q), N, K, _p(a8), _p(s), T, _p(y))
    return y


def qgemv(W, x) -> np.ndarray:
    """C3: y fp32 [T][N] = W . q8(x)."""
    d, dmin, sc, m, q = _fields(W)
    N, K = q.shape
    x = _c(np.atleast_2d(x), np.float32)
    T = x.shape[0]
    assert x.shape[1] == K
    y = np.empty((T, N), np.float32)
    _load().orc_qgemv(_p(d), _p(dmin), _p(sc), _p(m), _p(q), N, K, _p(x), T, _p(y))
    return y


def q4k_partials(W, a8) -> np.ndarray:
    """Exact integer partial sums P[t][o][g] = sum_{i<32} q*a8 over group g."""
    q = _c(W["q"], np.uint8)
    N, K = q.shape
    a8 = _c(a8, np.int8)
    T = a8.shape[0]
    P = np.empty((T, N, K // 32), np.int32)
    _load().orc_q4k_partials(_p(q), N, K, _p(a8), T, _p(P))
    return P


def silu_mul(g, u) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.empty_like(g)
    _load().orc_silu_mul(_p(g), _p(u), g.size, _p(h))
    return h


def ffn(Wg, Wu, Wd, x, return_h=False):
    """C4: y = W_d . q8(SiLU(W_g . q8(x)) * (W_u . q8(x)))."""
    x = _c(np.atleast_2d(x), np.float32)
    T, H = x.shape
    F = Wg["q"].shape[0]
    arrs = list(_fields(Wg)) + list(_fields(Wu)) + list(_fields(Wd))
    y = np.empty((T, H), np.float32)
    h = np.empty((T, F), np.float32)
    _load().orc_ffn(*[_p(a) for a in arrs], H, F, _p(x), T, _p(y), _p(h))
    return (y, h) if return_h else y


def rmsnorm(x, eps=RMS_EPS) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    T, K = x.shape
    a = np.empty_like(x)
    _load().orc_rmsnorm(_p(x), T, K, eps, _p(a))
    return a


def residual_add(x, y) -> np.ndarray:
    out = _c(x, np.float32).copy()
    y = _c(y, np.float32)
    _load().orc_residual_add(_p(out), _p(y), out.size)
    return out


def layer(x, Wl) -> np.ndarray:
    """C5 (one synthetic layer; the glue is a reading of the pages: the
    workload lists only the projections and the FFN): pre-RMSNorm with unit
    gain, identity mixer, fp32 residual:
    x += P_out.q8(P_in.q8(RMSNorm x)); x += FFN(RMSNorm x)."""
    u = qgemv(Wl["p_in"], rmsnorm(x))
    x = residual_add(x, qgemv(Wl["p_out"], u))
    return residual_add(x, ffn(Wl["gate"], Wl["up"], Wl["down"], rmsnorm(x)))


def decode_step(x, layers, W16, group_start, drafts, gdn=None, n_layers=None, teacher=None, progress=None) -> dict:
    """C8: one whole decode step, composed in the pages' order (richland.au
    single-stream article, "What shipped"; the 4-agent article, "Why it
    matters"): the T rows x [T][H] pass every layer (C5); the final residual
    is RMSNorm'ed and goes through lm_head with its argmax (C6); each group's
    drafts are verified against its rows' argmax (C6); then each agent's Gated
    DeltaNet state absorbs the agent's rows 0..n_acc of this step (C7), so the
    committed state ends at the accepted token.

    layers: list of per-layer field dicts (p_in, p_out, gate, up, down), or a
    callable l -> dict (then n_layers is required) so that a large stack is
    generated one layer at a time.
    teacher: optional [L][T][H] residuals of another path; layer l > 0 then
    starts from teacher[l - 1] instead of the oracle's own layer l - 1, and
    the lm_head input is teacher[L - 1] (stage-wise comparison).
    gdn: None, or a dict with "S" (list of per-agent states [nh][dk][dv]) and
    the step's rows "q", "k", "v" [T][nh][d], "g", "beta" [T][nh].
    progress: optional callable (l, trace_l) run after each layer.
    Returns trace [L][T][H] (residual after each layer), hid, argmax, n_acc,
    tokens and, with gdn, the committed states "S" and outputs "gdn_o"."""
    x = _c(np.atleast_2d(x), np.float32)
    if callable(layers):
        if n_layers is None:
            raise ValueError("n_layers is required with a layer generator")
        get = layers
    else:
        n_layers = len(layers)
        get = layers.__getitem__
    trace = np.empty((n_layers,) + x.shape, np.float32)
    cur = x
    for l in range(n_layers):
        if teacher is not None and l > 0:
            cur = _c(teacher[l - 1], np.float32)
        cur = layer(cur, get(l))
        trace[l] = cur
        if progress is not None:
            progress(l, cur)
    final = trace[-1] if teacher is None else _c(teacher[-1], np.float32)
    hid = rmsnorm(final)
    r = lmhead(W16, hid)
    n_acc, tokens = verify(r["top1"], group_start, drafts)
    out = {"trace": trace, "hid": hid, "argmax": r["top1"], "lm": r, "n_acc": n_acc, "tokens": tokens}
    if gdn is not None:
        gs = list(group_start)
        S_new, o_all = [], np.empty_like(_c(gdn["v"], np.float32))
        for a in range(len(gs) - 1):
            r0, r1 = gs[a], gs[a + 1]
            S1, o = gdn_step(gdn["S"][a], gdn["q"][r0:r1], gdn["k"][r0:r1], gdn["v"][r0:r1], gdn["g"][r0:r1],
                             gdn["beta"][r0:r1], int(n_acc[a]))
            S_new.append(S1)
            o_all[r0:r1] = o
        out["S"], out["gdn_o"] = S_new, o_all
    return out


def mtp_block(mtp, E16, tokens, h_rows) -> np.ndarray:
    """M1: one pass of the synthetic MTP draft head over rows (token, hidden):
    z = [RMSNorm(f32 E[token]) ; RMSNorm(hidden)] (2H), u = fc . q8(z),
    x' = u + FFN(RMSNorm(u)).  A token outside [0, V) contributes a zero
    embedding.  Returns x' [rows][H] (rounded to fp32 at every stage the GPU
    stores).  The head's layers are a reading: the pages name only the
    head's work (richland.au single-stream article, "What shipped": MTP
    catch-up rows for accepted tokens, then n_draft draft steps)."""
    tokens = np.asarray(tokens, np.int64)
    h_rows = _c(np.atleast_2d(h_rows), np.float32)
    V, H = E16.shape
    e = np.zeros((len(tokens), H), np.float32)
    for i, t in enumerate(tokens):
        if 0 <= t < V:
            e[i] = np.asarray(E16[t], np.uint16).view(np.float16).astype(np.float32)
    z = np.concatenate([rmsnorm(e), rmsnorm(h_rows)], axis=1)
    u = qgemv(mtp["fc"], z)
    return residual_add(u, ffn(mtp["gate"], mtp["up"], mtp["down"], rmsnorm(u)))


def mtp_draft(mtp, E16, V_draft, hidden, tokens, group_start, n_acc, n_draft) -> dict:
    """M2: the on-device MTP draft loop of one step (richland.au single-stream
    article, "What shipped": catch-up rows for the accepted tokens, then the
    draft steps, drafting over the 32,768 most frequent tokens).  Group g's
    catch-up rows are its rows i = 0..n_acc[g]: main-model hidden (final
    residual) of row i with the token emitted after it, tokens[gs[g] + i] (the
    accepted drafts, then the bonus token).  The last catch-up row gives
    draft 1 = argmax over the first V_draft rows of E16 (tied lm_head) of
    RMSNorm(x'); draft k + 1 comes from a pass over (draft k, x' of draft k's
    pass), one row per group.  Returns drafts [n_draft][G], "catchup" (x' of
    every catch-up row, dict row -> [H]) and "chain" (x' [n_draft][G][H] of
    the row that produced each draft)."""
    gs = list(group_start)
    G = len(gs) - 1
    hidden = _c(np.atleast_2d(hidden), np.float32)
    drafts = np.zeros((n_draft, G), np.int32)
    chain = np.zeros((n_draft, G, hidden.shape[1]), np.float32)
    catchup = {}
    Wd = E16[:V_draft]
    for g in range(G):
        rows = list(range(gs[g], gs[g] + int(n_acc[g]) + 1))
        xp = mtp_block(mtp, E16, [tokens[r] for r in rows], hidden[rows])
        for j, r in enumerate(rows):
            catchup[r] = xp[j]
        chain[0, g] = xp[-1]
    drafts[0] = lmhead(Wd, rmsnorm(chain[0]))["top1"]
    for k in range(1, n_draft):
        chain[k] = mtp_block(mtp, E16, drafts[k - 1], chain[k - 1])
        drafts[k] = lmhead(Wd, rmsnorm(chain[k]))["top1"]
    return {"drafts": drafts, "catchup": catchup, "chain": chain}


def lmhead(W16, hid, return_logits=False) -> dict:
    """C6 logits: argmax (lowest index on ties, NaN never wins), runner-up and
    the sums of |W*hid| of both (for the near-tie bound)."""
    W16 = _c(W16, np.uint16)
    V, H = W16.shape
    hid = _c(np.atleast_2d(hid), np.float32)
    T = hid.shape[0]
    out = {k: np.empty(T, np.int32) for k in ("top1", "top2")}
    for k in ("top1_val", "top2_val", "abs1", "abs2"):
        out[k] = np.empty(T, np.float64)
    lg = np.empty((T, V), np.float64) if return_logits else None
    _load().orc_lmhead(_p(W16), V, H, _p(hid), T, _p(lg), _p(out["top1"]), _p(out["top1_val"]),
                       _p(out["top2"]), _p(out["top2_val"]), _p(out["abs1"]), _p(out["abs2"]))
    if return_logits:
        out["logits"] = lg
    return out


def near_tie_tau(H, abs1, abs2):
    """Near-tie bound per row: 8 * 2^-24 * sqrt(H) * max(sum|W h|) of the top two."""
    return 8.0 * 2.0 ** -24 * np.sqrt(H) * np.maximum(abs1, abs2)


def verify(argmax, group_start, drafts):
    """C6 verify: (n_acc [G], tokens [T]); unused token slots are -1."""
    argmax = _c(argmax, np.int32)
    gs = _c(group_start, np.int32)
    G = len(gs) - 1
    drafts = _c(drafts, np.int32)
    n_acc = np.empty(G, np.int32)
    tokens = np.full(len(argmax), -1, np.int32)
    _load().orc_verify(_p(argmax), _p(gs), G, _p(drafts), _p(n_acc), _p(tokens))
    return n_acc, tokens


def topk_rows(logits, k):
    """F1: per row, the k largest logits (NaN never counts), ties broken
    towards the lower vocabulary index; returns (idx, val) [T][k], each row's
    candidates in ascending vocabulary order (the order the sampler walks),
    padded with idx -1 and val -inf when a row has fewer than k non-NaN
    logits."""
    lg = np.atleast_2d(np.asarray(logits, np.float64))
    T, V = lg.shape
    out_i = np.full((T, k), -1, np.int32)
    out_v = np.full((T, k), -np.inf)
    for t in range(T):
        ok = np.flatnonzero(~np.isnan(lg[t]))
        order = ok[np.lexsort((ok, -lg[t, ok]))][:k]  # value descending, then index ascending
        sel = np.sort(order)
        out_i[t, :len(sel)] = sel
        out_v[t, :len(sel)] = lg[t, sel]
    return out_i, out_v


def sample_weights(vals, temperature):
    """F2: unnormalised target weights of one row's top-k candidates,
    exp((l - max l) / temperature), in float64 (padding slots, -inf, weigh 0)."""
    v = np.asarray(vals, np.float64)
    if not np.isfinite(v).any():
        return np.zeros_like(v)
    return np.exp((v - v[np.isfinite(v)].max()) / float(temperature))


def _inverse_cdf(w, u, skip=None):
    """Index j of the candidate picked by u in [0, 1): walk the candidates in
    the given (ascending vocabulary) order, the first whose cumulative
    weight exceeds u * total; candidate `skip` has weight 0.  Also returns
    the distance of u * total from the nearest cumulative boundary, relative
    to the total (for the comparison carve-out)."""
    w = np.array(w, np.float64)
    if skip is not None:
        w[skip] = 0.0
    tot = w.sum()
    x = u * tot
    c = np.cumsum(w)
    j = int(np.searchsorted(c, x, side="right"))
    j = min(j, len(w) - 1)
    while w[j] == 0.0 and j > 0:  # past the end by rounding: the last candidate with weight
        j -= 1
    gap = float(np.min(np.abs(c - x)) / tot) if tot > 0 else 0.0
    return j, gap


def sample_verify(topk_idx, topk_val, group_start, drafts, temperature, u_acc, u_samp):
    """F3: sampling-mode verification of drafted rows, keeping the target
    distribution (pulse-3k2, "UPDATE: ... KL divergence 0.0009 vs llama.cpp",
    "Decode accuracy vs llama.cpp": sampling keeps the same distribution as
    without drafts; top_k capped at 32 per the single-stream and 4-agent
    pages' limits).  The rule (a reading: the pages give none) is
    speculative sampling with each draft a deterministic proposal.  Row i of
    a group has the target p_i = softmax(top-k logits / temperature).  For
    i = 0, 1, ...: draft d_i is accepted when u_acc[i] < p_i(d_i)
    (p_i(d) = 0 for a token outside the top-k or outside [0, V)); at the
    first rejection the row emits a sample of p_i with d_i removed and
    renormalised (u_samp[i], inverse CDF over the candidates in ascending
    vocabulary order) and the group stops; if every draft is accepted, the
    last row emits a sample of p (its bonus token).  Each emitted token is
    then distributed exactly as p_i: P(d) = p(d) + 0, and for x != d,
    (1 - p(d)) p(x) / (1 - p(d)) = p(x).
    Returns n_acc [G], tokens [T] (-1 past the emitted ones) and, per row, the
    decision margin (distance of u from its decision boundary, relative)."""
    gs = list(group_start)
    G = len(gs) - 1
    T = gs[-1]
    drafts = np.asarray(drafts, np.int64)
    n_acc = np.zeros(G, np.int32)
    tokens = np.full(T, -1, np.int32)
    margin = np.full(T, np.inf)
    for g in range(G):
        r, n = gs[g], gs[g + 1] - gs[g]
        a = 0
        while True:
            t = r + a
            w = sample_weights(topk_val[t], temperature)
            tot = w.sum()
            if tot == 0.0:  # no candidate (every logit NaN): the draft is rejected and nothing is emitted
                tokens[t] = -1
                margin[t] = np.inf
                break
            if a < n - 1:
                d = int(drafts[r - g + a])
                hit = np.flatnonzero((topk_idx[t] == d) & (d >= 0))
                pd = w[hit[0]] / tot if len(hit) else 0.0
                margin[t] = abs(u_acc[t] - pd)
                if u_acc[t] < pd:
                    tokens[t] = d
                    a += 1
                    continue
                j, gap = _inverse_cdf(w, u_samp[t], skip=hit[0] if len(hit) else None)
            else:
                j, gap = _inverse_cdf(w, u_samp[t])
            margin[t] = min(margin[t], gap)
            tokens[t] = int(topk_idx[t][j])
            break
        n_acc[g] = a
    return n_acc, tokens, margin


def gdn_rows(S, q, k, v, g, beta, literal=False):
    """C7 rows on one head: S (float64 [dk][dv]) is updated in place; returns o [n][dv]."""
    assert S.dtype == np.float64 and S.flags["C_CONTIGUOUS"]
    dk, dv = S.shape
    k = _c(np.atleast_2d(k), np.float32)
    v = _c(np.atleast_2d(v), np.float32)
    n = k.shape[0]
    q = _c(np.atleast_2d(q), np.float32) if q is not None else None
    g = _c(np.atleast_1d(g), np.float32)
    beta = _c(np.atleast_1d(beta), np.float32)
    o = np.empty((n, dv), np.float32) if q is not None else None
    _load().orc_gdn_rows(_p(S), dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta), n, dk, dv, 1, _p(o), dv,
                         int(bool(literal)))
    return o


def gdn_step(S, q, k, v, g, beta, a):
    """C7 + C8 on nh heads: S fp32 [nh][dk][dv] (or [L][H][dk][dv]) is replaced
    by the state committed through row a; returns o [T][nh][dv]."""
    S32 = _c(S, np.float32).copy()
    shp = S32.shape
    dk, dv = shp[-2], shp[-1]
    nh = S32.size // (dk * dv)
    q = _c(q, np.float32).reshape(-1, nh, dk)
    T = q.shape[0]
    k = _c(k, np.float32).reshape(T, nh, dk)
    v = _c(v, np.float32).reshape(T, nh, dv)
    g = _c(g, np.float32).reshape(T, nh)
    beta = _c(beta, np.float32).reshape(T, nh)
    if not 0 <= a < T:
        raise ValueError("accept length out of range")
    o = np.empty((T, nh, dv), np.float32)
    _load().orc_gdn_step(_p(S32), nh, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta), T, int(a), _p(o))
    return S32.reshape(shp), o


def attn_decode(q, gate, kc, vc, ctx, group_start=None) -> np.ndarray:
    """A1: full-attention decode.  q, gate (or None) fp32 [T][Hq][d]; kc fp16
    bits [G][Hkv][cap][d]; vc fp16 bits [G][Hkv][d][cap] (dimension-major);
    ctx [G] positions cached before the step; group_start [G+1] (None = one
    group).  Row i of group g sees positions 0..ctx[g]+i.  Returns o fp32
    [T][Hq][d]."""
    q = _c(q, np.float32)
    T, Hq, d = q.shape
    kc = _c(kc, np.uint16)
    vc = _c(vc, np.uint16)
    G, Hkv, cap, dk = kc.shape
    if dk != d or vc.shape != (G, Hkv, d, cap) or Hq % Hkv:
        raise ValueError("attention: shape mismatch")
    ctx = _c(np.asarray(ctx), np.int32)
    gs = _c(np.asarray([0, T] if group_start is None else group_start), np.int32)
    if len(ctx) != G or len(gs) != G + 1 or gs[0] != 0 or gs[-1] != T or np.any(np.diff(gs) <= 0):
        raise ValueError("attention: bad groups")
    if np.any(ctx < 0) or np.any(ctx + np.diff(gs) > cap):
        raise ValueError("attention: context exceeds the cache")
    gate = _c(gate, np.float32) if gate is not None else None
    o = np.empty((T, Hq, d), np.float32)
    _load().orc_attn_decode(_p(q), _p(gate), T, Hq, _p(kc), _p(vc), Hkv, d, cap, _p(ctx), _p(gs), G, _p(o))
    return o


def attn_decode_q8(q, gate, k8, ks, v8, vs, ctx, group_start=None) -> np.ndarray:
    """A2: attention over q8_0 caches.  k8 int8 [G][Hkv][cap][d] with ks fp16
    bits [G][Hkv][cap][d/32]; v8 int8 [G][Hkv][cap/64][d][64] (tile-major)
    with vs fp16 bits [G][Hkv][cap/32][d]; otherwise as attn_decode."""
    q = _c(q, np.float32)
    T, Hq, d = q.shape
    k8 = _c(k8, np.int8)
    v8 = _c(v8, np.int8)
    ks = _c(ks, np.uint16)
    vs = _c(vs, np.uint16)
    G, Hkv, cap, dk = k8.shape
    if (dk != d or d % 32 or cap % 64 or v8.shape != (G, Hkv, cap // 64, d, 64) or ks.shape != (G, Hkv, cap, d // 32)
            or vs.shape != (G, Hkv, cap // 32, d) or Hq % Hkv):
        raise ValueError("attention q8: shape mismatch")
    ctx = _c(np.asarray(ctx), np.int32)
    gs = _c(np.asarray([0, T] if group_start is None else group_start), np.int32)
    if len(ctx) != G or len(gs) != G + 1 or gs[0] != 0 or gs[-1] != T or np.any(np.diff(gs) <= 0):
        raise ValueError("attention q8: bad groups")
    if np.any(ctx < 0) or np.any(ctx + np.diff(gs) > cap):
        raise ValueError("attention q8: context exceeds the cache")
    gate = _c(gate, np.float32) if gate is not None else None
    o = np.empty((T, Hq, d), np.float32)
    _load().orc_attn_decode_q8(_p(q), _p(gate), T, Hq, _p(k8), _p(ks), _p(v8), _p(vs), Hkv, d, cap, _p(ctx),
                               _p(gs), G, _p(o))
    return o
