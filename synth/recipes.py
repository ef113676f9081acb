"""Workload recipes: which seeded streams and distributions each synthetic
workload draws.  Shapes mirror a 27B dense hybrid decoder (hidden 5120,
FFN 17408, 64 layers of which 48 are Gated DeltaNet layers, 32 heads of
128, vocabulary 151,936).  Every tensor is regenerable on its own from
(seed, tensor id); nothing here computes any part of the decode method.
"""
from __future__ import annotations

import numpy as np

from . import gdn_step_inputs, normal_f16, normal_f32, q4k_fields, uniform_f64, uniform_i32

HIDDEN = 5120
FFN = 17408
PROJ = 10240
VOCAB = 151936
DRAFT_VOCAB = 32768
N_LAYERS = 64
GDN_HEADS = 32
GDN_DK = 128
GDN_DV = 128


def gdn_layers(n_layers: int = N_LAYERS) -> list[int]:
    """Layers that carry a Gated DeltaNet mixer: three of every four (the
    fourth is a full-attention layer), giving 48 of 64."""
    return [l for l in range(n_layers) if l % 4 != 3]


# ---------------------------------------------------------------- single GEMV
def gemv_weight(n_out=HIDDEN, n_in=HIDDEN, seed=0, tensor=1, r0=0, r1=None):
    return q4k_fields(seed, tensor, n_out, n_in, r0, r1)


def rows_f32(T, K, seed=0, tensor=2):
    """T activation rows ~ N(0, 1), fp32, [T][K]."""
    return normal_f32(seed, tensor, 0, T * K).reshape(T, K)


# ---------------------------------------------------------------- FFN block
def ffn_weights(hidden=HIDDEN, ffn=FFN, seed=1, base=11):
    return {
        "gate": q4k_fields(seed, base + 0, ffn, hidden),
        "up": q4k_fields(seed, base + 1, ffn, hidden),
        "down": q4k_fields(seed, base + 2, hidden, ffn),
    }


# ---------------------------------------------------------------- layer stack
STACK_SEED = 2
STACK_MATS = ("p_in", "p_out", "gate", "up", "down")


def stack_tensor_id(layer: int, mat: str) -> int:
    return 100 + 8 * layer + STACK_MATS.index(mat)


def stack_shapes(hidden=HIDDEN, proj=PROJ, ffn=FFN) -> dict:
    return {"p_in": (proj, hidden), "p_out": (hidden, proj), "gate": (ffn, hidden),
            "up": (ffn, hidden), "down": (hidden, ffn)}


def stack_weight(layer, mat, hidden=HIDDEN, proj=PROJ, ffn=FFN, r0=0, r1=None, seed=STACK_SEED, out=None):
    n_out, n_in = stack_shapes(hidden, proj, ffn)[mat]
    return q4k_fields(seed, stack_tensor_id(layer, mat), n_out, n_in, r0, r1, out=out)


def stack_step_input(step, T, hidden=HIDDEN, seed=STACK_SEED):
    return normal_f32(seed, 10000 + step, 0, T * hidden).reshape(T, hidden)


def stack_gdn_inputs(step, T, n_gdn_layers, heads=GDN_HEADS, dk=GDN_DK, dv=GDN_DV, seed=STACK_SEED):
    return gdn_step_inputs(seed, 20000 + step, T, n_gdn_layers * heads, dk, dv)


def stack_gdn_state(agent, n_gdn_layers, heads=GDN_HEADS, dk=GDN_DK, dv=GDN_DV, seed=STACK_SEED):
    n = n_gdn_layers * heads * dk * dv
    return normal_f32(seed, 40000 + agent, 0, n, 0.0, 0.01).reshape(n_gdn_layers, heads, dk, dv)


def stack_lm_head(vocab=VOCAB, hidden=HIDDEN, seed=STACK_SEED, r0=0, r1=None):
    r1 = vocab if r1 is None else r1
    return normal_f16(seed, 30000, 0, (r1 - r0) * hidden, 0.0, 0.02, start=r0 * hidden).reshape(r1 - r0, hidden)


# ---------------------------------------------------------------- MTP draft head
MTP_BASE = 60000


def mtp_weights(hidden=HIDDEN, ffn=FFN, seed=STACK_SEED, base=MTP_BASE):
    """The synthetic MTP draft head: fc (hidden x 2 hidden) and one FFN of
    the stack's shape, Q4_K-style fields with the stack's distributions."""
    return {"fc": q4k_fields(seed, base + 0, hidden, 2 * hidden),
            "gate": q4k_fields(seed, base + 1, ffn, hidden),
            "up": q4k_fields(seed, base + 2, ffn, hidden),
            "down": q4k_fields(seed, base + 3, hidden, ffn)}


# ---------------------------------------------------------------- lm_head + verify
LM_SEED = 3


def lm_head_weight(vocab=VOCAB, hidden=HIDDEN, seed=LM_SEED, r0=0, r1=None):
    """fp16 bit patterns ~ N(0, 0.02), [vocab][hidden]; rows [r0, r1)."""
    r1 = vocab if r1 is None else r1
    return normal_f16(seed, 1, 0, (r1 - r0) * hidden, 0.0, 0.02, start=r0 * hidden).reshape(r1 - r0, hidden)


def lm_hidden(T, hidden=HIDDEN, seed=LM_SEED, trial=0):
    return normal_f32(seed, 2, trial, T * hidden).reshape(T, hidden)


def drafts_from_argmax(true_argmax, vocab, p_match=0.7, seed=LM_SEED, trial=0):
    """Draft i equals the true argmax of row i with probability p_match,
    otherwise a uniform id in [0, vocab).  ``true_argmax`` has T-1 entries."""
    n = len(true_argmax)
    u = uniform_f64(seed, 3, trial, n)
    rnd = uniform_i32(seed, 4, trial, n, 0, vocab - 1)
    return np.where(u < p_match, np.asarray(true_argmax, np.int32), rnd).astype(np.int32)


# ---------------------------------------------------------------- Gated DeltaNet
GDN_SEED = 4


def gdn_initial_state(n_layers=48, heads=GDN_HEADS, dk=GDN_DK, dv=GDN_DV, seed=GDN_SEED):
    n = n_layers * heads * dk * dv
    return normal_f32(seed, 1, 0, n, 0.0, 0.01).reshape(n_layers, heads, dk, dv)


def gdn_step(step, T, n_layers=48, heads=GDN_HEADS, dk=GDN_DK, dv=GDN_DV, seed=GDN_SEED):
    return gdn_step_inputs(seed, 100 + step, T, n_layers * heads, dk, dv)


def gdn_accept_lengths(n_steps, T=5, seed=GDN_SEED):
    """Seeded accept lengths, uniform on 0..T-1."""
    return uniform_i32(seed, 2, 0, n_steps, 0, T - 1)


# ---------------------------------------------------------------- full attention
# 16 of the 64 layers run full attention.  Head geometry (a reading: the
# pages give none): 32 query heads and 8 KV heads of 128, which with an
# output gate of the query's width fills the 10240-wide input projection
# exactly (q 4096 + gate 4096 + k 1024 + v 1024).
ATTN_SEED = 5
ATTN_Q_HEADS = 32
ATTN_KV_HEADS = 8
ATTN_D = 128
F16_NAN = 0x7E00


def attn_cap(ctx, sizes, align=64):
    need = max(int(c) + int(n) for c, n in zip(ctx, sizes))
    return (need + align - 1) // align * align


def attn_inputs(ctx, sizes, Hq=ATTN_Q_HEADS, Hkv=ATTN_KV_HEADS, d=ATTN_D, cap=None, seed=ATTN_SEED, layer=0,
                gate=True, fill=F16_NAN):
    """One attention layer's decode inputs for G agents.

    Agent g has ctx[g] cached positions and sizes[g] new rows (token +
    drafts), whose k and v already sit at positions ctx[g] .. ctx[g] +
    sizes[g] - 1.  K cache [G][Hkv][cap][d] and V cache [G][Hkv][d][cap]
    (dimension-major) hold fp16 N(0, 1) values; slots past an agent's last
    position hold ``fill`` (a NaN by default, so that a kernel that reads
    them into its result is caught).  q and gate are fp32 N(0, 1)
    [T][Hq][d].  Returns q, gate (or None), k, v, ctx, group_start.
    """
    G = len(ctx)
    if cap is None:
        cap = attn_cap(ctx, sizes)
    kc = np.full((G, Hkv, cap, d), fill, np.uint16)
    vc = np.full((G, Hkv, d, cap), fill, np.uint16)
    for g in range(G):
        n = int(ctx[g]) + int(sizes[g])
        for h in range(Hkv):
            sub = g * Hkv + h
            kc[g, h, :n, :] = normal_f16(seed, 100 + layer, sub, n * d).reshape(n, d)
            vc[g, h, :, :n] = normal_f16(seed, 200 + layer, sub, n * d).reshape(n, d).T
    T = int(sum(sizes))
    q = normal_f32(seed, 300 + layer, 0, T * Hq * d).reshape(T, Hq, d)
    gt = normal_f32(seed, 400 + layer, 0, T * Hq * d).reshape(T, Hq, d) if gate else None
    gs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return {"q": q, "gate": gt, "k": kc, "v": vc, "ctx": np.asarray(ctx, np.int32), "group_start": gs}


def step_attn_inputs(n_layers, ctx, sizes, cap=None, gate=True, q8=False):
    """The full-attention layers of a decode step: q and gate [n_layers][T][Hq][d]
    with per-layer seeds (as attn_inputs with layer = i), and one layer's
    caches (attn_inputs, or attn_inputs_q8 when q8, with layer = 0), which the
    caller copies into every layer's cache: generating all of them takes a
    minute at 4 x 32768 positions, and the bytes each layer reads are the same
    either way."""
    first = (attn_inputs_q8 if q8 else attn_inputs)(ctx, sizes, cap=cap, layer=0, gate=gate)
    T = int(sum(sizes))
    n = T * ATTN_Q_HEADS * ATTN_D
    q = np.stack([normal_f32(ATTN_SEED, 300 + i, 0, n).reshape(T, ATTN_Q_HEADS, ATTN_D) for i in range(n_layers)])
    gt = np.stack([normal_f32(ATTN_SEED, 400 + i, 0, n).reshape(T, ATTN_Q_HEADS, ATTN_D)
                   for i in range(n_layers)]) if gate else None
    out = {"q": q, "gate": gt, "ctx": first["ctx"], "group_start": first["group_start"]}
    for k in (("k8", "ks", "v8", "vs") if q8 else ("k", "v")):
        out[k] = first[k]
    return out


def attn_inputs_q8(ctx, sizes, Hq=ATTN_Q_HEADS, Hkv=ATTN_KV_HEADS, d=ATTN_D, cap=None, seed=ATTN_SEED, layer=0,
                   gate=True, fill_scale=F16_NAN):
    """The same workload over q8_0 caches: codes uniform in -127..127 and
    fp16 scales |N(0, 0.01)| (values of about the fp16 cache's spread).
    K codes [G][Hkv][cap][d] with scales [G][Hkv][cap][d/32]; V codes
    tile-major [G][Hkv][cap/64][d][64] (positions 64t..64t+63 of every
    dimension together) with scales [G][Hkv][cap/32][d].  Codes past an agent's
    last position are 0x80 (-128, outside the codes' range) and scales of
    slots or blocks holding no position are ``fill_scale`` (a NaN)."""
    G = len(ctx)
    if cap is None:
        cap = attn_cap(ctx, sizes)
    nb = d // 32
    k8 = np.full((G, Hkv, cap, d), -128, np.int8)
    v8 = np.full((G, Hkv, d, cap), -128, np.int8)
    ks = np.full((G, Hkv, cap, nb), fill_scale, np.uint16)
    vs = np.full((G, Hkv, cap // 32, d), fill_scale, np.uint16)
    for g in range(G):
        n = int(ctx[g]) + int(sizes[g])
        nblk = (n + 31) // 32
        for h in range(Hkv):
            sub = g * Hkv + h
            k8[g, h, :n, :] = uniform_i32(seed, 500 + layer, sub, n * d, -127, 127).reshape(n, d)
            v8[g, h, :, :n] = uniform_i32(seed, 600 + layer, sub, n * d, -127, 127).reshape(n, d).T
            ks[g, h, :n, :] = normal_f16(seed, 700 + layer, sub, n * nb, 0.0, 0.01, absval=True).reshape(n, nb)
            vs[g, h, :nblk, :] = normal_f16(seed, 800 + layer, sub, nblk * d, 0.0, 0.01, absval=True).reshape(nblk, d)
    v8 = np.ascontiguousarray(v8.reshape(G, Hkv, d, cap // 64, 64).transpose(0, 1, 3, 2, 4))
    T = int(sum(sizes))
    q = normal_f32(seed, 300 + layer, 0, T * Hq * d).reshape(T, Hq, d)
    gt = normal_f32(seed, 400 + layer, 0, T * Hq * d).reshape(T, Hq, d) if gate else None
    gs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    return {"q": q, "gate": gt, "k8": k8, "ks": ks, "v8": v8, "vs": vs, "ctx": np.asarray(ctx, np.int32),
            "group_start": gs}
