"""GPU parity of the persistent decode step (mk_decode_step): every layer is
checked teacher-forced against the oracle (the oracle's layer applied to the
GPU's residual entering it), then the final RMSNorm + lm_head argmax, the
verification, and the Gated DeltaNet outputs and committed state across steps
(with the accept lengths the step itself produced)."""
import numpy as np
import pytest

import oracle
import synth
from tests._util import FP32_TOL, need_gpu, rel_err, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _mk():
    import bit_weight_streaming_q4_amd as mk
    return mk


MATS = ("p_in", "p_out", "gate", "up", "down")


def small_stack(mk, seed, L, H, P, F, V, n_agents, T_max=5, gdn=True):
    shapes = {"p_in": (P, H), "p_out": (H, P), "gate": (F, H), "up": (F, H), "down": (H, F)}
    fields = [{m: synth.q4k_fields(seed, 100 + 8 * l + i, *shapes[m]) for i, m in enumerate(MATS)}
              for l in range(L)]
    layers = [{m: mk.Q4K.from_fields(fields[l][m]) for m in MATS} for l in range(L)]
    W16 = synth.normal_f16(seed, 30000, 0, V * H, 0.0, 0.02).reshape(V, H)
    lm = to_dev(W16)
    gl = [l for l in range(L) if l % 4 != 3] if gdn else []
    nh = len(gl) * 32
    S0 = [synth.normal_f32(seed, 40000 + a, 0, nh * 128 * 128, 0.0, 0.01).reshape(nh, 128, 128)
          for a in range(n_agents)] if gdn else []
    agents = [mk.DeltaNetState(nh, T_max, S=to_dev(S0[a].copy())) for a in range(n_agents)] if gdn else []
    st = mk.Stack(layers, lm, gdn_layers=gl if gdn else None, agents=agents)
    dry = mk.Stack(layers, lm)  # same weights, no mixer: used to preview the argmax for drafts
    return st, dry, fields, W16, S0, nh


def _check_layers(fields, x_in, trace):
    L = len(fields)
    prev = x_in
    worst = 0.0
    for l in range(L):
        ref = oracle.layer(prev, fields[l])
        e = rel_err(trace[l], ref)
        worst = max(worst, e)
        assert e <= FP32_TOL, (l, e)
        prev = trace[l]
    return worst


def _check_head(W16, x_final, am, na, tok, gs, drafts):
    hid = oracle.rmsnorm(x_final)
    r = oracle.lmhead(W16, hid)
    tau = oracle.near_tie_tau(W16.shape[1], r["abs1"], r["abs2"])
    near = (r["top1_val"] - r["top2_val"]) <= tau
    for t in range(len(am)):
        assert am[t] == r["top1"][t] or (near[t] and am[t] == r["top2"][t]), (t, am[t], r["top1"][t])
    n_ref, t_ref = oracle.verify(am, gs, drafts)
    assert np.array_equal(na, n_ref) and np.array_equal(tok, t_ref)
    return r["top1"]


# T = 1 runs the dot4 engine; T = 2..8 the packed matrix-core engine (8
# padded rows, two sub-blocks per product); T = 9..16 the 16-row engine.
# 2 and 9 are the first instances of the two matrix-core engines, 8 and 16
# their largest; 6 has three agents of unequal size (1, 2 and 3 rows), 11 one
# group that fills neither the rows nor a whole agent count.  The last two
# run eight agents of two rows, and a ten-row chunk of a new prompt riding
# beside two agents of three rows (each group with its own GDN state).  Above
# 16 rows the record has two 16-row halves and the lm_head is streamed once
# per half: 17 (one row in the second half), 20, eight agents of three rows
# (24), and a twelve-row chunk beside four agents of three rows.  The other
# row counts complete the set, so that every instance of the step (T = 1 to
# 24) runs: 13 is the first with the epilogue's six-partial batches, 19 and 23
# put a full 16-row group beside a short one.
@pytest.mark.parametrize("T,gs", [(1, [0, 1]), (2, [0, 2]), (3, [0, 3]), (5, [0, 5]), (6, [0, 1, 3, 6]),
                                  (8, [0, 2, 4, 6, 8]), (9, [0, 9]), (11, [0, 11]), (12, [0, 3, 6, 9, 12]),
                                  (16, [0, 4, 8, 12, 16]), (16, list(range(0, 17, 2))), (16, [0, 10, 13, 16]),
                                  (17, [0, 8, 17]), (20, [0, 4, 8, 12, 16, 20]), (24, list(range(0, 25, 3))),
                                  (24, [0, 3, 6, 9, 12, 24]),
                                  (4, [0, 4]), (7, [0, 3, 7]), (10, [0, 5, 10]), (13, [0, 13]), (14, [0, 7, 14]),
                                  (15, [0, 3, 6, 9, 12, 15]), (18, [0, 9, 18]), (19, [0, 16, 19]),
                                  (21, list(range(0, 22, 3))), (22, [0, 11, 22]), (23, [0, 16, 23])])
def test_decode_step_small_stack(T, gs):
    torch = need_gpu()
    mk = _mk()
    L, H, P, F, V = 4, 512, 1024, 768, 1000
    G = len(gs) - 1
    T_max = max(5, max(gs[g + 1] - gs[g] for g in range(G)))  # each agent's ring holds its longest group
    st, dry, fields, W16, S0, nh = small_stack(mk, 21, L, H, P, F, V, G, T_max=T_max)
    S_ref = [s.copy() for s in S0]
    for step in range(3):
        x = synth.normal_f32(21, 10000 + step, 0, T * H).reshape(T, H)
        # preview the argmax (the layer path does not depend on the mixer), then
        # draft so that some groups accept some drafts
        xd = to_dev(x)
        am_prev = torch.empty(T, dtype=torch.int32, device="cuda")
        drafts0 = np.zeros(max(T - G, 1), np.int32)
        mk.mk_decode_step(dry, xd, gs, to_dev(drafts0), argmax=am_prev)
        amp = to_np(am_prev)
        drafts = []
        for g in range(G):
            n = gs[g + 1] - gs[g]
            for i in range(n - 1):
                drafts.append(int(amp[gs[g] + i]) if (i + g + step) % 3 != 2 else 3)
        drafts = np.asarray(drafts if drafts else [0], np.int32)
        inp = synth.gdn_step_inputs(21, 20000 + step, T, nh, 128, 128)
        gin = {k: to_dev(inp[k]) for k in ("q", "k", "v", "g", "beta")}
        go = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
        xd = to_dev(x)
        trace = torch.empty(L, T, H, dtype=torch.float32, device="cuda")
        am = torch.empty(T, dtype=torch.int32, device="cuda")
        say("decode small", T, step)
        tok, na = mk.mk_decode_step(st, xd, gs, to_dev(drafts), gdn=gin, gdn_o=go, argmax=am, trace=trace)
        tr = to_np(trace)
        assert np.array_equal(to_np(xd), tr[L - 1])
        assert np.array_equal(to_np(am), amp)
        _check_layers(fields, x, tr)
        _check_head(W16, tr[L - 1], to_np(am), na, tok, gs, drafts[:T - G])
        # Gated DeltaNet per agent: outputs of this step and (below) the committed state
        og = to_np(go)
        for a in range(G):
            r0, r1 = gs[a], gs[a + 1]
            sl = {k: inp[k][r0:r1] for k in inp}
            S_ref[a], o_ref = oracle.gdn_step(S_ref[a], sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], int(na[a]))
            assert rel_err(og[r0:r1], o_ref) <= FP32_TOL, (a, rel_err(og[r0:r1], o_ref))
    for a in range(G):
        mk.mk_deltanet_commit(st.agents[a])
        assert rel_err(to_np(st.agents[a].S), S_ref[a]) <= FP32_TOL


# ---------------------------------------------------------------- full size
# The benchmark's own workload and launch configuration: the 64-layer stack
# (hidden 5120, projections 10240, FFN 17408), the 151,936-row lm_head and 48
# Gated DeltaNet layers, one state per agent.  The oracle checks whole layers
# teacher-forced at sampled depths, all rows of the argmax / verification,
# and sampled GDN heads (outputs and the committed state).

@pytest.fixture(scope="module")
def full_stack():
    torch = need_gpu()
    import bench
    from synth import recipes
    mk = _mk()
    mk.mk_init(0)
    layers, lm = bench.build_stack(progress=False)
    return {"layers": layers, "lm": lm, "gl": recipes.gdn_layers(bench.LAYERS)}


@pytest.mark.parametrize("T,gs", [(12, [0, 3, 6, 9, 12]), (1, [0, 1]), (5, [0, 5]), (24, list(range(0, 25, 3)))])
def test_decode_step_full_size(full_stack, T, gs):
    torch = need_gpu()
    import bench
    from synth import recipes
    mk = _mk()
    layers, lm, gl = full_stack["layers"], full_stack["lm"], full_stack["gl"]
    G = len(gs) - 1
    H, L = bench.HIDDEN, bench.LAYERS
    say("decode full", T)
    agents = bench.make_agents(G, len(gl), 5)
    st = mk.Stack(layers, lm, gdn_layers=gl, agents=agents)
    dry = mk.Stack(layers, lm)
    x = recipes.stack_step_input(0, T)
    # preview the argmax, then draft so that some groups accept some drafts
    am_prev = torch.empty(T, dtype=torch.int32, device="cuda")
    mk.mk_decode_step(dry, to_dev(x), gs, to_dev(np.zeros(max(T - G, 1), np.int32)), argmax=am_prev)
    amp = to_np(am_prev)
    drafts = []
    for g in range(G):
        for i in range(gs[g + 1] - gs[g] - 1):
            drafts.append(int(amp[gs[g] + i]) if (i + g) % 3 != 2 else 7)
    drafts = np.asarray(drafts if drafts else [0], np.int32)
    inp = recipes.stack_gdn_inputs(0, T, len(gl))
    gin = {k: to_dev(inp[k]) for k in ("q", "k", "v", "g", "beta")}
    nh = len(gl) * 32
    go = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
    trace = torch.empty(L, T, H, dtype=torch.float32, device="cuda")
    am = torch.empty(T, dtype=torch.int32, device="cuda")
    xd = to_dev(x)
    tok, na = mk.mk_decode_step(st, xd, gs, to_dev(drafts), gdn=gin, gdn_o=go, argmax=am, trace=trace)
    tr = to_np(trace)
    assert np.array_equal(to_np(xd), tr[L - 1])
    assert np.array_equal(to_np(am), amp)
    # layers teacher-forced: every layer at T = 12 (the benchmark's rows),
    # sampled depths at T = 1, 5 and 24 (eight agents of three rows)
    bufs = {}
    for l in (range(L) if T == 12 else (0, 21, 42, L - 1)):
        for m in MATS:
            bufs[m] = recipes.stack_weight(l, m, out=bufs.get(m))
        prev = x if l == 0 else tr[l - 1]
        e = rel_err(tr[l], oracle.layer(prev, bufs))
        say("layer", l, "err", e)
        assert e <= FP32_TOL, (l, e)
    del bufs
    # final RMSNorm + lm_head argmax over the full vocabulary, verification
    _check_head(recipes.stack_lm_head(), tr[L - 1], to_np(am), na, tok, gs, drafts[:T - G])
    # Gated DeltaNet, sampled heads of every agent: outputs and committed state
    og = to_np(go)
    heads = [0, 517, nh - 1]
    for a in range(G):
        mk.mk_deltanet_commit(st.agents[a])
    for a in range(G):
        S0 = recipes.stack_gdn_state(a, len(gl)).reshape(nh, 128, 128)
        S1 = to_np(st.agents[a].S)
        r0, r1 = gs[a], gs[a + 1]
        for hh in heads:
            sl = {k: inp[k][r0:r1, hh:hh + 1] for k in inp}
            Sref, oref = oracle.gdn_step(S0[hh:hh + 1].copy(), sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                         int(na[a]))
            assert rel_err(og[r0:r1, hh:hh + 1], oref) <= FP32_TOL, (a, hh)
            assert rel_err(S1[hh:hh + 1], Sref) <= FP32_TOL, (a, hh)
    del st, dry, agents
    torch.cuda.empty_cache()


def test_decode_step_workspace_bound_to_its_stack():
    """Two stacks that share one workspace each get their own results (the
    tables are uploaded again when the other stack ran last); a workspace
    that another call overwrote is refused (MK_ERR_WORKSPACE, nothing runs)
    and the next call runs normally."""
    torch = need_gpu()
    mk = _mk()
    L, H, P, F, V, T = 2, 512, 1024, 768, 1000, 5
    gs = [0, T]
    stA, _, _, _, _, _ = small_stack(mk, 41, L, H, P, F, V, 1, gdn=False)
    stB, _, _, _, _, _ = small_stack(mk, 42, L, H, P, F, V, 1, gdn=False)
    drafts = to_dev(np.array([1, 2, 3, 4], np.int32))
    x = synth.normal_f32(41, 10000, 0, T * H).reshape(T, H)

    def run(st, ws):
        xd = to_dev(x)
        tr = torch.empty(L, T, H, dtype=torch.float32, device="cuda")
        tok, na = mk.mk_decode_step(st, xd, gs, drafts, trace=tr, ws=ws)
        return to_np(tr), tok, na

    refA = run(stA, stA.workspace(T))
    refB = run(stB, stB.workspace(T))
    assert not np.array_equal(refA[0], refB[0])
    shared = mk.workspace(max(stA.workspace_bytes(T), stB.workspace_bytes(T)))
    for st, ref in ((stA, refA), (stB, refB), (stA, refA), (stA, refA), (stB, refB)):
        say("shared workspace", "A" if st is stA else "B")
        got = run(st, shared)
        assert all(np.array_equal(g, r) for g, r in zip(got, ref))
    shared.zero_()  # another call wrote the workspace
    with pytest.raises(mk.MkError) as ei:
        run(stB, shared)
    assert ei.value.status == mk.MK_ERR_WORKSPACE
    got = run(stB, shared)
    assert all(np.array_equal(g, r) for g, r in zip(got, refB))


def test_decode_step_accept_length_out_of_range():
    """An agent state whose accept length is outside 0..T_max-1 is reported
    (MK_ERR_RANGE) and that agent replays nothing."""
    torch = need_gpu()
    mk = _mk()
    L, H, P, F, V, T = 4, 512, 1024, 768, 1000, 6
    gs = [0, 3, 6]
    st, _, _, _, S0, nh = small_stack(mk, 43, L, H, P, F, V, 2)
    x = synth.normal_f32(43, 10000, 0, T * H).reshape(T, H)
    inp = synth.gdn_step_inputs(43, 20000, T, nh, 128, 128)
    gin = {k: to_dev(inp[k]) for k in ("q", "k", "v", "g", "beta")}
    go = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
    drafts = to_dev(np.array([1, 2, 3, 4], np.int32))
    st.agents[1].n_acc[0] = 9
    say("decode accept out of range")
    with pytest.raises(mk.MkError) as ei:
        mk.mk_decode_step(st, to_dev(x), gs, drafts, gdn=gin, gdn_o=go)
    assert ei.value.status == mk.MK_ERR_RANGE
    assert mk.mk_deltanet_status(st.agents[1]) == mk.MK_ERR_RANGE
    assert mk.mk_deltanet_status(st.agents[0]) == mk.MK_OK
    # agent 1 replayed nothing: its outputs are those of its rows on S0
    og = to_np(go)
    _, o_ref = oracle.gdn_step(S0[1], inp["q"][3:], inp["k"][3:], inp["v"][3:], inp["g"][3:], inp["beta"][3:], 0)
    assert rel_err(og[3:], o_ref) <= FP32_TOL


@pytest.mark.parametrize("gs_ride,rows", [([0, 10, 13, 16], (0, 10)), ([0, 3, 6, 16], (6, 16)),
                                          ([0, 3, 6, 9, 12, 24], (12, 24))])
def test_decode_step_prompt_chunk_is_bit_identical(gs_ride, rows):
    """A new prompt's chunk riding in a step beside other agents' rows gives,
    bit for bit, what the chunk gives when the step processes it on its own:
    residuals after every layer, argmax, Gated DeltaNet outputs and the
    chunk's committed state (the 4-agent article, "Why it matters").  Every
    step here runs the 16-row matrix-core engine: on the whole record (T = 16,
    10 and 12) or on each of its two halves (T = 24, the chunk's rows 12..23
    straddling them)."""
    torch = need_gpu()
    mk = _mk()
    L, H, P, F, V = 4, 512, 1024, 768, 1000
    T = gs_ride[-1]
    r0, r1 = rows
    n = r1 - r0
    ci = [g for g in range(len(gs_ride) - 1) if gs_ride[g] == r0][0]  # the chunk's group
    x = synth.normal_f32(51, 10000, 0, T * H).reshape(T, H)
    ride, _, _, _, S0, nh = small_stack(mk, 51, L, H, P, F, V, len(gs_ride) - 1, T_max=n)
    inp = synth.gdn_step_inputs(51, 20000, T, nh, 128, 128)
    # the chunk alone: one agent whose state is the riding chunk's agent state
    alone, _, _, _, _, _ = small_stack(mk, 51, L, H, P, F, V, 1, T_max=n)
    alone.agents[0].S.copy_(to_dev(S0[ci].copy()))
    out = {}
    for name, st, xs, gs, sl in (("ride", ride, x, gs_ride, slice(0, T)), ("alone", alone, x[r0:r1], [0, n],
                                                                          slice(r0, r1))):
        Tn = xs.shape[0]
        G = len(gs) - 1
        drafts = to_dev(np.arange(1, Tn - G + 1, dtype=np.int32) if Tn > G else np.zeros(1, np.int32))
        gin = {k: to_dev(np.ascontiguousarray(inp[k][sl])) for k in ("q", "k", "v", "g", "beta")}
        go = torch.empty(Tn, nh, 128, dtype=torch.float32, device="cuda")
        tr = torch.empty(L, Tn, H, dtype=torch.float32, device="cuda")
        am = torch.empty(Tn, dtype=torch.int32, device="cuda")
        say("prompt chunk", name, gs)
        mk.mk_decode_step(st, to_dev(xs), gs, drafts, gdn=gin, gdn_o=go, argmax=am, trace=tr)
        a = st.agents[ci if name == "ride" else 0]
        st.agents[ci if name == "ride" else 0].n_acc[0] = n - 1  # commit the whole chunk
        mk.mk_deltanet_commit(a)
        out[name] = (to_np(tr), to_np(am), to_np(go), to_np(a.S))
    tr_r, am_r, go_r, S_r = out["ride"]
    tr_a, am_a, go_a, S_a = out["alone"]
    assert np.array_equal(tr_r[:, r0:r1], tr_a)
    assert np.array_equal(am_r[r0:r1], am_a)
    assert np.array_equal(go_r[r0:r1], go_a)
    assert np.array_equal(S_r, S_a)


@pytest.mark.parametrize("fmt", ["f16", "q8"])
@pytest.mark.parametrize("ctx,sizes,cap,n_layers", [([0, 100, 517, 1000], [3, 3, 3, 3], 1024, 2),
                                                    ([0, 64, 200, 4999], [1, 4, 3, 4], 5056, 1),
                                                    ([32768, 32768, 30000, 12345], [3, 3, 3, 3], 32832, 1),
                                                    ([0, 7, 64, 129, 500, 1000, 2047, 3000], [3] * 8, 3008, 2),
                                                    ([500], [1], 512, 1),
                                                    ([77, 1000], [1, 4], 1024, 1),
                                                    ([100, 300], [4, 4], 320, 1),
                                                    (list(range(0, 480, 30)), [1] * 16, 512, 1)])
def test_decode_step_attention_beside_the_pipeline(ctx, sizes, cap, n_layers, fmt):
    """The full-attention layers' split-K flash decoding inside the persistent
    step (four agents of 12 rows in all, or eight agents of 3 rows = 24 rows
    on the two-record path; 32 query and 8 KV heads of 128, gated; fp16
    caches whose unused slots hold NaN, or q8_0 caches whose unused codes are
    out of range and unused scales NaN; an agent with no cached position and
    one row; ragged groups of 1 to 4 rows; the instances at T = 1, 5, 8 and
    16, the last with sixteen agents of one row): every layer's
    output equals the oracle's attention on that layer's inputs, and the rest
    of the step is bit-identical to the same step without attention."""
    torch = need_gpu()
    mk = _mk()
    from synth import recipes
    L, H, P, F, V = 4, 512, 1024, 768, 1000
    gs = [0] + list(np.cumsum(sizes))
    T, G = int(gs[-1]), len(sizes)
    gen = recipes.attn_inputs if fmt == "f16" else recipes.attn_inputs_q8
    layers_in = [gen(ctx, sizes, cap=cap, layer=i) for i in range(n_layers)]
    q = to_dev(np.stack([a["q"] for a in layers_in]))
    gate = to_dev(np.stack([a["gate"] for a in layers_in]))
    caches = [to_dev(np.stack([a[k] for a in layers_in]))
              for k in (("k", "v") if fmt == "f16" else ("k8", "ks", "v8", "vs"))]
    o = torch.full((n_layers, T, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    runs = {}
    for name in ("plain", "attn"):
        st, _, fields, W16, S0, nh = small_stack(mk, 61, L, H, P, F, V, G, T_max=max(2, max(sizes)))
        x = synth.normal_f32(61, 10000, 0, T * H).reshape(T, H)
        inp = synth.gdn_step_inputs(61, 20000, T, nh, 128, 128)
        gin = {k: to_dev(inp[k]) for k in ("q", "k", "v", "g", "beta")}
        go = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
        tr = torch.empty(L, T, H, dtype=torch.float32, device="cuda")
        drafts = to_dev(np.arange(1, T - G + 1, dtype=np.int32))
        at = None
        if name == "attn":
            at = mk.step_attn(q, *caches, o, ctx, gate=gate) if fmt == "f16" else \
                mk.step_attn_q8(q, *caches, o, ctx, gate=gate)
        say("decode with attention", name, ctx)
        tok, na = mk.mk_decode_step(st, to_dev(x), gs, drafts, gdn=gin, gdn_o=go, trace=tr, attn=at)
        for ag in st.agents:
            mk.mk_deltanet_commit(ag)
        runs[name] = (tok, na, to_np(tr), to_np(go)) + tuple(to_np(ag.S) for ag in st.agents)
        del st
    for a, b in zip(runs["plain"], runs["attn"]):
        assert np.array_equal(a, b)
    og = to_np(o)
    for i, a in enumerate(layers_in):
        if fmt == "f16":
            ref = oracle.attn_decode(a["q"], a["gate"], a["k"], a["v"], a["ctx"], a["group_start"])
        else:
            ref = oracle.attn_decode_q8(a["q"], a["gate"], a["k8"], a["ks"], a["v8"], a["vs"], a["ctx"],
                                        a["group_start"])
        e = rel_err(og[i], ref)
        say("attention layer", i, "err", e)
        assert e <= FP32_TOL, (i, e)


def test_decode_step_attention_cache_format_checks():
    """mk_step_attn takes exactly one cache format: neither, both, or a
    partial set of pointers gives no workspace (the call fails with
    MK_ERR_ARG); a misaligned q8_0 pointer fails the alignment check; shapes
    beyond the items' limits give no workspace.  Only the host checks run (no
    launch)."""
    torch = need_gpu()
    mk = _mk()
    import ctypes
    st, *_ = small_stack(mk, 61, 4, 512, 1024, 768, 1000, 4, T_max=3)
    gs = np.array([0, 3, 6, 9, 12], np.int32)
    ctx = np.array([0, 10, 20, 30], np.int32)
    P = 1 << 20  # aligned stand-in addresses: the checks read no memory

    def ws(k=None, v=None, k8=None, ks=None, v8=None, vs=None):
        a = mk.mk_step_attn(1, 32, 8, 64, ctx.ctypes.data, P, None, k, v, P, k8, ks, v8, vs)
        return mk.lib().mk_decode_step_attn_workspace(st.h, 12, gs.ctypes.data, 4, ctypes.byref(a))

    assert ws(k=P, v=P) > 0
    assert ws(k8=P, ks=P, v8=P, vs=P) > 0
    assert ws() == 0
    assert ws(k=P, v=P, k8=P, ks=P, v8=P, vs=P) == 0
    assert ws(k=P) == 0
    assert ws(k8=P, ks=P, v8=P) == 0
    assert ws(k8=P, ks=P + 2, v8=P, vs=P) == 0

    # shapes: an agent's rows x Hq/Hkv above 16 query columns, a cache length
    # that is not a multiple of 64 or is above MK_ATTN_CAP_MAX, cached
    # positions + new rows above the cache length, Hq not a multiple of Hkv
    def ws2(T, groups, ctx2, Hq=32, Hkv=8, cap=64):
        g2 = np.array(groups, np.int32)
        c2 = np.array(ctx2, np.int32)
        a = mk.mk_step_attn(1, Hq, Hkv, cap, c2.ctypes.data, P, None, P, P, P, None, None, None, None)
        return mk.lib().mk_decode_step_attn_workspace(st.h, T, g2.ctypes.data, len(groups) - 1, ctypes.byref(a))

    g12, g8 = [0, 3, 6, 9, 12], [0, 2, 4, 6, 8]
    assert ws2(12, g12, [0, 10, 20, 30]) > 0
    assert ws2(12, g12, [0, 10, 20, 30], Hq=64) == 0  # 3 rows x 8 = 24 columns
    assert ws2(8, g8, [0, 10, 20, 30], Hq=64) > 0  # 2 rows x 8 = 16 columns
    assert ws2(12, g12, [0, 10, 20, 30], cap=100) == 0
    assert ws2(12, g12, [0, 10, 20, 30], cap=mk.MK_ATTN_CAP_MAX + 64) == 0
    assert ws2(12, g12, [0, 10, 20, 62]) == 0  # 62 + 3 > 64
    assert ws2(12, g12, [0, 10, 20, 61]) > 0
    assert ws2(12, g12, [0, 10, 20, 30], Hkv=12) == 0
