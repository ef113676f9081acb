"""GPU parity of full-attention decode (mk_attn_decode) against the oracle
(A1), element by element, with the comparison rule of fp32 outputs."""
import numpy as np
import pytest

from synth import recipes
from tests._util import FP32_TOL, need_gpu, norm_err, rel_err, say

pytestmark = pytest.mark.gpu


def _run(torch, mk, a, ws=None):
    dev = "cuda"
    q = torch.from_numpy(a["q"]).to(dev)
    gate = torch.from_numpy(a["gate"]).to(dev) if a["gate"] is not None else None
    k = torch.from_numpy(a["k"].view(np.int16)).to(dev)
    v = torch.from_numpy(a["v"].view(np.int16)).to(dev)
    o = torch.full_like(q, float("nan"))
    mk.mk_attn_decode(q, gate, k, v, a["ctx"], a["group_start"], o, ws=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def _check(orc, torch, mk, a, label):
    say("attention", label, "ctx", list(a["ctx"]), "groups", list(a["group_start"]), "Hq", a["q"].shape[1],
        "Hkv", a["k"].shape[1], "cap", a["k"].shape[2], "gate", a["gate"] is not None)
    y = _run(torch, mk, a)
    ref = orc.attn_decode(a["q"], a["gate"], a["k"], a["v"], a["ctx"], a["group_start"])
    assert np.isfinite(y).all(), label
    e, n = rel_err(y, ref), norm_err(y, ref)
    say(label, "rel", e, "norm", n)
    assert e <= FP32_TOL, (label, e)
    assert n <= 1e-5, (label, n)
    return y


CASES = [
    # (label, ctx per agent, rows per agent, Hq, Hkv, gate)
    ("4 agents x 3 rows, ragged contexts", [100, 37, 0, 250], [3, 3, 3, 3], 32, 8, True),
    ("1 agent x 5 rows (two column blocks)", [1000], [5], 32, 8, False),
    ("T = 1, empty cache", [0], [1], 32, 8, True),
    ("T = 1, ragged tail", [4095], [1], 32, 8, True),
    ("T = 16, one group (four column blocks)", [300], [16], 32, 8, True),
    ("T = 16, no grouped queries", [517], [16], 8, 8, False),
    ("unequal groups, many splits", [20000, 3, 777], [2, 5, 1], 32, 8, True),
    ("16 agents x 1 row", list(range(0, 1600, 100)), [1] * 16, 32, 8, True),
    ("1 agent x 10 rows (three column blocks)", [2000], [10], 32, 8, True),
]


@pytest.mark.parametrize("label,ctx,sizes,Hq,Hkv,gate", CASES, ids=[c[0] for c in CASES])
def test_attn_parity(orc, label, ctx, sizes, Hq, Hkv, gate):
    torch = need_gpu()
    import bit_weight_streaming_q4_amd as mk
    a = recipes.attn_inputs(ctx, sizes, Hq=Hq, Hkv=Hkv, gate=gate)
    _check(orc, torch, mk, a, label)


def test_attn_full_size_four_agents(orc):
    """The measured workload: 4 agents x 32768 cached positions, 3 rows each
    (T = 12), 32 query / 8 KV heads of 128, gated; every output compared."""
    torch = need_gpu()
    import bit_weight_streaming_q4_amd as mk
    a = recipes.attn_inputs([32768] * 4, [3] * 4)
    y1 = _check(orc, torch, mk, a, "full size T = 12")
    y2 = _run(torch, mk, a)
    assert np.array_equal(y1, y2), "two calls differ"


def test_attn_full_size_long_context(orc):
    """One agent at 81920 cached positions (the long end of the fp16 cache), T = 5."""
    torch = need_gpu()
    import bit_weight_streaming_q4_amd as mk
    a = recipes.attn_inputs([81920], [5])
    _check(orc, torch, mk, a, "long context T = 5")


def test_attn_rejects_bad_arguments():
    torch = need_gpu()
    import bit_weight_streaming_q4_amd as mk
    a = recipes.attn_inputs([10], [2], Hq=8, Hkv=2, gate=False)
    q = torch.from_numpy(a["q"]).cuda()
    k = torch.from_numpy(a["k"].view(np.int16)).cuda()
    v = torch.from_numpy(a["v"].view(np.int16)).cuda()
    o = torch.empty_like(q)
    L = mk.lib()
    ctx = np.array([10], np.int32)
    gs = np.array([0, 2], np.int32)
    ws = mk.workspace(1 << 20)

    def call(cap=k.shape[2], d=128, ctx_=ctx, Hkv=2, wsz=ws.numel()):
        return L.mk_attn_decode(mk._ptr(q), None, 2, 8, mk._ptr(k), mk._ptr(v), Hkv, d, cap, ctx_.ctypes.data,
                                gs.ctypes.data, 1, mk._ptr(o), mk._ptr(ws), wsz, None)

    assert call() == 0
    assert call(cap=100) == -2          # cap not a multiple of 64
    assert call(d=64) == -2             # head size
    assert call(Hkv=3) == -2            # Hq % Hkv
    assert call(ctx_=np.array([63], np.int32)) == -4   # ctx + rows > cap
    assert call(wsz=16) == -5           # workspace too small
    torch.cuda.synchronize()


# ------------------------------------------------------------------ q8_0 cache
def _run_q8(torch, mk, a):
    dev = "cuda"
    q = torch.from_numpy(a["q"]).to(dev)
    gate = torch.from_numpy(a["gate"]).to(dev) if a["gate"] is not None else None
    k8 = torch.from_numpy(a["k8"]).to(dev)
    v8 = torch.from_numpy(a["v8"]).to(dev)
    ks = torch.from_numpy(a["ks"].view(np.int16)).to(dev)
    vs = torch.from_numpy(a["vs"].view(np.int16)).to(dev)
    o = torch.full_like(q, float("nan"))
    mk.mk_attn_decode_q8(q, gate, k8, ks, v8, vs, a["ctx"], a["group_start"], o)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def _check_q8(orc, torch, mk, a, label):
    say("attention q8", label, "ctx", list(a["ctx"])[:4], "groups", list(a["group_start"])[:5],
        "Hq", a["q"].shape[1], "Hkv", a["k8"].shape[1], "cap", a["k8"].shape[2])
    y = _run_q8(torch, mk, a)
    ref = orc.attn_decode_q8(a["q"], a["gate"], a["k8"], a["ks"], a["v8"], a["vs"], a["ctx"], a["group_start"])
    assert np.isfinite(y).all(), label
    e, n = rel_err(y, ref), norm_err(y, ref)
    say(label, "rel", e, "norm", n)
    assert e <= FP32_TOL, (label, e)
    assert n <= 1e-5, (label, n)
    return y


Q8_CASES = [c for c in CASES if c[0] in ("4 agents x 3 rows, ragged contexts", "1 agent x 5 rows (two column blocks)",
                                         "T = 1, ragged tail", "T = 16, one group (four column blocks)",
                                         "unequal groups, many splits", "16 agents x 1 row",
                                         "1 agent x 10 rows (three column blocks)")]


@pytest.mark.parametrize("label,ctx,sizes,Hq,Hkv,gate", Q8_CASES, ids=[c[0] for c in Q8_CASES])
def test_attn_q8_parity(orc, label, ctx, sizes, Hq, Hkv, gate):
    torch = need_gpu()
    import bit_weight_streaming_q4_amd as mk
    a = recipes.attn_inputs_q8(ctx, sizes, Hq=Hq, Hkv=Hkv, gate=gate)
    _check_q8(orc, torch, mk, a, label)


def test_attn_q8_full_size_long_context(orc):
    """One agent at 131072 cached positions in q8_0 (the pages' long-context
    setting), T = 5; every output compared, two calls bit-identical."""
    torch = need_gpu()
    import bit_weight_streaming_q4_amd as mk
    a = recipes.attn_inputs_q8([131072], [5])
    y1 = _check_q8(orc, torch, mk, a, "q8 long context T = 5")
    assert np.array_equal(y1, _run_q8(torch, mk, a)), "two calls differ"


def test_attn_graph_replay_matches_eager():
    """Both attention entry points captured in a HIP graph: three replays,
    with eager calls on other inputs in between, each bit-identical to the
    eager call (the calls use no memset and no allocation)."""
    torch = need_gpu()
    import bit_weight_streaming_q4_amd as mk
    a = recipes.attn_inputs([300, 41, 1000], [3, 2, 3])
    b = recipes.attn_inputs_q8([300, 41, 1000], [3, 2, 3])
    dev = "cuda"
    q = torch.from_numpy(a["q"]).to(dev)
    gt = torch.from_numpy(a["gate"]).to(dev)
    k = torch.from_numpy(a["k"].view(np.int16)).to(dev)
    v = torch.from_numpy(a["v"].view(np.int16)).to(dev)
    t8 = [torch.from_numpy(b["k8"]).to(dev), torch.from_numpy(b["ks"].view(np.int16)).to(dev),
          torch.from_numpy(b["v8"]).to(dev), torch.from_numpy(b["vs"].view(np.int16)).to(dev)]
    ctx, gs = a["ctx"], a["group_start"]
    ws = mk.workspace(mk.mk_attn_decode_workspace(8, 32, 8, ctx, gs))
    o, o8 = torch.empty_like(q), torch.empty_like(q)

    def calls():
        mk.mk_attn_decode(q, gt, k, v, ctx, gs, o, ws=ws)
        mk.mk_attn_decode_q8(q, gt, *t8, ctx, gs, o8, ws=ws)

    say("attention graph capture", "ctx", list(ctx))
    calls()
    torch.cuda.synchronize()
    ref, ref8 = o.clone(), o8.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    other = recipes.attn_inputs([50], [2], gate=False)
    oq = torch.from_numpy(other["q"]).to(dev)
    ok_ = torch.from_numpy(other["k"].view(np.int16)).to(dev)
    ov = torch.from_numpy(other["v"].view(np.int16)).to(dev)
    for _ in range(3):
        o.fill_(float("nan"))
        o8.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(o8, ref8)
        mk.mk_attn_decode(oq, None, ok_, ov, other["ctx"], other["group_start"], torch.empty_like(oq))
        torch.cuda.synchronize()
