"""GPU parity of the activation quantizer, the T-row Q4_K-style GEMV (both
engines) and the FFN block, against the CPU oracle on the same seeded inputs."""
import numpy as np
import pytest

import oracle
import synth
from synth import recipes
from tests._util import FP32_TOL, need_gpu, norm_err, rel_err, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _mk():
    import bit_weight_streaming_q4_amd as mk
    return mk


def test_quantize_bit_exact():
    torch = need_gpu()
    mk = _mk()
    T, K = 16, 655360  # 1.05e7 values
    x = synth.normal_f32(5, 1, 0, T * K).reshape(T, K)
    x[0, :32] = 0.0  # all-zero group
    # exact half-way cases: group max 127 gives s = 1, then n + 0.5 values
    x[1, :32] = np.arange(32) - 15.5
    x[1, 0] = 127.0
    x[2, :32] = (np.arange(32) - 16) * 3.0 + 1.5
    x[2, 31] = -127.0 * 3.0
    x[3, :32] *= 1e-30  # tiny magnitudes (s subnormal-adjacent)
    # groups with no usable scale and non-finite elements
    tiny = np.float32(2.0 ** -149)
    k = np.arange(32) - 16
    x[4, :32] = (k % 4) * tiny  # amax/127 underflows: s = 0, zero codes
    x[4, 32:64] = np.where(k == 0, 63, -(k % 7)) * tiny  # the largest amax that underflows
    x[4, 64:96] = np.clip(k * 4, -64, 64) * tiny  # s = 2^-149 exactly
    x[4, 96:128] *= 1e-40  # subnormal inputs with a subnormal scale
    x[5, 5] = np.nan  # one NaN element
    x[5, 32:64] = np.nan  # a group of NaN only
    x[5, 70] = np.inf  # infinite amax
    x[5, 71] = -np.inf
    say("quantize", T, K)
    xd = to_dev(x)
    a8 = torch.empty(T, K, dtype=torch.int8, device="cuda")
    s = torch.empty(T, K // 32, dtype=torch.float32, device="cuda")
    gs = torch.empty(T, K // 32, dtype=torch.int32, device="cuda")
    mk.mk_quantize_rows(xd, a8, s, gs)
    ra8, rs, rgs = oracle.quantize_rows(x)
    assert np.array_equal(to_np(a8), ra8)
    assert np.array_equal(to_np(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(to_np(gs), rgs)


def _gemv_gpu(mk, W, x, path, torch):
    Wd = mk.Q4K.from_fields(W)
    xd = to_dev(x)
    y = torch.empty(x.shape[0], W["n_out"], dtype=torch.float32, device="cuda")
    mk.mk_qgemv_rows(Wd, xd, y, path=path)
    return to_np(y)


@pytest.mark.parametrize("N,K", [(200, 768), (64, 256), (130, 2304)])
def test_gemv_vs_oracle_shapes_and_paths(N, K):
    torch = need_gpu()
    mk = _mk()
    W = synth.q4k_fields(7, N + K, N, K)
    for T in (1, 2, 3, 5, 7, 8, 12, 16):
        x = synth.normal_f32(7, 900 + T, 0, T * K).reshape(T, K)
        ref = oracle.qgemv(W, x)
        paths = [mk.MK_PATH_MFMA] + ([mk.MK_PATH_DOT4] if T <= 8 else [])
        for path in paths:
            say("gemv", N, K, T, path)
            y = _gemv_gpu(mk, W, x, path, torch)
            assert rel_err(y, ref) <= FP32_TOL, (T, path, rel_err(y, ref))
            assert norm_err(y, ref) <= 1e-5


def _int_rows(T, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.integers(-127, 128, size=(T, K)).astype(np.float32)
    x.reshape(T, -1, 32)[:, :, 7] = 127.0  # max |x| = 127 in every group -> s = 1
    return x


def _family(N, K, d_bits, dmin_bits, sc, m, seed):
    rng = np.random.default_rng(seed)
    nsb = K // 256
    return {"d": np.full((N, nsb), d_bits, np.uint16), "dmin": np.full((N, nsb), dmin_bits, np.uint16),
            "sc": sc if np.ndim(sc) == 3 else np.full((N, nsb, 8), sc, np.uint8),
            "m": m if np.ndim(m) == 3 else np.full((N, nsb, 8), m, np.uint8),
            "q": rng.integers(0, 16, size=(N, K)).astype(np.uint8), "n_out": N, "n_in": K}


def test_gemv_integer_families_are_exact():
    """The integer sub-block sums are exact: with d, dmin, sc, m and the
    activation scale chosen so every partial result is an integer below 2^24,
    the fp32 outputs equal the exact integer results bit for bit."""
    torch = need_gpu()
    mk = _mk()
    N, K = 192, 1024
    one = 0x3C00
    rng = np.random.default_rng(11)
    sc = rng.integers(0, 64, size=(N, K // 256, 8)).astype(np.uint8)
    m = rng.integers(0, 64, size=(N, K // 256, 8)).astype(np.uint8)
    fams = {"E1": _family(N, K, one, 0, 1, 0, 1), "E2": _family(N, K, 0, one, 0, 1, 2),
            "E3": _family(N, K, one, one, sc, m, 3)}
    for T in (1, 5, 12):
        x = _int_rows(T, K, 40 + T)
        xi = x.astype(np.int64).reshape(T, K // 32, 32)
        for name, W in fams.items():
            qi = W["q"].astype(np.int64).reshape(N, K // 32, 32)
            P = np.einsum("tgi,ogi->tog", xi, qi)
            scg = W["sc"].reshape(N, -1).astype(np.int64)
            mg = W["m"].reshape(N, -1).astype(np.int64)
            dd = 1 if name != "E2" else 0
            dm = 1 if name != "E1" else 0
            exp = dd * (P * scg[None]).sum(-1) - dm * (xi.sum(-1)[:, None, :] * mg[None]).sum(-1)
            # every partial sum the kernel can form is an integer below 2^24
            bound = dd * (np.abs(P) * scg[None]).sum(-1) + dm * (np.abs(xi.sum(-1))[:, None, :] * mg[None]).sum(-1)
            assert bound.max() < 2 ** 24
            for path in [mk.MK_PATH_MFMA] + ([mk.MK_PATH_DOT4] if T <= 8 else []):
                say("family", name, T, path)
                y = _gemv_gpu(mk, W, x, path, torch)
                assert np.array_equal(y, exp.astype(np.float32)), (name, T, path)


def test_gemv_rows_paths_and_reruns_bit_identical():
    torch = need_gpu()
    mk = _mk()
    N, K = 320, 1536
    W = synth.q4k_fields(8, 1, N, K)
    Wd = mk.Q4K.from_fields(W)
    x = synth.normal_f32(8, 2, 0, 8 * K).reshape(8, K)
    xd = to_dev(x)
    outs = {}
    for path in (mk.MK_PATH_DOT4, mk.MK_PATH_MFMA):
        y = torch.empty(8, N, dtype=torch.float32, device="cuda")
        mk.mk_qgemv_rows(Wd, xd, y, path=path)
        outs[path] = to_np(y)
        y2 = torch.empty_like(y)
        mk.mk_qgemv_rows(Wd, xd, y2, path=path)
        assert np.array_equal(to_np(y2), outs[path]), "rerun differs"
        for t in range(8):
            y1 = torch.empty(1, N, dtype=torch.float32, device="cuda")
            mk.mk_qgemv_rows(Wd, xd[t:t + 1].contiguous(), y1, path=path)
            assert np.array_equal(to_np(y1)[0], outs[path][t]), ("row", t, path)
    say("paths agree bitwise")
    assert np.array_equal(outs[mk.MK_PATH_DOT4], outs[mk.MK_PATH_MFMA])


def test_gemv_full_size_single_row():
    """5120 x 5120 weight, one fp32 row ~ N(0, 1), seed 0: every output."""
    torch = need_gpu()
    mk = _mk()
    W = recipes.gemv_weight()
    x = recipes.rows_f32(1, 5120)
    ref = oracle.qgemv(W, x)
    for path in (mk.MK_PATH_AUTO, mk.MK_PATH_MFMA):
        say("gemv 5120x5120 T=1", path)
        y = _gemv_gpu(mk, W, x, path, torch)
        assert rel_err(y, ref) <= FP32_TOL
        assert norm_err(y, ref) <= 1e-6


def test_ffn_full_size_five_rows():
    """gate/up 5120 -> 17408 and down 17408 -> 5120, T = 5 (token + 4 drafts).
    The intermediate h is compared at tolerance; the down projection is checked
    teacher-forced (oracle applied to the GPU's h) and end to end."""
    torch = need_gpu()
    mk = _mk()
    Ws = recipes.ffn_weights()
    x = recipes.rows_f32(5, 5120, seed=1, tensor=14)
    say("ffn cfg1 T=5")
    g, u, d = (mk.Q4K.from_fields(Ws[k]) for k in ("gate", "up", "down"))
    xd = to_dev(x)
    y = torch.empty(5, 5120, dtype=torch.float32, device="cuda")
    h = torch.empty(5, 17408, dtype=torch.float32, device="cuda")
    mk.mk_ffn_rows(g, u, d, xd, y, h_out=h)
    yg, hg = to_np(y), to_np(h)
    ref_y, ref_h = oracle.ffn(Ws["gate"], Ws["up"], Ws["down"], x, return_h=True)
    assert rel_err(hg, ref_h) <= FP32_TOL
    assert rel_err(yg, oracle.qgemv(Ws["down"], hg)) <= FP32_TOL
    assert rel_err(yg, ref_y) <= FP32_TOL, rel_err(yg, ref_y)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 12, 16])
def test_ffn_small_rows_vs_oracle(T):
    """FFN block at H = 512, F = 768 (gate/up 3 tiles x 2 superblocks per row,
    down 8 tiles x 3): h at tolerance; y teacher-forced on the GPU's h and end
    to end; a call without h_out gives the same y bit for bit."""
    torch = need_gpu()
    mk = _mk()
    H, F = 512, 768
    Ws = {m: synth.q4k_fields(20 + i, T, n_out, n_in)
          for i, (m, n_out, n_in) in enumerate([("gate", F, H), ("up", F, H), ("down", H, F)])}
    x = synth.normal_f32(23, T, 0, T * H).reshape(T, H)
    say("ffn small", T)
    g, u, d = (mk.Q4K.from_fields(Ws[k]) for k in ("gate", "up", "down"))
    xd = to_dev(x)
    y = torch.empty(T, H, dtype=torch.float32, device="cuda")
    h = torch.empty(T, F, dtype=torch.float32, device="cuda")
    mk.mk_ffn_rows(g, u, d, xd, y, h_out=h)
    yg, hg = to_np(y), to_np(h)
    ref_y, ref_h = oracle.ffn(Ws["gate"], Ws["up"], Ws["down"], x, return_h=True)
    assert rel_err(hg, ref_h) <= FP32_TOL
    assert rel_err(yg, oracle.qgemv(Ws["down"], hg)) <= FP32_TOL
    assert rel_err(yg, ref_y) <= FP32_TOL, rel_err(yg, ref_y)
    y2 = torch.empty_like(y)
    mk.mk_ffn_rows(g, u, d, xd, y2)
    assert np.array_equal(to_np(y2), yg)


def test_gemv_ffn_graph_replay_matches_eager():
    """The GEMV and FFN entry points captured in one HIP graph (no memset
    nodes: the quantizer clears the tile counters) and replayed three times,
    with eager calls in between, give the eager results bit for bit."""
    torch = need_gpu()
    mk = _mk()
    N, K, T = 320, 1536, 5
    W = synth.q4k_fields(30, 1, N, K)
    Wd = mk.Q4K.from_fields(W)
    H, F = 512, 768
    Ws = {m: synth.q4k_fields(31 + i, 1, n_out, n_in)
          for i, (m, n_out, n_in) in enumerate([("gate", F, H), ("up", F, H), ("down", H, F)])}
    g, u, d = (mk.Q4K.from_fields(Ws[k]) for k in ("gate", "up", "down"))
    xa = to_dev(synth.normal_f32(32, 1, 0, T * K).reshape(T, K))
    xb = to_dev(synth.normal_f32(33, 1, 0, T * H).reshape(T, H))
    ya = torch.empty(T, N, dtype=torch.float32, device="cuda")
    yb = torch.empty(T, H, dtype=torch.float32, device="cuda")
    wsa = mk.workspace(mk.mk_qgemv_rows_workspace(T, N, K))
    wsb = mk.workspace(mk.mk_ffn_rows_workspace(T, H, F))

    def calls():
        mk.mk_qgemv_rows(Wd, xa, ya, ws=wsa)
        mk.mk_ffn_rows(g, u, d, xb, yb, ws=wsb)

    calls()
    torch.cuda.synchronize()
    ref_a, ref_b = to_np(ya), to_np(yb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(3):
        ya.zero_()
        yb.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say("graph replay", rep)
        assert np.array_equal(to_np(ya), ref_a), rep
        assert np.array_equal(to_np(yb), ref_b), rep
        calls()
        torch.cuda.synchronize()


# --------------------------------------------------------- the step's engines
def _step_path(mk, torch, W, x, ws=None):
    Wd = mk.Q4K.from_fields(W)
    T = x.shape[0]
    y = torch.empty(T, W["n_out"], dtype=torch.float32, device="cuda")
    if ws is None:
        ws = mk.workspace(mk.mk_qgemv_rows_workspace(T, W["n_out"], W["n_in"]), "cuda")
    mk.mk_qgemv_rows(Wd, to_dev(x), y, ws=ws, path=mk.MK_PATH_STEP)
    return to_np(y), ws


def _decode_records(ws, T, K):
    """The step's activation records at the start of the workspace, decoded
    into a8 [16][K], s and s*gsum [16][K/32] (layout stated in mk.h)."""
    nsb = K // 256
    raw = to_np(ws)[: nsb * 5120].reshape(nsb, 5120)
    codes = raw[:, :4096].view(np.int8).reshape(nsb, 8, 4, 16, 8)  # [b][j][q][t][e]
    a8 = codes.transpose(3, 0, 1, 2, 4).reshape(16, K)
    s = raw[:, 4096:4608].copy().view(np.float32).reshape(nsb, 8, 16).transpose(2, 0, 1).reshape(16, K // 32)
    sg = raw[:, 4608:].copy().view(np.float32).reshape(nsb, 8, 16).transpose(2, 0, 1).reshape(16, K // 32)
    return a8, s, sg


@pytest.mark.parametrize("T", [1, 2, 5, 8, 9, 12, 16])
def test_step_engines_integer_families_are_exact(T):
    """The decode step's three engines (dot4 at T = 1, the packed 16x16x64
    matrix-core engine up to 8 padded rows, the 16x16x32 engine above) give
    the exact integer results of the E1-E3 families bit for bit, like the
    standalone engines."""
    torch = need_gpu()
    mk = _mk()
    N, K = 192, 1024
    one = 0x3C00
    rng = np.random.default_rng(11)
    sc = rng.integers(0, 64, size=(N, K // 256, 8)).astype(np.uint8)
    m = rng.integers(0, 64, size=(N, K // 256, 8)).astype(np.uint8)
    fams = {"E1": _family(N, K, one, 0, 1, 0, 1), "E2": _family(N, K, 0, one, 0, 1, 2),
            "E3": _family(N, K, one, one, sc, m, 3)}
    x = _int_rows(T, K, 40 + T)
    xi = x.astype(np.int64).reshape(T, K // 32, 32)
    for name, W in fams.items():
        qi = W["q"].astype(np.int64).reshape(N, K // 32, 32)
        P = np.einsum("tgi,ogi->tog", xi, qi)
        dd = 1 if name != "E2" else 0
        dm = 1 if name != "E1" else 0
        exp = dd * (P * W["sc"].reshape(N, -1).astype(np.int64)[None]).sum(-1) - \
            dm * (xi.sum(-1)[:, None, :] * W["m"].reshape(N, -1).astype(np.int64)[None]).sum(-1)
        say("step engine family", name, T)
        y, _ = _step_path(mk, torch, W, x)
        assert np.array_equal(y, exp.astype(np.float32)), (name, T)


@pytest.mark.parametrize("T", [1, 2, 5, 8, 9, 12, 16])
def test_step_records_bit_exact(T):
    """The step's fused epilogue quantizer (store_q8) writes records whose
    codes, scales and scaled code sums equal the oracle's quantizer bit for
    bit, edge groups included; rows T..15 are zero."""
    torch = need_gpu()
    mk = _mk()
    K = 2048
    x = synth.normal_f32(6, 100 + T, 0, T * K).reshape(T, K)
    tiny = np.float32(2.0 ** -149)
    k = np.arange(32) - 16
    x[0, :32] = 0.0
    x[0, 32:64] = (k % 4) * tiny
    x[0, 64:96] = np.clip(k * 4, -64, 64) * tiny
    x[0, 96:128] *= 1e-40
    x[-1, 130] = np.nan
    x[-1, 160:192] = np.nan
    x[-1, 200] = np.inf
    x[0, 256:288] = np.arange(32) - 15.5
    x[0, 256] = 127.0
    W = synth.q4k_fields(6, 7, 64, K)
    say("step records", T)
    _, ws = _step_path(mk, torch, W, x)
    a8, s, sg = _decode_records(ws, T, K)
    ra8, rs, rgs = oracle.quantize_rows(x)
    assert np.array_equal(a8[:T], ra8)
    assert np.array_equal(s[:T].view(np.uint32), rs.view(np.uint32))
    with np.errstate(invalid="ignore"):
        rsg = (rs * rgs.astype(np.float32)).astype(np.float32)
    assert np.array_equal(sg[:T], rsg, equal_nan=True)
    assert not a8[T:].any() and not s[T:].any() and not sg[T:].any()


@pytest.mark.parametrize("N,K", [(200, 768), (64, 256)])
def test_step_engines_vs_oracle(N, K):
    torch = need_gpu()
    mk = _mk()
    W = synth.q4k_fields(9, N + K, N, K)
    for T in range(1, 17):  # every instance of the streaming kernel
        x = synth.normal_f32(9, 900 + T, 0, T * K).reshape(T, K)
        say("step engine vs oracle", N, K, T)
        y, _ = _step_path(mk, torch, W, x)
        assert rel_err(y, oracle.qgemv(W, x)) <= FP32_TOL, T
