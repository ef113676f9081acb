"""Python binding of libmk, the MI355X (gfx950) library of the multi-row
speculative-verification decode step (C ABI in ``include/mk.h``).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libmk.so``.  Device buffers are torch tensors on the ROCm device; the
current torch stream is passed to every call.  There is no CPU fallback: if
``libmk.so`` is missing, importing the compute functions raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_OK, MK_ERR_ARG, MK_ERR_SHAPE, MK_ERR_ALIGN, MK_ERR_RANGE = 0, -1, -2, -3, -4
MK_ERR_WORKSPACE, MK_ERR_LAUNCH, MK_ERR_COOP, MK_ERR_DEVICE = -5, -6, -7, -8
MK_PATH_AUTO, MK_PATH_DOT4, MK_PATH_MFMA, MK_PATH_STEP = 0, 1, 2, 3
MK_T_MAX = 16
MK_STEP_T_MAX = 24
MK_ATTN_CAP_MAX = 1 << 26


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class mk_q4k(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_void_p), ("n_out", ctypes.c_int32), ("n_in", ctypes.c_int32)]


class mk_deltanet(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("ring", ctypes.c_void_p), ("n_acc", ctypes.c_void_p),
                ("nh", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("T_max", ctypes.c_int32)]


class mk_step_attn(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("cap", ctypes.c_int32),
                ("h_ctx", ctypes.c_void_p), ("q", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p)]


class mk_mtp(ctypes.Structure):
    _fields_ = [("fc", mk_q4k), ("gate", mk_q4k), ("up", mk_q4k), ("down", mk_q4k)]


class mk_stack_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("proj", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("p_in", ctypes.POINTER(mk_q4k)), ("p_out", ctypes.POINTER(mk_q4k)),
                ("gate", ctypes.POINTER(mk_q4k)), ("up", ctypes.POINTER(mk_q4k)),
                ("down", ctypes.POINTER(mk_q4k)), ("lm_head", ctypes.c_void_p),
                ("h_gdn_layer", ctypes.c_void_p), ("n_agents", ctypes.c_int32),
                ("dn", ctypes.POINTER(mk_deltanet))]


_lib = None


def lib():
    """The loaded libmk.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with bit_weight_streaming_q4_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.mk_status_string.argtypes = [ctypes.c_int]
    L.mk_status_string.restype = ctypes.c_char_p
    L.mk_last_error.restype = ctypes.c_char_p
    L.mk_init.argtypes = [ctypes.c_int]
    L.mk_q4k_bytes.argtypes = [i32, i32]
    L.mk_q4k_bytes.restype = sz
    L.mk_q4k_pack.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P]
    L.mk_q4k_unpack.argtypes = [P, i32, i32, P, P, P, P, P]
    L.mk_quantize_rows.argtypes = [P, i32, i32, P, P, P, P]
    L.mk_qgemv_rows_workspace.argtypes = [i32, i32, i32]
    L.mk_qgemv_rows_workspace.restype = sz
    L.mk_qgemv_rows.argtypes = [ctypes.POINTER(mk_q4k), P, i32, P, P, sz, P]
    L.mk_qgemv_rows_ex.argtypes = [ctypes.POINTER(mk_q4k), P, i32, P, i32, P, sz, P]
    L.mk_qgemv_rows_noalloc.argtypes = [ctypes.POINTER(mk_q4k), P, i32, P, i32, P]
    L.mk_ffn_rows_workspace.argtypes = [i32, i32, i32]
    L.mk_ffn_rows_workspace.restype = sz
    L.mk_ffn_rows.argtypes = [ctypes.POINTER(mk_q4k)] * 3 + [P, i32, P, P, P, sz, P]
    L.mk_lmhead_verify_workspace.argtypes = [i32, i32, i32]
    L.mk_lmhead_verify_workspace.restype = sz
    L.mk_lmhead_verify.argtypes = [P, i32, i32, P, i32, P, i32, P, P, P, P, P, sz, P]
    L.mk_lmhead_sample_workspace.argtypes = [i32, i32, i32]
    L.mk_lmhead_sample_workspace.restype = sz
    L.mk_lmhead_sample.argtypes = [P, i32, i32, P, i32, P, i32, P, i32, ctypes.c_float, P, P, P, P, P, P, P, sz, P]
    L.mk_mtp_draft_workspace.argtypes = [ctypes.POINTER(mk_mtp), i32, i32, i32]
    L.mk_mtp_draft_workspace.restype = sz
    L.mk_mtp_draft.argtypes = [ctypes.POINTER(mk_mtp), P, i32, i32, P, i32, P, i32, P, P, i32, P, P, P, sz, P]
    L.mk_deltanet_step.argtypes = [ctypes.POINTER(mk_deltanet), i32, P, P, P, P, P, i32, P, P]
    L.mk_deltanet_commit.argtypes = [ctypes.POINTER(mk_deltanet), P]
    L.mk_deltanet_status.argtypes = [ctypes.POINTER(mk_deltanet), P]
    L.mk_stack_create.argtypes = [ctypes.POINTER(mk_stack_desc), ctypes.POINTER(ctypes.c_void_p)]
    L.mk_stack_destroy.argtypes = [P]
    L.mk_decode_step_workspace.argtypes = [P, i32]
    L.mk_decode_step_workspace.restype = sz
    L.mk_decode_step.argtypes = [P, P, i32, P, i32, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    L.mk_decode_step_attn.argtypes = [P, P, i32, P, i32, P, P, P, P, P, P, P, P, P, P, P, ctypes.POINTER(mk_step_attn),
                                      P, sz, P]
    L.mk_decode_step_attn_workspace.argtypes = [P, i32, P, i32, ctypes.POINTER(mk_step_attn)]
    L.mk_decode_step_attn_workspace.restype = sz
    L.mk_decode_step_stamps.argtypes = [P, i32, P, P, i32, P]
    L.mk_decode_step_last_ms.argtypes = [P]
    L.mk_decode_step_last_ms.restype = ctypes.c_float
    L.mk_read_probe.argtypes = [P, sz, P, P]
    L.mk_attn_decode_workspace.argtypes = [i32, i32, i32, P, P, i32]
    L.mk_attn_decode_workspace.restype = sz
    L.mk_attn_decode.argtypes = [P, P, i32, i32, P, P, i32, i32, i32, P, P, i32, P, P, sz, P]
    L.mk_attn_decode_q8.argtypes = [P, P, i32, i32, P, P, P, P, i32, i32, i32, P, P, i32, P, P, sz, P]
    _lib = L
    return L


def _check(status: int, what: str):
    if status != MK_OK:
        msg = lib().mk_last_error().decode(errors="replace")
        raise MkError(status, f"{what}: {msg or lib().mk_status_string(status).decode()}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _np_ptr(a):
    return a.ctypes.data


def mk_init(device: int = 0):
    _check(lib().mk_init(device), "mk_init")


# --------------------------------------------------------------------- weights
def mk_q4k_bytes(n_out: int, n_in: int) -> int:
    return int(lib().mk_q4k_bytes(n_out, n_in))


def mk_q4k_pack(fields: dict, r0: int = 0, r1: int | None = None) -> np.ndarray:
    """Host packing of field arrays (rows [r0, r1) of an n_out x n_in matrix;
    the arrays hold exactly those rows) into the device layout."""
    n_in = int(fields["n_in"])
    n_out = int(fields.get("n_out_total", fields["n_out"]))
    r1 = n_out if r1 is None else r1
    if r0 % 64 or (r1 % 64 and r1 != n_out):
        raise ValueError("row slices must be 64-row aligned")
    rows_t = (r1 - r0 + 63) // 64
    out = np.empty(rows_t * (n_in // 256) * 9216, np.uint8)
    arrs = [np.ascontiguousarray(fields[k]) for k in ("d", "dmin", "sc", "m", "q")]
    _check(lib().mk_q4k_pack(*[_np_ptr(a) for a in arrs], n_out, n_in, r0, r1, _np_ptr(out)), "mk_q4k_pack")
    return out


def mk_q4k_unpack(blocks: np.ndarray, n_out: int, n_in: int) -> dict:
    nsb = n_in // 256
    f = {"d": np.empty((n_out, nsb), np.uint16), "dmin": np.empty((n_out, nsb), np.uint16),
         "sc": np.empty((n_out, nsb, 8), np.uint8), "m": np.empty((n_out, nsb, 8), np.uint8),
         "q": np.empty((n_out, n_in), np.uint8)}
    blocks = np.ascontiguousarray(blocks)
    _check(lib().mk_q4k_unpack(_np_ptr(blocks), n_out, n_in, *[_np_ptr(f[k]) for k in ("d", "dmin", "sc", "m", "q")]),
           "mk_q4k_unpack")
    return f


class Q4K:
    """A packed Q4_K-style matrix resident in device memory."""

    def __init__(self, blocks, n_out: int, n_in: int):
        self.blocks = blocks  # torch uint8 tensor on the device
        self.n_out, self.n_in = n_out, n_in
        self.c = mk_q4k(blocks.data_ptr(), n_out, n_in)

    @classmethod
    def from_fields(cls, fields: dict, device="cuda"):
        import torch
        host = mk_q4k_pack(fields)
        return cls(torch.from_numpy(host).to(device), int(fields["n_out"]), int(fields["n_in"]))

    @classmethod
    def empty(cls, n_out: int, n_in: int, device="cuda"):
        import torch
        return cls(torch.empty(mk_q4k_bytes(n_out, n_in), dtype=torch.uint8, device=device), n_out, n_in)


def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------- compute
def mk_read_probe(buf, sink, stream=None):
    """Reads every byte of the device tensor buf once (measurement aid);
    sink is a 1-element int32 device tensor."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().mk_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "mk_read_probe")


def mk_quantize_rows(x, a8, s, gsum, stream=None):
    T, K = x.shape
    _check(lib().mk_quantize_rows(_ptr(x), T, K, _ptr(a8), _ptr(s), _ptr(gsum), _stream(stream)),
           "mk_quantize_rows")


def mk_qgemv_rows_workspace(T: int, n_out: int, n_in: int) -> int:
    return int(lib().mk_qgemv_rows_workspace(T, n_out, n_in))


def mk_qgemv_rows(W: Q4K, x, y, ws=None, path: int = MK_PATH_AUTO, stream=None):
    T = x.shape[0]
    if ws is None:
        ws = workspace(mk_qgemv_rows_workspace(T, W.n_out, W.n_in), x.device)
    _check(lib().mk_qgemv_rows_ex(ctypes.byref(W.c), _ptr(x), T, _ptr(y), path, _ptr(ws), ws.numel(),
                                  _stream(stream)), "mk_qgemv_rows")


def mk_qgemv_rows_noalloc(W: Q4K, x, y, path: int = MK_PATH_AUTO, stream=None):
    """mk_qgemv_rows with its workspace in the library's static per-GPU
    scratch array (allocates nothing; calls on one GPU must not overlap)."""
    T = x.shape[0]
    _check(lib().mk_qgemv_rows_noalloc(ctypes.byref(W.c), _ptr(x), T, _ptr(y), path, _stream(stream)),
           "mk_qgemv_rows_noalloc")


def mk_ffn_rows_workspace(T: int, H: int, F: int) -> int:
    return int(lib().mk_ffn_rows_workspace(T, H, F))


def mk_ffn_rows(gate: Q4K, up: Q4K, down: Q4K, x, y, h_out=None, ws=None, stream=None):
    T, H = x.shape
    if ws is None:
        ws = workspace(mk_ffn_rows_workspace(T, H, gate.n_out), x.device)
    _check(lib().mk_ffn_rows(ctypes.byref(gate.c), ctypes.byref(up.c), ctypes.byref(down.c), _ptr(x), T, _ptr(y),
                             _ptr(h_out), _ptr(ws), ws.numel(), _stream(stream)), "mk_ffn_rows")


def mk_lmhead_verify_workspace(V: int, H: int, T: int) -> int:
    return int(lib().mk_lmhead_verify_workspace(V, H, T))


def mk_lmhead_verify(W16, hid, group_start, drafts, argmax, n_acc, tokens, ws=None, V=None, stream=None):
    """W16: int16/uint16-bit fp16 tensor [V][H] (V may be a prefix of its rows)."""
    H = W16.shape[1]
    V = W16.shape[0] if V is None else V
    T = hid.shape[0]
    if group_start is None:
        gs, G = None, 1
    else:
        gs_np = np.ascontiguousarray(group_start, np.int32)
        gs, G = gs_np.ctypes.data, len(gs_np) - 1
    if ws is None:
        ws = workspace(mk_lmhead_verify_workspace(V, H, T), hid.device)
    _check(lib().mk_lmhead_verify(_ptr(W16), V, H, _ptr(hid), T, gs, G, _ptr(drafts), _ptr(argmax), _ptr(n_acc),
                                  _ptr(tokens), _ptr(ws), ws.numel(), _stream(stream)), "mk_lmhead_verify")


def mk_lmhead_sample_workspace(V: int, H: int, T: int) -> int:
    return int(lib().mk_lmhead_sample_workspace(V, H, T))


def mk_lmhead_sample(W16, hid, group_start, drafts, top_k, temperature, u_acc, u_samp, n_acc, tokens,
                     topk_idx=None, topk_logit=None, ws=None, V=None, stream=None):
    """Sampling-mode verification: u_acc, u_samp fp32 [T] device tensors of
    the caller's uniforms; topk_idx int32 [T][32] / topk_logit fp32 [T][32]
    optional outputs."""
    H = W16.shape[1]
    V = W16.shape[0] if V is None else V
    T = hid.shape[0]
    if group_start is None:
        gs, G = None, 1
    else:
        gs_np = np.ascontiguousarray(group_start, np.int32)
        gs, G = gs_np.ctypes.data, len(gs_np) - 1
    if ws is None:
        ws = workspace(mk_lmhead_sample_workspace(V, H, T), hid.device)
    _check(lib().mk_lmhead_sample(_ptr(W16), V, H, _ptr(hid), T, gs, G, _ptr(drafts), int(top_k), float(temperature),
                                  _ptr(u_acc), _ptr(u_samp), _ptr(topk_idx), _ptr(topk_logit), _ptr(n_acc),
                                  _ptr(tokens), _ptr(ws), ws.numel(), _stream(stream)), "mk_lmhead_sample")


class MtpHead:
    """The synthetic MTP draft head on the device: fc (H x 2H) and one FFN
    (gate, up: F x H; down: H x F), each a Q4K."""

    def __init__(self, fc: Q4K, gate: Q4K, up: Q4K, down: Q4K):
        self.fc, self.gate, self.up, self.down = fc, gate, up, down
        self.c = mk_mtp(fc.c, gate.c, up.c, down.c)

    @classmethod
    def from_fields(cls, f: dict, device="cuda"):
        return cls(*[Q4K.from_fields(f[k], device) for k in ("fc", "gate", "up", "down")])


def mk_mtp_draft_workspace(head: MtpHead, V_draft: int, T: int, G: int) -> int:
    return int(lib().mk_mtp_draft_workspace(ctypes.byref(head.c), V_draft, T, G))


def mk_mtp_draft(head: MtpHead, embed16, V_draft, hidden, group_start, tokens, n_acc, n_draft, drafts, trace=None,
                 ws=None, stream=None):
    """On-device MTP draft loop: hidden fp32 [T][H], tokens int32 [T],
    n_acc int32 [G] and drafts int32 [n_draft][G] are device tensors."""
    V = embed16.shape[0]
    T = hidden.shape[0]
    if group_start is None:
        gs, G = None, 1
    else:
        gs_np = np.ascontiguousarray(group_start, np.int32)
        gs, G = gs_np.ctypes.data, len(gs_np) - 1
    if ws is None:
        ws = workspace(mk_mtp_draft_workspace(head, V_draft, T, G), hidden.device)
    _check(lib().mk_mtp_draft(ctypes.byref(head.c), _ptr(embed16), V, V_draft, _ptr(hidden), T, gs, G, _ptr(tokens),
                              _ptr(n_acc), int(n_draft), _ptr(drafts), _ptr(trace), _ptr(ws), ws.numel(),
                              _stream(stream)), "mk_mtp_draft")


def _attn_groups(T, ctx, group_start):
    ctx_np = np.ascontiguousarray(ctx, np.int32)
    gs_np = np.ascontiguousarray([0, T] if group_start is None else group_start, np.int32)
    return ctx_np, gs_np, len(gs_np) - 1


def mk_attn_decode_workspace(T: int, Hq: int, Hkv: int, ctx, group_start=None) -> int:
    ctx_np, gs_np, G = _attn_groups(T, ctx, group_start)
    return int(lib().mk_attn_decode_workspace(T, Hq, Hkv, ctx_np.ctypes.data, gs_np.ctypes.data, G))


def mk_attn_decode(q, gate, k_cache, v_cache, ctx, group_start, o, ws=None, stream=None):
    """q, gate (or None), o: fp32 [T][Hq][128]; k_cache int16/uint16 bits
    [G][Hkv][cap][128]; v_cache [G][Hkv][128][cap]; ctx, group_start: host
    sequences (group_start None = one group)."""
    T, Hq, d = q.shape
    G_, Hkv, cap, _ = k_cache.shape
    ctx_np, gs_np, G = _attn_groups(T, ctx, group_start)
    if ws is None:
        ws = workspace(max(mk_attn_decode_workspace(T, Hq, Hkv, ctx_np, gs_np), 256), q.device)
    _check(lib().mk_attn_decode(_ptr(q), _ptr(gate), T, Hq, _ptr(k_cache), _ptr(v_cache), Hkv, d, cap,
                                ctx_np.ctypes.data, gs_np.ctypes.data, G, _ptr(o), _ptr(ws), ws.numel(),
                                _stream(stream)), "mk_attn_decode")


def mk_attn_decode_q8(q, gate, k_codes, k_scales, v_codes, v_scales, ctx, group_start, o, ws=None, stream=None):
    """As mk_attn_decode over q8_0 caches: k_codes int8 [G][Hkv][cap][128] with
    k_scales fp16 bits [G][Hkv][cap][4]; v_codes int8 [G][Hkv][cap/64][128][64]
    (tile-major) with v_scales [G][Hkv][cap/32][128]."""
    T, Hq, d = q.shape
    G_, Hkv, cap, _ = k_codes.shape
    ctx_np, gs_np, G = _attn_groups(T, ctx, group_start)
    if ws is None:
        ws = workspace(max(mk_attn_decode_workspace(T, Hq, Hkv, ctx_np, gs_np), 256), q.device)
    _check(lib().mk_attn_decode_q8(_ptr(q), _ptr(gate), T, Hq, _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                   _ptr(v_scales), Hkv, d, cap, ctx_np.ctypes.data, gs_np.ctypes.data, G, _ptr(o),
                                   _ptr(ws), ws.numel(), _stream(stream)), "mk_attn_decode_q8")


class DeltaNetState:
    """Device buffers of one Gated DeltaNet state: S [nh][128][128], the
    two-half ring [2][nh][T_max-1][258] and n_acc = [accept length, ring half,
    status word, unused]."""

    def __init__(self, nh: int, T_max: int, device="cuda", S=None):
        import torch
        self.S = torch.zeros(nh, 128, 128, dtype=torch.float32, device=device) if S is None else S
        self.ring = torch.zeros(2, nh, T_max - 1, 258, dtype=torch.float32, device=device)
        self.n_acc = torch.zeros(4, dtype=torch.int32, device=device)
        self.nh, self.T_max = nh, T_max
        self.c = mk_deltanet(self.S.data_ptr(), self.ring.data_ptr(), self.n_acc.data_ptr(), nh, 128, 128, T_max)


def mk_deltanet_step(st: DeltaNetState, q, k, v, g, beta, o, use_prev_acc: bool = True, stream=None):
    T = q.shape[0]
    _check(lib().mk_deltanet_step(ctypes.byref(st.c), int(use_prev_acc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), T, _ptr(o), _stream(stream)), "mk_deltanet_step")


def mk_deltanet_commit(st: DeltaNetState, stream=None):
    _check(lib().mk_deltanet_commit(ctypes.byref(st.c), _stream(stream)), "mk_deltanet_commit")


def mk_deltanet_status(st: DeltaNetState, stream=None) -> int:
    """Synchronises, reads and clears the state's status word; returns
    MK_ERR_RANGE if an out-of-range accept length was read since the last
    call (nothing was replayed then), else MK_OK."""
    r = lib().mk_deltanet_status(ctypes.byref(st.c), _stream(stream))
    if r not in (MK_OK, MK_ERR_RANGE):
        _check(r, "mk_deltanet_status")
    return int(r)


# --------------------------------------------------------------------- decode step
class Stack:
    """A synthetic layer stack for mk_decode_step: per layer p_in, p_out, gate,
    up, down (Q4K), an fp16 lm_head [vocab][hidden], the layers that carry a
    Gated DeltaNet mixer, and one DeltaNetState per agent (verify group)."""

    def __init__(self, layers, lm_head, gdn_layers=None, agents=None):
        import torch
        self.layers = layers
        L = len(layers)
        self.d_layers = L
        self.hidden, self.proj = layers[0]["p_in"].n_in, layers[0]["p_in"].n_out
        self.ffn = layers[0]["gate"].n_out
        self.lm_head = lm_head
        self.vocab = lm_head.shape[0]
        self.agents = agents or []
        arr = {k: (mk_q4k * L)(*[layers[l][k].c for l in range(L)]) for k in ("p_in", "p_out", "gate", "up", "down")}
        self._arr = arr
        flags = np.zeros(L, np.uint8)
        if gdn_layers is not None:
            for l in gdn_layers:
                flags[l] = 1
        self._flags = flags
        self._dn = (mk_deltanet * max(1, len(self.agents)))(*[a.c for a in self.agents])
        desc = mk_stack_desc(L, self.hidden, self.proj, self.ffn, self.vocab, arr["p_in"], arr["p_out"],
                             arr["gate"], arr["up"], arr["down"], lm_head.data_ptr(),
                             flags.ctypes.data if gdn_layers is not None else None, len(self.agents), self._dn)
        self._desc = desc
        h = ctypes.c_void_p()
        _check(lib().mk_stack_create(ctypes.byref(desc), ctypes.byref(h)), "mk_stack_create")
        self.h = h
        self._ws = {}

    def close(self):
        """Destroys the host-side descriptor (and its two HIP events) now."""
        if getattr(self, "h", None):
            lib().mk_stack_destroy(self.h)
            self.h = None

    def __del__(self):
        # No HIP call while the interpreter is finalizing: the runtime (or a
        # profiler wrapped around it) may already be tearing down.  The
        # descriptor is then left to the process exit.
        import sys
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, T: int) -> int:
        return int(lib().mk_decode_step_workspace(self.h, T))

    def workspace(self, T: int, device="cuda"):
        if T not in self._ws:
            self._ws[T] = workspace(self.workspace_bytes(T), device)
        return self._ws[T]


def step_attn(q, k_cache, v_cache, o, ctx, gate=None):
    """The attention of a step's full-attention layers (mk_step_attn): q, gate,
    o [n_layers][T][Hq][128] fp32; k_cache [n_layers][G][Hkv][cap][128] and
    v_cache [n_layers][G][Hkv][128][cap] fp16 (device); ctx: cached positions
    per agent.  The returned structure keeps its arguments alive."""
    ctx = np.ascontiguousarray(ctx, np.int32)
    a = mk_step_attn(int(q.shape[0]), int(q.shape[2]), int(k_cache.shape[2]), int(k_cache.shape[3]), ctx.ctypes.data,
                     _ptr(q), _ptr(gate), _ptr(k_cache), _ptr(v_cache), _ptr(o), None, None, None, None)
    a._keep = (ctx, q, gate, k_cache, v_cache, o)
    return a


def step_attn_q8(q, k_codes, k_scales, v_codes, v_scales, o, ctx, gate=None):
    """The same over a q8_0 cache: k_codes [n_layers][G][Hkv][cap][128] int8,
    k_scales [n_layers][G][Hkv][cap][4] fp16 bits, v_codes
    [n_layers][G][Hkv][cap/64][128][64] int8, v_scales
    [n_layers][G][Hkv][cap/32][128] fp16 bits (device)."""
    ctx = np.ascontiguousarray(ctx, np.int32)
    a = mk_step_attn(int(q.shape[0]), int(q.shape[2]), int(k_codes.shape[2]), int(k_codes.shape[3]), ctx.ctypes.data,
                     _ptr(q), _ptr(gate), None, None, _ptr(o), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                     _ptr(v_scales))
    a._keep = (ctx, q, gate, k_codes, k_scales, v_codes, v_scales, o)
    return a


def mk_decode_step(st: Stack, x, group_start=None, drafts=None, gdn=None, gdn_o=None, argmax=None, trace=None,
                   ws=None, stream=None, attn=None):
    """One decode step in one persistent launch.  x [T][hidden] (in/out).
    gdn: dict of q, k, v, g, beta device tensors [T][nh][..] (None without GDN
    layers).  attn: a step_attn(...) for the full-attention layers (None:
    none).  Returns (tokens [T] int32 host, n_acc [G] int32 host)."""
    T = x.shape[0]
    if group_start is None:
        gs, G = None, 1
        gsa = None
    else:
        gsa = np.ascontiguousarray(group_start, np.int32)
        gs, G = gsa.ctypes.data, len(gsa) - 1
    tokens = np.full(T, -1, np.int32)
    n_acc = np.zeros(G, np.int32)
    g = gdn or {}
    if attn is None:
        if ws is None:
            ws = st.workspace(T, x.device)
        _check(lib().mk_decode_step(st.h, _ptr(x), T, gs, G, _ptr(drafts), _ptr(g.get("q")), _ptr(g.get("k")),
                                    _ptr(g.get("v")), _ptr(g.get("g")), _ptr(g.get("beta")), _ptr(gdn_o),
                                    tokens.ctypes.data, n_acc.ctypes.data, _ptr(argmax), _ptr(trace), _ptr(ws),
                                    ws.numel(), _stream(stream)), "mk_decode_step")
        return tokens, n_acc
    if ws is None:
        need = int(lib().mk_decode_step_attn_workspace(st.h, T, gs, G, ctypes.byref(attn)))
        if need == 0:
            raise MkError(MK_ERR_ARG, "mk_decode_step_attn_workspace: invalid attention arguments")
        ws = workspace(need, x.device)
    _check(lib().mk_decode_step_attn(st.h, _ptr(x), T, gs, G, _ptr(drafts), _ptr(g.get("q")), _ptr(g.get("k")),
                                     _ptr(g.get("v")), _ptr(g.get("g")), _ptr(g.get("beta")), _ptr(gdn_o),
                                     tokens.ctypes.data, n_acc.ctypes.data, _ptr(argmax), _ptr(trace),
                                     ctypes.byref(attn), _ptr(ws), ws.numel(), _stream(stream)),
           "mk_decode_step_attn")
    return tokens, n_acc


def mk_decode_step_last_ms(st: Stack) -> float:
    """Event-timed duration (ms) of the last persistent launch on this stack."""
    return float(lib().mk_decode_step_last_ms(st.h))


def mk_decode_step_stamps(st: Stack, T: int, ws=None, n_max: int = 520):
    """Device clock stamps of the last step on this workspace (seconds from
    the launch start): [0] start, [i] after barrier i, [-1] end."""
    ws = st.workspace(T) if ws is None else ws
    h = np.zeros(n_max, np.uint64)
    hz = ctypes.c_int64()
    n = lib().mk_decode_step_stamps(st.h, T, _ptr(ws), h.ctypes.data, n_max, ctypes.byref(hz))
    if n < 0:
        _check(n, "mk_decode_step_stamps")
    return (h[:n].astype(np.float64) - float(h[0])) / float(hz.value)


def pack_to_device(fields: dict, device="cuda", host_buf=None) -> Q4K:
    """Packs a field-array matrix on the host and uploads it (host_buf: an
    optional reusable uint8 numpy buffer of at least mk_q4k_bytes bytes)."""
    import torch
    n_out, n_in = int(fields["n_out"]), int(fields["n_in"])
    nb = mk_q4k_bytes(n_out, n_in)
    blocks = host_buf[:nb] if host_buf is not None and host_buf.size >= nb else np.empty(nb, np.uint8)
    arrs = [np.ascontiguousarray(fields[k]) for k in ("d", "dmin", "sc", "m", "q")]
    _check(lib().mk_q4k_pack(*[_np_ptr(a) for a in arrs], n_out, n_in, 0, n_out, _np_ptr(blocks)), "mk_q4k_pack")
    return Q4K(torch.from_numpy(blocks).to(device), n_out, n_in)
