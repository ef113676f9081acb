"""GPU check of mk_qgemv_rows_noalloc (the T-row GEMV whose workspace is the
library's static per-GPU scratch array): through the C ABI, its output equals
mk_qgemv_rows_ex's (own workspace) bit for bit, on two calls in a row, the
second with a smaller input; a shape whose workspace exceeds the array is
refused before anything runs."""
import numpy as np
import pytest

import oracle
import synth
from tests._util import FP32_TOL, need_gpu, rel_err, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _mk():
    import bit_weight_streaming_q4_amd as mk
    return mk


def _pair(mk, torch, W, x, path):
    Wd = mk.Q4K.from_fields(W)
    xd = to_dev(x)
    T, N = x.shape[0], W["n_out"]
    y_ref = torch.empty(T, N, dtype=torch.float32, device="cuda")
    mk.mk_qgemv_rows(Wd, xd, y_ref, path=path)
    y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    mk.mk_qgemv_rows_noalloc(Wd, xd, y, path=path)
    return to_np(y), to_np(y_ref)


@pytest.mark.parametrize("path", ["auto", "dot4", "mfma", "step"])
def test_noalloc_equals_workspace_call_twice(path):
    torch = need_gpu()
    mk = _mk()
    p = {"auto": mk.MK_PATH_AUTO, "dot4": mk.MK_PATH_DOT4, "mfma": mk.MK_PATH_MFMA, "step": mk.MK_PATH_STEP}[path]
    # first call: the model's 5120 x 5120 shape (several tiles); second: a
    # smaller ragged one, so the array holds the first call's leftovers
    for (N, K, T) in ((5120, 5120, 8 if path == "dot4" else 12), (130, 768, 3)):
        W = synth.q4k_fields(61, N + K, N, K)
        x = synth.normal_f32(61, 7 + T, 0, T * K).reshape(T, K)
        say("noalloc", path, N, K, T)
        y, y_ref = _pair(mk, torch, W, x, p)
        assert np.array_equal(y, y_ref)
        assert rel_err(y, oracle.qgemv(W, x)) <= FP32_TOL


def test_noalloc_refuses_shapes_above_the_scratch_array():
    torch = need_gpu()
    mk = _mk()
    big = mk.Q4K(torch.empty(256, dtype=torch.uint8, device="cuda"), 32768, 32768)  # never read
    assert mk.mk_qgemv_rows_workspace(16, 32768, 32768) > (16 << 20)
    x = torch.zeros(16, 32768, dtype=torch.float32, device="cuda")
    y = torch.zeros(16, 32768, dtype=torch.float32, device="cuda")
    with pytest.raises(mk.MkError) as ei:
        mk.mk_qgemv_rows_noalloc(big, x, y)
    assert ei.value.status == mk.MK_ERR_WORKSPACE
    assert to_np(y).max() == 0.0
