"""CPU checks of bench.py's contract that need no GPU: several GPUs are
refused with a message, and the algorithmic byte counts behind the reported
GB/s follow the shapes they describe."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_follow_the_shapes():
    # 64 layers x (10240x5120 + 5120x10240 + 3 x 17408x5120) weights at 4.5 bit
    assert bench.stack_bytes() == 64 * (2 * 10240 * 5120 + 3 * 17408 * 5120) // 256 * 144 == 13_400_801_280
    # attention: every visible K and V row once in fp16, plus q, gate, o in fp32
    assert bench.attn_bytes([32768] * 4, [3] * 4) == 4 * 32771 * 8 * 128 * 4 + 12 * 32 * 128 * 12
    # q8_0: one byte per code, an fp16 scale per 32 dims of a K row and per 32
    # positions of a V dimension
    L = 131077
    assert bench.attn_bytes_q8([131072], [5]) == (L * 8 * 128 * 2 + L * 8 * 4 * 2 + ((L + 31) // 32) * 8 * 128 * 2
                                                  + 5 * 32 * 128 * 12)


def test_oracle_beside_every_timed_call_has_a_sample_and_a_rate():
    """The CPU leg that times the oracle beside the standalone calls runs on
    the CPU alone and names calls that the GPU leg times, each with a
    positive time, a rate consistent with the call's bytes, and its sample."""
    r = bench.cpu_entry_points()
    gpu_names = {"qgemv_5120x5120_T1", "qgemv_5120x5120_T5", "qgemv_5120x5120_T12", "ffn_5120_17408_T5",
                 f"lmhead_verify_V{bench.VOCAB}_T5", f"lmhead_sample_V{bench.VOCAB}_T12_k32",
                 "deltanet_step_48x32_T5", "attn_decode_4x32768_T12", "attn_decode_q8_4x32768_T12",
                 "mtp_draft_T12_G4_n2"}
    assert set(r) == gpu_names
    for name, v in r.items():
        assert v["us"] > 0 and v["oracle_s_per_sample"] > 0 and v["sample"], name
        # scaled up, never down (oracle_s_per_sample is rounded to 0.1 ms)
        assert v["us"] + 60 >= v["oracle_s_per_sample"] * 1e6, name
    # the whole 5120^2 GEMV call: its rate is its bytes over its time
    g = r["qgemv_5120x5120_T1"]
    nbytes = 5120 * 5120 // 256 * 144 + 2 * 5120 * 4
    assert abs(g["gb_s"] - nbytes / (g["us"] * 1e-6) / 1e9) <= 1e-3 * g["gb_s"] + 1e-4
