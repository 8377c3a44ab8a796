"""bench.py's contract, checked without a GPU: one GPU only (any other count
exits with a message), and the algorithmic bytes per launch that the roofline
figures divide by.

The byte counts follow from the tensor shapes alone: the prefill reads q, k,
z, v and beta and writes o (bf16), reads S0 and writes S_T (fp32) and reads A;
the decode step reads and writes the fp32 state once and moves one token of
q, k, v, z, beta and o per head; the prologue reads and writes q, k and v once
and the convolution states and taps.
"""
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_bytes_k3_shape():
    B, T, H, d = 1, 4096, 96, 128
    per_token_head = 4 * d * 2 + d * 2 + 2          # q, k, z, v in; o out; beta
    per_head = 2 * d * d * 4                        # S0 in, S_T out
    assert bench.prefill_bytes(B, T, H, d) == B * T * H * per_token_head + B * H * per_head + H * 4
    assert bench.prefill_bytes(B, T, H, d) == 516_686_208


def test_decode_bytes_k3_shape():
    B, H, d = 64, 96, 128
    per_update = 2 * d * d * 4 + 4 * d * 2 + 2 + d * 2   # S in + out; q, k, v, z; beta; o
    assert per_update == 132_354
    assert bench.decode_bytes(B, H, d) == B * H * per_update + H * 4 == 813_183_360


def test_prologue_bytes_k3_shape():
    assert bench.conv_norm_bytes(1, 4096, 96, 128, 4) == 605_011_968


def test_prefill_flops_k3_shape():
    # 6 d^2 + 5 C d + C^2 / 3 per token-head: the three d x d state products of a
    # token (U, O and the update), the chunk-local products and the inverse
    B, T, H, d, C = 1, 4096, 96, 128, 16
    per = 6 * d * d + 5 * C * d + C * C / 3
    assert abs(bench.prefill_flops(B, T, H, d, C) - B * T * H * per) < 1.0
    assert round(bench.prefill_flops(B, T, H, d, C)) == 42_714_791_936
