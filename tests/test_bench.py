"""The measurement's own arithmetic, checked on the CPU against closed forms: the
visible (query, key) pairs behind every TFLOP/s figure, the algorithmic bytes
behind every roofline fraction, and the refusal of a multi-GPU run."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_visible_pairs_closed_forms():
    bench = _bench()
    from workloads import WORKLOADS
    # causal, Sq == Sk: row i sees i + 1 keys
    w = WORKLOADS["causal_prefill_bf16"]
    assert bench.visible_pairs(w) == w.Hq * w.B * w.Sq * (w.Sq + 1) // 2
    assert 4 * w.d * bench.visible_pairs(w) == 549822922752
    # causal with a left window of W: min(i + 1, W + 1) keys
    w = WORKLOADS["window_prefill_bf16"]
    W = w.window_left
    per_row = sum(min(i + 1, W + 1) for i in range(w.Sq))
    assert bench.visible_pairs(w) == w.B * w.Hq * per_row
    # decode, no mask: every key
    w = WORKLOADS["gqa_decode_bf16"]
    assert bench.visible_pairs(w) == w.B * w.Hq * w.Sq * w.Sk
    # Sq > Sk with a causal mask: the first Sq - Sk rows see nothing
    class P:
        B, Sq, Sk, Hq, causal, window_left = 1, 10, 4, 3, True, -1
    assert bench.visible_pairs(P) == 3 * (1 + 2 + 3 + 4)


def test_algorithmic_bytes_of_the_decode_headline():
    pytest.importorskip("torch")
    bench = _bench()
    from workloads import WORKLOADS
    w = WORKLOADS["gqa_decode_bf16"]
    kv = 2 * w.B * w.Sk * w.Hkv * w.d * 2
    q = w.B * w.Sq * w.Hq * w.d * 2
    rows = w.B * w.Sq * w.Hq
    read, write = bench.algorithmic_bytes("attn_decode_kdma_kernel", "gqa_decode_bf16")
    assert read == kv + q == 67117056
    import tiled_prefill_amd as tpa
    S = tpa.plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left, 0, w.dtype)["num_splits"]
    assert S > 1 and write == S * rows * (w.d + 1) * 4
    # the combine reads exactly what the decode kernel wrote, and writes O and lse
    c_read, c_write = bench.algorithmic_bytes("lse_combine_kernel", "gqa_decode_bf16")
    assert c_read == write and c_write == q + rows * 4
    # the streaming-read reference reads K and V only
    assert bench.algorithmic_bytes("stream_read_kernel", "gqa_decode_bf16") == (kv, 0)
