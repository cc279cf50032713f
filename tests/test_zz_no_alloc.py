"""attn_fwd_noalloc (the forward whose scratch is the library's static device array)
against attn_fwd, through the C-ABI: two calls in a row, the second smaller; the
static array keeps the first call's contents, which must not leak into the second."""
import ctypes
import math

import pytest
import torch

import oracle
import tiled_prefill_amd as tpa
from workloads import small_case

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _call(entry, q, k, v, o, lse, causal, wl, S):
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    fn = getattr(tpa.load(), entry)
    return fn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
              ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
              ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, Sq, Sk, d, int(causal), wl,
              1.0 / math.sqrt(d), S, tpa.BF16 if q.dtype == torch.bfloat16 else tpa.FP32,
              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (dtype, B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits): the first of each
# pair needs the larger scratch
PAIRS = [
    [("bf16", 1, 32, 4, 1, 32768, 128, False, -1, 0), ("bf16", 1, 16, 2, 1, 3000, 128, False, -1, 0)],
    [("fp32", 2, 16, 16, 17, 2065, 128, True, -1, 0), ("fp32", 1, 4, 4, 1, 256, 64, False, -1, 5)],
    [("bf16", 1, 8, 2, 700, 900, 128, True, -1, 0), ("bf16", 1, 4, 4, 150, 150, 64, True, 40, 3)],
]


@pytest.mark.parametrize("pair", PAIRS, ids=["decode", "verify_fp32", "prefill"])
def test_noalloc_matches_attn_fwd_on_two_calls(pair):
    for n, (dtype, B, Hq, Hkv, Sq, Sk, d, causal, wl, S) in enumerate(pair):
        q, k, v = small_case(50 + n, dtype, B, Hq, Hkv, Sq, Sk, d)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        need = tpa.plan(B, Hq, Hkv, Sq, Sk, d, causal, wl, S, dtype)["workspace_bytes"]
        assert need <= 16 << 20
        print(f"noalloc call {n}: {dtype} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} d={d} "
              f"causal={causal} wl={wl} S={S} scratch={need}", flush=True)
        o_ref = torch.empty_like(qd)
        lse_ref = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV)
        assert _call("attn_fwd", qd, kd, vd, o_ref, lse_ref, causal, wl, S) == 0
        assert _call("attn_fwd_noalloc", qd, kd, vd, o, lse, causal, wl, S) == 0
        torch.cuda.synchronize()
        # the same kernels on the same plan: the same bits
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        ro, rl = oracle.attn_ref(q, k, v, causal, wl, 1.0 / math.sqrt(d))
        err = (o.float().cpu().double() - torch.from_numpy(ro)).abs().max().item()
        assert err <= (1e-5 if dtype == "fp32" else 2e-2)


def test_noalloc_refuses_problems_beyond_its_scratch():
    # 256 forced splits of 64 x 32 rows of 128 fp32 values: ~269 MB of partials
    q, k, v = small_case(60, "bf16", 64, 32, 32, 1, 4096, 128)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    assert tpa.plan(64, 32, 32, 1, 4096, 128, num_splits=256)["workspace_bytes"] > 16 << 20
    o = torch.empty_like(qd)
    lse = torch.empty((64, 32, 1), dtype=torch.float32, device=DEV)
    assert _call("attn_fwd_noalloc", qd, kd, vd, o, lse, False, -1, 256) == -1
    assert "noalloc" in tpa.load().attn_last_error().decode()
