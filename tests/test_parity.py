"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Tolerances (from the stated accuracy targets and the arithmetic):
  fp32 inputs: max |o - ref| <= 1e-5.
  bf16 inputs (fp32 accumulation): max |o - ref| <= 2e-2, and
      max |o - ref| / |ref| <= 1e-2 where |ref| > 0.1.
  lse: fp32 inputs |lse - ref| <= 2e-5 * max(1, |ref|) (fp32 accumulation);
      bf16 inputs |lse - ref| <= 1e-3 * max(1, |ref|): the bf16 prefill path sums
      P after rounding it to fp16 (relative error <= 2^-11 per term, so
      |d lse| <= 2^-11 ~ 4.9e-4); -inf exactly where the row sees no key (and
      then o == 0 exactly).
Small cases are compared element by element; full-size workloads run in the
launch configuration the benchmark times and are compared on sampled query
rows, each recomputed by the oracle on its own.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_prefill_amd as tpa
from workloads import WORKLOADS, make_inputs, random_partials, small_case

pytestmark = pytest.mark.gpu

DEV = "cuda"


def assert_parity(o, lse, ro, rl, dtype, what=""):
    o = o.detach().float().cpu().double().numpy()
    err = np.abs(o - ro)
    if dtype == "fp32":
        assert err.max(initial=0.0) <= 1e-5, f"{what}: max abs {err.max()}"
    else:
        assert err.max(initial=0.0) <= 2e-2, f"{what}: max abs {err.max()}"
        big = np.abs(ro) > 0.1
        if big.any():
            rel = (err[big] / np.abs(ro[big])).max()
            assert rel <= 1e-2, f"{what}: max rel {rel}"
    if lse is not None:
        lse = lse.detach().cpu().double().numpy()
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(lse), fin), f"{what}: masked-row pattern differs"
        assert np.all(lse[~fin] == -np.inf)
        if fin.any():
            d = np.abs(lse[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))
            assert d.max() <= (2e-5 if dtype == "fp32" else 1e-3), f"{what}: lse err {d.max()}"


def run_case(dtype, B, Hq, Hkv, Sq, Sk, d, causal, wl, S, seed=0, std=1.0):
    q, k, v = small_case(seed, dtype, B, Hq, Hkv, Sq, Sk, d, std=std)
    scale = 1.0 / math.sqrt(d)
    print(f"case {dtype} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} d={d} causal={causal} "
          f"wl={wl} S={S} seed={seed}", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_left=wl,
                     scale=scale, num_splits=S)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_ref(q, k, v, causal, wl, scale)
    assert_parity(o, lse, ro, rl, dtype, f"{dtype} {B},{Hq},{Hkv},{Sq},{Sk},{d} c={causal} wl={wl} S={S}")
    return o, lse


@pytest.mark.parametrize("S", [0, 1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_fp32_split_sweep(S):
    # tiny fp32 decode, every split count 1..8 (4 key blocks: 5..8 leave empty splits)
    w = WORKLOADS["decode_fp32"]
    q, k, v, _ = make_inputs(w, seed=0)
    print(f"decode_fp32 S={S}", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, num_splits=S)
    ro, rl = oracle.attn_ref(q, k, v, False, -1, w.scale)
    assert_parity(o, lse, ro, rl, "fp32", f"decode_fp32 S={S}")


@pytest.mark.parametrize("S", [0, 1])
def test_spec_verify_fp32_full(S):
    w = WORKLOADS["spec_verify_fp32"]
    q, k, v, _ = make_inputs(w, seed=1)
    print(f"spec_verify_fp32 S={S}", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, num_splits=S)
    ro, rl = oracle.attn_ref(q, k, v, True, -1, w.scale)
    assert_parity(o, lse, ro, rl, "fp32", f"spec_verify S={S}")


@pytest.mark.parametrize("B,H,q_len,kv_len", [(2, 16, 17, 2065), (1, 64, 33, 161),
                                              (2, 64, 9, 521), (2, 8, 9, 9)])
def test_verify_page_shapes_fp32(B, H, q_len, kv_len):
    # shapes of the verify-attention parity run on the occupancy blog page
    run_case("fp32", B, H, H, q_len, kv_len, 128, True, -1, 0, seed=2)


@pytest.mark.parametrize("tile", ["0", "2"], ids=["widest_rows", "waves_2x4"])
@pytest.mark.parametrize("case", [(2, 16, 16, 17, 2065, 128, True, -1, 0), (1, 8, 2, 9, 521, 128, True, -1, 3),
                                  (2, 4, 4, 20, 300, 64, False, -1, 0), (1, 4, 1, 5, 77, 128, True, 2, 2),
                                  (1, 2, 2, 32, 129, 64, True, 40, 1)])
def test_verify_tile_choices_fp32(tile, case, attn_options):
    # the general kernel's other tiles for <= 32 query rows per KV head (the
    # planner's default there is the LDS-copy kernel, switched off here)
    attn_options("ATTN_F32_DMA", 0)
    attn_options("ATTN_VERIFY_TILE", tile)
    run_case("fp32", *case, seed=4)


F32_LDS_CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, d, causal, wl, S: the fp32 kernel that copies K/V
    # into per-wave LDS stages (<= 32 query rows per KV head)
    ("fp32", 2, 16, 16, 17, 2065, 128, True, -1, 0),   # the verify workload's shape
    ("fp32", 1, 4, 4, 32, 100, 128, True, -1, 0),      # exactly 32 rows
    ("fp32", 1, 8, 2, 4, 333, 128, True, -1, 0),       # GQA packed: 16 rows
    ("fp32", 1, 4, 2, 9, 521, 64, True, 30, 3),        # packed 18 rows, window, d 64
    ("fp32", 2, 6, 3, 1, 77, 128, False, -1, 2),       # decode, ragged last block
    ("fp32", 1, 2, 2, 30, 20, 128, True, -1, 1),       # Sq > Sk: fully masked rows
    ("fp32", 1, 2, 1, 3, 5, 64, False, 1, 1),          # fewer keys than one block
    ("fp32", 1, 4, 4, 5, 1000, 128, False, -1, 37),    # many splits, empty ones
    ("fp32", 1, 4, 4, 5, 1000, 64, True, 100, 0),
    ("fp32", 3, 4, 4, 12, 4100, 128, False, -1, 1),    # one split: many blocks per wave
]


@pytest.mark.parametrize("waves", [4, 8])  # waves per workgroup, one LDS stage each
@pytest.mark.parametrize("case", F32_LDS_CASES)
def test_f32_lds_kernel_shapes(case, waves, attn_options):
    attn_options("ATTN_F32_DMA", 2)  # decode's row counts too
    attn_options("ATTN_F32_WAVES", waves)
    if waves == 8 and case[6] == 64:
        pytest.skip("d 64 has only the 4-wave form")
    assert tpa.plan(*case[1:7], case[7], case[8], case[9], "fp32")["block_n"] == 16  # that kernel
    run_case(*case, seed=8)


SMALL = [
    # dtype, B, Hq, Hkv, Sq, Sk, d, causal, wl, S
    ("bf16", 2, 4, 4, 200, 200, 128, True, -1, 1),
    ("bf16", 1, 8, 2, 130, 300, 128, True, 50, 1),
    ("bf16", 1, 8, 2, 130, 300, 64, False, -1, 3),
    ("bf16", 2, 16, 2, 3, 500, 128, True, -1, 0),
    ("bf16", 1, 32, 4, 1, 1000, 128, False, -1, 0),
    ("bf16", 1, 32, 4, 1, 1000, 64, False, -1, 7),
    ("bf16", 1, 4, 4, 300, 100, 128, True, -1, 1),
    ("bf16", 1, 4, 1, 5, 77, 128, True, 2, 2),
    ("bf16", 3, 6, 3, 40, 40, 64, True, 0, 1),
    ("bf16", 1, 2, 2, 1, 1, 128, False, -1, 1),
    ("bf16", 2, 8, 8, 64, 64, 128, False, 10, 1),
    ("bf16", 1, 16, 16, 257, 1025, 128, True, 300, 4),
    ("bf16", 2, 4, 2, 16, 700, 128, True, -1, 0),
    ("bf16", 1, 16, 2, 2, 333, 128, True, -1, 0),   # decode tile: 2 positions x 8 heads, ragged halves
    ("bf16", 2, 8, 2, 4, 95, 64, True, 20, 3),      # decode tile: 16 packed rows, window, d 64
    ("bf16", 1, 8, 1, 2, 333, 128, False, -1, 0),   # decode tile: one KV head (grid-y divisor 1)
    ("fp32", 1, 4, 2, 33, 70, 64, True, 5, 0),
    ("fp32", 2, 2, 2, 20, 150, 128, False, -1, 4),
    ("fp32", 1, 8, 1, 2, 333, 128, False, -1, 0),
    ("fp32", 1, 4, 4, 90, 60, 64, True, -1, 1),
    ("fp32", 1, 2, 2, 130, 130, 128, True, 17, 2),
]


@pytest.mark.parametrize("case", SMALL)
def test_small_shapes(case):
    run_case(*case, seed=3)


def _random_cases(n, seed):
    """n forward problems from a fixed generator, spanning every kernel family
    (decode tiles, the fp32 verify kernel, prefill tiles, the general kernel):
    GQA groups of 1..8 heads (3 included), ragged query and key counts (more
    queries than keys too), both masks and windows, automatic and forced split
    counts; each small enough for the oracle to take well under a second."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = "bf16" if rng.random() < 0.65 else "fp32"
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.integers(1, 4))
        kind = rng.random()
        Sq = 1 if kind < 0.25 else (int(rng.integers(2, 33)) if kind < 0.5 else int(rng.integers(33, 600)))
        Sk = int(rng.integers(1, 1500))
        causal = bool(rng.random() < 0.6)
        wl = -1 if rng.random() < 0.6 else int(rng.integers(0, Sk + 1))
        S = 0 if rng.random() < 0.6 else int(rng.integers(1, 10))
        if B * Hkv * G * Sq * Sk * d > 1e8:
            continue
        cases.append((dtype, B, Hkv * G, Hkv, Sq, Sk, d, causal, wl, S))
    return cases


RANDOM = _random_cases(96, 20261203)


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: "%s_B%d_H%d-%d_q%d_k%d_d%d_c%d_w%d_S%d" % c)
def test_random_shapes(case):
    run_case(*case, seed=7)


def test_empty_keys_give_masked_rows():
    for dtype in ("fp32", "bf16"):
        q, k, v = small_case(4, dtype, 1, 4, 2, 3, 0, 64)
        o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV))
        torch.cuda.synchronize()
        assert torch.all(o.float().cpu() == 0)
        assert torch.all(lse.cpu() == float("-inf"))


def test_empty_query_is_noop():
    q, k, v = small_case(5, "bf16", 1, 4, 4, 0, 16, 64)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert o.numel() == 0


def test_lse_not_requested():
    q, k, v = small_case(6, "bf16", 1, 8, 2, 70, 90, 128)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, return_lse=False)
    assert lse is None
    ro, _ = oracle.attn_ref(q, k, v, True, -1, 1 / math.sqrt(128))
    assert_parity(o, None, ro, None, "bf16", "no lse")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_split_invariance(dtype):
    q, k, v = small_case(7, dtype, 1, 8, 2, 4, 1500, 128)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ro, rl = oracle.attn_ref(q, k, v, False, -1, 1 / math.sqrt(128))
    outs = []
    for S in (1, 2, 3, 7, 16, 64, 256):
        o, lse = tpa.fwd(qd, kd, vd, num_splits=S)
        assert_parity(o, lse, ro, rl, dtype, f"S={S}")
        outs.append(o.float().cpu())
    tol = 1e-5 if dtype == "fp32" else 2e-2
    for x in outs[1:]:
        assert (x - outs[0]).abs().max().item() <= tol


def test_deterministic():
    q, k, v = small_case(8, "bf16", 2, 8, 4, 100, 300, 128)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for S in (1, 5):
        o1, l1 = tpa.fwd(qd, kd, vd, causal=True, num_splits=S)
        o2, l2 = tpa.fwd(qd, kd, vd, causal=True, num_splits=S)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_non_default_stream():
    q, k, v = small_case(9, "bf16", 1, 32, 4, 1, 2048, 128)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        o, lse = tpa.fwd(qd, kd, vd, stream=s)
    s.synchronize()
    ro, rl = oracle.attn_ref(q, k, v, False, -1, 1 / math.sqrt(128))
    assert_parity(o, lse, ro, rl, "bf16", "stream")


@pytest.mark.parametrize("cols", ["0", "1", "1l", "rows"],
                         ids=["split_groups", "columns", "columns_looped", "rows"])
@pytest.mark.parametrize("S,d,dtype", [(1, 128, "fp32"), (2, 64, "bf16"), (5, 128, "bf16"),
                                       (8, 128, "fp32"), (9, 64, "bf16"), (16, 128, "fp32"),
                                       (64, 128, "fp32"), (256, 64, "fp32"), (128, 128, "bf16"),
                                       (7, 512, "bf16"), (51, 512, "bf16"), (256, 512, "fp32"),
                                       (1, 512, "fp32")])
def test_combine_kernel_parity(S, d, dtype, cols, attn_options):
    # four kernels: split groups; columns, with every partial of a thread in flight
    # at once (up to 16 splits) or looped; (512-wide rows only) one workgroup per row
    if cols == "rows":
        if d != 512:
            pytest.skip("the row-parallel combine serves 512-wide rows")
        attn_options("ATTN_COMBINE_ROWS", "1")
    else:
        attn_options("ATTN_COMBINE_ROWS", "0")
        attn_options("ATTN_COMBINE_COLS", cols[0])
        attn_options("ATTN_COMBINE_SMALL", "0" if cols == "1l" else "1")
    B, Sq, Hq = 2, 3, 5
    rows = B * Sq * Hq
    o_part, lse_part = random_partials(10 + S, S, rows, d, p_empty=0.3)
    lse_part[:, 0] = float("-inf")  # a row with every split empty
    o_part[:, 0] = 0
    # an empty split leaves its O_s unwritten: NaN there must never reach the output
    o_dev = o_part.clone()
    o_dev[torch.isneginf(lse_part)] = float("nan")
    out = torch.empty((B, Sq, Hq, d), dtype=torch.float32 if dtype == "fp32" else torch.bfloat16,
                      device=DEV)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=DEV)
    tpa.lse_combine(o_dev.to(DEV), lse_part.to(DEV), out, lse, B, Sq, Hq)
    ro, rl = oracle.lse_combine_ref(o_part, lse_part)
    ro = ro.reshape(B, Sq, Hq, d)
    rl = rl.reshape(B, Sq, Hq).transpose(0, 2, 1)
    got = out.float().cpu().double().numpy()
    tol = 1e-5 if dtype == "fp32" else 2e-2
    assert np.abs(got - ro).max() <= tol * max(1.0, np.abs(ro).max())
    lg = lse.cpu().double().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.abs(lg[fin] - rl[fin]).max() <= 2e-5 * max(1.0, np.abs(rl[fin]).max())


def test_varlen_small():
    B, Hq, Hkv, Sk, d = 5, 8, 2, 700, 128
    q, k, v = small_case(11, "bf16", B, Hq, Hkv, 1, Sk, d)
    seqlens = torch.tensor([700, 1, 0, 257, 513], dtype=torch.int32)
    ro, rl = oracle.attn_ref(q, k, v, False, -1, 1 / math.sqrt(d), seqlens_k=seqlens)
    for S in (0, 1, 3):
        o, lse = tpa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), seqlens.to(DEV), num_splits=S,
                                sum_seqlens_k=int(seqlens.sum()))
        assert_parity(o, lse, ro, rl, "bf16", f"varlen S={S}")


def _random_varlen(n, seed):
    """variable-length decode batches from a fixed generator: 2..24 sequences,
    1 or 2 query positions, GQA groups of 1..8 heads, both head dims, both masks
    and windows, automatic and forced split counts"""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B = int(rng.integers(2, 25))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        Sq = int(rng.choice([1, 2]))
        Sk = int(rng.integers(64, 4000))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.5)
        wl = -1 if rng.random() < 0.7 else int(rng.integers(0, Sk + 1))
        S = 0 if rng.random() < 0.7 else int(rng.integers(1, 17))
        if B * Hkv * G * Sq * Sk * d > 1e8:
            continue
        cases.append((B, Hkv * G, Hkv, Sq, Sk, d, causal, wl, S, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _random_varlen(12, 5077),
                         ids=lambda c: "B%d_H%d-%d_q%d_k%d_d%d_c%d_w%d_S%d_%d" % c)
def test_varlen_random_batches(case):
    B, Hq, Hkv, Sq, Sk, d, causal, wl, S, lseed = case
    q, k, v = small_case(lseed % 1000, "bf16", B, Hq, Hkv, Sq, Sk, d)
    g = torch.Generator().manual_seed(lseed)
    seqlens = torch.randint(0, Sk + 1, (B,), generator=g, dtype=torch.int32)
    seqlens[0] = Sk
    seqlens[B // 2] = 0
    print(f"varlen random {case} lengths {seqlens.tolist()}", flush=True)
    scale = 1.0 / math.sqrt(d)
    o, lse = tpa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), seqlens.to(DEV), causal=causal,
                            window_left=wl, scale=scale, num_splits=S, sum_seqlens_k=int(seqlens.sum()))
    torch.cuda.synchronize()
    ro, rl = oracle.attn_ref(q, k, v, causal, wl, scale, seqlens_k=seqlens)
    assert_parity(o, lse, ro, rl, "bf16", f"varlen random {case}")


@pytest.mark.parametrize("units", [1, 0], ids=["unit_grid", "split_grid"])
@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Sq, Sk, d, causal, wl, lengths seed, sum given
    (5, 8, 2, 1, 700, 128, False, -1, 1, "exact"),
    (70, 8, 2, 1, 300, 128, False, -1, 2, "exact"),     # more sequences than lanes: two scan steps
    (70, 8, 2, 1, 300, 64, False, -1, 3, "none"),       # no sum: B x S units
    (9, 16, 2, 2, 900, 128, True, -1, 4, "exact"),      # two positions x 8 heads per tile, causal
    (9, 8, 2, 1, 900, 128, False, 200, 5, "exact"),     # window: fewer blocks than the length
    (12, 8, 2, 1, 600, 128, False, -1, 6, "short"),     # sum understated: workgroups take several units
])
def test_varlen_work_units(case, units, attn_options):
    B, Hq, Hkv, Sq, Sk, d, causal, wl, seed, given = case
    attn_options("ATTN_VARLEN_UNITS", units)
    attn_options("ATTN_VARLEN_CHUNK", 128)  # small chunks: many splits per sequence
    q, k, v = small_case(30 + seed, "bf16", B, Hq, Hkv, Sq, Sk, d)
    g = torch.Generator().manual_seed(seed)
    seqlens = torch.randint(0, Sk + 1, (B,), generator=g, dtype=torch.int32)
    seqlens[0] = 0
    seqlens[-1] = Sk
    total = int(seqlens.sum())
    sum_arg = {"exact": total, "none": -1, "short": max(1, total // 10)}[given]
    pl = tpa.plan(B, Hq, Hkv, Sq, Sk, d, causal, wl, 0, "bf16", varlen=True, sum_seqlens_k=sum_arg)
    assert (pl["work_units"] > 0) == bool(units) and pl["num_splits"] > 1
    if units and given == "exact":
        assert pl["grid_x"] <= total // (64 * pl["chunk_blocks"]) + B
    print(f"varlen units={units} {case} plan {pl['grid_x']}x{pl['grid_y']} S={pl['num_splits']}", flush=True)
    ro, rl = oracle.attn_ref(q, k, v, causal, wl, 1 / math.sqrt(d), seqlens_k=seqlens)
    o, lse = tpa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), seqlens.to(DEV), causal=causal,
                            window_left=wl, sum_seqlens_k=sum_arg)
    assert_parity(o, lse, ro, rl, "bf16", f"varlen units={units} {case}")


@pytest.mark.parametrize("factor,causal,wl,d", [(8.0, True, -1, 128), (4.0, True, -1, 128),
                                                (8.0, False, -1, 128), (8.0, True, 1000, 128),
                                                (16.0, False, 300, 64), (2.0, True, -1, 64)])
def test_prefill_score_jumps(factor, causal, wl, d):
    # Keys are walked from the last block to the first. Scaling the first 64 keys
    # (exact in bf16: a power of two) makes their scores jump far above the
    # reference max the later keys set: x8 and x16 overflow the fp16 P of the
    # steady-tile form (that tile runs again with the exact max), x4 and x2 stay
    # inside fp16 with large P. The result must not depend on either.
    B, H, S = 1, 4, 600
    q, k, v = small_case(15, "bf16", B, H, H, S, S, d)
    k[:, :64] = (k[:, :64].float() * factor).to(k.dtype)
    scale = 1.0 / math.sqrt(d)
    print(f"score jumps factor={factor} causal={causal} wl={wl} d={d}", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_left=wl, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_ref(q, k, v, causal, wl, scale)
    assert_parity(o, lse, ro, rl, "bf16", f"jumps x{factor} c={causal} wl={wl} d={d}")


# ---------------------------------------------------------------------------
# full-size workloads in the benchmark's launch configuration
# ---------------------------------------------------------------------------
def _sampled_rows_check(w, q, k, v, o, lse, rows):
    """Recompute chosen query rows one by one with the oracle and compare."""
    delta = w.Sk - w.Sq
    for i in rows:
        if w.causal:
            kl = i + delta + 1  # keys the row can see, so the row aligns at the bottom right
            ro, rl = oracle.attn_ref(q[:, i:i + 1], k[:, :kl], v[:, :kl], True, w.window_left, w.scale)
        else:
            ro, rl = oracle.attn_ref(q[:, i:i + 1], k, v, False, w.window_left, w.scale)
        assert_parity(o[:, i:i + 1], lse[:, :, i:i + 1], ro, rl, w.dtype, f"{w.name} row {i}")


def _full_props(o, v):
    of = o.float()
    assert torch.isfinite(of).all()
    assert of.abs().max().item() <= v.float().abs().max().item() + 1e-3


def test_gqa_decode_full():
    w = WORKLOADS["gqa_decode_bf16"]
    q, k, v, _ = make_inputs(w, seed=0)
    print("gqa_decode_bf16 full", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    ro, rl = oracle.attn_ref(q, k, v, False, -1, w.scale)
    assert_parity(o, lse, ro, rl, "bf16", "gqa_decode full")


def test_varlen_decode_full():
    w = WORKLOADS["varlen_decode_bf16"]
    q, k, v, seqlens = make_inputs(w, seed=0)
    print("varlen_decode_bf16 full", flush=True)
    o, lse = tpa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), seqlens.to(DEV),
                            sum_seqlens_k=int(seqlens.sum()))
    ro, rl = oracle.attn_ref(q, k, v, False, -1, w.scale, seqlens_k=seqlens)
    assert_parity(o, lse, ro, rl, "bf16", "varlen_decode full")


@pytest.mark.parametrize("name", ["causal_prefill_bf16", "window_prefill_bf16"])
def test_prefill_full_sampled(name):
    w = WORKLOADS[name]
    q, k, v, _ = make_inputs(w, seed=0)
    print(f"{name} full", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, window_left=w.window_left)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    _full_props(o, v)
    S = w.Sq
    rows = sorted({0, 1, 15, 16, 63, 64, 127, 128, 129, 1000, 1023, 1024, 1025, 2047, 2048,
                   S // 2 + 7, S - 129, S - 128, S - 65, S - 2, S - 1})
    _sampled_rows_check(w, q, k, v, o, lse, rows)


# ---------------------------------------------------------------------------
# every kernel path a planner switch can select (ablations included)
# ---------------------------------------------------------------------------
ABLATIONS = [
    {"ATTN_PREFILL_SKIP": "1"},             # prefill with raised wave priority
    {"ATTN_PREFILL_WAVES": "4"},            # 128-row tiles (default with a window)
    {"ATTN_PREFILL_WAVES": "8"},            # 256-row tiles (default without one)
    {"ATTN_PREFILL_PERSIST": "1"},          # persistent workgroups, per-XCD tile queues
    {"ATTN_PREFILL_PERSIST": "1", "ATTN_PREFILL_WAVES": "8"},
    {"ATTN_GENERIC_PREFILL": "1"},          # general tile kernel for bf16 prefill
    {"ATTN_GENERIC_DECODE": "1"},           # general tile kernel for bf16 decode
    {"ATTN_DECODE_WAVES": "8"},             # 8-wave decode workgroups
    {"ATTN_DECODE_KDMA": "0"},              # decode with K straight into registers, 16-row V tiles
    {"ATTN_DECODE_KDMA": "1"},              # decode with K and V through LDS in 32-key halves
    {"ATTN_SPLIT_RULE": "1"},               # split-count rule of the tiling page
    {"ATTN_SPLIT_RULE": "2"},               # NSPLIT rule of the occupancy blog
    {"ATTN_SPLIT_RULE": "3"},               # occupancy first, below the 256-key chunk
    {"ATTN_SPLIT_MAJOR": "0"},              # head-major decode grid order
    {"ATTN_COMBINE_COLS": "0"},             # split-group combine kernel everywhere
    {"ATTN_COMBINE_COLS": "1"},             # column-parallel combine kernel everywhere
]


@pytest.mark.parametrize("S", [2, 15, 16, 17, 31, 64, 200, 256])
def test_decode_forced_split_counts(S):
    # forced split counts on both sides of the combine kernels' switch (16);
    # 2100 keys make 33 key blocks, so S > 33 leaves empty splits
    for seed in (13, 14):
        run_case("bf16", 2, 16, 2, 1, 2100, 128, False, -1, S, seed=seed)
        run_case("bf16", 1, 8, 8, 1, 700, 64, False, 100, S, seed=seed)


DECODE_FORM_CASES = [
    # dtype, B, Hq, Hkv, Sq, Sk, d, causal, wl, S
    ("bf16", 1, 32, 4, 1, 3000, 128, False, -1, 0),    # ragged last block, planner splits
    ("bf16", 2, 16, 2, 1, 2100, 128, False, -1, 1),    # one split: 33 blocks, several per wave
    ("bf16", 2, 16, 2, 1, 2100, 128, False, -1, 37),   # more splits than blocks: empty splits
    ("bf16", 1, 8, 8, 1, 700, 64, False, 100, 3),      # d 64, window
    ("bf16", 2, 16, 2, 2, 333, 128, True, -1, 0),      # two positions x 8 heads, causal
    ("bf16", 1, 8, 1, 1, 5, 128, False, -1, 0),        # fewer keys than one block
    ("bf16", 1, 32, 8, 1, 64, 128, False, -1, 2),      # exactly one block, split in two
]


@pytest.mark.parametrize("form", [2, 1], ids=["k_in_registers", "halves_through_lds"])
@pytest.mark.parametrize("case", DECODE_FORM_CASES)
def test_decode_forms(case, form, attn_options):
    attn_options("ATTN_DECODE_KDMA", form)
    run_case(*case, seed=21)


@pytest.mark.parametrize("form", [2, 1], ids=["k_in_registers", "halves_through_lds"])
def test_decode_forms_varlen(form, attn_options):
    attn_options("ATTN_DECODE_KDMA", form)
    B, Hq, Hkv, Sk, d = 20, 16, 4, 1500, 128
    q, k, v = small_case(22, "bf16", B, Hq, Hkv, 1, Sk, d)
    seqlens = torch.randint(0, Sk + 1, (B,), generator=torch.Generator().manual_seed(22), dtype=torch.int32)
    seqlens[3] = 0
    ro, rl = oracle.attn_ref(q, k, v, False, -1, 1 / math.sqrt(d), seqlens_k=seqlens)
    print(f"decode form {form} varlen", flush=True)
    o, lse = tpa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), seqlens.to(DEV), sum_seqlens_k=int(seqlens.sum()))
    assert_parity(o, lse, ro, rl, "bf16", f"decode form {form} varlen")


@pytest.mark.parametrize("env", ABLATIONS, ids=lambda e: ",".join(f"{k}={v}" for k, v in e.items()))
def test_ablation_paths(env, attn_options):
    for k_, v_ in env.items():
        attn_options(k_, v_)
    for case in [("bf16", 1, 8, 2, 300, 300, 128, True, 40, 0), ("bf16", 2, 16, 2, 200, 333, 64, True, -1, 0),
                 ("bf16", 1, 32, 4, 1, 3000, 128, False, -1, 0), ("bf16", 1, 4, 4, 130, 520, 128, False, -1, 0)]:
        run_case(*case, seed=12)


# --- values of their own width: the latent-attention verify shapes --------------
from workloads import latent_case  # noqa: E402

# the verify parity shapes printed on the occupancy blog page (B, H, q_len, kv_len),
# at the latent-attention widths (keys 576 = 512 latent + 64 rotary, values 512)
LATENT_SHAPES = [(2, 16, 17, 2065), (1, 64, 33, 161), (2, 64, 9, 521), (2, 8, 9, 9)]


def run_latent(B, Hq, Sq, Sk, causal=True, wl=-1, S=0, seed=0):
    q, k, v = latent_case(seed, B, Hq, Sq, Sk)
    scale = 1.0 / math.sqrt(576)
    print(f"latent B={B} Hq={Hq} Sq={Sq} Sk={Sk} causal={causal} wl={wl} S={S} seed={seed}", flush=True)
    o, lse = tpa.fwd_dv(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_left=wl, scale=scale,
                        num_splits=S)
    torch.cuda.synchronize()
    assert o.shape == (B, Sq, Hq, 512)
    ro, rl = oracle.attn_ref(q, k, v, causal, wl, scale)
    assert_parity(o, lse, ro, rl, "bf16", f"latent {B},{Hq},{Sq},{Sk} c={causal} wl={wl} S={S}")


# the latent kernel's two forms: 4 waves (all 512 output columns each), 8 waves
# (a row block's two waves split the output columns)
MLA_WAVES = pytest.mark.parametrize("mla_waves", [4, 8], ids=["w4", "w8"])


@MLA_WAVES
@pytest.mark.parametrize("shape", LATENT_SHAPES, ids=lambda s: "B%d_H%d_q%d_kv%d" % s)
def test_latent_verify_shapes(shape, mla_waves, attn_options):
    attn_options("ATTN_MLA_WAVES", mla_waves)
    run_latent(*shape)


@MLA_WAVES
@pytest.mark.parametrize("S", [1, 2, 3, 7])
def test_latent_split_sweep(S, mla_waves, attn_options):
    attn_options("ATTN_MLA_WAVES", mla_waves)
    run_latent(2, 16, 17, 2065, S=S, seed=1)


@MLA_WAVES
def test_latent_noncausal_window_and_ragged(mla_waves, attn_options):
    attn_options("ATTN_MLA_WAVES", mla_waves)
    run_latent(1, 8, 5, 77, causal=False, seed=2)           # ragged last key tile
    run_latent(1, 8, 12, 300, causal=True, wl=50, seed=3)   # sliding window
    run_latent(1, 3, 30, 20, causal=True, seed=4)           # Sq > Sk: fully masked rows


def _random_latent(n, seed):
    """latent-width problems (keys 576, values 512, one KV head) from a fixed
    generator: 1..16 heads, 1..40 query positions, ragged key counts, both masks
    and windows, automatic and forced split counts"""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        B = int(rng.integers(1, 3))
        Hq = int(rng.integers(1, 17))
        Sq = int(rng.integers(1, 41))
        Sk = int(rng.integers(1, 3000))
        causal = bool(rng.random() < 0.7)
        wl = -1 if rng.random() < 0.7 else int(rng.integers(0, Sk + 1))
        S = 0 if rng.random() < 0.6 else int(rng.integers(1, 9))
        if B * Hq * Sq * Sk > 4e5:
            continue
        cases.append((B, Hq, Sq, Sk, causal, wl, S))
    return cases


@pytest.mark.parametrize("case", _random_latent(16, 7031),
                         ids=lambda c: "B%d_H%d_q%d_k%d_c%d_w%d_S%d" % c)
def test_latent_random_shapes(case):
    B, Hq, Sq, Sk, causal, wl, S = case
    run_latent(B, Hq, Sq, Sk, causal=causal, wl=wl, S=S, seed=9)


def test_latent_long_prefix_sampled():
    # the 65,536-key prefix at full size (103 splits), checked on sampled query
    # positions: each recomputed by the oracle over exactly its visible keys
    from workloads import LATENT_WORKLOADS
    B, Hq, Sq, Sk = LATENT_WORKLOADS["latent_verify_long_bf16"]
    q, k, v = latent_case(0, B, Hq, Sq, Sk)
    scale = 1.0 / math.sqrt(576)
    print(f"latent long B={B} Hq={Hq} Sq={Sq} Sk={Sk}", flush=True)
    o, lse = tpa.fwd_dv(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for i in (0, 8, Sq - 1):
        kl = i + Sk - Sq + 1  # causal, bottom-right: row i sees keys [0, kl)
        ro, rl = oracle.attn_ref(q[:, i:i + 1], k[:, :kl], v[:, :kl], False, -1, scale)
        assert_parity(o[:, i:i + 1], lse[:, :, i:i + 1], ro, rl, "bf16", f"latent long row {i}")


# ---------------------------------------------------------------------------
# V beyond fp16's range: legal bf16 values the fp16 P.V operands cannot hold
# ---------------------------------------------------------------------------
BIG = 2.0 ** 17  # a power of two: scaled bf16 values stay exact


def _assert_scaled_parity(o, lse, q, k, v, causal, wl, scale, what, dv_path=False):
    """Tolerance in units of the row's value magnitude: the stated bars (max-abs 2e-2;
    max-rel 1e-2 where |ref| > 0.1) applied to o / m, m = max(1, sum_j P_ij |v_j|) per
    element, where the oracle gives sum_j P_ij |v_j| as attention over |v|. For inputs of
    unit scale m = 1 and this is the ordinary check; attention is linear in V, so
    scaling rows of V by 2^17 scales their share of each output by the same factor."""
    ro, rl = oracle.attn_ref(q, k, v, causal, wl, scale)
    mag, _ = oracle.attn_ref(q, k, v.abs(), causal, wl, scale)
    m = np.maximum(1.0, mag)
    of = o.detach().float().cpu().double().numpy()
    assert np.isfinite(of).all(), f"{what}: non-finite output"
    err = np.abs(of - ro) / m
    assert err.max() <= 2e-2, f"{what}: max scaled abs {err.max()}"
    big = np.abs(ro) / m > 0.1
    if big.any():
        rel = (np.abs(of - ro)[big] / np.abs(ro[big])).max()
        assert rel <= 1e-2, f"{what}: max rel {rel}"
    lse = lse.detach().cpu().double().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    if fin.any():
        d = np.abs(lse[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))
        assert d.max() <= 1e-3, f"{what}: lse err {d.max()}"


@pytest.mark.parametrize("rows,causal,wl,d,Hkv", [
    ("all", True, -1, 128, 4),       # every tile overflows: the bf16 form runs them all
    ("tail", True, -1, 128, 4),      # only tiles that see the last keys overflow
    ("tail", True, 300, 128, 2),     # sliding window: the scaled keys leave most windows
    ("some", False, -1, 128, 4),     # scattered rows, dense mask
    ("some", True, -1, 64, 4),
    ("tail", True, 200, 64, 1),
])
def test_prefill_values_beyond_fp16_range(rows, causal, wl, d, Hkv):
    B, Hq, S = 1, 4, 1100
    q, k, v = small_case(21, "bf16", B, Hq, Hkv, S, S, d)
    vf = v.float()
    if rows == "all":
        vf = vf * BIG
    elif rows == "tail":
        vf[:, 1000:1040] *= BIG
    else:
        vf[:, 3::97] *= BIG
    v = vf.to(torch.bfloat16)
    assert v.float().abs().max().item() > 65504.0
    scale = 1.0 / math.sqrt(d)
    print(f"V beyond fp16 rows={rows} causal={causal} wl={wl} d={d} Hkv={Hkv}", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window_left=wl, scale=scale)
    torch.cuda.synchronize()
    _assert_scaled_parity(o, lse, q, k, v, causal, wl, scale, f"prefill rows={rows}")
    if rows == "all":
        # linearity: O(V * 2^17) / 2^17 is O(V), at the ordinary tolerance
        ro, rl = oracle.attn_ref(q, k, (v.float() / BIG).to(torch.bfloat16), causal, wl, scale)
        assert_parity((o.float() / BIG), lse, ro, rl, "bf16", "prefill all rows / 2^17")


@pytest.mark.parametrize("env", [{"PREFILL_WAVES": 4}, {"PREFILL_WAVES": 8},
                                 {"PREFILL_PERSIST": 1}, {"PREFILL_SKIP": 1}],
                         ids=lambda e: ",".join(f"{k}={v}" for k, v in e.items()))
def test_prefill_values_beyond_fp16_range_every_variant(env, attn_options):
    for k_, v_ in env.items():
        attn_options(k_, v_)
    q, k, v = small_case(22, "bf16", 2, 8, 2, 700, 900, 128)
    vf = v.float()
    vf[:, 850:870] *= BIG
    v = vf.to(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    print(f"V beyond fp16, variant {env}", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale)
    torch.cuda.synchronize()
    _assert_scaled_parity(o, lse, q, k, v, True, -1, scale, f"variant {env}")


def test_decode_and_verify_values_beyond_fp16_range():
    # decode tiles keep V in bf16; the split combine sees large partials
    q, k, v = small_case(23, "bf16", 1, 32, 4, 1, 5000, 128)
    vf = v.float()
    vf[:, 4000:4100] *= BIG
    v = vf.to(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    print("decode V beyond fp16", flush=True)
    for S in (0, 1, 7):
        o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, num_splits=S)
        torch.cuda.synchronize()
        _assert_scaled_parity(o, lse, q, k, v, False, -1, scale, f"decode S={S}")


@MLA_WAVES
@pytest.mark.parametrize("rows", ["all", "tail"])
def test_latent_values_beyond_fp16_range(rows, mla_waves, attn_options):
    attn_options("ATTN_MLA_WAVES", mla_waves)
    B, Hq, Sq, Sk = 2, 16, 17, 2065
    q, k, v = latent_case(5, B, Hq, Sq, Sk)
    vf = v.float()
    if rows == "all":
        vf = vf * BIG
    else:
        vf[:, 2000:2030] *= BIG
    v = vf.to(torch.bfloat16)
    scale = 1.0 / math.sqrt(576)
    print(f"latent V beyond fp16 rows={rows}", flush=True)
    o, lse = tpa.fwd_dv(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale)
    torch.cuda.synchronize()
    _assert_scaled_parity(o, lse, q, k, v, True, -1, scale, f"latent rows={rows}")


# ---------------------------------------------------------------------------
# caller-owned workspaces (attn_set_workspace)
# ---------------------------------------------------------------------------
def test_caller_workspaces_on_two_streams():
    """Two decode problems on two streams, each with its own workspace bound at its
    launch, run concurrently; both match the oracle, twice in a row."""
    cases = [(small_case(31, "bf16", 1, 32, 4, 1, 20000, 128), 0),
             (small_case(32, "bf16", 2, 16, 2, 1, 9000, 64), 5)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs, outs, refs = [], [], []
    for (q, k, v), S in cases:
        B, Sq, Hq, d = q.shape
        need = tpa.plan(B, Hq, k.shape[2], Sq, k.shape[1], d, num_splits=S)["workspace_bytes"]
        assert need > 0
        bufs.append(torch.empty(need, dtype=torch.uint8, device=DEV))
        refs.append(oracle.attn_ref(q, k, v, False, -1, 1.0 / math.sqrt(d)))
    dev_in = [tuple(t.to(DEV) for t in qkv) for qkv, _ in cases]
    torch.cuda.synchronize()
    print("two streams, two workspaces", flush=True)
    try:
        for _ in range(2):
            outs = []
            for (q, k, v), (_, S), buf, st in zip(dev_in, cases, bufs, streams):
                tpa.set_workspace(buf)
                outs.append(tpa.fwd(q, k, v, num_splits=S, stream=st))
            torch.cuda.synchronize()
            for (o, lse), (ro, rl) in zip(outs, refs):
                assert_parity(o, lse, ro, rl, "bf16", "caller workspace")
        # a workspace one byte too small is refused
        q, k, v = dev_in[0]
        tpa.set_workspace(bufs[0][: bufs[0].numel() - 256])
        with pytest.raises(tpa.AttnError):
            tpa.fwd(q, k, v)
    finally:
        tpa.set_workspace(None)


# ---------------------------------------------------------------------------
# the persistent scheduler with several tiles per resident workgroup
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,Hq,Hkv,S,wl", [(4, 32, 32, 2048, -1), (4, 32, 8, 2048, 512)])
def test_persistent_several_tiles_per_workgroup(B, Hq, Hkv, S, wl, attn_options):
    q, k, v = small_case(41, "bf16", B, Hq, Hkv, S, S, 128)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_ref, lse_ref = tpa.fwd(qd, kd, vd, causal=True, window_left=wl)
    attn_options("PREFILL_PERSIST", 1)
    p = tpa.plan(B, Hq, Hkv, S, S, 128, causal=True, window_left=wl)
    tiles = B * p["grid_heads"] * p["num_m_blocks"] * p["num_splits"]
    assert tiles >= 2 * p["grid_x"], (tiles, p["grid_x"])  # several tiles per workgroup
    print(f"persistent B={B} Hq={Hq} Hkv={Hkv} S={S} wl={wl}: {tiles} tiles on {p['grid_x']} "
          "workgroups", flush=True)
    for _ in range(2):  # the queue counters are reset before every launch
        o, lse = tpa.fwd(qd, kd, vd, causal=True, window_left=wl)
        torch.cuda.synchronize()
        # the same per-tile arithmetic as the one-tile-per-workgroup grid: same bits
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    o, lse = o.cpu(), lse.cpu()
    scale = 1.0 / math.sqrt(128)
    for b, i in [(0, 0), (1, 255), (2, 256), (3, 1023), (3, S - 1), (0, S // 2 + 3)]:
        ro, rl = oracle.attn_ref(q[b:b + 1, i:i + 1], k[b:b + 1, :i + 1], v[b:b + 1, :i + 1],
                                 True, wl, scale)
        assert_parity(o[b:b + 1, i:i + 1], lse[b:b + 1, :, i:i + 1], ro, rl, "bf16",
                      f"persistent row {b},{i}")


# ---------------------------------------------------------------------------
# the largest sizes the planner takes on one call
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [0, 256])
def test_decode_256k_keys(S):
    # 262,144 keys: the planner's 128 splits give 2048 keys per split (eight blocks
    # per wave, the longest decode pipelines); 256 is the split cap
    B, Hq, Hkv, Sk, d = 1, 32, 4, 262144, 128
    pl = tpa.plan(B, Hq, Hkv, 1, Sk, d, False, -1, S, "bf16")
    assert pl["num_splits"] == (S or 128)
    run_case("bf16", B, Hq, Hkv, 1, Sk, d, False, -1, S, seed=41)


def test_varlen_200_sequences():
    # more sequences than two 64-lane scan steps of the work-unit search, many short
    B, Hq, Hkv, Sk, d = 200, 8, 2, 2500, 128
    q, k, v = small_case(42, "bf16", B, Hq, Hkv, 1, Sk, d)
    g = torch.Generator().manual_seed(42)
    seqlens = torch.randint(0, Sk + 1, (B,), generator=g, dtype=torch.int32)
    seqlens[::17] = 0
    seqlens[5] = Sk
    pl = tpa.plan(B, Hq, Hkv, 1, Sk, d, False, -1, 0, "bf16", varlen=True, sum_seqlens_k=int(seqlens.sum()))
    print(f"varlen 200 sequences plan {pl['grid_x']} units x {pl['grid_y']}, S={pl['num_splits']}", flush=True)
    ro, rl = oracle.attn_ref(q, k, v, False, -1, 1 / math.sqrt(d), seqlens_k=seqlens)
    o, lse = tpa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), seqlens.to(DEV), sum_seqlens_k=int(seqlens.sum()))
    assert_parity(o, lse, ro, rl, "bf16", "varlen 200 sequences")


@pytest.mark.parametrize("d", [128, 64])
def test_causal_prefill_32k_sampled(d):
    # 32,768 positions: 128 query blocks per head, the longest key ranges
    B, H, S = 1, 4, 32768
    q, k, v = small_case(43, "bf16", B, H, H, S, S, d, std=0.5)
    scale = 1.0 / math.sqrt(d)
    print(f"causal prefill 32k d={d}", flush=True)
    o, lse = tpa.fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for i in (0, 255, 256, 16383, 16384, 32511, S - 1):
        ro, rl = oracle.attn_ref(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], True, -1, scale)
        assert_parity(o[:, i:i + 1], lse[:, :, i:i + 1], ro, rl, "bf16", f"32k row {i} d={d}")
