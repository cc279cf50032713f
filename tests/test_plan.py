"""Host planner: block ranges, split partition, PackGQA and split-count rules.

Checked against the oracle's brute-force visible key blocks and against the
worked examples printed on the tiling-strategy page (tests/golden/).
"""
import json
import os

import pytest

import oracle
import tiled_prefill_amd as tpa
from workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ranges(Sq, Skb, G, pack, causal, wl, BM, BN):
    rows = Sq * (G if pack else 1)
    return [tpa.n_block_range(Sq, Skb, G, pack, causal, wl, BM, BN, m)
            for m in range((rows + BM - 1) // BM)]


def test_printed_causal_block_count():
    # "分块策略与调度" §3.3: N = 4096, B_r = B_c = 128 -> 528 of 1024 blocks.
    g = json.load(open(os.path.join(GOLDEN, "causal_block_count.json")))
    rng = _ranges(g["N"], g["N"], 1, False, True, -1, g["block_m"], g["block_n"])
    assert sum(hi - lo for lo, hi in rng) == g["blocks_computed"]
    assert len(rng) * len(rng) == g["blocks_total"]


def test_printed_split_heuristic_example():
    # "分块策略与调度" §5.2: 108 SMs, 48 tiles -> 2 splits (efficiencies 44%, 89%, 67%).
    g = json.load(open(os.path.join(GOLDEN, "split_heuristic_example.json")))
    s = tpa.num_splits_fa3(g["total_mblocks"], g["num_sms"], 64, 1, 1 << 20, False, 128)
    assert s == g["chosen_splits"]
    for k, pct in g["efficiency_percent"].items():
        w = g["total_mblocks"] * int(k) / g["num_sms"]
        assert round(100 * w / -(-w // 1)) == pct


def test_printed_pack_gqa_example():
    # "分块策略与调度" §6.2: Sq = 100, kBlockM = 128, G = 8 -> pack (78.1% < 0.9 x 89.3%).
    g = json.load(open(os.path.join(GOLDEN, "pack_gqa_example.json")))
    assert tpa.should_pack_gqa(False, g["seqlen_q"], g["qhead_per_khead"], g["block_m"]) == g["pack"]
    assert round(100 * 100 / 128, 1) == g["nopack_efficiency_percent"]
    assert round(100 * 800 / 896, 1) == g["pack_efficiency_percent"]
    assert tpa.should_pack_gqa(True, 4096, 8, 128)      # varlen always packs
    assert not tpa.should_pack_gqa(False, 4096, 8, 128)  # full tiles either way


def test_fa3_rule_branches():
    assert tpa.num_splits_fa3(200, 108, 64, 200, 1 << 20, False, 128) == 1  # grid already full
    assert tpa.num_splits_fa3(10, 108, 4, 1, 1 << 20, False, 128) == 1     # too few key blocks
    # long non-causal KV beyond the L2 budget splits by ceil(KV / 50 MB)
    assert tpa.num_splits_fa3(500, 108, 64, 500, 120 << 20, False, 128) == 3
    assert tpa.num_splits_fa3(500, 108, 64, 500, 120 << 20, True, 128) == 1


CASES = [(Sq, Skb, G, pack, causal, wl, BM, BN)
         for Sq, Skb in [(1, 1), (1, 37), (5, 5), (9, 40), (33, 17), (64, 64), (70, 200), (3, 130)]
         for G, pack in [(1, False), (4, False), (4, True)]
         for causal, wl in [(False, -1), (True, -1), (True, 0), (True, 7), (False, 5), (True, 64)]
         for BM, BN in [(16, 16), (32, 64), (128, 64), (16, 128)]]


@pytest.mark.parametrize("case", CASES[::3] + CASES[1::7])
def test_block_ranges_cover_every_visible_pair(case):
    Sq, Skb, G, pack, causal, wl, BM, BN = case
    need = oracle.needed_block_range(Sq, Skb, causal, wl, BM, BN, G=G, pack=pack)
    got = _ranges(Sq, Skb, G, pack, causal, wl, BM, BN)
    assert len(got) == len(need)
    vis = oracle.visible_mask(Sq, Skb, causal, wl)
    for m, ((lo, hi), nd) in enumerate(zip(got, need)):
        if nd is None:
            continue
        assert lo <= nd[0] and nd[1] <= hi, (m, (lo, hi), nd)
        # tight whenever the block's first row sees a key
        first_pos = (m * BM) // (G if pack else 1)
        if vis[first_pos].any():
            assert (lo, hi) == nd


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 64])
def test_splits_partition_the_block_range(S):
    for Sq, Skb, causal, wl in [(1, 300, False, -1), (17, 2065, True, -1), (200, 200, True, 30)]:
        for m in range((Sq + 15) // 16):
            lo, hi = tpa.n_block_range(Sq, Skb, 1, False, causal, wl, 16, 32, m)
            covered = []
            prev_end = lo
            for s in range(S):
                a, b = tpa.n_block_range(Sq, Skb, 1, False, causal, wl, 16, 32, m, s, S)
                if b <= a:  # empty split: only trailing ones may be empty
                    for s2 in range(s, S):
                        a2, b2 = tpa.n_block_range(Sq, Skb, 1, False, causal, wl, 16, 32, m, s2, S)
                        assert b2 <= a2
                    break
                assert a == prev_end
                covered.extend(range(a, b))
                prev_end = b
            assert covered == list(range(lo, max(lo, hi)))


def test_occupancy_rule():
    # toward 2 workgroups per CU, but every split keeps 256 keys
    assert tpa.num_splits_occupancy(4, 256, 256, 128) == 128     # 32K keys, 4 tiles
    assert tpa.num_splits_occupancy(4, 256, 512, 64) == 128      # the same keys in 64-key blocks
    assert tpa.num_splits_occupancy(32, 256, 65, 32) == 8        # the chunk bounds it (65 / 8)
    assert tpa.num_splits_occupancy(32, 256, 33, 64) == 8        # fp32 verify: 2065 keys, 32 tiles
    assert tpa.num_splits_occupancy(4, 256, 4, 64) == 1          # 256 keys: one chunk
    assert tpa.num_splits_occupancy(2048, 256, 128, 64) == 1     # grid already full
    assert tpa.num_splits_occupancy(4, 256, 1, 64) == 1          # one key block
    assert tpa.num_splits_occupancy(1, 256, 4096, 64) == 256     # capped at 256 splits
    assert tpa.num_splits_occupancy(300, 256, 4096, 64) == 2     # occupancy bounds it: ceil(512 / 300)
    assert tpa.num_splits_occupancy(4, 256, 4096, 64, min_chunk_rows=64) == 128  # 1-block chunks


def _plan(name, **kw):
    w = WORKLOADS[name]
    return tpa.plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left,
                    dtype=w.dtype, varlen=w.varlen, num_cus=256, **kw)


def test_workload_plans():
    p = _plan("gqa_decode_bf16")
    assert p["pack_gqa"] == 1 and p["grid_heads"] == 4 and p["num_m_blocks"] == 1
    assert p["num_splits"] == 128 and p["grid_y"] == 512  # 2 workgroups per CU, 256-key chunks
    p = _plan("causal_prefill_bf16")
    assert p["num_splits"] == 1 and p["pack_gqa"] == 0 and p["lpt"] == 1
    assert p["grid_x"] * p["grid_y"] * p["grid_z"] >= 2 * 256
    p = _plan("window_prefill_bf16")
    assert p["num_splits"] == 1
    p = _plan("spec_verify_fp32")
    assert p["num_splits"] == 8 and p["grid_x"] * p["grid_y"] * p["grid_z"] == 256  # 258-key splits
    p = _plan("decode_fp32")
    assert p["num_splits"] == 1  # 256 keys: a single chunk
    p = _plan("varlen_decode_bf16", sum_seqlens_k=16 * 8448)
    assert p["pack_gqa"] == 1 and p["chunk_blocks"] * p["block_n"] >= 256
    p = _plan("decode_fp32", num_splits=8)
    assert p["num_splits"] == 8


def test_causal_visited_blocks_about_half():
    p = _plan("causal_prefill_bf16", num_splits=1)
    dense = p["num_m_blocks"] * (8192 // p["block_n"]) * 32
    assert 0.5 < p["visited_blocks"] / dense < 0.52


def test_persistent_grid_is_resident_workgroups(attn_options):
    """Persistent prefill: one workgroup per resident slot (8-wave: 1 per CU, 4-wave: 2), a
    multiple of the 8 XCDs, never more than the tiles; the workspace holds the 8 queue counters."""
    attn_options("ATTN_PREFILL_PERSIST", "1")
    p = tpa.plan(1, 32, 32, 8192, 8192, 128, causal=True, num_cus=256)
    assert p["block_m"] == 256 and p["grid_x"] == 256
    assert p["workspace_bytes"] >= 8 * 4
    p = tpa.plan(4, 32, 8, 4096, 4096, 128, causal=True, window_left=1024, num_cus=256)
    assert p["block_m"] == 128 and p["grid_x"] == 512
    p = tpa.plan(1, 2, 2, 300, 300, 128, causal=True, num_cus=256)  # few tiles: all of them, rounded to 8
    tiles = p["grid_heads"] * p["num_m_blocks"] * p["num_splits"]
    assert tiles < 256 and p["grid_x"] == -(-tiles // 8) * 8
    attn_options("ATTN_PREFILL_PERSIST", "0")
    p = tpa.plan(1, 32, 32, 8192, 8192, 128, causal=True, num_cus=256)
    assert p["grid_x"] == 1024 and p["workspace_bytes"] == 0


# ---------------------------------------------------------------------------
# backward: query-block range of each key block ([FA-tiling] §3.4)
# ---------------------------------------------------------------------------
M_CASES = [
    (64, 64, True, -1, 16, 16), (37, 53, True, -1, 8, 16), (53, 37, True, 5, 16, 8),
    (40, 40, False, 7, 8, 8), (9, 30, True, 0, 4, 4), (100, 100, False, -1, 64, 64),
    (130, 129, True, 33, 64, 64), (1, 300, True, -1, 64, 64), (300, 1, True, -1, 64, 64),
    (17, 2065, True, -1, 64, 64), (200, 150, False, 20, 64, 32),
]


@pytest.mark.parametrize("case", M_CASES)
def test_m_block_range_matches_brute_force(case):
    Sq, Sk, causal, wl, BM, BN = case
    want = oracle.needed_m_block_range(Sq, Sk, causal, wl, BM, BN)
    for n, w in enumerate(want):
        lo, hi = tpa.m_block_range(Sq, Sk, causal, wl, BM, BN, n)
        if w is None:
            assert hi <= lo, (n, lo, hi)
        else:
            assert (lo, hi) == w, (n, lo, hi, w)


def test_bwd_plan_visits_the_printed_block_count_and_the_forward_pairs():
    g = json.load(open(os.path.join(GOLDEN, "causal_block_count.json")))
    N, bm, bn = g["N"], g["block_m"], g["block_n"]
    total = sum(max(0, hi - lo) for lo, hi in
                (tpa.m_block_range(N, N, True, -1, bm, bn, n) for n in range(N // bn)))
    assert total == g["blocks_computed"]
    for name in ("causal_prefill_bf16", "window_prefill_bf16"):
        w = WORKLOADS[name]
        p = tpa.plan_bwd(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left, w.dtype)
        fwd = oracle.needed_block_range(w.Sq, w.Sk, w.causal, w.window_left,
                                        p["block_m"], p["block_n"])
        pairs = sum(hi - lo for r in fwd if r for lo, hi in [r])
        assert p["visited_blocks"] == pairs * w.Hq * w.B
        assert p["grid_x"] == p["num_n_blocks"] * w.Hkv * w.B
        rows = w.B * w.Sq * w.Hq
        assert p["workspace_bytes"] >= rows * 2 * 4  # lse2 and the row sums


def test_bwd_plan_atomic_form_needs_the_accumulator(attn_options):
    w = WORKLOADS["causal_prefill_bf16"]
    attn_options("ATTN_BWD_ATOMIC", "1")
    p = tpa.plan_bwd(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, w.window_left, w.dtype)
    assert p["dq_block_m"] == 0
    assert p["workspace_bytes"] >= w.B * w.Sq * w.Hq * (w.d + 2) * 4


@pytest.mark.parametrize("seed", range(6))
def test_varlen_work_unit_grid_covers_every_split(seed, attn_options):
    # The unit grid holds one workgroup per (sequence, split); sequence b has
    # S_b = min(S, max(1, ceil(blocks_b / chunk))) splits, so with the exact sum
    # of the key lengths the host's count must reach sum_b S_b, and the fixed
    # grid (B * S) must be the bound when no sum is given.
    import numpy as np
    attn_options("ATTN_VARLEN_CHUNK", 128 * (1 + seed % 3))
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Sk = int(rng.integers(1, 200)), 32, 8, int(rng.integers(64, 20000))
    lens = rng.integers(0, Sk + 1, B)
    total = int(lens.sum())
    pl = tpa.plan(B, Hq, Hkv, 1, Sk, 128, False, -1, 0, "bf16", varlen=True, sum_seqlens_k=max(total, 1))
    if pl["num_splits"] == 1:
        assert pl["work_units"] == 0
        return
    cb, S = pl["chunk_blocks"], pl["num_splits"]
    need = sum(min(S, max(1, -(-(-(-int(n) // 64)) // cb))) for n in lens)
    assert need <= pl["work_units"] == pl["grid_x"] <= B * S
    assert pl["grid_y"] == Hkv and pl["grid_z"] == 1
    pl0 = tpa.plan(B, Hq, Hkv, 1, Sk, 128, False, -1, 0, "bf16", varlen=True, sum_seqlens_k=-1)
    assert pl0["work_units"] == B * pl0["num_splits"]
