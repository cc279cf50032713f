"""Pins for the fp64 oracle: checks it against facts fixed outside itself.

Each test ties an oracle function to something it does not compute itself:
a closed form, an invariant of softmax attention, a library routine (torch
fp64 scaled_dot_product_attention, logsumexp, tril/triu masks) or a value
printed on the pages (tests/golden/). A plausible slip in the oracle (a
dropped term, a wrong sign or mask offset, a transposed head mapping) fails
at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import random_partials, small_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _visible_interval(i, Sq, Skb, causal, wl):
    """Closed-form visible key interval [lo, hi] of row i (hi < lo: empty)."""
    delta = Skb - Sq
    hi = min(Skb - 1, i + delta) if causal else Skb - 1
    lo = max(0, i + delta - wl) if wl >= 0 else 0
    return lo, hi


MASKS = [(False, -1), (True, -1), (True, 0), (True, 3), (True, 100), (False, 2)]


@pytest.mark.parametrize("causal,wl", MASKS)
@pytest.mark.parametrize("Sq,Sk", [(1, 37), (5, 5), (7, 20), (12, 4)])
def test_constant_keys_average_visible_values(causal, wl, Sq, Sk):
    # With every key equal, all visible scores tie: the output is the plain mean
    # of the visible value rows and lse = score + ln(#visible).
    q, k, v = small_case(1, "fp32", 1, 2, 1, Sq, Sk, 16)
    k[:] = k[:, :1]
    scale = 0.3
    o, lse = oracle.attn_ref(q, k, v, causal, wl, scale)
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    for h in range(2):
        for i in range(Sq):
            lo, hi = _visible_interval(i, Sq, Sk, causal, wl)
            if hi < lo:
                assert np.all(o[0, i, h] == 0.0) and lse[0, h, i] == -np.inf
                continue
            mean = v64[0, lo:hi + 1, 0].mean(axis=0)
            np.testing.assert_allclose(o[0, i, h], mean, rtol=0, atol=1e-12)
            s = scale * float(q64[0, i, h] @ k64[0, 0, 0])
            assert abs(lse[0, h, i] - (s + math.log(hi - lo + 1))) < 1e-12


@pytest.mark.parametrize("jstar", [0, 17, 63])
def test_one_hot_dominant_key_selects_its_value(jstar):
    # One key aligned with q and long enough that its score beats every other
    # by a margin >= 40: the output is that key's value row within 2e^-40.
    q, k, v = small_case(2, "fp32", 1, 1, 1, 1, 64, 32)
    q64 = q.double()
    qn = q64[0, 0, 0] / q64[0, 0, 0].norm()
    scale = 1.0 / math.sqrt(32)
    k64 = k.double()
    others = (k64[0, :, 0] @ q64[0, 0, 0]).abs().max().item() * scale
    alpha = (others + 60.0) / (scale * q64[0, 0, 0].norm().item())
    k64[0, jstar, 0] = alpha * qn
    o, lse = oracle.attn_ref(q64, k64, v.double(), False, -1, scale)
    s_star = scale * alpha * q64[0, 0, 0].norm().item()
    margin = s_star - max(scale * float(k64[0, j, 0] @ q64[0, 0, 0]) for j in range(64) if j != jstar)
    assert margin >= 40
    bound = 2 * math.exp(-margin) * float(v.abs().max())
    np.testing.assert_allclose(o[0, 0, 0], v.double()[0, jstar, 0].numpy(), rtol=0, atol=bound + 1e-15)
    assert abs(lse[0, 0, 0] - s_star) <= math.exp(-margin) * 64 + 1e-12


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (6, 6), (4, 11)])
def test_single_visible_key_is_exact(Sq, Sk):
    # window_left = 0 with causal leaves exactly the diagonal key i + (Sk - Sq).
    q, k, v = small_case(3, "fp32", 2, 3, 3, Sq, Sk, 8)
    scale = 0.7
    o, lse = oracle.attn_ref(q, k, v, True, 0, scale)
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    for b in range(2):
        for h in range(3):
            for i in range(Sq):
                j = i + Sk - Sq
                assert np.array_equal(o[b, i, h], v64[b, j, h])
                s = scale * float(np.dot(q64[b, i, h], k64[b, j, h]))
                assert abs(lse[b, h, i] - s) < 1e-12


@pytest.mark.parametrize("causal,wl", MASKS)
def test_key_shift_invariance(causal, wl):
    # Adding the same vector u to every key shifts all scores of a row by
    # scale*q.u: the softmax is unchanged and lse moves by exactly that amount.
    q, k, v = small_case(4, "fp32", 1, 2, 2, 6, 13, 16)
    scale = 0.25
    u = torch.linspace(-1, 1, 16, dtype=torch.float64)
    o1, l1 = oracle.attn_ref(q, k, v, causal, wl, scale)
    o2, l2 = oracle.attn_ref(q.double(), k.double() + u, v, causal, wl, scale)
    shift = scale * np.einsum("bihc,c->bhi", q.double().numpy(), u.numpy())
    finite = np.isfinite(l1)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2[finite], (l1 + shift)[finite], rtol=0, atol=1e-12)
    assert np.array_equal(np.isfinite(l2), finite)


def test_key_value_permutation_invariance():
    q, k, v = small_case(5, "fp32", 2, 2, 1, 3, 29, 16)
    perm = torch.randperm(29, generator=torch.Generator().manual_seed(0))
    o1, l1 = oracle.attn_ref(q, k, v, False, -1, 0.3)
    o2, l2 = oracle.attn_ref(q, k[:, perm], v[:, perm], False, -1, 0.3)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,wl", [(False, -1), (True, -1), (True, 2)])
def test_gqa_equals_mha_with_repeated_heads(causal, wl):
    # Query head h reads key/value head h // G: identical to MHA whose key/value
    # heads are each repeated G times in a row.
    q, k, v = small_case(6, "fp32", 2, 8, 2, 5, 9, 16)
    o1, l1 = oracle.attn_ref(q, k, v, causal, wl, 0.4)
    kr, vr = k.repeat_interleave(4, dim=2), v.repeat_interleave(4, dim=2)
    o2, l2 = oracle.attn_ref(q, kr, vr, causal, wl, 0.4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def _torch_reference(q, k, v, causal, wl, scale):
    """torch fp64 SDPA with an explicit mask built from tril/triu offsets."""
    B, Sq, H, d = q.shape
    Sk = k.shape[1]
    delta = Sk - Sq
    mask = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        mask = torch.tril(mask, diagonal=delta)
    if wl >= 0:
        mask = mask & torch.triu(torch.ones(Sq, Sk, dtype=torch.bool), diagonal=delta - wl)
    qt = q.double().permute(0, 2, 1, 3)
    kt = k.double().permute(0, 2, 1, 3)
    vt = v.double().permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    scores = (qt @ kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy(), mask.numpy()


def test_masks_brute_force_against_torch_sdpa():
    # Every tiny shape Sq, Sk in 1..9, causal on/off, every window width.
    torch.manual_seed(0)
    n = 0
    for Sq in range(1, 10):
        for Sk in range(1, 10):
            q, k, v = small_case(100 + 10 * Sq + Sk, "fp32", 2, 2, 2, Sq, Sk, 8)
            for causal in (False, True):
                for wl in [-1] + list(range(0, Sk + 1)):
                    o, lse = oracle.attn_ref(q, k, v, causal, wl, 0.5)
                    ro, rl, mask = _torch_reference(q, k, v, causal, wl, 0.5)
                    rows = mask.any(axis=1)  # [Sq]
                    np.testing.assert_allclose(o[:, rows], ro[:, rows], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(lse[:, :, rows], rl[:, :, rows], rtol=0, atol=1e-12)
                    assert np.all(o[:, ~rows] == 0.0)
                    assert np.all(lse[:, :, ~rows] == -np.inf)
                    n += 1
    assert n > 500


@pytest.mark.parametrize("causal,wl", [(False, -1), (True, -1), (True, 4), (False, 3)])
def test_visible_sets_agree_between_c_oracle_and_mask_helper(causal, wl):
    # With constant keys and value rows e_j (one-hot), o[i] * |V_i| is the
    # indicator of the visible set: the C oracle and visible_mask must agree.
    Sq, Sk = 9, 14
    q, k, v = small_case(7, "fp32", 1, 1, 1, Sq, Sk, Sk)
    k[:] = k[:, :1]
    v = torch.eye(Sk, dtype=torch.float64).reshape(1, Sk, 1, Sk)
    o, _ = oracle.attn_ref(q, k, v, causal, wl, 1.0)
    mask = oracle.visible_mask(Sq, Sk, causal, wl)
    got = o[0, :, 0, :] > 0
    np.testing.assert_array_equal(got, mask)


def test_printed_causal_block_count():
    # "分块策略与调度" §3.3: N = 4096 with 128 x 128 blocks computes 528 of 1024.
    g = json.load(open(os.path.join(GOLDEN, "causal_block_count.json")))
    rng = oracle.needed_block_range(g["N"], g["N"], True, -1, g["block_m"], g["block_n"])
    assert len(rng) * ((g["N"] + g["block_n"] - 1) // g["block_n"]) == g["blocks_total"]
    computed = sum(hi - lo for lo, hi in rng)
    assert computed == g["blocks_computed"]
    assert round(100.0 * computed / g["blocks_total"], 1) == g["fraction_percent"]


def _window_block_pairs(N, B, wl):
    """(query block, key block) pairs a causal sliding window needs, counted by hand for
    Sq = Sk = N and square B x B blocks: query block m holds rows mB .. mB + B - 1, whose
    keys run from max(0, mB - wl) to the diagonal, so it needs key blocks
    max(0, m - ceil(wl / B)) .. m, i.e. min(m, c) + 1 of them with c = ceil(wl / B).
    Summed over the M = N / B query blocks: (c + 1)(c + 2) / 2 + (M - 1 - c)(c + 1) when
    c < M, else the causal M (M + 1) / 2."""
    M = N // B
    c = -(-wl // B)
    if c >= M:
        return M * (M + 1) // 2
    return (c + 1) * (c + 2) // 2 + (M - 1 - c) * (c + 1)


@pytest.mark.parametrize("wl,expected", [(1024, 252), (1000, 252), (1025, 275), (0, 32),
                                         (127, 63), (128, 63), (4095, 528), (100000, 528)])
def test_window_block_count_closed_form(wl, expected):
    # the causal example of "分块策略与调度" §3.3 (N = 4096, 128 x 128 blocks) with a
    # left window: the brute-force ranges of needed_block_range against the count above
    assert _window_block_pairs(4096, 128, wl) == expected
    rng = oracle.needed_block_range(4096, 4096, True, wl, 128, 128)
    assert sum(hi - lo for lo, hi in rng) == expected
    # every block's range by the same reasoning: [max(0, m - c), m + 1)
    c = -(-wl // 128)
    assert rng == [(max(0, m - c), m + 1) for m in range(32)]


@pytest.mark.parametrize("Sq,Skb,causal,wl,BM,BN,G", [
    (5, 9, True, -1, 4, 3, 3), (7, 7, True, 2, 8, 4, 4), (3, 20, False, 5, 5, 4, 2),
    (9, 5, True, -1, 16, 2, 8), (6, 13, True, 0, 3, 5, 3), (4, 4, False, -1, 2, 2, 5),
    (11, 17, True, 6, 7, 3, 2), (1, 30, True, 4, 16, 8, 8)])
def test_packed_block_range_is_the_hull_of_its_positions(Sq, Skb, causal, wl, BM, BN, G):
    # "分块策略与调度" §6.3: packed row r is query position r // G, so a packed block of
    # rows [r0, r1) needs the union (hull) of the key-block ranges of positions
    # r0 // G .. (r1 - 1) // G, each taken from the unpacked ranges with one row per block
    packed = oracle.needed_block_range(Sq, Skb, causal, wl, BM, BN, G=G, pack=True)
    per_pos = oracle.needed_block_range(Sq, Skb, causal, wl, 1, BN)
    assert len(packed) == -(-(Sq * G) // BM)
    for m, got in enumerate(packed):
        p0, p1 = (m * BM) // G, (min((m + 1) * BM, Sq * G) - 1) // G
        rs = [per_pos[p] for p in range(p0, p1 + 1) if per_pos[p] is not None]
        want = (min(r[0] for r in rs), max(r[1] for r in rs)) if rs else None
        assert got == want, (m, got, want)
    assert oracle.needed_block_range(Sq, Skb, causal, wl, BM, BN, G=1, pack=True) == \
        oracle.needed_block_range(Sq, Skb, causal, wl, BM, BN)


def test_varlen_equals_truncated_fixed_length():
    q, k, v = small_case(8, "fp32", 3, 4, 2, 3, 20, 16)
    seqlens = [20, 5, 11]
    for causal, wl in [(False, -1), (True, -1), (True, 2)]:
        o, lse = oracle.attn_ref(q, k, v, causal, wl, 0.3, seqlens_k=seqlens)
        for b, L in enumerate(seqlens):
            ob, lb = oracle.attn_ref(q[b:b + 1], k[b:b + 1, :L], v[b:b + 1, :L], causal, wl, 0.3)
            np.testing.assert_array_equal(o[b:b + 1], ob)
            np.testing.assert_array_equal(lse[b:b + 1], lb)


@pytest.mark.parametrize("causal,wl", [(False, -1), (True, -1), (True, 5)])
def test_partition_merge_reproduces_full_result(causal, wl):
    # The flash-decoding identity: partials over any partition of the keys
    # (empty pieces allowed), merged by log-sum-exp, equal the full result.
    q, k, v = small_case(9, "fp32", 2, 4, 2, 6, 41, 16)
    o, lse = oracle.attn_ref(q, k, v, causal, wl, 0.3)
    cuts = [0, 0, 7, 8, 8, 30, 41, 41]
    parts = [oracle.attn_ref(q, k, v, causal, wl, 0.3, key_range=(a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    S = len(parts)
    rows = 2 * 6 * 4
    # partial layout [S, rows, d] with rows ordered (b, i, h) as in o
    op = np.stack([p[0].reshape(rows, 16) for p in parts])
    lp = np.stack([p[1].transpose(0, 2, 1).reshape(rows) for p in parts])
    om, lm = oracle.lse_combine_ref(op, lp)
    np.testing.assert_allclose(om, o.reshape(rows, 16), rtol=0, atol=1e-12)
    ref_l = lse.transpose(0, 2, 1).reshape(rows)
    finite = np.isfinite(ref_l)
    np.testing.assert_allclose(lm[finite], ref_l[finite], rtol=0, atol=1e-12)
    assert np.all(lm[~finite] == -np.inf)
    # one split holding every key is the full result itself
    o1, l1 = oracle.attn_ref(q, k, v, causal, wl, 0.3, key_range=(0, 41))
    np.testing.assert_array_equal(o1, o)
    np.testing.assert_array_equal(l1, lse)


def test_combine_closed_forms():
    o_part, lse_part = random_partials(0, 5, 7, 4, p_empty=0.0)
    # equal lse: plain mean of the partial outputs, lse + ln S
    lse_eq = torch.full((5, 7), 1.25)
    o, lse = oracle.lse_combine_ref(o_part, lse_eq)
    np.testing.assert_allclose(o, o_part.double().mean(0).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, 1.25 + math.log(5), rtol=0, atol=1e-12)
    # a single split is the identity
    o1, l1 = oracle.lse_combine_ref(o_part[:1], lse_part[:1])
    np.testing.assert_array_equal(o1, o_part[0].double().numpy())
    np.testing.assert_array_equal(l1, lse_part[0].double().numpy())
    # all splits empty: o = 0, lse = -inf (no -inf - -inf)
    o2, l2 = oracle.lse_combine_ref(torch.zeros(3, 2, 4), torch.full((3, 2), float("-inf")))
    assert np.all(o2 == 0) and np.all(l2 == -np.inf)
    # split order does not matter; empty splits carry zero weight
    o_part, lse_part = random_partials(1, 6, 9, 8, p_empty=0.3)
    oa, la = oracle.lse_combine_ref(o_part, lse_part)
    ob, lb = oracle.lse_combine_ref(o_part.flip(0), lse_part.flip(0))
    np.testing.assert_allclose(oa, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)
    keep = torch.isfinite(lse_part).any(0)
    two_ref = torch.logsumexp(lse_part.double(), dim=0).numpy()
    np.testing.assert_allclose(la[keep.numpy()], two_ref[keep.numpy()], rtol=0, atol=1e-12)


# --- values of their own width (the latent-attention verify shape: one shared KV
# head, 576-wide keys, 512-wide values) --------------------------------------------

def _values(seed, B, Sk, Hkv, dv):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(B, Sk, Hkv, dv, generator=g)


@pytest.mark.parametrize("d,dv", [(8, 24), (24, 8), (576, 512)])
def test_value_width_brute_force_against_torch_sdpa(d, dv):
    # torch fp64 SDPA accepts values of another width; every mask on tiny shapes,
    # all query heads sharing one KV head (repeated for torch)
    n = 0
    for Sq, Sk in [(1, 5), (3, 7), (5, 5), (4, 9)]:
        q, k, _ = small_case(7 + Sq * Sk, "fp32", 2, 4, 1, Sq, Sk, d)
        v = _values(3 + Sk, 2, Sk, 1, dv)
        for causal, wl in [(False, -1), (True, -1), (True, 1), (False, 2)]:
            o, lse = oracle.attn_ref(q, k, v, causal, wl, 0.07)
            assert o.shape == (2, Sq, 4, dv)
            ro, rl, mask = _torch_reference(q, k.repeat_interleave(4, dim=2), v.repeat_interleave(4, dim=2),
                                            causal, wl, 0.07)
            rows = mask.any(axis=1)
            np.testing.assert_allclose(o[:, rows], ro[:, rows], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[:, :, rows], rl[:, :, rows], rtol=0, atol=1e-12)
            assert np.all(o[:, ~rows] == 0.0)
            n += 1
    assert n == 16


def test_value_columns_are_independent():
    # softmax weights do not depend on V: attention with values [V1 | V2] is the
    # concatenation of the results for V1 (same width as the keys, the plain
    # path) and V2 (a width of its own) -- pins the value-row stride and offsets
    q, k, v1 = small_case(21, "fp32", 2, 8, 2, 6, 11, 16)
    v2 = _values(5, 2, 11, 2, 40)
    o, lse = oracle.attn_ref(q, k, torch.cat([v1, v2], dim=-1), True, 4, 0.25)
    o1, l1 = oracle.attn_ref(q, k, v1, True, 4, 0.25)
    o2, l2 = oracle.attn_ref(q, k, v2, True, 4, 0.25)
    np.testing.assert_allclose(o, np.concatenate([o1, o2], axis=-1), rtol=0, atol=1e-14)
    np.testing.assert_array_equal(lse, l1)
    np.testing.assert_array_equal(lse, l2)


def test_value_width_constant_keys_average_values():
    q, k, _ = small_case(31, "fp32", 1, 4, 1, 3, 10, 576)
    k[:] = k[:, :1]
    v = _values(9, 1, 10, 1, 512)
    o, _ = oracle.attn_ref(q, k, v, True, -1, 0.04)
    v64 = v.double().numpy()
    for i in range(3):
        hi = i + 7  # causal, delta = 7
        np.testing.assert_allclose(o[0, i, 2], v64[0, :hi + 1, 0].mean(axis=0), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# backward pass (attn_bwd_ref): gradients of L = <dout, attn(q, k, v)>
# ---------------------------------------------------------------------------
BWD_MASKS = [(False, -1), (True, -1), (True, 2), (False, 3)]


def _bwd_inputs(seed, B, Hq, Hkv, Sq, Sk, d):
    q, k, v = small_case(seed, "fp32", B, Hq, Hkv, Sq, Sk, d)
    rng = np.random.default_rng(seed + 101)
    g = rng.standard_normal((B, Sq, Hq, d))
    return q.double().numpy(), k.double().numpy(), v.double().numpy(), g


def _loss(q, k, v, g, causal, wl, scale):
    o, _ = oracle.attn_ref(q, k, v, causal, wl, scale)
    return float(np.sum(o * g))


@pytest.mark.parametrize("causal,wl", BWD_MASKS)
@pytest.mark.parametrize("Sq,Sk", [(3, 5), (6, 4)])
def test_bwd_matches_finite_differences(causal, wl, Sq, Sk):
    # Central differences of the forward oracle, entry by entry (error O(h^2)).
    # (6, 4) with a causal mask has rows that see no key: their gradient is 0.
    q, k, v, g = _bwd_inputs(3, 1, 2, 1, Sq, Sk, 3)
    scale = 0.7
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, g, causal, wl, scale)
    h = 1e-5
    for x, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            up = _loss(q, k, v, g, causal, wl, scale)
            x[idx] = old - h
            dn = _loss(q, k, v, g, causal, wl, scale)
            x[idx] = old
            assert abs((up - dn) / (2 * h) - grad[idx]) < 1e-7, idx


def _torch_attn_fp64(q, k, v, causal, wl, scale):
    """Explicitly masked softmax attention with torch fp64 ops (GQA by repeating
    the KV heads); rows with no visible key give 0."""
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kk = k.repeat_interleave(G, dim=2)
    vv = v.repeat_interleave(G, dim=2)
    s = torch.einsum("bihc,bjhc->bhij", q, kk) * scale
    delta = Sk - Sq
    mask = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        mask &= torch.tril(torch.ones(Sq, Sk, dtype=torch.bool), diagonal=delta)
    if wl >= 0:
        mask &= torch.triu(torch.ones(Sq, Sk, dtype=torch.bool), diagonal=delta - wl)
    rowok = mask.any(dim=-1)
    s = torch.where(mask, s, torch.tensor(float("-inf"), dtype=s.dtype))
    s = torch.where(rowok[:, None], s, torch.zeros((), dtype=s.dtype))
    p = torch.softmax(s, dim=-1) * rowok[:, None].to(s.dtype)
    return torch.einsum("bhij,bjhc->bihc", p, vv)


@pytest.mark.parametrize("causal,wl", BWD_MASKS + [(True, 0)])
def test_bwd_against_torch_autograd(causal, wl):
    # A library routine: torch autograd (fp64, CPU) through an explicitly masked
    # softmax, GQA with group 3, Sq > Sk so that causal masks empty some rows.
    q, k, v, g = _bwd_inputs(5, 2, 6, 2, 13, 9, 16)
    scale = 0.25
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, g, causal, wl, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = _torch_attn_fp64(tq, tk, tv, causal, wl, scale)
    (o * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("causal,wl", BWD_MASKS)
def test_bwd_invariants(causal, wl):
    q, k, v, g = _bwd_inputs(9, 2, 4, 2, 7, 11, 8)
    scale = 0.4
    dq, dk, dv = oracle.attn_bwd_ref(q, k, v, g, causal, wl, scale)
    # Shifting every key of a head by one vector moves all scores of a row by the
    # same amount, so the key gradients of a head sum to zero.
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # Each row's probabilities sum to one: the value gradients of a KV head sum
    # to the output gradients of the rows (of its query heads) that see a key.
    vis = oracle.visible_mask(7, 11, causal, wl)
    rows = vis.any(axis=1)
    G = 2
    for hkv in range(2):
        want = g[:, rows][:, :, hkv * G:(hkv + 1) * G].sum(axis=(1, 2))
        np.testing.assert_allclose(dv[:, :, hkv].sum(axis=1), want, atol=1e-12)
    # A constant added to every value row shifts each output by that constant,
    # whatever the probabilities: dq and dk do not change.
    dq2, dk2, dv2 = oracle.attn_bwd_ref(q, k, v + np.arange(8) * 0.37, g, causal, wl, scale)
    np.testing.assert_allclose(dq2, dq, atol=1e-12)
    np.testing.assert_allclose(dk2, dk, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, atol=1e-12)


def test_bwd_identical_keys_give_zero_query_gradient():
    # With every key equal, each visible score of a row ties whatever q is, so
    # the output does not depend on q.
    q, k, v, g = _bwd_inputs(11, 1, 2, 1, 6, 9, 8)
    k[:] = k[:, :1]
    for causal, wl in BWD_MASKS:
        dq, _, _ = oracle.attn_bwd_ref(q, k, v, g, causal, wl, 0.9)
        np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_bwd_block_ranges_visit_the_printed_block_count():
    # The backward loop (key block outside, the query blocks that see it inside,
    # "分块策略与调度" §3.4) visits the same (query block, key block) pairs as the
    # forward loop: 528 of 1024 for the causal example of §3.3.
    gd = json.load(open(os.path.join(GOLDEN, "causal_block_count.json")))
    N, bm, bn = gd["N"], gd["block_m"], gd["block_n"]
    mr = oracle.needed_m_block_range(N, N, True, -1, bm, bn)
    assert sum(hi - lo for lo, hi in mr) == gd["blocks_computed"]
    for Sq, Sk, causal, wl, BM, BN in [(37, 53, True, -1, 8, 16), (53, 37, True, 5, 16, 8),
                                       (40, 40, False, 7, 8, 8), (9, 30, True, 0, 4, 4)]:
        fwd = oracle.needed_block_range(Sq, Sk, causal, wl, BM, BN)
        bwd = oracle.needed_m_block_range(Sq, Sk, causal, wl, BM, BN)
        pf = {(m, n) for m, r in enumerate(fwd) if r for n in range(*r)}
        pb = {(m, n) for n, r in enumerate(bwd) if r for m in range(*r)}
        assert pf == pb
