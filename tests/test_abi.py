"""The C-ABI library loads on a machine without a GPU, exports every symbol its
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import re

import pytest

import tiled_prefill_amd as tpa

FAKE = 0x1000  # never dereferenced: every call below fails argument checks first


def declared_functions():
    text = open(tpa.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("attn_fwd", "attn_fwd_varlen", "attn_plan", "attn_plan_fwd", "attn_workspace_bytes",
                     "attn_set_workspace", "attn_lse_combine", "attn_last_error",
                     "attn_set_option", "attn_get_option"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tpa.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert missing == []


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=64,
             causal=0, wl=-1, scale=0.125, splits=0, dtype=tpa.BF16)
    a.update(kw)
    lib = tpa.load()
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Sq"], a["Sk"], a["d"], a["causal"], a["wl"], a["scale"],
                          a["splits"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1),
    (dict(o=None), -1),
    (dict(Hq=6, Hkv=4), -1),
    (dict(Hkv=0), -1),
    (dict(d=96), -2),
    (dict(d=256), -2),
    (dict(dtype=7), -2),
    (dict(wl=-2), -1),
    (dict(scale=0.0), -1),
    (dict(scale=float("inf")), -1),
    (dict(scale=float("nan")), -1),
    (dict(splits=257), -1),
    (dict(Sq=-1), -1),
    (dict(B=70000), -1),
])
def test_bad_arguments_are_rejected_without_launch(kw, code):
    assert _fwd(**kw) == code
    assert tpa.load().attn_last_error().decode() != ""


def test_varlen_requires_seqlens():
    lib = tpa.load()
    rc = lib.attn_fwd_varlen(FAKE, FAKE, FAKE, FAKE, None, 2, 4, 4, 1, 64, 64, 0, -1, 0.1, 0,
                               tpa.BF16, None, -1, None)
    assert rc == -1


def test_combine_rejects_bad_split_counts():
    lib = tpa.load()
    assert lib.attn_lse_combine(FAKE, FAKE, FAKE, None, 1, 1, 4, 128, 0, 1, None) == -1
    assert lib.attn_lse_combine(FAKE, FAKE, FAKE, None, 1, 1, 4, 128, 300, 1, None) == -1
    assert lib.attn_lse_combine(FAKE, FAKE, FAKE, None, 1, 1, 4, 80, 4, 1, None) == -2
    assert lib.attn_lse_combine(None, FAKE, FAKE, None, 1, 1, 4, 128, 4, 1, None) == -1


def test_plan_rejects_bad_arguments():
    with pytest.raises(tpa.AttnError):
        tpa.plan(1, 3, 2, 4, 4, 64, num_cus=256)
    with pytest.raises(tpa.AttnError):
        tpa.plan(1, 4, 4, 4, 4, 80, num_cus=256)


def test_workspace_bytes():
    assert tpa.workspace_bytes(1, 32, 1, 128, 1) == 0
    assert tpa.workspace_bytes(1, 32, 1, 128, 128) == 128 * 32 * 129 * 4


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        tpa.fwd(q, q, q)


def _bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1,
             Hq=4, Hkv=2, Sq=8, Sk=8, d=64, causal=0, wl=-1, scale=0.125, dtype=tpa.BF16)
    a.update(kw)
    return tpa.load().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                 a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
                                 a["d"], a["causal"], a["wl"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(do=None), -1), (dict(lse=None), -1), (dict(dq=None), -1),
    (dict(dk=None), -1), (dict(v=None), -1), (dict(Hq=6, Hkv=4), -1), (dict(d=96), -2),
    (dict(dtype=5), -2), (dict(wl=-3), -1), (dict(scale=-1.0), -1), (dict(Sk=-2), -1),
])
def test_bwd_bad_arguments_are_rejected_without_launch(kw, code):
    assert _bwd(**kw) == code
    assert tpa.load().attn_last_error().decode() != ""


def test_python_binding_refuses_cpu_tensors_in_every_entry_point():
    # no CPU fallback anywhere: every compute call raises on host tensors
    import torch
    q = torch.zeros(1, 2, 4, 64)
    k = torch.zeros(1, 3, 2, 64)
    lse = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError):
        tpa.fwd_varlen(q, k, k, torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        tpa.fwd_dv(q, k, torch.zeros(1, 3, 2, 32))
    with pytest.raises(ValueError):
        tpa.bwd(q, k, k, q, q, lse)


def test_host_block_range_mirrors_reject_bad_arguments():
    with pytest.raises(tpa.AttnError):
        tpa.m_block_range(8, 8, True, -2, 64, 64, 0)
    with pytest.raises(tpa.AttnError):
        tpa.m_block_range(8, 8, True, -1, 0, 64, 0)
    with pytest.raises(tpa.AttnError):
        tpa.plan_bwd(1, 6, 4, 8, 8, 64)
    assert tpa.m_block_range(0, 8, True, -1, 64, 64, 0)[1] == 0   # no query rows: empty


def test_caller_workspace_errors_launch_nothing():
    """A bound workspace that is too small (or misaligned) is refused before any GPU
    call: the decode problem below needs split partials."""
    lib = tpa.load()
    assert lib.attn_set_workspace(ctypes.c_void_p(FAKE + 8), 1 << 20) == -1  # not 256-byte aligned
    need = tpa.plan(1, 32, 4, 1, 32768, 128, num_cus=256)["workspace_bytes"]
    assert need > 0
    assert lib.attn_set_workspace(ctypes.c_void_p(FAKE), need - 1) == 0
    try:
        rc = lib.attn_fwd(FAKE, FAKE, FAKE, FAKE, None, 1, 32, 4, 1, 32768, 128, 0, -1, 0.088,
                          0, tpa.BF16, None)
        assert rc == -1
        assert "workspace" in lib.attn_last_error().decode()
        bneed = tpa.plan_bwd(1, 4, 2, 64, 64, 64, causal=True)["workspace_bytes"]
        assert lib.attn_set_workspace(ctypes.c_void_p(FAKE), bneed - 1) == 0
        rc = lib.attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 64, 64,
                          64, 1, -1, 0.125, tpa.BF16, None)
        assert rc == -1 and "workspace" in lib.attn_last_error().decode()
    finally:
        assert lib.attn_set_workspace(None, 0) == 0


def test_options_round_trip_and_reject_unknown_names(attn_options):
    assert tpa.get_option("ATTN_SPLIT_RULE") == tpa.get_option("SPLIT_RULE")
    attn_options("SPLIT_RULE", 3)
    assert tpa.get_option("ATTN_SPLIT_RULE") == 3
    with pytest.raises(tpa.AttnError):
        tpa.set_option("NO_SUCH_SWITCH", 1)
    with pytest.raises(tpa.AttnError):
        tpa.get_option("NO_SUCH_SWITCH")


def test_options_change_the_plan(attn_options):
    base = tpa.plan(1, 32, 32, 8192, 8192, 128, causal=True, num_cus=256)
    attn_options("PREFILL_WAVES", 4)
    assert tpa.plan(1, 32, 32, 8192, 8192, 128, causal=True, num_cus=256)["block_m"] == 128
    assert base["block_m"] == 256


def test_noalloc_refuses_a_problem_beyond_its_static_scratch():
    # 256 forced splits of 2048 decode rows need ~270 MB of partials: refused
    # before any GPU call
    lib = tpa.load()
    rc = lib.attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, None, 64, 32, 32, 1, 4096, 128, 0, -1,
                              0.088, 256, tpa.BF16, None)
    assert rc == -1
    assert "noalloc" in lib.attn_last_error().decode()


def test_stream_read_rejects_bad_buffers():
    lib = tpa.load()
    assert lib.attn_stream_read(None, 1024, 0, FAKE, None) == -1
    assert lib.attn_stream_read(FAKE, 1000, 0, FAKE, None) == -1       # not a multiple of 16
    assert lib.attn_stream_read(FAKE + 4, 1024, 0, FAKE, None) == -1   # misaligned
    assert lib.attn_stream_read(FAKE, 1 << 34, 4, FAKE, None) == -1    # > 2 GiB per workgroup
    assert lib.attn_stream_read(FAKE, 0, 0, FAKE, None) == 0           # nothing to read


def test_attn_plan_is_attn_plan_fwd():
    lib = tpa.load()
    for args in [(1, 32, 4, 1, 32768, 128, 0, -1, 0, tpa.BF16, 0, -1, 256),
                 (1, 32, 32, 8192, 8192, 128, 1, -1, 0, tpa.BF16, 0, -1, 256),
                 (16, 32, 8, 1, 16384, 128, 0, -1, 0, tpa.BF16, 1, 135000, 256),
                 (2, 16, 16, 17, 2065, 128, 1, -1, 0, tpa.FP32, 0, -1, 256),
                 (1, 4, 3, 8, 8, 64, 0, -1, 0, tpa.BF16, 0, -1, 256)]:  # Hq % Hkv != 0
        a, b = tpa.Plan(), tpa.Plan()
        ra = lib.attn_plan(*args, ctypes.byref(a))
        rb = lib.attn_plan_fwd(*args, ctypes.byref(b))
        assert ra == rb
        assert bytes(a) == bytes(b)
