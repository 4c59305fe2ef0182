"""Property tests of the tile-config factory and the split-K planner (host
code only, no GPU): for seeded random problems over the whole argument
space -- empty to 2^20-sized extents, both input formats and storage
orders, leading dimensions from packed to past 32-bit buffer offsets, alpha
zero or not -- the choice the library reports must obey the rules its
header and table state:

* nothing to do for an empty C, the scale-only kernel when K = 0 or alpha
  = 0;
* otherwise an entry of the call's input format; a tiled or narrow entry in
  the call's storage orders (a one-column row-major B with ldb = 1 may be
  read as column-major by the narrow kernel), whose 32-bit per-stage buffer
  offsets hold, with the grid its tile size gives; the narrow kernel only
  for N <= 16 with A row-major; the 64-bit direct kernel only when no tiled
  entry of the family fits; the largest tile only when three times its
  rounds of workgroups over the compute units (2.5 times with A row-major
  and B column-major) come to at most the 128x128 tiles' rounds;
* split-K: at least one piece, the workspace exactly pieces * M * N * 4
  bytes (none for one piece), pieces only of a tiled kernel, each but the
  last holding ceil(K tiles / pieces asked) K tiles (so a requested count
  n gives ceil(K tiles / ceil(K tiles / n)) pieces, at most n and at most
  one per K tile), and an automatic split only for K >= 4096, into at most
  32 pieces of at least 1024 K (of at least 512 K when that makes 6 or 8).
"""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import dense_mixed_precision_amd as mp

FAKE_A = 0x7F0000000000
FAKE_B = 0x7F1000000000
FAKE_C = 0x7F2000000000
NUM_CU = 256
LIMIT32 = 0x7FFFFFF0

SETTINGS = settings(max_examples=400, derandomize=True, deadline=None, database=None,
                    suppress_health_check=[HealthCheck.too_slow])

extent = st.one_of(st.integers(0, 20), st.integers(1, 700), st.integers(1, 1 << 14),
                   st.sampled_from([1, 15, 16, 17, 127, 128, 129, 255, 256, 257, 2048, 4096, 8192, 32768]))
pad = st.one_of(st.just(0), st.integers(0, 64), st.sampled_from([1 << 20, 1 << 24, 1 << 28]))


def cdiv(a, b):
    return -(-a // b)


def problem():
    return st.fixed_dictionaries(dict(
        in_type=st.sampled_from([mp.MPGEMM_IN_F16, mp.MPGEMM_IN_BF16]),
        la=st.sampled_from([0, 1]), lb=st.sampled_from([0, 1]),
        M=extent, N=extent, K=extent, pad_a=pad, pad_b=pad, pad_c=st.integers(0, 16),
        alpha=st.sampled_from([1.0, 0.0, -2.5]),
        off_a=st.sampled_from([0, 2]), off_b=st.sampled_from([0, 2])))


def lds(p):
    lda = max(p["M"] if p["la"] else p["K"], 1) + p["pad_a"]
    ldb = max(p["K"] if p["lb"] else p["N"], 1) + p["pad_b"]
    ldc = max(p["N"], 1) + p["pad_c"]
    return lda, ldb, ldc


def query(p):
    lda, ldb, ldc = lds(p)
    f = mp.mpgemm_bf16f32_layout_query if p["in_type"] == mp.MPGEMM_IN_BF16 else mp.mpgemm_f16f32_layout_query
    return f(p["la"], p["lb"], p["M"], p["N"], p["K"], FAKE_A + p["off_a"], lda, FAKE_B + p["off_b"], ldb,
             FAKE_C, ldc, p["alpha"], 0.0)


def spans_fit(c, la, lb, lda, ldb, ldc, M, N):
    """The 32-bit per-stage offsets of a tiled entry (and its C tile)."""
    a_span = ((c["bm"] * lda + c["bk"]) if la == 0 else (c["bk"] * lda + c["bm"])) * 2
    b_span = ((c["bk"] * ldb + c["bn"]) if lb == 0 else (c["bn"] * ldb + c["bk"])) * 2
    c_span = (c["bm"] * ldc + c["bn"]) * 4
    return (a_span < LIMIT32 and b_span < LIMIT32 and c_span < LIMIT32
            and cdiv(M, c["bm"]) * cdiv(N, c["bn"]) <= 0x7FFFFFFF)


def family_entries(in_type, la, lb):
    return [mp.mpgemm_config_info(i) for i in range(mp.mpgemm_num_configs())
            if mp.mpgemm_config_info(i)["kind_name"] == "pipe"
            and (mp.mpgemm_config_info(i)["in_type"], mp.mpgemm_config_info(i)["layout_a"],
                 mp.mpgemm_config_info(i)["layout_b"]) == (in_type, la, lb)]


@SETTINGS
@given(problem())
def test_factory_choice_obeys_the_table_rules(p):
    c = query(p)
    M, N, K = p["M"], p["N"], p["K"]
    lda, ldb, ldc = lds(p)
    if M == 0 or N == 0:
        assert c["id"] == -1 and c["kind_name"] == "none"
        return
    if K == 0 or p["alpha"] == 0.0:
        assert c["kind_name"] == "scale"
        return
    assert c["in_type"] == p["in_type"]
    kind = c["kind_name"]
    assert kind in ("pipe", "narrow", "direct")
    if kind == "narrow":
        assert N <= 16 and p["la"] == 0 and c["grid"] == cdiv(M, 16)
        one_column = N == 1 and p["lb"] == 0 and ldb == 1
        assert c["layout_b"] == p["lb"] or (one_column and c["layout_b"] == 1)
        return
    assert c["grid"] == cdiv(M, c["bm"]) * cdiv(N, c["bn"])
    if kind == "direct":
        # only when no tiled entry of the family fits
        assert not any(spans_fit(e, p["la"], p["lb"], lda, ldb, ldc, M, N)
                       for e in family_entries(p["in_type"], p["la"], p["lb"]))
        return
    assert (c["layout_a"], c["layout_b"]) == (p["la"], p["lb"])
    assert spans_fit(c, p["la"], p["lb"], lda, ldb, ldc, M, N)
    if c["bm"] == 256:
        # the big tile only where its rounds of workgroups over the compute
        # units come to at most a third of the 128x128 tiles' rounds
        r256 = cdiv(cdiv(M, 256) * cdiv(N, 256), NUM_CU)
        r128 = cdiv(cdiv(M, 128) * cdiv(N, 128), NUM_CU)
        assert (5 * r256 <= 2 * r128) if (p["la"], p["lb"]) == (0, 1) else (3 * r256 <= r128)


@SETTINGS
@given(problem(), st.sampled_from([0, 0, 1, 2, 3, 7, 32, 100]))
def test_splitk_plan_obeys_its_contract(p, requested):
    lda, ldb, _ = lds(p)
    M, N, K = p["M"], p["N"], p["K"]
    plan = mp.mpgemm_splitk_plan(p["in_type"], p["la"], p["lb"], M, N, K, FAKE_A + p["off_a"], lda,
                                 FAKE_B + p["off_b"], ldb, requested)
    s = plan["splits"]
    assert s >= 1
    assert plan["workspace_bytes"] == (0 if s == 1 else s * M * N * 4)
    if s == 1:
        return
    c = mp.mpgemm_config_info(plan["config_id"])
    assert c["kind_name"] == "pipe" and c["in_type"] == p["in_type"]
    k_tiles = cdiv(K, c["bk"])
    if requested > 0:
        n = min(requested, k_tiles)
        assert s == cdiv(k_tiles, cdiv(k_tiles, n)) and s <= n
    else:
        # K of at least 4096, pieces of at least 1024 K (512 K for the floors
        # of 6 and 8 pieces), at most 32
        assert s <= 32 and K >= 4096 and s <= max(K // 1024, 8) and s <= K // 512


def test_strategies_reach_every_kind():
    """Every kind the rules above speak of is reachable from the argument
    space the strategies draw from (fixed representatives), so no branch of
    the properties is vacuous."""
    base = dict(in_type=0, la=0, lb=0, pad_a=0, pad_b=0, pad_c=0, alpha=1.0, off_a=0, off_b=0)
    kinds = {query(dict(base, M=M, N=N, K=K, **kw))["kind_name"]
             for M, N, K, kw in [(64, 64, 0, {}), (4096, 16, 4096, {}), (300, 300, 64, {}),
                                 (300, 300, 64, dict(pad_a=1 << 28)), (0, 5, 5, {})]}
    assert kinds == {"scale", "narrow", "pipe", "direct", "none"}


@pytest.mark.parametrize("M,N", [(16 * 256, 16 * 256), (256 * 16, 256 * 15), (256 * 16, 256 * 8),
                                 (256 * 12, 256 * 11), (256 * 11, 256 * 11), (256 * 17, 256 * 16)])
def test_largest_tile_by_rounds_over_the_compute_units(M, N):
    """256x256 tiles exactly when three times their rounds of workgroups over
    the compute units come to at most the 128x128 tiles' rounds (4096 x 3840:
    240 big tiles, one round, against 960 tiles in four; 4096 x 2048: 128
    big tiles against two rounds; 4352 x 4096: two rounds against five)."""
    base = dict(in_type=0, la=0, lb=0, pad_a=0, pad_b=0, pad_c=0, alpha=1.0, off_a=0, off_b=0, K=512)
    c = query(dict(base, M=M, N=N))
    big = 3 * cdiv(cdiv(M, 256) * cdiv(N, 256), NUM_CU) <= cdiv(cdiv(M, 128) * cdiv(N, 128), NUM_CU)
    assert (c["bm"] == 256) == big
