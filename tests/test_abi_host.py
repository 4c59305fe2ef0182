"""Host-side tests of the C ABI (no GPU): the library loads, exports every
function include/mpgemm.h declares, rejects bad arguments before any HIP call,
and the tile-config factory picks the intended entry per shape/alignment.
Pointers here are fake integers: only validation and the factory run, both
pure host code."""
import ctypes
import os
import re

import pytest

import dense_mixed_precision_amd as mp
from dense_mixed_precision_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpgemm.h")
PROBES_HEADER = os.path.join(ROOT, "include", "mpgemm_probes.h")
TIMELINE_HEADER = os.path.join(ROOT, "include", "mpgemm_timeline.h")

FAKE_A = 0x7F0000000000   # 256-byte aligned fake device addresses
FAKE_B = 0x7F1000000000
FAKE_C = 0x7F2000000000


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpgemm_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("mpgemm_f16f32", "mpgemm_f16f32_query", "mpgemm_f16f32_with_config",
                 "mpgemm_num_configs", "mpgemm_config_info", "mpgemm_strerror", "mpgemm_version"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mp.lib_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_probes_library_exports_its_header_and_the_product_none_of_it():
    probes = declared_functions(PROBES_HEADER)
    assert {"mpgemm_probe_mfma_layout", "mpgemm_probe_mfma_rate", "mpgemm_probe_fill"} <= set(probes)
    lib = mp.load_probes()
    assert not [n for n in probes if not hasattr(lib, n)]
    product = ctypes.CDLL(mp.lib_path())
    assert not [n for n in probes if hasattr(product, n)]


def test_timeline_build_exports_its_header_and_the_product_none_of_it():
    names = declared_functions(TIMELINE_HEADER)
    assert names == ["mpgemm_timeline_clear", "mpgemm_timeline_entries", "mpgemm_timeline_read"]
    lib = mp.load_timeline()
    assert not [n for n in names + declared_functions() if not hasattr(lib, n)]
    product = ctypes.CDLL(mp.lib_path())
    assert not [n for n in names if hasattr(product, n)]
    assert lib.mpgemm_timeline_entries() == 4096 * mp.TIMELINE_SLOTS
    # argument checks come before any HIP call
    assert lib.mpgemm_timeline_read(None, 1) == mp.MPGEMM_ENULL
    out = (ctypes.c_uint64 * 4)()
    assert lib.mpgemm_timeline_read(out, -1) == mp.MPGEMM_EDIM
    assert lib.mpgemm_timeline_read(out, 4096 * mp.TIMELINE_SLOTS + 1) == mp.MPGEMM_EDIM
    assert lib.mpgemm_timeline_read(out, 0) == mp.MPGEMM_OK


def test_version_and_strerror():
    assert "gfx950" in mp.mpgemm_version()
    for code in range(-11, 1):
        assert mp.mpgemm_strerror(code)
    assert mp.mpgemm_strerror(-99) == "unknown error code"


def q(M, N, K, A=FAKE_A, lda=None, B=FAKE_B, ldb=None, C=FAKE_C, ldc=None, alpha=1.0, beta=0.0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return mp.mpgemm_f16f32_query(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta)


def code(M, N, K, A=FAKE_A, lda=None, B=FAKE_B, ldb=None, C=FAKE_C, ldc=None, alpha=1.0, beta=0.0):
    try:
        q(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta)
        return 0
    except mp.MpgemmError as e:
        return e.code


@pytest.mark.parametrize("args,expect", [
    (dict(M=-1, N=4, K=4), mp.MPGEMM_EDIM),
    (dict(M=4, N=-1, K=4), mp.MPGEMM_EDIM),
    (dict(M=4, N=4, K=-3), mp.MPGEMM_EDIM),
    (dict(M=4, N=4, K=8, lda=7), mp.MPGEMM_ELD),
    (dict(M=4, N=8, K=4, ldb=7), mp.MPGEMM_ELD),
    (dict(M=4, N=8, K=4, ldc=7), mp.MPGEMM_ELD),
    (dict(M=4, N=4, K=0, lda=0), mp.MPGEMM_ELD),
    (dict(M=4, N=4, K=4, A=0), mp.MPGEMM_ENULL),
    (dict(M=4, N=4, K=4, B=0), mp.MPGEMM_ENULL),
    (dict(M=4, N=4, K=4, C=0), mp.MPGEMM_ENULL),
    (dict(M=4, N=4, K=4, C=FAKE_C + 2), mp.MPGEMM_EALIGN),
    (dict(M=4, N=4, K=4, A=FAKE_A + 1), mp.MPGEMM_EALIGN),
    (dict(M=4, N=4, K=4, B=FAKE_B + 1), mp.MPGEMM_EALIGN),
    # A and B are not read when alpha == 0 or K == 0: NULL is fine there
    (dict(M=4, N=4, K=4, A=0, B=0, alpha=0.0, beta=0.5), 0),
    (dict(M=4, N=4, K=0, A=0, B=0), 0),
    # nothing to do at all: C may be NULL
    (dict(M=0, N=4, K=4, C=0), 0),
    (dict(M=4, N=0, K=4, C=0), 0),
])
def test_validation_codes(args, expect):
    assert code(**args) == expect


def test_validation_happens_before_launch():
    # the launching entry point returns the same codes without touching HIP
    rc = mp.mpgemm_f16f32(-1, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0, 0)
    assert rc == mp.MPGEMM_EDIM
    rc = mp.mpgemm_f16f32(4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C + 1, 4, 1.0, 0.0, 0)
    assert rc == mp.MPGEMM_EALIGN
    rc = mp.mpgemm_f16f32_with_config(999, 4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0, 0)
    assert rc == mp.MPGEMM_ECONFIG
    rc = mp.mpgemm_f16f32_with_config(-1, 4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0, 0)
    assert rc == mp.MPGEMM_ECONFIG


def test_config_table_is_consistent():
    n = mp.mpgemm_num_configs()
    assert n >= 4
    kinds = set()
    for i in range(n):
        c = mp.mpgemm_config_info(i)
        assert c["id"] == i
        kinds.add(c["kind_name"])
        if c["kind_name"] == "pipe":
            assert (c["mfma_m"], c["mfma_n"], c["mfma_k"]) in ((32, 32, 16), (16, 16, 32))
            assert c["bm"] % (c["mfma_m"] * c["waves_m"]) == 0 and c["bn"] % (c["mfma_n"] * c["waves_n"]) == 0
            assert c["bk"] % c["mfma_k"] == 0
            assert c["wave_m"] * c["waves_m"] == c["bm"] and c["wave_n"] * c["waves_n"] == c["bn"]
            assert c["threads"] == 64 * c["waves_m"] * c["waves_n"] * c["k_groups"]
            assert c["lds_bytes"] == c["stages"] * (c["bm"] + c["bn"]) * c["bk"] * 2
            assert c["lds_bytes"] <= 160 * 1024
            assert (c["vec_a"], c["vec_b"]) == (8, 8)
            # only the 128x128x128 tile staggers its K order
            assert c["k_order"] == (2 if (c["bm"], c["bn"], c["bk"]) == (128, 128, 128) else 0)
        else:
            assert c["k_order"] == 0
    assert kinds == {"pipe", "direct", "scale", "narrow"}
    with pytest.raises(mp.MpgemmError):
        mp.mpgemm_config_info(n)


def _pick(w):
    return q(w.M, w.N, w.K, alpha=w.alpha, beta=w.beta)


def test_factory_choices_for_the_workloads():
    c = _pick(WORKLOADS["square8192"])
    assert (c["kind_name"], c["bm"], c["bn"], c["vec_a"], c["vec_b"]) == ("pipe", 256, 256, 8, 8)
    assert c["grid"] == 32 * 32
    assert (c["mfma_m"], c["mfma_n"], c["mfma_k"]) == (16, 16, 32)
    c = _pick(WORKLOADS["square2048"])
    assert (c["bm"], c["bn"], c["bk"]) == (128, 128, 128) and c["grid"] == 256
    c = _pick(WORKLOADS["tallskinny32768x128x4096"])
    assert c["kind_name"] == "pipe" and c["grid"] >= 256 and c["bk"] == 64
    c = _pick(WORKLOADS["ragged1000x800x617"])
    # lda = 617 is odd: A rows are only 2-byte aligned, which 16-byte loads
    # serve on gfx950 (unaligned mode), so A keeps the vector copy path.
    assert c["kind_name"] == "pipe" and c["vec_a"] == 8 and c["vec_b"] == 8
    # 208 tiles of 64x64 fill more than half the chip: 64x64, 8 waves, 2 stages
    assert (c["bm"], c["bn"], c["bk"], c["stages"], c["threads"], c["mfma_m"]) == (64, 64, 128, 2, 512, 16)
    c = _pick(WORKLOADS["square256"])
    # 16 tiles of 64x64 would leave most of the chip idle: 16x64 tiles on 4 waves
    assert c["kind_name"] == "pipe" and c["grid"] == 64
    assert (c["bm"], c["bn"], c["bk"], c["stages"], c["threads"], c["mfma_m"]) == (16, 64, 128, 2, 256, 16)
    # ... unless N is not a multiple of 8 (partial B vectors on every K tile): 32x64 on 8 waves
    c = q(200, 300, 400)
    assert (c["bm"], c["bn"], c["bk"], c["stages"], c["threads"]) == (32, 64, 128, 3, 512)
    # one K tile of 64 or less keeps the 64-deep tile
    assert q(256, 256, 64)["bk"] == 64
    # the 2048-class tile (128x128x128) is chosen by panel reuse
    c = _pick(WORKLOADS["square2048"])
    assert (c["bm"], c["bn"], c["bk"], c["stages"], c["k_order"]) == (128, 128, 128, 2, 2)


@pytest.mark.parametrize("M,N,K,shape", [
    # half a wave of 128x128 tiles whose 64x64 tiles come to two per unit: 64x64
    (1024, 2048, 2048, (64, 64, 128, 2)), (2048, 1024, 512, (64, 64, 128, 2)),
    # more than half a wave otherwise: 128x128
    (1536, 1536, 2048, (128, 128, 128, 2)), (1280, 2048, 8192, (128, 128, 128, 2)),
    # short K over at least two 64x64 tiles per unit: 64x64x64 tiles, unless
    # the big tiles come to nearly a full round or the 128x128 class has
    # whole 128-deep K tiles
    (3072, 3072, 128, (64, 64, 64, 2)), (2048, 2048, 192, (64, 64, 64, 2)), (2048, 1024, 64, (64, 64, 64, 2)),
    (5907, 1622, 137, (64, 64, 64, 2)), (3328, 3328, 256, (64, 64, 64, 2)),
    (4096, 4096, 64, (256, 256, 64, 2)), (1457, 10609, 128, (256, 256, 64, 2)),
    (2048, 2048, 128, (128, 128, 128, 2)), (2048, 2048, 256, (128, 128, 128, 2)),
    (3072, 3072, 384, (256, 256, 64, 2)), (1024, 1024, 128, (64, 64, 128, 2)),
    # B rows not 16-byte aligned with a second round of at most 64 128x128
    # tiles: 64x64x128 tiles; aligned B rows or a fuller second round keep
    # the 128x128 tiles
    (2049, 2049, 2048, (64, 64, 128, 2)), (2100, 2100, 2048, (64, 64, 128, 2)),
    (2049, 2048, 2048, (128, 128, 128, 2)), (2304, 2305, 2048, (128, 128, 128, 2)),
    # 256x256 tiles where 3 x their rounds over the compute units <= the
    # 128x128 tiles' rounds, even with fewer big tiles than units
    (3072, 2816, 4096, (256, 256, 64, 2)), (4096, 2304, 1024, (256, 256, 64, 2)),
    (3328, 3328, 4096, (256, 256, 64, 2)), (2816, 2816, 4096, (128, 128, 128, 2)),
    (4096, 2048, 4096, (128, 128, 128, 2)), (4352, 4096, 4096, (128, 128, 128, 2)),
    (5376, 5376, 4096, (256, 256, 64, 2)),
    # 128-deep K tiles with at least two tile rows and columns; with one tile
    # column (A streamed once) only up to K 1024, with one tile row (B
    # streamed once) up to K 4096; else the 3-deep ring of 64-deep tiles
    (16384, 256, 4096, (128, 128, 128, 2)), (8192, 384, 1024, (128, 128, 128, 2)),
    (32768, 256, 8192, (128, 128, 64, 3)), (16384, 384, 8192, (128, 128, 128, 2)),
    (16384, 192, 4096, (128, 128, 128, 2)), (256, 16384, 4096, (128, 128, 128, 2)),
    (32768, 128, 1024, (128, 128, 128, 2)), (32768, 128, 4096, (128, 128, 64, 3)),
    (32768, 128, 8192, (128, 128, 64, 3)), (128, 32768, 2048, (128, 128, 128, 2)),
    (128, 32768, 4096, (128, 128, 64, 3)), (128, 32768, 8192, (128, 128, 64, 3)),
    # one 128-row or 128-column band takes 128x128 tiles even where enough
    # 256x256 tiles would fill the chip (they would be half empty)
    (65536, 128, 1024, (128, 128, 128, 2)), (65536, 128, 4096, (128, 128, 64, 3)),
    (128, 65536, 4096, (128, 128, 64, 3)), (65536, 192, 4096, (256, 256, 64, 2)),
    # fewer 64x64 tiles than units: 16x64 on 4 waves while at most one per
    # unit and K moderate
    (512, 512, 2048, (16, 64, 128, 2)), (384, 384, 2048, (16, 64, 128, 2)), (256, 256, 4096, (16, 64, 128, 2)),
    # ... else 32x64 with 3 stages while at most one per unit or K long
    (512, 512, 8192, (32, 64, 128, 3)), (384, 384, 4096, (32, 64, 128, 3)), (512, 768, 1024, (32, 64, 128, 3)),
    (512, 1024, 512, (32, 64, 128, 3)), (768, 768, 4096, (32, 64, 128, 3)),
    # ... else 64x64
    (768, 768, 1024, (64, 64, 128, 2)), (768, 1024, 2048, (64, 64, 128, 2)),
])
def test_factory_small_and_mid_shapes(M, N, K, shape):
    """The measured choices for small and mid-size row-major FP16 products
    (graph-replayed sweeps over the three small entries and the 128x128
    one)."""
    c = q(M, N, K)
    assert (c["bm"], c["bn"], c["bk"], c["stages"]) == shape, (M, N, K, c["id"])


def test_one_column_row_major_b_is_read_as_column_major():
    """A (K x 1) row-major B with ldb 1 is K consecutive values: when the
    narrow kernel takes the product, the factory reads the column-major form
    of the same bytes (K-contiguous loads); a strided column, a wider B, or
    a product another kernel takes keeps the order it was given."""
    c = q(4096, 1, 4096, ldb=1)
    assert c["kind_name"] == "narrow" and c["layout_b"] == mp.MPGEMM_COL_MAJOR
    c = q(4096, 1, 4096, ldb=8)
    assert c["kind_name"] == "narrow" and c["layout_b"] == mp.MPGEMM_ROW_MAJOR
    assert q(4096, 2, 4096)["layout_b"] == mp.MPGEMM_ROW_MAJOR
    # only the narrow kernel takes the other form: a column-major A keeps B as given
    c = ql(mp.MPGEMM_COL_MAJOR, mp.MPGEMM_ROW_MAJOR, 2048, 1, 2048, ldb=1)
    assert c["kind_name"] == "pipe" and c["layout_b"] == mp.MPGEMM_ROW_MAJOR
    # the caller's arguments are validated as given: ldb 0 is still refused
    assert code(4096, 1, 4096, ldb=0) == mp.MPGEMM_ELD
    plan = mp.mpgemm_splitk_plan(mp.MPGEMM_IN_F16, 0, 0, 4096, 1, 4096, FAKE_A, 4096, FAKE_B, 1, 0)
    assert mp.mpgemm_config_info(plan["config_id"])["layout_b"] == mp.MPGEMM_COL_MAJOR


@pytest.mark.parametrize("M,N,K,ldc,c_off,stores", [
    # 128x128 and smaller tiles: non-temporal stores only
    (2048, 2048, 2048, None, 0, 1), (32768, 128, 4096, None, 0, 1), (1000, 800, 617, None, 0, 1),
    (2049, 2049, 2048, None, 0, 1),
    # 256x256: non-temporal over several rounds at K >= 2048 or with at most 176 tiles
    (8192, 8192, 8192, None, 0, 1), (8192, 8192, 2048, None, 0, 1), (3072, 2816, 1024, None, 0, 1),
    (3328, 3328, 512, None, 0, 1), (3584, 4096, 384, None, 0, 0),
    # ... plain for a full round at shorter K
    (8192, 8192, 512, None, 0, 0), (4096, 4096, 4096, None, 0, 0), (4096, 4096, 1024, None, 0, 0),
    (1456, 10608, 512, None, 0, 0),
    # ... and whenever the rows of C start mid-line
    (8192, 8192, 8192, 8200, 0, 0), (8192, 8192, 8192, None, 4, 0), (1457, 10609, 128, None, 0, 0),
])
def test_factory_c_store_policy(M, N, K, ldc, c_off, stores):
    """The cache policy of the C stores the query reports (1 non-temporal,
    0 plain), by the measured rule; the table marks the entries built with
    both (the 256x256 tiles) with 2."""
    c = q(M, N, K, ldc=ldc, C=FAKE_C + c_off)
    assert c["c_stores"] == stores, (M, N, K, ldc, c_off, c["bm"])
    kinds = {mp.mpgemm_config_info(i)["bm"]: mp.mpgemm_config_info(i)["c_stores"]
             for i in range(mp.mpgemm_num_configs()) if mp.mpgemm_config_info(i)["kind_name"] == "pipe"}
    assert kinds[256] == 2 and all(v == 1 for bm, v in kinds.items() if bm != 256)
    assert mp.mpgemm_config_info(0)["c_stores"] == 0      # the direct kernel's plain stores


def test_factory_alignment_and_degenerate_cases():
    # any 2-byte aligned operand takes the 16-byte copy path
    assert q(512, 512, 512, A=FAKE_A + 2)["vec_a"] == 8
    assert q(512, 512, 512, B=FAKE_B + 8)["vec_b"] == 8
    assert q(512, 512, 512, lda=515)["vec_a"] == 8
    assert q(512, 512, 512, lda=520)["vec_a"] == 8
    assert code(512, 512, 512, A=FAKE_A + 1) == mp.MPGEMM_EALIGN
    assert q(512, 512, 0)["kind_name"] == "scale"
    assert q(512, 512, 64, alpha=0.0, beta=2.0)["kind_name"] == "scale"
    assert q(0, 512, 64)["kind_name"] == "none"


def test_factory_falls_back_to_direct_for_huge_strides():
    # a 256-row A stage with lda = 2^23 spans 4 GiB: 32-bit buffer offsets
    # cannot reach it, so only the 64-bit direct kernel fits.
    c = q(300, 300, 64, lda=1 << 23)
    assert c["kind_name"] in ("pipe", "direct")
    if c["kind_name"] == "pipe":
        assert (c["bm"] * (1 << 23) + c["bk"]) * 2 < 0x7FFFFFF0
    c = q(300, 300, 64, lda=1 << 30)
    assert c["kind_name"] == "direct"


@pytest.mark.parametrize("ld", [1 << 62, (1 << 63) - 1, (1 << 32) + 3])
def test_size_checks_do_not_overflow(ld):
    # bm * lda for these strides is past 2^63: the span checks must see a
    # huge stage (64-bit direct kernel), not a wrapped-around small one
    for kw in ({"lda": ld}, {"ldb": ld}, {"ldc": ld}):
        c = q(1, 1, 64, **kw)
        assert c["kind_name"] == "direct", (kw, c)
    for la, lb in [(1, 0), (0, 1), (1, 1)]:
        c = ql(la, lb, 1, 1, 64, lda=ld, ldb=ld)
        assert c["kind_name"] == "direct", (la, lb, c)
    # tile counts past 2^63 and workspaces past 2^63 bytes: no split, and the
    # only kernel that could take the shape reports a grid it cannot launch
    big = 1 << 62
    c = q(big, big, 64, ldc=big)
    assert c["kind_name"] == "direct" and c["grid"] > 0x7FFFFFFF
    p = plan(1 << 40, 1 << 40, 1 << 20, ldb=1 << 40)
    assert p["splits"] == 1 and p["workspace_bytes"] == 0
    p = plan(64, 64, (1 << 62) + 5, splits=3, la=1)   # A column-major: lda = M
    assert p["splits"] == 3 and p["workspace_bytes"] == 3 * 64 * 64 * 4


# ----------------------------------------------------------------------------
# Column-major operands
# ----------------------------------------------------------------------------

def ql(la, lb, M, N, K, A=FAKE_A, lda=None, B=FAKE_B, ldb=None, C=FAKE_C, ldc=None,
       alpha=1.0, beta=0.0):
    lda = max(M if la else K, 1) if lda is None else lda
    ldb = max(K if lb else N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return mp.mpgemm_f16f32_layout_query(la, lb, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta)


def code_l(*args, **kw):
    try:
        ql(*args, **kw)
        return 0
    except mp.MpgemmError as e:
        return e.code


@pytest.mark.parametrize("args,kw,expect", [
    ((2, 0, 4, 4, 4), {}, mp.MPGEMM_ELAYOUT),
    ((0, -1, 4, 4, 4), {}, mp.MPGEMM_ELAYOUT),
    # column-major A: lda counts M, not K
    ((1, 0, 8, 4, 4), dict(lda=7), mp.MPGEMM_ELD),
    ((1, 0, 8, 4, 16), dict(lda=8), 0),
    # column-major B: ldb counts K, not N
    ((0, 1, 4, 8, 16), dict(ldb=15), mp.MPGEMM_ELD),
    ((0, 1, 4, 32, 16), dict(ldb=16), 0),
    ((1, 1, 4, 4, 4), dict(A=FAKE_A + 1), mp.MPGEMM_EALIGN),
    ((1, 1, 4, 4, 4), dict(C=0), mp.MPGEMM_ENULL),
])
def test_layout_validation_codes(args, kw, expect):
    assert code_l(*args, **kw) == expect


def test_layout_launch_validates_before_hip():
    rc = mp.mpgemm_f16f32_layout(3, 0, 4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0, 0)
    assert rc == mp.MPGEMM_ELAYOUT
    rowmajor_id = q(8192, 8192, 8192)["id"]
    rc = mp.mpgemm_f16f32_layout_with_config(rowmajor_id, 1, 0, 4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4,
                                             1.0, 0.0, 0)
    assert rc == mp.MPGEMM_ECONFIG  # a row-major entry asked to read a column-major A


def test_every_layout_pair_has_pipelined_entries():
    pairs = {}
    for i in range(mp.mpgemm_num_configs()):
        c = mp.mpgemm_config_info(i)
        assert c["layout_a"] in (0, 1) and c["layout_b"] in (0, 1)
        if c["kind_name"] == "pipe":
            pairs.setdefault((c["layout_a"], c["layout_b"]), set()).add((c["bm"], c["bn"]))
    for pair in [(0, 0), (0, 1), (1, 0), (1, 1)]:
        assert {(256, 256), (128, 128), (64, 64)} <= pairs[pair], pair


@pytest.mark.parametrize("la,lb", [(0, 1), (1, 0), (1, 1)])
def test_layout_factory_choices(la, lb):
    c = ql(la, lb, 8192, 8192, 8192)
    assert (c["kind_name"], c["bm"], c["bn"], c["vec_a"], c["vec_b"]) == ("pipe", 256, 256, 8, 8)
    assert (c["layout_a"], c["layout_b"]) == (la, lb) and c["grid"] == 1024
    c = ql(la, lb, 2048, 2048, 2048)
    assert (c["bm"], c["bn"], c["bk"]) == (128, 128, 128) and c["grid"] == 256
    # every storage order: 128-deep tiles with two or more tile rows and
    # columns, the 64-deep ring for one tile column at long K, 256x256 tiles
    # by rounds over the compute units
    assert ql(la, lb, 16384, 256, 4096)["bk"] == 128
    assert ql(la, lb, 32768, 128, 4096)["bk"] == 64
    assert ql(la, lb, 3072, 2816, 4096)["bm"] == 256
    assert ql(la, lb, 4096, 2048, 4096)["bm"] == 128
    # two rounds of 256x256 tiles against five of 128x128: the big tile for
    # A row-major with B column-major only
    assert ql(la, lb, 1504, 12052, 2229)["bm"] == (256 if (la, lb) == (0, 1) else 128)
    c = ql(la, lb, 1000, 800, 617, lda=(1001 if la else 617), ldb=(617 if lb else 800))
    assert c["kind_name"] == "pipe" and (c["vec_a"], c["vec_b"]) == (8, 8)
    # a stored stage beyond 32-bit offsets leaves only the 64-bit direct kernel
    c = ql(la, lb, 300, 300, 64, lda=(1 << 30), ldb=(1 << 30))
    assert c["kind_name"] == "direct" and (c["layout_a"], c["layout_b"]) == (la, lb)


# ----------------------------------------------------------------------------
# BF16 inputs
# ----------------------------------------------------------------------------

def qb(la, lb, M, N, K, A=FAKE_A, lda=None, B=FAKE_B, ldb=None, C=FAKE_C, ldc=None,
       alpha=1.0, beta=0.0):
    lda = max(M if la else K, 1) if lda is None else lda
    ldb = max(K if lb else N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return mp.mpgemm_bf16f32_layout_query(la, lb, M, N, K, A, lda, B, ldb, C, ldc, alpha, beta)


@pytest.mark.parametrize("la,lb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_bf16_factory_choices(la, lb):
    c = qb(la, lb, 8192, 8192, 8192)
    assert (c["kind_name"], c["bm"], c["bn"], c["in_type"]) == ("pipe", 256, 256, mp.MPGEMM_IN_BF16)
    assert (c["layout_a"], c["layout_b"]) == (la, lb)
    assert mp.mpgemm_config_info(c["id"])["in_type"] == mp.MPGEMM_IN_BF16
    c = qb(la, lb, 2048, 2048, 2048)
    assert (c["bm"], c["bk"], c["in_type"]) == (128, 128, mp.MPGEMM_IN_BF16)
    c = qb(la, lb, 1000, 800, 617, lda=(1001 if la else 617), ldb=(617 if lb else 800))
    assert (c["vec_a"], c["vec_b"], c["in_type"]) == (8, 8, mp.MPGEMM_IN_BF16)
    c = qb(la, lb, 300, 300, 64, lda=(1 << 30), ldb=(1 << 30))
    assert c["kind_name"] == "direct" and c["in_type"] == mp.MPGEMM_IN_BF16
    assert qb(la, lb, 64, 64, 0)["kind_name"] == "scale"


def test_bf16_and_f16_entries_do_not_mix():
    f16_id = q(8192, 8192, 8192)["id"]
    bf16_id = qb(0, 0, 8192, 8192, 8192)["id"]
    assert f16_id != bf16_id
    args = (8192, 8192, 8192, FAKE_A, 8192, FAKE_B, 8192, FAKE_C, 8192, 1.0, 0.0, 0)
    assert mp.mpgemm_bf16f32_layout_with_config(f16_id, 0, 0, *args) == mp.MPGEMM_ECONFIG
    assert mp.mpgemm_f16f32_layout_with_config(bf16_id, 0, 0, *args) == mp.MPGEMM_ECONFIG
    assert mp.mpgemm_bf16f32(-1, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0, 0) == mp.MPGEMM_EDIM
    assert mp.mpgemm_bf16f32_layout(5, 0, 4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0, 0) \
        == mp.MPGEMM_ELAYOUT


def test_gemm_ex_validation_before_launch():
    args = (4, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0)
    assert mp.mpgemm_gemm_ex(2, 0, 0, *args, 0, 0) == mp.MPGEMM_ETYPE
    assert mp.mpgemm_gemm_ex(0, 2, 0, *args, 0, 0) == mp.MPGEMM_ELAYOUT
    assert mp.mpgemm_gemm_ex(0, 0, 0, *args, FAKE_C + 0x1000 + 2, 0) == mp.MPGEMM_EALIGN
    assert mp.mpgemm_gemm_ex(0, 0, 0, -1, 4, 4, FAKE_A, 4, FAKE_B, 4, FAKE_C, 4, 1.0, 0.0, 0, 0) \
        == mp.MPGEMM_EDIM
    assert mp.mpgemm_gemm_ex_with_config(999, 0, 0, 0, *args, 0, 0) == mp.MPGEMM_ECONFIG


# ----------------------------------------------------------------------------
# Split-K plans
# ----------------------------------------------------------------------------

def plan(M, N, K, splits=0, la=0, lb=0, in_type=0, lda=None, ldb=None):
    lda = max(M if la else K, 1) if lda is None else lda
    ldb = max(K if lb else N, 1) if ldb is None else ldb
    return mp.mpgemm_splitk_plan(in_type, la, lb, M, N, K, FAKE_A, lda, FAKE_B, ldb, splits)


def test_splitk_plan_skinny_case_fills_the_chip():
    # 4096 x 16 x 4096: the narrow kernel (256 workgroups of 16 rows, K split
    # over each one's 8 waves) fills the chip in one launch, so no pieces
    p = plan(4096, 16, 4096)
    assert mp.mpgemm_config_info(p["config_id"])["kind_name"] == "narrow"
    assert (p["splits"], p["workspace_bytes"]) == (1, 0)
    # 256 x 16 x 65536: 16 narrow workgroups would leave the chip idle, so
    # the plan splits a tile kernel into pieces of about 1024 K, at most ~4
    # workgroups per compute unit and at most 32
    p = plan(256, 16, 65536)
    c = mp.mpgemm_config_info(p["config_id"])
    tiles = -(-256 // c["bm"])
    assert c["kind_name"] == "pipe" and p["splits"] == min(32, 65536 // 1024, -(-4 * 256 // tiles))
    assert p["workspace_bytes"] == p["splits"] * 256 * 16 * 4
    # a requested piece count splits a tile kernel whatever the shape
    p = plan(4096, 16, 4096, splits=4)
    assert p["splits"] == 4 and mp.mpgemm_config_info(p["config_id"])["kind_name"] == "pipe"


@pytest.mark.parametrize("M,N,K,pieces", [
    (512, 512, 2048, 1), (512, 512, 1024, 1),          # K < 4096 stays whole
    (256, 256, 8192, 8), (256, 256, 16384, 16),        # pieces of 1024 K
    (256, 256, 65536, 32),                             # at most 32
    (1024, 1024, 8192, 4), (2048, 256, 8192, 8),       # at most ~4 workgroups per unit
    (2048, 2048, 8192, 1),                             # a full wave of 128x128 tiles
    (256, 256, 4096, 8), (256, 96, 5000, 8),           # at least 8 on grids of <= 64 tiles
    (512, 48, 4096, 8),
    (768, 768, 6144, 6), (1024, 512, 4096, 6),         # at least 6 on larger grids ...
    (640, 640, 4096, 6), (1280, 512, 4096, 6),
    (1024, 1024, 4096, 4),                             # ... within 4 workgroups per unit
])
def test_splitk_automatic_plan(M, N, K, pieces):
    """The automatic plan, by graph-replayed sweeps of forced piece counts."""
    assert plan(M, N, K)["splits"] == pieces


def test_splitk_plan_keeps_full_grids_whole():
    for shape in [(2048, 2048, 2048), (8192, 8192, 8192), (32768, 128, 4096)]:
        p = plan(*shape)
        assert (p["splits"], p["workspace_bytes"]) == (1, 0), shape


def test_splitk_plan_forced_and_capped():
    p = plan(300, 200, 1234, splits=3)
    assert p["splits"] == 3 and p["workspace_bytes"] == 3 * 300 * 200 * 4
    bk = mp.mpgemm_config_info(p["config_id"])["bk"]
    p = plan(300, 200, 100, splits=64)           # at most one piece per K tile
    assert p["splits"] == -(-100 // bk)
    assert plan(300, 200, 1234, splits=1)["splits"] == 1
    assert plan(300, 200, 0)["splits"] == 1      # K == 0 is the scale path
    with pytest.raises(mp.MpgemmError) as e:
        plan(300, 200, 1234, splits=-1)
    assert e.value.code == mp.MPGEMM_ESPLIT
    with pytest.raises(mp.MpgemmError) as e:
        plan(300, 200, 1234, la=3)
    assert e.value.code == mp.MPGEMM_ELAYOUT


def test_static_splitk_refuses_before_hip():
    """The allocation-free split-K checks its arguments and the plan's size
    against the static scratch before any HIP call."""
    args = (0, 0, 0, 256, 16, 65536, FAKE_A, 65536, FAKE_B, 16, FAKE_C, 16, 1.0, 0.0, 0)
    assert mp.mpgemm_gemm_splitk_static(*args, -1, 0) == mp.MPGEMM_ESPLIT
    assert mp.mpgemm_gemm_splitk_static(3, *args[1:], 0, 0) == mp.MPGEMM_ETYPE
    assert mp.mpgemm_gemm_splitk_static(0, 0, 0, 256, 16, 65536, FAKE_A, 65536, FAKE_B, 16, FAKE_C + 2, 16,
                                        1.0, 0.0, 0, 0, 0) == mp.MPGEMM_EALIGN
    # 4 pieces of 2048 x 2048: 64 MiB of partial products
    big = (0, 0, 0, 2048, 2048, 8192, FAKE_A, 8192, FAKE_B, 2048, FAKE_C, 2048, 1.0, 0.0, 0)
    assert plan(2048, 2048, 8192, splits=4)["workspace_bytes"] > mp.MPGEMM_STATIC_SCRATCH_BYTES
    assert mp.mpgemm_gemm_splitk_static(*big, 4, 0) == mp.MPGEMM_ESCRATCH
    assert mp.mpgemm_strerror(mp.MPGEMM_ESCRATCH) != "unknown error code"


def test_splitk_launch_checks_the_workspace_before_hip():
    # a shape the plan splits (four 64-row tiles, deep K)
    args = (0, 0, 0, 256, 16, 65536, FAKE_A, 65536, FAKE_B, 16, FAKE_C, 16, 1.0, 0.0, 0, 0)
    assert mp.mpgemm_gemm_splitk(*args, 0, 0, 0) == mp.MPGEMM_ENULL
    assert mp.mpgemm_gemm_splitk(*args, FAKE_C + 0x100000, 1024, 0) == mp.MPGEMM_EWORKSPACE
    assert mp.mpgemm_gemm_splitk(*args, FAKE_C + 0x100002, 1 << 30, 0) == mp.MPGEMM_EALIGN


def test_mfma_rate_probe_rejects_bad_arguments_before_launch():
    ok = (mp.MPGEMM_IN_F16, 16, FAKE_A, 4096, 10, 256, FAKE_C, 256 * 512, 0)

    def call(**kw):
        names = ("in_type", "shape", "ops", "ops_len", "iters", "workgroups", "out", "out_len", "stream")
        args = dict(zip(names, ok))
        args.update(kw)
        return mp.mpgemm_probe_mfma_rate(*(args[n] for n in names))

    assert call(in_type=7) == mp.MPGEMM_ECONFIG
    assert call(shape=8) == mp.MPGEMM_ECONFIG
    assert call(ops=0) == mp.MPGEMM_ENULL
    assert call(out=0) == mp.MPGEMM_ENULL
    assert call(ops_len=4095) == mp.MPGEMM_EDIM
    assert call(out_len=256 * 512 - 1) == mp.MPGEMM_EDIM
    assert call(iters=-1) == mp.MPGEMM_EDIM
    assert call(iters=(1 << 24) + 1) == mp.MPGEMM_EDIM
    assert call(workgroups=0) == mp.MPGEMM_EDIM
    assert call(workgroups=65536) == mp.MPGEMM_EDIM


def test_fill_probe_rejects_bad_arguments_before_launch():
    names = ("mode", "depth", "buf", "buf_bytes", "footprint", "shared", "replicas", "passes", "workgroups",
             "sink", "sink_len", "clocks", "clocks_len", "stream")
    ok = dict(zip(names, (mp.MPGEMM_FILL_LDS16, 8, FAKE_A, 8 << 20, 1 << 20, 0, 1, 4, 256, FAKE_C,
                          256 * 512, FAKE_C, 4 * 256, 0)))

    def call(**kw):
        args = dict(ok)
        args.update(kw)
        return mp.mpgemm_probe_fill(*(args[n] for n in names))

    assert call(mode=3) == mp.MPGEMM_ECONFIG
    assert call(depth=3) == mp.MPGEMM_ECONFIG
    assert call(buf=0) == mp.MPGEMM_ENULL
    assert call(sink=0) == mp.MPGEMM_ENULL
    assert call(buf=FAKE_A + 8) == mp.MPGEMM_EALIGN
    assert call(workgroups=252) == mp.MPGEMM_EDIM          # not a multiple of 8
    assert call(replicas=3) == mp.MPGEMM_EDIM              # does not divide 32 per XCD
    assert call(footprint=(1 << 20) + 1024) == mp.MPGEMM_EDIM
    assert call(footprint=2 << 20) == mp.MPGEMM_EDIM       # 8 distinct regions exceed the buffer
    assert call(buf_bytes=1 << 31, footprint=1 << 20) == mp.MPGEMM_EDIM
    assert call(passes=0) == mp.MPGEMM_EDIM
    assert call(sink_len=256 * 512 - 1) == mp.MPGEMM_EDIM
    assert call(clocks_len=4 * 256 - 1) == mp.MPGEMM_EDIM   # too short for the clock spans


def test_factory_gives_narrow_products_the_narrow_kernel():
    """N <= 16 with A row-major takes the narrow kernel of the call's input
    format and B storage order, one workgroup per 16 rows; N = 17, a
    column-major A, or 16 rows of A past 32-bit offsets take another kind."""
    for N in (1, 2, 8, 15, 16):
        for lb in (0, 1):
            if lb and N == 1:
                continue
            c = ql(0, lb, 1000, N, 617)
            # a packed one-column row-major B is read in its column-major form
            want = 1 if N == 1 else lb
            assert c["kind_name"] == "narrow" and c["layout_b"] == want and c["grid"] == -(-1000 // 16), (N, lb, c)
            assert c["in_type"] == mp.MPGEMM_IN_F16
            c = mp.mpgemm_bf16f32_layout_query(0, lb, 1000, N, 617, FAKE_A, 617, FAKE_B, 617 if lb else N,
                                               FAKE_C, N, 1.0, 0.0)
            assert c["kind_name"] == "narrow" and c["in_type"] == mp.MPGEMM_IN_BF16 and c["layout_b"] == want
    assert ql(0, 0, 1000, 17, 617)["kind_name"] == "pipe"
    assert ql(1, 0, 1000, 16, 617)["kind_name"] != "narrow"
    assert ql(0, 0, 1000, 16, 617, lda=1 << 27)["kind_name"] == "direct"
    assert ql(0, 0, 0, 16, 617)["kind_name"] == "none"
    assert ql(0, 0, 1000, 16, 0)["kind_name"] == "scale"


def test_product_table_holds_what_the_factory_can_choose():
    """Every table entry except the scale-only one is the factory's choice
    for some call (the direct kernels by huge strides, the tile entries by
    shape, the narrow ones by N <= 16), so nothing in the product library is
    unreachable."""
    chosen = set()
    for in_type in (0, 1):
        for la in (0, 1):
            for lb in (0, 1):
                f = mp.mpgemm_bf16f32_layout_query if in_type else mp.mpgemm_f16f32_layout_query
                for M, N, K in [(8192, 8192, 8192), (2048, 2048, 2048), (32768, 128, 4096), (256, 256, 256), (1000, 800, 617),
                                (256, 256, 64), (1000, 16, 617), (300, 300, 64), (200, 300, 400)]:
                    lda = M if la else K
                    ldb = K if lb else N
                    chosen.add(f(la, lb, M, N, K, FAKE_A, lda, FAKE_B, ldb, FAKE_C, N, 1.0, 0.0)["id"])
                chosen.add(f(la, lb, 300, 300, 64, FAKE_A, 1 << 30, FAKE_B, 1 << 30, FAKE_C, 300, 1.0, 0.0)["id"])
    chosen.add(q(64, 64, 0)["id"])
    assert chosen == set(range(mp.mpgemm_num_configs()))


def test_candidates_library_extends_the_product_table():
    """The candidates build (tile sweeps) holds the product entries with the
    same ids and fields, then the sweep-only shapes."""
    path = mp.CANDIDATES_PATH
    if not os.path.exists(path):
        pytest.skip("candidates library not built (python -m dense_mixed_precision_amd.build --candidates)")
    lib = ctypes.CDLL(path)
    lib.mpgemm_num_configs.restype = ctypes.c_int
    lib.mpgemm_config_info.argtypes = [ctypes.c_int, ctypes.POINTER(mp._binding.MpgemmConfig)]
    n = lib.mpgemm_num_configs()
    assert n > mp.mpgemm_num_configs()
    for i in range(n):
        out = mp._binding.MpgemmConfig()
        assert lib.mpgemm_config_info(i, ctypes.byref(out)) == 0
        d = mp._binding._cfg_dict(out)
        if i < mp.mpgemm_num_configs():
            assert d == mp.mpgemm_config_info(i)
        else:
            assert d["id"] == i and d["kind_name"] in ("pipe", "narrow")


# ----------------------------------------------------------------------------
# The tensor binding refuses what the library would misread
# ----------------------------------------------------------------------------

@pytest.fixture
def fake_cuda(monkeypatch):
    """Host tensors pass the binding's is-on-the-GPU checks (there is no GPU
    here), except those tagged ``_host_for_test``; nothing reaches the GPU
    because the library entry points are replaced in each test."""
    import torch
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda t: not getattr(t, "_host_for_test", False)))


def test_binding_refuses_overlapping_rows(fake_cuda):
    import torch
    from dense_mixed_precision_amd import _binding as b

    ok = torch.zeros(8, 16, dtype=torch.float32)
    assert b._check_tensor(ok, "C", torch.float32) == (0, 16)
    # a broadcast C: every row is the same 16 floats
    bcast = torch.zeros(1, 16).expand(4096, 16)
    with pytest.raises(ValueError, match="overlap"):
        b._check_tensor(bcast, "C", torch.float32)
    # overlapping rows of A (stride 4 < 16 columns) and a broadcast column
    over = torch.as_strided(torch.zeros(64, dtype=torch.float16), (8, 16), (4, 1))
    with pytest.raises(ValueError, match="overlap"):
        b._check_tensor(over, "A", torch.float16, allow_col_major=True)
    col = torch.zeros(1, dtype=torch.float16).expand(8, 1)
    with pytest.raises(ValueError, match="overlap"):
        b._check_tensor(col, "B", torch.float16, allow_col_major=True)
    # column-major views: overlapping columns refused, a padded one accepted
    over_t = torch.as_strided(torch.zeros(64, dtype=torch.float16), (16, 8), (1, 4))
    with pytest.raises(ValueError, match="overlap"):
        b._check_tensor(over_t, "A", torch.float16, allow_col_major=True)
    padded_t = torch.zeros(8, 20, dtype=torch.float16)[:, :16].t()
    assert b._check_tensor(padded_t, "A", torch.float16, allow_col_major=True) == (1, 20)


def test_binding_refuses_overlaps_before_the_c_abi(fake_cuda, monkeypatch):
    """gemm() with an expanded C raises before any library call."""
    import torch
    from dense_mixed_precision_amd import _binding as b

    called = []
    monkeypatch.setattr(b, "mpgemm_f16f32", lambda *a: called.append(a) or 0)
    A = torch.zeros(4096, 8, dtype=torch.float16)
    B = torch.zeros(8, 16, dtype=torch.float16)
    C = torch.zeros(1, 16).expand(4096, 16)
    with pytest.raises(ValueError, match="overlap"):
        b.gemm(A, B, C, stream=0)
    assert not called


def test_splitk_binding_checks_the_workspace(fake_cuda, monkeypatch):
    import torch
    from dense_mixed_precision_amd import _binding as b

    called = []
    monkeypatch.setattr(b, "mpgemm_gemm_splitk", lambda *a: called.append(a) or 0)
    monkeypatch.setattr(b, "mpgemm_splitk_plan", lambda *a: {"splits": 4, "workspace_bytes": 4096,
                                                                "config_id": 3})
    A = torch.zeros(64, 256, dtype=torch.float16)
    B = torch.zeros(256, 16, dtype=torch.float16)
    C = torch.zeros(64, 16)
    host = torch.zeros(1024)
    host._host_for_test = True
    with pytest.raises(TypeError, match="GPU"):
        b.gemm_splitk(A, B, C, workspace=host, stream=0)
    with pytest.raises(TypeError, match="float32"):
        b.gemm_splitk(A, B, C, workspace=torch.zeros(2048, dtype=torch.float16), stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        b.gemm_splitk(A, B, C, workspace=torch.zeros(2048)[::2], stream=0)
    assert not called
    b.gemm_splitk(A, B, C, workspace=torch.zeros(1024), stream=0)
    assert len(called) == 1
