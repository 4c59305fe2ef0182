"""Seeded random sweep through the public entry points, every element against
the CPU oracle ("Capstone 4: a tensor-core GEMM", Compare like with like:
every element against the double-precision result).

Each case draws, from its own seed:
* M, N, K: small (1..16), near a tile edge (16..512 plus or minus 2) or
  anywhere up to 640, with M*N*K capped so the oracle's loop stays fast;
* the storage order of A and of B, and FP16 or BF16 inputs;
* alpha (0 included) and beta (0 included; C is NaN-poisoned when beta = 0,
  so a read of C shows);
* leading dimensions padded past the extents, and operands starting 2 bytes
  past an aligned address (no 16-byte vector path then);
* a per-column bias or none;
* the entry point: the factory (through the tensor binding) or split-K with
  the library's plan or a requested number of pieces.
A second sweep forces a random entry of the product table on each case (in
its input format and storage orders; N <= 16 for the narrow kernel, alpha
= 0 for the scale-only kernel), so every kernel variant meets shapes the
factory would not give it.
Every element must meet the acceptance rule and the accumulation diagnostic,
and nothing outside C's window (guards, the ldc gap) may change.  Each case
prints its draw before it runs.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
import oracle
from dense_mixed_precision_amd.workloads import bits, make_inputs
from tests.gpu_util import Guarded, assert_close, device, stored

pytestmark = pytest.mark.gpu

CASES = 600
BASE_SEED = 7300
MAX_MNK = 20_000_000


def _dim(rng):
    r = rng.random()
    if r < 0.25:
        return int(rng.integers(1, 17))
    if r < 0.55:
        edge = int(rng.choice([16, 32, 64, 128, 256, 512]))
        return max(1, edge + int(rng.integers(-2, 3)))
    return int(rng.integers(1, 641))


def draw(idx):
    rng = np.random.default_rng(BASE_SEED + idx)
    M, N, K = _dim(rng), _dim(rng), _dim(rng)
    while M * N * K > MAX_MNK:
        K = max(1, K // 2)
    return dict(
        M=M, N=N, K=K,
        la=int(rng.integers(0, 2)), lb=int(rng.integers(0, 2)),
        fmt=str(rng.choice(["f16", "bf16"])),
        alpha=float(rng.choice([1.0, 1.0, -0.5, 1.5, 0.0])),
        beta=float(rng.choice([0.0, 0.0, 1.0, -0.25])),
        pad_a=int(rng.choice([0, 0, 1, 8, 13])), pad_b=int(rng.choice([0, 0, 1, 8, 13])),
        pad_c=int(rng.choice([0, 0, 3, 16])),
        off_a=int(rng.random() < 0.2), off_b=int(rng.random() < 0.2),
        bias=bool(rng.random() < 0.3),
        splitk=bool(rng.random() < 0.25), splits=int(rng.choice([0, 0, 2, 3, 7])),
        seed=BASE_SEED + idx,
    )


def forced_draw(idx):
    """A case for a random table entry: the entry's input format and storage
    orders; M, N, K >= 2 so the binding reads the storage order from the
    strides; N <= 16 for the narrow kernel; alpha = 0 for the scale kernel."""
    d = draw(FORCED_SEED_OFFSET + idx)
    rng = np.random.default_rng(BASE_SEED + FORCED_SEED_OFFSET + idx)
    cfg = int(rng.integers(0, mp.mpgemm_num_configs()))
    c = mp.mpgemm_config_info(cfg)
    d.update(config=cfg, splitk=False, M=max(d["M"], 2), N=max(d["N"], 2), K=max(d["K"], 2))
    d["fmt"] = "bf16" if c["in_type"] == mp.MPGEMM_IN_BF16 else "f16"
    if c["kind_name"] in ("pipe", "narrow"):
        d["la"], d["lb"] = c["layout_a"], c["layout_b"]
    if c["kind_name"] == "narrow":
        d["N"] = int(rng.integers(2, 17))
    if c["kind_name"] == "scale":
        d["alpha"] = 0.0
    while d["M"] * d["N"] * d["K"] > MAX_MNK:
        d["K"] = max(2, d["K"] // 2)
    return d


FORCED_CASES = 400
FORCED_SEED_OFFSET = 100_000


@pytest.mark.parametrize("idx", range(CASES), ids=lambda i: f"case{i:03d}")
def test_random_case(idx):
    d = draw(idx)
    print(f"[sweep {idx}] {d}", flush=True)
    check(idx, d)


@pytest.mark.parametrize("idx", range(FORCED_CASES), ids=lambda i: f"forced{i:03d}")
def test_random_forced_config(idx):
    d = forced_draw(idx)
    print(f"[forced {idx}] {d}", flush=True)
    check(f"forced {idx}", d)


def check(idx, d):
    M, N, K = d["M"], d["N"], d["K"]
    dtype = torch.bfloat16 if d["fmt"] == "bf16" else torch.float16
    A, B, C = make_inputs(M, N, K, "uniform", seed=d["seed"], c_init="uniform" if d["beta"] != 0 else None,
                          dtype=dtype)
    la, lb = d["la"], d["lb"]
    As, Bs = stored(A, la), stored(B, lb)
    gA = Guarded(As, ld=As.shape[1] + d["pad_a"], offset=d["off_a"])
    gB = Guarded(Bs, ld=Bs.shape[1] + d["pad_b"], offset=d["off_b"])
    if C is None:
        gC = Guarded(torch.zeros((M, N), dtype=torch.float32), ld=N + d["pad_c"], fill=float("nan"))
    else:
        gC = Guarded(C, ld=N + d["pad_c"])
    a_view = gA.view().t() if la else gA.view()
    b_view = gB.view().t() if lb else gB.view()
    bias = None
    bias_d = None
    if d["bias"]:
        g = torch.Generator().manual_seed(d["seed"] + 1)
        bias = (torch.rand(N, generator=g) * 2 - 1).numpy().astype(np.float32)
        bias_d = torch.from_numpy(bias).to(device())
    if d["splitk"]:
        mp.gemm_splitk(a_view, b_view, gC.view(), d["alpha"], d["beta"], bias=bias_d, splits=d["splits"])
    else:
        mp.gemm(a_view, b_view, gC.view(), d["alpha"], d["beta"], bias=bias_d, config=d.get("config"))
    torch.cuda.synchronize()
    got = gC.result()
    assert gC.untouched_outside_window(), f"case {idx}: a write outside C's window"
    ref, absdot = oracle.gemm(bits(As), bits(Bs), None if C is None else C.numpy(), d["alpha"], d["beta"],
                              layout_a=la, layout_b=lb, in_type=d["fmt"], bias=bias)
    assert_close(f"sweep {idx}", got, ref, absdot, K=K, alpha=d["alpha"], beta=d["beta"], C0=C, bias=bias)
