"""CPU model of the pipelined kernel's LDS ring protocol (no GPU needed).

The pipelined kernel (`gemm_pipe` in csrc/kernels.hpp) keeps STAGES K tiles
in an LDS ring.  Its copies into LDS are issued through inline assembly, so
the compiler does not track them: the kernel itself waits on the vector
memory counter (`s_waitcnt vmcnt(n)`: at most n of this wave's vector memory
operations still outstanding; they complete in issue order) before the
barrier that publishes a tile, and it starts refilling a buffer right after
the barrier that follows the last read of the tile in it.

This model replays the kernel's schedule for one wave (every wave of a
workgroup runs the same schedule; a barrier orders everything before it in
every wave before everything after it) and checks, for every table entry,
every K-tile count up to a few times the ring depth, with and without a
register fill of partial vectors on every tile and with and without early
K-tail loads:

* when a tile is published, every copy of it has completed and all of its
  copy positions were issued;
* every operand read of a tile comes after the barrier that published it
  and reads the buffer that tile was copied into;
* no copy or fill store into a buffer is issued before a barrier that
  follows every read of the tile previously held there;
* every wait count fits the 6-bit counter.

The per-config quantities (copies per wave, waits per tile, copy window)
are computed from the library's own config table with the kernel's
formulas.  Planted mistakes (a wait one too loose, copies started before the
barrier, a window too wide for the k-steps) must each make the model fail.
"""
from collections import deque

import pytest

import dense_mixed_precision_amd as mp


def params(c):
    """Schedule constants of a pipelined table entry, as the kernel derives them."""
    MI = c["mfma_m"]
    KD = 16 if MI == 32 else 32
    S = c["stages"]
    KS = c["bk"] // KD
    KG = c["k_groups"]
    KSL = KS // KG
    FM = c["wave_m"] // MI
    NW = c["waves_m"] * c["waves_n"] * KG

    def pw(BX, k_contig):
        rows = BX if k_contig else c["bk"]
        rowb = 2 * (c["bk"] if k_contig else BX)
        ch = rowb // 16
        rpi = 64 // ch
        return rows // rpi // NW

    APW = pw(c["bm"], c["layout_a"] == mp.MPGEMM_ROW_MAJOR)
    BPW = pw(c["bn"], c["layout_b"] == mp.MPGEMM_COL_MAJOR)
    NCOPY = APW + BPW
    NL = APW + BPW
    if S == 2:
        W = (max(NCOPY, 1) if NCOPY < KSL * FM else KSL * FM)
    else:
        W = KSL * FM
    return dict(S=S, KSL=KSL, FM=FM, APW=APW, BPW=BPW, NCOPY=NCOPY, NL=NL, W=W, roll_a=MI == 16)


def wait_count(p, newer):
    """The immediate of the wait in publish() for `newer` younger tiles."""
    S, NL = p["S"], p["NL"]
    if newer <= 0:
        return 0
    if newer == 1:
        return NL
    if newer == 2:
        return (2 if S > 2 else 1) * NL
    if newer == 3:
        return (3 if S > 3 else 1) * NL
    return (4 if S > 4 else 1) * NL


def simulate(p, num_k, fill_every, tail_early, wait_slack=0, copy_before_barrier=False, window_extra=0):
    S, KSL, FM, NCOPY, APW = p["S"], p["KSL"], p["FM"], p["NCOPY"], p["APW"]
    W = p["W"] + window_extra
    q = deque()          # this wave's outstanding vector memory operations, oldest first
    events = []          # program order: ("read"|"copy"|"fillstore", tile, buf) or ("barrier",)
    calls = {}           # copy positions issued per tile
    buf_tile = [None] * S
    published = set()
    cur = {"t": None, "b": None, "live": False}

    def wait(n):
        assert 0 <= n < 64, f"vmcnt {n} does not fit 6 bits"
        while len(q) > n:
            q.popleft()

    def begin_copies(t, b):
        if cur["live"]:
            assert calls[cur["t"]] == NCOPY, f"tile {cur['t']}: copy window left {NCOPY - calls[cur['t']]} copies"
        live = t < num_k
        cur.update(t=t, b=b, live=live)
        if live:
            calls[t] = 0
            buf_tile[b] = t

    def copy_one(c):
        if not cur["live"]:
            return
        t, b = cur["t"], cur["b"]
        assert c < NCOPY
        calls[t] += 1
        events.append(("copy", t, b))
        q.append(("copy", t))

    def copy_slice(pos):
        for c in range(NCOPY):
            if -(-pos * NCOPY // W) <= c < -(-(pos + 1) * NCOPY // W):
                copy_one(c)

    def publish(t, b, newer):
        if fill_every:
            wait(0)
            events.append(("fillstore", t, b))
        else:
            wait(max(0, wait_count(p, newer) + wait_slack))
        assert not any(op[0] == "copy" and op[1] == t for op in q), f"tile {t} published before it landed"
        assert calls.get(t) == NCOPY, f"tile {t} published with {calls.get(t)} of {NCOPY} copies issued"
        events.append(("barrier",))
        published.add(t)

    def read(t, b):
        assert t in published, f"tile {t} read before it was published"
        assert buf_tile[b] == t, f"buffer {b} holds tile {buf_tile[b]}, read as tile {t}"
        events.append(("read", t, b))

    if tail_early:
        q.append(("tail",))
    if num_k > 0:
        for t in range(S):
            begin_copies(t, t)
            for c in range(NCOPY):
                copy_one(c)
        publish(0, 0, min(num_k - 1, S - 1))
        for _ in range(FM):
            read(0, 0)
    buf = 0
    for kt in range(num_k):
        nbuf = 0 if buf + 1 == S else buf + 1
        for ks in range(KSL):
            last = ks + 1 == KSL
            if copy_before_barrier and last:
                begin_copies(kt + S, buf)
                copy_slice(0)
            if last and kt + 1 < num_k:
                publish(kt + 1, nbuf, min(num_k - 2 - kt, S - 2))
            if last and not copy_before_barrier:
                begin_copies(kt + S, buf)
            # operand reads of the next k-step (B only when A rolls)
            for _ in range(FM):
                if not last:
                    read(kt, buf)
                elif kt + 1 < num_k:
                    read(kt + 1, nbuf)
            for grp in range(FM):
                if p["roll_a"]:
                    if not last:
                        read(kt, buf)
                    elif kt + 1 < num_k:
                        read(kt + 1, nbuf)
                if last:
                    if not (copy_before_barrier and grp == 0):
                        copy_slice(grp)
                elif kt > 0:
                    copy_slice(FM + ks * FM + grp)
        buf = nbuf
    if cur["live"]:
        assert calls[cur["t"]] == NCOPY

    # a buffer is refilled only after a barrier that follows every read of
    # the tile it held before
    last_read = {}
    last_barrier = -1
    for i, e in enumerate(events):
        if e[0] == "barrier":
            last_barrier = i
        elif e[0] == "read":
            last_read[(e[1], e[2])] = i
        elif e[0] in ("copy", "fillstore"):
            prev = (e[1] - S, e[2])
            if prev in last_read:
                assert last_read[prev] < last_barrier, \
                    f"{e[0]} of tile {e[1]} into buffer {e[2]} before every wave finished reading tile {prev[0]}"


def _pipe_configs():
    return [mp.mpgemm_config_info(i) for i in range(mp.mpgemm_num_configs())
            if mp.mpgemm_config_info(i)["kind_name"] == "pipe"]


@pytest.mark.parametrize("cid", [c["id"] for c in _pipe_configs()])
def test_ring_protocol_every_pipe_config(cid):
    p = params(mp.mpgemm_config_info(cid))
    assert p["NL"] * (p["S"] - 1) < 64
    for num_k in range(1, 3 * p["S"] + 4):
        for fill_every in (False, True):
            for tail in (False, True):
                simulate(p, num_k, fill_every, tail)


def _deep_config():
    # a three-stage entry
    for c in _pipe_configs():
        if c["stages"] == 3:
            return params(c)
    raise AssertionError("no three-stage entry")


def test_model_rejects_a_wait_one_too_loose():
    p = _deep_config()
    simulate(p, 6, False, False)
    with pytest.raises(AssertionError, match="published before it landed"):
        simulate(p, 6, False, False, wait_slack=1)


def test_model_rejects_copies_before_the_barrier():
    p = _deep_config()
    with pytest.raises(AssertionError, match="before every wave finished reading"):
        simulate(p, 6, False, False, copy_before_barrier=True)


def test_model_rejects_a_window_wider_than_the_k_steps():
    p = _deep_config()
    with pytest.raises(AssertionError, match="copy window left|published with|published before it landed"):
        simulate(p, 8, False, False, window_extra=p["W"])   # twice as wide
