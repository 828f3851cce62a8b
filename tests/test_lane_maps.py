"""The lane maps of the scan backward's channel reduce-scatter, taken from the kernels'
own header (tests/lane_maps_dump.cpp, compiled for the host with hipcc, prints
perm_quarter, perm_xor, perm_partial_lane and chan_partial_lane<V>), checked on a
64-lane wavefront emulated in numpy with DPP's lane semantics.

Permuted order (four states per lane, N = 16, the plain backward): lane l holds channel
l // 4 and, in register r, state 4*Q + (r ^ m) with Q = perm_quarter(l) and
m = perm_xor(l).  Each lane's eight values are (register r, type t) at index 2r + t.  The
reduce-scatter halves across lane ^ 8 (keeping the first four values), across lane ^ 7
(keeping the first two), then swaps the pair across lane ^ 16 (bit 4 clear keeps type 0).
Afterwards the lanes perm_partial_lane(t, n, p) must hold, for p = 0 and 1, the sums of
(type t, state n) over the two halves of the channels.  The documented formulas (below)
are checked against the C++ maps too.

Natural order (chan_reduce_scatter<V>, V = 2, 4, 8): halvings across lane bits 3, 2 (two
bank-masked DPP adds) and 4 (lane swap); the lanes chan_partial_lane<V>(k, p, q) must
hold the partial sums of value k of quad lane q over the channel groups p.
"""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def maps(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available to build the lane-map dump")
    exe = str(tmp_path_factory.mktemp("lanemaps") / "dump")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
                    os.path.join(HERE, "lane_maps_dump.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return json.loads(subprocess.run([exe], check=True, capture_output=True, text=True).stdout)


# the documented formulas of the permuted order (cross-checked against the C++ maps)
def quarter_formula(l):
    return (l & 3) ^ (3 * ((l >> 2) & 1))


def xor_formula(l):
    return ((l >> 2) & 1) | (((l >> 3) & 1) << 1)


def partial_formula(t, n, p):
    m = n & 3
    b2, b3 = m & 1, m >> 1
    q = (n >> 2) ^ (3 * b2)
    return q | (b2 << 2) | (b3 << 3) | (t << 4) | (p << 5)


def test_cpp_maps_match_the_documented_formulas(maps):
    assert maps["quarter"] == [quarter_formula(l) for l in range(64)]
    assert maps["xor"] == [xor_formula(l) for l in range(64)]
    for t, n, p, lane in maps["partial"]:
        assert lane == partial_formula(t, n, p)


def test_every_channel_holds_all_sixteen_states(maps):
    quarter, xm = maps["quarter"], maps["xor"]
    for ch in range(16):
        states = sorted(4 * quarter[4 * ch + q] + (r ^ xm[4 * ch + q])
                        for q in range(4) for r in range(4))
        assert states == list(range(16))


def test_reduce_scatter_leaves_the_channel_sums_where_the_tile_sum_reads_them(maps):
    quarter, xm = maps["quarter"], maps["xor"]
    plane = {(t, n, p): lane for t, n, p, lane in maps["partial"]}

    def state_of(l, r):
        return 4 * quarter[l] + (r ^ xm[l])
    rng = np.random.default_rng(0)
    # value[channel][type][state], integers so that every sum is exact
    value = rng.integers(-1000, 1000, size=(16, 2, 16)).astype(np.int64)
    v = np.zeros((64, 8), dtype=np.int64)
    for l in range(64):
        for r in range(4):
            for t in range(2):
                v[l, 2 * r + t] = value[l >> 2, t, state_of(l, r)]

    def partner(l, mask):  # DPP row_ror:8 and row_half_mirror stay inside a row of 16
        return (l & ~15) | ((l & 15) ^ mask)

    w = v.copy()
    for l in range(64):  # lane ^ 8: keep values 0..3, add the partner's 4..7
        w[l, :4] = v[l, :4] + v[partner(l, 8), 4:8]
    v, w = w, w.copy()
    for l in range(64):  # lane ^ 7: keep values 0, 1, add the partner's 2, 3
        w[l, :2] = v[l, :2] + v[partner(l, 7), 2:4]
    v = w
    out = np.zeros(64, dtype=np.int64)
    for l in range(64):  # lane swap across bit 4: bit clear keeps type 0, set keeps type 1
        if (l >> 4) & 1 == 0:
            out[l] = v[l, 0] + v[l + 16, 0]
        else:
            out[l] = v[l - 16, 1] + v[l, 1]

    seen = set()
    for t in range(2):
        for n in range(16):
            lanes = [plane[(t, n, p)] for p in range(2)]
            seen.update(lanes)
            for p, l in enumerate(lanes):
                assert (l >> 4) & 1 == t and 4 * quarter[l] + xm[l] == n
                chans = [c for c in range(16) if (c >> 3) & 1 == p]
                assert out[l] == value[chans, t, n].sum(), (t, n, p)
            assert out[lanes[0]] + out[lanes[1]] == value[:, t, n].sum()
    assert seen == set(range(64))


@pytest.mark.parametrize("V", [2, 4, 8])
def test_natural_order_reduce_scatter_matches_chan_partial_lane(maps, V):
    rng = np.random.default_rng(V)
    value = rng.integers(-1000, 1000, size=(64, V)).astype(np.int64)  # [lane][value index]

    def row_partner(l, mask):
        return (l & ~15) | ((l & 15) ^ mask)

    def halve(v, bit, half):
        # lanes with the bit clear keep values k < half and add the partner's copy of them,
        # the others keep k + half likewise (dpp_halve: row_ror:8 for bit 3; row_shl:4 /
        # row_shr:4 by bank for bit 2, i.e. the partner lane ^ 4)
        w = v.copy()
        for l in range(64):
            q = row_partner(l, 1 << bit)
            off = half if (l >> bit) & 1 else 0
            for k in range(half):
                w[l, k] = v[l, k + off] + v[q, k + off]
        return w

    v = halve(value, 3, V // 2)
    if V >= 4:
        v = halve(v, 2, V // 4)
    out = v[:, 0].copy()
    if V == 8:  # swap16: bit 4 clear keeps (a, a of lane + 16), set (b of lane - 16, b)
        for l in range(64):
            out[l] = v[l, 0] + v[l + 16, 0] if (l >> 4) & 1 == 0 else v[l - 16, 1] + v[l, 1]
    used = [3, 2, 4][: {2: 1, 4: 2, 8: 3}[V]]
    free = [b for b in range(2, 6) if b not in used]
    lanes = {}
    for k, p, q, lane in maps[f"chan{V}"]:
        lanes[(k, p, q)] = lane
        # the channels summed: those agreeing with the lane in the bits the butterfly left
        chans = [c for c in range(16)
                 if all(((c >> (b - 2)) & 1) == ((lane >> b) & 1) for b in free)]
        assert lane & 3 == q
        assert out[lane] == value[[4 * c + q for c in chans], k].sum(), (V, k, p, q)
    assert sorted(lanes.values()) == list(range(64))
    for k in range(V):
        for q in range(4):
            total = sum(out[lanes[(k, p, q)]] for p in range(16 // V))
            assert total == value[q::4, k].sum()

