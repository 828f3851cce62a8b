"""Host model of the permuted state order of the scan backward's channel reduce-scatter
(four states per lane, N = 16), checked on a 64-lane wavefront emulated in numpy.

Lane l holds channel l // 4 and, in register r, state 4*Q + (r ^ m) with
Q = (l & 3) ^ 3*b2 and m = 2*b3 + b2 (b2, b3 = lane bits 2, 3).  Each lane's eight values
are (register r, type t) at index 2r + t.  The reduce-scatter halves across lane ^ 8
(keeping the first four values), across lane ^ 7 (keeping the first two), then swaps the
pair across lane ^ 16 (bit 4 clear keeps type 0).  Afterwards lane l must hold, for
type t = bit 4 of l and state n = 4*Q + m, the sum over the 8 channels that agree with
its channel in channel bit 3 (lane bit 5); the two partials of (t, n) sit at the lanes
the kernel's post-tile sum reads.
"""
import numpy as np


def quarter(l):
    return (l & 3) ^ (3 * ((l >> 2) & 1))


def xor_m(l):
    return ((l >> 2) & 1) | (((l >> 3) & 1) << 1)


def state_of(l, r):
    return 4 * quarter(l) + (r ^ xor_m(l))


def partial_lane(t, n, p):
    m = n & 3
    b2, b3 = m & 1, m >> 1
    q = (n >> 2) ^ (3 * b2)
    return q | (b2 << 2) | (b3 << 3) | (t << 4) | (p << 5)


def test_every_channel_holds_all_sixteen_states():
    for ch in range(16):
        states = sorted(state_of(4 * ch + q, r) for q in range(4) for r in range(4))
        assert states == list(range(16))


def test_reduce_scatter_leaves_the_channel_sums_where_the_tile_sum_reads_them():
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
            lanes = [partial_lane(t, n, p) for p in range(2)]
            seen.update(lanes)
            for p, l in enumerate(lanes):
                assert (l >> 4) & 1 == t and 4 * quarter(l) + xor_m(l) == n
                chans = [c for c in range(16) if (c >> 3) & 1 == p]
                assert out[l] == value[chans, t, n].sum(), (t, n, p)
            assert out[lanes[0]] + out[lanes[1]] == value[:, t, n].sum()
    assert seen == set(range(64))
