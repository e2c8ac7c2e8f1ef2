"""Host-side model of the bf16 kernel's barrier schedule (no GPU).

The kernel runs two groups of waves offset by one barrier interval; each tile
j has an MFMA phase and a VALU phase per group.  K and V tiles stream from
HBM into two rings of NBUF LDS buffers.  This model enumerates, for every
barrier interval, which tile each group reads, when each tile is requested
and when its requester waits for it, and checks the two properties the
kernel relies on:

1. every LDS read of a tile happens in an interval after the one whose
   closing barrier follows the requester's wait for that tile (group 0 waits
   for K_{j+1} at the end of its MFMA phase j, group 1 for V_j);
2. a buffer is refilled only after every read of its previous tile is done,
   in an earlier interval: a group is four waves (one per SIMD) that are in
   step only at barriers, so a refill requested in the same interval as a
   read of the previous tile can overtake another wave's read.

The per-phase lists mirror the kernel in fa2_fwd_amd/csrc/attn_bf16.hpp (a
change there must be mirrored here); the ring depth NBUF is a build option
there, with AHEAD = NBUF - 1 tiles requested ahead, and both depths the
kernel is built with are checked.
"""

import pytest

RINGS = [(4, 3), (5, 4)]  # (NBUF, AHEAD)


def intervals(group, phase, j):
    """Barrier interval of group `group`'s `phase` ("mfma"/"valu") of tile j."""
    base = 2 * j + group
    return base if phase == "mfma" else base + 1


def build_events(ntiles, AHEAD):
    reads = []      # (interval, stream, tile)
    requests = []   # (interval, stream, tile)
    waits = []      # (interval, stream, tile): requester's wait completes this tile
    streams = {0: "K", 1: "V"}
    for g in (0, 1):
        s = streams[g]
        # prologue (interval -1): request tiles 0..AHEAD-1; group 0 waits for K_0
        for t in range(min(AHEAD, ntiles)):
            requests.append((-1, s, t))
        if g == 0:
            waits.append((-1, s, 0))
        for j in range(ntiles):
            mi = intervals(g, "mfma", j)
            vi = intervals(g, "valu", j)
            # MFMA phase j: K_j; V_{j-1} for j >= 1 (tile 0 reads its own K operands)
            reads.append((mi, "K", j))
            if j >= 1:
                reads.append((mi, "V", j - 1))
            # end of MFMA phase j: group 0 waits for K_{j+1}, group 1 for V_j
            need = j + 1 if g == 0 else j
            for t in range(0, min(need, ntiles - 1) + 1):
                waits.append((mi, s, t))
            # VALU phase j: K operands of MFMA phase j+1 read ahead, request of tile j+AHEAD
            if j + 1 < ntiles:
                reads.append((vi, "K", j + 1))
            if j + AHEAD < ntiles:
                requests.append((vi, s, j + AHEAD))
        # final P V of the last tile, in the slot of MFMA phase ntiles
        reads.append((intervals(g, "mfma", ntiles), "V", ntiles - 1))
    return reads, requests, waits


@pytest.mark.parametrize("ring", RINGS)
@pytest.mark.parametrize("ntiles", list(range(1, 14)))
def test_reads_after_completion_and_no_early_refill(ntiles, ring):
    NBUF, AHEAD = ring
    reads, requests, waits = build_events(ntiles, AHEAD)
    first_wait = {}
    for i, s, t in waits:
        first_wait[(s, t)] = min(first_wait.get((s, t), i), i)
    req = {(s, t): i for i, s, t in requests}
    # every tile that is read was requested
    for i, s, t in reads:
        assert (s, t) in req, f"{s}{t} read but never requested"
        # 1. completed by a wait in an earlier interval (the barrier closing it publishes the tile)
        assert (s, t) in first_wait and first_wait[(s, t)] < i, \
            f"{s}{t} read in interval {i} but completed only in {first_wait.get((s, t))}"
        assert req[(s, t)] <= first_wait[(s, t)]
    # 2. a refill of buffer t % NBUF is requested after the last read of tile t - NBUF
    last_read = {}
    for i, s, t in reads:
        last_read[(s, t)] = max(last_read.get((s, t), i), i)
    for i, s, t in requests:
        prev = t - NBUF
        if prev >= 0:
            assert last_read.get((s, prev), -9) < i, \
                f"{s}{t} requested in interval {i} while {s}{prev} is read in {last_read[(s, prev)]}"


@pytest.mark.parametrize("ring", RINGS)
def test_wait_counts_within_spelled_out_cases(ring):
    # the kernel spells out waits with at most min(AHEAD - 1, 3) newer tiles
    # of the group's own stream in flight
    _, AHEAD = ring
    for ntiles in range(1, 14):
        for j in range(-1, ntiles):
            if j < 0:
                checks = [(AHEAD - 1, 0)]  # prologue, group 0: K_0
            else:
                newest = j - 1 + AHEAD  # requested by the end of MFMA phase j
                checks = [(newest, j + 1), (newest, j)]
            for newest, need in checks:
                after = min(newest, ntiles - 1) - need
                assert after <= min(AHEAD - 1, 3)


# ---- the 128-row 4-wave kernel (attn_bf16_solo.hpp): one barrier per step.
# Step j: each wave waits for its own requests of tile j (at most the
# requests of tile j + 1 may stay in flight), barrier, then requests tile
# j + AHEAD (K into slot (j + AHEAD) % NBUF_K, V into slot (j + AHEAD) %
# NBUF_V), reads K_j for the scores and V_{j-1} for the output products of
# the previous tile; V_{ntiles-1} is read after the last step.
SOLO_NBUF_K, SOLO_NBUF_V, SOLO_AHEAD = 3, 4, 2


def solo_events(ntiles):
    requested = {t: -1 for t in range(min(SOLO_AHEAD, ntiles))}  # tile -> step (-1: prologue)
    reads = []  # (step, tensor, tile); step ntiles = after the loop
    in_flight = {}
    for j in range(ntiles):
        in_flight[j] = len([t for t in requested if t > j])
        if j + SOLO_AHEAD < ntiles:
            requested[j + SOLO_AHEAD] = j
        reads.append((j, "K", j))
        if j > 0:
            reads.append((j, "V", j - 1))
    reads.append((ntiles, "V", ntiles - 1))
    return requested, reads, in_flight


@pytest.mark.parametrize("ntiles", range(1, 12))
def test_solo_ring(ntiles):
    requested, reads, in_flight = solo_events(ntiles)
    assert sorted(requested) == list(range(ntiles))
    for j in range(ntiles):
        # the kernel lets exactly one newer tile stay in flight (none on the last step)
        assert in_flight[j] == (0 if j == ntiles - 1 else 1)
    for step, tensor, tile in reads:
        # complete by the wait of step `tile`, whose barrier precedes the read
        assert tile <= step and (requested[tile] < tile or requested[tile] == -1)
    for t, step in requested.items():
        if step < 0:
            continue
        for tensor, depth in (("K", SOLO_NBUF_K), ("V", SOLO_NBUF_V)):
            # the slot's previous tile is last read before this step's barrier,
            # and no read in this step uses the slot being refilled
            prev = t - depth
            if prev >= 0:
                assert all(r_step < step for r_step, r_tensor, r_tile in reads if r_tensor == tensor and r_tile == prev)
            assert all(r_tile % depth != t % depth for r_step, r_tensor, r_tile in reads
                       if r_step == step and r_tensor == tensor)
