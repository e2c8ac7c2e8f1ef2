"""Host-side model of the bf16 kernel's barrier schedule (no GPU).

The kernel runs two groups of waves offset by one barrier interval; each tile
j has an MFMA phase and a VALU phase per group.  K and V tiles stream from
HBM into two rings of NBUF LDS buffers.  This model enumerates, for every
barrier interval, which tile each group reads, when each tile is requested
and when its requester waits for it, and checks the two properties the
kernel relies on:

1. every LDS read of a tile happens in an interval after the one whose
   closing barrier follows the requester's wait for that tile;
2. a buffer is refilled only after every read of its previous tile is done.

The constants and the per-phase lists mirror the kernel in
fa2_fwd_amd/csrc/attn_bf16.hpp; a change there must be mirrored here.
"""

import pytest

NBUF = 4
AHEAD = 3


def intervals(group, phase, j):
    """Barrier interval of group `group`'s `phase` ("mfma"/"valu") of tile j."""
    base = 2 * j + group
    return base if phase == "mfma" else base + 1


def build_events(ntiles):
    reads = []      # (interval, stream, tile)
    requests = []   # (interval, stream, tile)
    waits = []      # (interval, stream, tile): requester's wait completes this tile
    streams = {0: "K", 1: "V"}
    for g in (0, 1):
        s = streams[g]
        # prologue (interval -1): request tiles 0..AHEAD-1, wait K_0..K_1 / V_0
        for t in range(min(AHEAD, ntiles)):
            requests.append((-1, s, t))
        for t in (range(0, 2) if g == 0 else range(0, 1)):
            if t < ntiles:
                waits.append((-1, s, t))
        for j in range(ntiles):
            mi = intervals(g, "mfma", j)
            vi = intervals(g, "valu", j)
            # MFMA phase j: K_j; V_{j-1} for j >= 1 (tile 0 prefetches its own K operands)
            reads.append((mi, "K", j))
            if j >= 1:
                reads.append((mi, "V", j - 1))
            # VALU phase j: prefetch of MFMA phase j+1 operands, request, wait
            if j + 1 < ntiles:
                reads.append((vi, "K", j + 1))
                reads.append((vi, "V", j))
            if j + AHEAD < ntiles:
                requests.append((vi, s, j + AHEAD))
            need = j + 2 if g == 0 else j + 1
            for t in range(0, min(need, ntiles - 1) + 1):
                waits.append((vi, s, t))
        # final P V of the last tile, in the slot of MFMA phase ntiles
        reads.append((intervals(g, "mfma", ntiles), "V", ntiles - 1))
    return reads, requests, waits


@pytest.mark.parametrize("ntiles", list(range(1, 14)))
def test_reads_after_completion_and_no_early_refill(ntiles):
    reads, requests, waits = build_events(ntiles)
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


def test_wait_counts_within_vmcnt_encoding():
    # the kernel waits with at most two newer tiles in flight (vmcnt(2*LD))
    for ntiles in range(1, 14):
        for j in range(ntiles):
            for g, need in ((0, j + 2), (1, j + 1)):
                after = min(j + AHEAD, ntiles - 1) - need
                assert after <= 2
