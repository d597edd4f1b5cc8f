"""Host logic of the simulated ring (no GPU): critical path, overlapped
communication, block sizes and the projection, checked on small hand-made
time tables whose answers follow from the definitions."""

import pytest

from striped_ring_attention_amd import ring_sim


def test_critical_path_takes_slowest_device_per_round():
    t = [[1.0, 3.0, 2.0], [4.0, 1.0, 1.0], [2.0, 2.0, 2.0]]   # t[round][device]
    assert ring_sim.critical_path(t) == 3.0 + 4.0 + 2.0
    assert ring_sim.mean_path(t) == pytest.approx(2.0 + 2.0 + 2.0)


def test_ring_time_overlaps_transfer_with_compute():
    t = [[1.0, 3.0], [0.5, 0.25]]
    assert ring_sim.ring_time(t, 0.0) == 3.5
    assert ring_sim.ring_time(t, 1.0) == 3.0 + 1.0      # second round waits for its transfer
    assert ring_sim.ring_time(t, 10.0) == 20.0


def test_kv_block_bytes():
    # K and V of one device: 2 tensors x (S/N rows) x H x D x 2 bytes
    assert ring_sim.kv_block_bytes(1, 8192, 16, 128, 8) == 2 * 1024 * 16 * 128 * 2
    assert ring_sim.kv_block_bytes(2, 300, 3, 64, 3, elem_bytes=4) == 2 * 2 * 100 * 3 * 64 * 4


def test_project_balanced_vs_triangular():
    """Contiguous causal work per round is triangular-like (one device busy,
    the rest partly idle); striped is flat with the same total. The projected
    compute-bound speedup is the ratio of sums of per-round maxima."""
    n = 4
    contig = [[1.0 if d >= r else 0.0 for d in range(n)] for r in range(n)]
    total = sum(map(sum, contig))
    striped = [[total / (n * n)] * n for _ in range(n)]
    p = ring_sim.project(striped, contig, block_bytes=0)
    assert p["t_comm_ms"] == 0.0
    assert p["contiguous"]["critical_path_ms"] == n * 1.0
    assert p["striped"]["critical_path_ms"] == pytest.approx(total / n)
    assert p["speedup_compute_bound"] == pytest.approx(n / (total / n))
    assert p["striped"]["round_max_over_mean"] == [pytest.approx(1.0)] * n
    # a transfer slower than every round makes both layouts transfer-bound
    slow = ring_sim.project(striped, contig, block_bytes=int(153e9 * 5e-3))   # 5 ms per hop at 153 GB/s
    assert slow["speedup_with_comm"] == pytest.approx(1.0)


def test_prefetch_time_waits_only_for_blocks_not_yet_in():
    """Direct-link prefetch: round r starts when round r-1 has ended and its
    block has arrived after ceil(r / links) transfers; worked by hand."""
    t = [[1.0], [1.0], [1.0]]          # three rounds of 1 ms, one device
    # two links: blocks 1 and 2 both arrive at 2 ms -> rounds on [0,1], [2,3], [3,4]
    assert ring_sim.prefetch_time(t, 2.0, links=2) == 4.0
    # one link: block 1 at 2 ms, block 2 at 4 ms -> [0,1], [2,3], [4,5]
    assert ring_sim.prefetch_time(t, 2.0, links=1) == 5.0
    # transfers shorter than a round are hidden entirely
    assert ring_sim.prefetch_time(t, 0.5, links=1) == ring_sim.critical_path(t)
    # the plain ring charges the slower of compute and transfer in every round
    assert ring_sim.ring_time(t, 2.0) == 6.0


def test_project_reports_prefetch_model():
    n = 4
    contig = [[1.0 if d >= r else 0.0 for d in range(n)] for r in range(n)]
    striped = [[10.0 / 16] * n for _ in range(n)]
    # 2 ms per hop: a plain ring is transfer-bound in both layouts, the direct
    # links (3 for 4 devices) deliver every block by 2 ms
    p = ring_sim.project(striped, contig, block_bytes=int(153e9 * 2e-3), links=3)
    assert p["direct_links"] == 3
    assert p["speedup_with_comm"] == pytest.approx(1.0)
    assert p["contiguous"]["prefetch_ms"] == pytest.approx(2.0 + 3 * 1.0)
    assert p["striped"]["prefetch_ms"] == pytest.approx(2.0 + 3 * 10.0 / 16)
    assert p["speedup_with_prefetch"] == pytest.approx(5.0 / (2.0 + 30.0 / 16))
