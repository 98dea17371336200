"""Host-thread model of the single-pass forward's statistics exchange
(csrc/sa_fused_bf16.hip), run on the CPU.

Each thread plays one workgroup: chunk c of a token segment.  It walks the
segment's 32-token tiles (cut at user boundaries) in the kernel's order:
  prologue:  publish tiles 0 and 1, read back tile 0;
  step t:    publish tile t + 2 (if any), read back tile t + 1 (if any),
             aggregate tile t.
A read-back waits until every chunk's word for each row of the tile is
there (ready bit), up to a wait budget; past it the thread stops waiting for
good and flags the exchange status.  Words live in one zeroed array,
[nchunks][T], indexed by (chunk, token), as in the kernel.

Checked: no deadlock under random delays (every thread finishes), every word
is written once, every read-back sees all chunks' words of its tile, all
indices stay inside the array, and a partner that stops publishing makes the
others time out, flag the status and still finish.
"""

import random
import threading
import time

import numpy as np
import pytest

TILE = 32


def seg_lo(T, G, s):
    return (T * s) // G


def tiles(offsets, lo, hi):
    """The kernel's tile walk of segment [lo, hi): 32-token tiles, cut at
    user boundaries, in token order.  Returns [(t0, t1, user)]."""
    out = []
    B = len(offsets) - 1
    t0 = lo
    while t0 < hi:
        u = int(np.searchsorted(offsets[1:], t0, side="right"))   # first user with end > t0
        u = min(u, B - 1)
        piece_end = min(int(offsets[u + 1]), hi)
        t1 = min(t0 + TILE, piece_end)
        out.append((t0, t1, u))
        t0 = t1
    return out


class Exchange:
    def __init__(self, nchunks, T):
        self.words = np.zeros(nchunks * T, dtype=np.uint64)
        self.writes = np.zeros(nchunks * T, dtype=np.int64)
        self.T = T
        self.lock = threading.Lock()
        self.status_timeout = False

    def publish(self, c, t0, t1):
        for r in range(t0, t1):
            i = c * self.T + r
            assert 0 <= i < self.words.size
            with self.lock:
                self.words[i] = (1 << 32) | (r & 0xFFFF)
                self.writes[i] += 1

    def ready(self, c, r):
        i = c * self.T + r
        assert 0 <= i < self.words.size
        return int(self.words[i]) >> 32 == 1


def workgroup(ex, nchunks, c, tl, budget_s, rng, stop_after=None, failed_box=None):
    failed = False

    def delay():
        if rng.random() < 0.3:
            time.sleep(rng.random() * 2e-4)

    def publish(j):
        if stop_after is not None and j >= stop_after:
            return                         # a partner that stops publishing
        ex.publish(c, tl[j][0], tl[j][1])

    def gather(j):
        nonlocal failed
        t0, t1, _ = tl[j]
        start = None
        while True:
            ok = all(ex.ready(cc, r) for cc in range(nchunks) for r in range(t0, t1))
            if ok or failed:
                return ok
            now = time.perf_counter()
            if start is None:
                start = now
            elif now - start > budget_s:
                failed = True
                ex.status_timeout = True
                return False
            time.sleep(1e-5)

    n = len(tl)
    publish(0)
    if n > 1:
        publish(1)
    seen = [gather(0)]
    for t in range(n):
        delay()
        if t + 2 < n:
            publish(t + 2)
        if t + 1 < n:
            seen.append(gather(t + 1))
        delay()
    if failed_box is not None:
        failed_box[c] = failed
    return seen


def run_model(lengths, nchunks, G, budget_s=2.0, seed=0, stop=None):
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offsets[-1])
    G = min(G, T)
    ex = Exchange(nchunks, T)
    results, threads, fails = {}, [], {}
    for s in range(G):
        tl = tiles(offsets, seg_lo(T, G, s), seg_lo(T, G, s + 1))
        assert tl, "every segment holds at least one token"
        boxes = {}
        fails[s] = boxes
        for c in range(nchunks):
            rng = random.Random(seed * 7919 + s * 31 + c)
            stop_after = stop[1] if (stop is not None and stop[0] == (s, c)) else None

            def body(c=c, tl=tl, rng=rng, stop_after=stop_after, s=s, boxes=boxes):
                results[(s, c)] = workgroup(ex, nchunks, c, tl, budget_s, rng, stop_after, boxes)

            th = threading.Thread(target=body, daemon=True)
            threads.append(th)
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
        assert not th.is_alive(), "a workgroup never finished (deadlock)"
    return offsets, T, ex, results, fails


@pytest.mark.parametrize("lengths,nchunks,G", [
    ([1000], 4, 8),                       # one user, k = 1024
    ([0, 31, 33, 0, 64, 65, 500, 1], 4, 6),   # ragged, empty users, ragged tails
    ([700, 2, 300], 2, 16),               # k = 512
    ([5, 5, 5], 8, 3),                    # k = 2048, one tile per segment
    ([3], 1, 3),                          # more segments than tokens: G = T
])
def test_exchange_completes_and_every_word_is_written_once(lengths, nchunks, G):
    offsets, T, ex, results, _ = run_model(lengths, nchunks, G, seed=len(lengths))
    assert not ex.status_timeout
    assert np.all(ex.writes == 1), "every (chunk, token) word is written exactly once"
    for key, seen in results.items():
        assert all(seen), f"workgroup {key} read back an incomplete tile"


def test_a_silent_partner_makes_the_others_time_out_and_finish():
    # chunk 2 of segment 1 stops publishing after its third tile
    offsets, T, ex, results, fails = run_model([2000], 4, 4, budget_s=0.05, seed=3,
                                               stop=((1, 2), 3))
    assert ex.status_timeout
    assert any(fails[1].values()), "segment 1's workgroups flagged the timeout"
    # the other segments never waited on the silent partner
    for s in (0, 2, 3):
        assert not any(fails[s].values())
        for c in range(4):
            assert all(results[(s, c)])


def test_tile_walk_covers_each_segment_exactly():
    rng = np.random.default_rng(0)
    lengths = rng.integers(0, 300, size=40)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offsets[-1])
    G = 37
    covered = np.zeros(T, dtype=int)
    for s in range(G):
        for t0, t1, u in tiles(offsets, seg_lo(T, G, s), seg_lo(T, G, s + 1)):
            assert 0 < t1 - t0 <= TILE
            assert offsets[u] <= t0 and t1 <= offsets[u + 1], "a tile never straddles two users"
            covered[t0:t1] += 1
    assert np.all(covered == 1)
