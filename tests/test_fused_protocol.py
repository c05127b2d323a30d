"""Host model of the fused decode-batch FFN launch's block protocol.

The fused kernel (launch_ffn_fused in ffn.hip) is one grid: d_ff / 16
columns, min(E, P) + down_rows rows; the first n_active rows are gate/up
blocks (slot s, neuron tile), the rows right after them down units (pair
position q, column block c), the trailing rows empty.  A gate/up block of an
active slot adds one to cnt_e[expert]; a down unit waits until cnt_e of its
pair's expert reaches d_ff / 16, then adds one to cnt_tc[t, c]; the unit
that brings it to top_k combines the token's partials.

This model runs that protocol on the host with the kernel's grid mapping,
dispatching blocks per XCD in id order (round robin over 8 XCDs) with a cap
on resident blocks, random run times, and waiting blocks holding their
slot.  It checks that every wait is eventually satisfied (no deadlock even
with one resident block per XCD), that every counter ends at its target
exactly, that every counter index stays inside the region the workspace
reserves (E + T * (H / 64) + 1 words), and that each (token, column block)
is combined exactly once.  A dispatcher that broke id order could deadlock
the same grid (shown below with a reversed order); the kernel's waits are
time-bounded for that case.
"""
import random

import numpy as np
import pytest

N_XCD = 8


def fused_cols(T, top_k, H):
    P = T * top_k
    if T > 2 and H % 256 == 0 and P * (H // 256) >= 512:
        return 256
    if T > 2 and H % 128 == 0 and P * (H // 128) >= 512:
        return 128
    return 64


def grid(T, E, top_k, d_ff, H, ids):
    """Blocks of the fused launch in linear id order: ("gu", expert), ("down",
    pair, token, column block, expert) or ("none",).  The grid has min(E, P)
    + down_rows rows; the first n_active rows run gate/up, the down units
    follow directly, and the trailing rows are empty."""
    P = T * top_k
    nt = d_ff // 16
    gu_rows = min(E, P)
    sw = fused_cols(T, top_k, H)
    ncb = H // sw
    down_rows = -(-P * ncb // nt)
    active = sorted(set(int(e) for e in ids.ravel()))
    nrows = min(len(active), gu_rows)
    # pairs grouped by expert, then pair id (the router's stable order)
    pairs = sorted(range(P), key=lambda p: (int(ids.ravel()[p]), p))
    blocks = []
    for y in range(gu_rows + down_rows):
        for x in range(nt):
            if y < nrows:
                blocks.append(("gu", active[y]))
            else:
                u = (y - nrows) * nt + x
                if u >= P * ncb:
                    blocks.append(("none",))
                    continue
                q, c = divmod(u, ncb)
                p = pairs[q]
                blocks.append(("down", p, p // top_k, c, int(ids.ravel()[p])))
    return blocks, nt, ncb


def simulate(blocks, T, E, top_k, nt, ncb, H, cap, order=None, seed=0, max_steps=10**6):
    rng = random.Random(seed)
    queues = [[] for _ in range(N_XCD)]
    ids_order = order if order is not None else range(len(blocks))
    for b in ids_order:
        queues[b % N_XCD].append(b)
    cnt_e = np.zeros(E, dtype=np.int64)
    cnt_tc = np.zeros(T * (H // 64), dtype=np.int64)
    region = E + T * (H // 64) + 1
    combined = {}
    resident = [[] for _ in range(N_XCD)]     # [block, remaining work or None while waiting]
    done = 0
    total = len(blocks)
    for step in range(max_steps):
        progress = False
        for x in range(N_XCD):
            while queues[x] and len(resident[x]) < cap:
                b = queues[x].pop(0)
                resident[x].append([b, None])
                progress = True
            keep = []
            for ent in resident[x]:
                b, rem = ent
                kind = blocks[b][0]
                if kind == "down" and rem is None:
                    e = blocks[b][4]
                    if cnt_e[e] < nt:           # still waiting
                        keep.append(ent)
                        continue
                    ent[1] = rem = rng.randint(1, 4)
                    progress = True
                if rem is None:
                    ent[1] = rem = rng.randint(1, 4)
                ent[1] -= 1
                progress = True
                if ent[1] > 0:
                    keep.append(ent)
                    continue
                done += 1
                if kind == "gu" and blocks[b][1] is not None:
                    e = blocks[b][1]
                    assert 0 <= e < region
                    cnt_e[e] += 1
                elif kind == "down":
                    _, p, t, c, e = blocks[b]
                    i = t * ncb + c                    # index inside cnt_tc
                    assert 0 <= E + i < region - 1
                    cnt_tc[i] += 1
                    if cnt_tc[i] == top_k:
                        combined[(t, c)] = combined.get((t, c), 0) + 1
            resident[x] = keep
        if done == total:
            return cnt_e, cnt_tc, combined
        if not progress:
            return None                                    # deadlock
    return None


CASES = [(1, 64, 8, 1024, 2048), (2, 64, 8, 1024, 2048), (4, 64, 8, 1024, 2048),
         (16, 64, 8, 1024, 2048), (8, 128, 8, 768, 2048), (3, 160, 6, 1536, 5120),
         (16, 160, 6, 1536, 5120), (5, 8, 2, 512, 256), (16, 16, 1, 2048, 5120)]


@pytest.mark.parametrize("T,E,top_k,d_ff,H", CASES)
@pytest.mark.parametrize("cap", [1, 4, 64])
def test_protocol_completes_and_counts_exactly(T, E, top_k, d_ff, H, cap):
    rng = np.random.default_rng(T * 1000 + E + cap)
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)])
    blocks, nt, ncb = grid(T, E, top_k, d_ff, H, ids)
    out = simulate(blocks, T, E, top_k, nt, ncb, H, cap, seed=cap)
    assert out is not None, "deadlock under in-order dispatch"
    cnt_e, cnt_tc, combined = out
    active = set(int(e) for e in ids.ravel())
    for e in range(E):
        assert cnt_e[e] == (nt if e in active else 0)
    assert all(cnt_tc[t * ncb + c] == top_k for t in range(T) for c in range(ncb))
    assert combined == {(t, c): 1 for t in range(T) for c in range(ncb)}


def test_reversed_dispatch_can_deadlock():
    # the dependency the kernel relies on: with down units dispatched before
    # the gate/up blocks they wait on and one resident block per XCD, the
    # waiters hold every slot (the kernel's waits give up after a bound)
    T, E, top_k, d_ff, H = 1, 64, 8, 1024, 2048
    ids = np.arange(top_k)[None, :]
    blocks, nt, ncb = grid(T, E, top_k, d_ff, H, ids)
    order = list(range(len(blocks)))[::-1]
    assert simulate(blocks, T, E, top_k, nt, ncb, H, cap=1, order=order, max_steps=5000) is None
