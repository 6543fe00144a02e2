"""The unit schedule the routed attention call writes into its workspace,
read back and compared entry by entry with a host re-statement of its rules:
each XCD takes a contiguous range of (head, pair) ids; a pair is the rows of
ranks 2 pr and 2 pr + 1 of its head ordered by route length (longest first,
ties by row); a unit costs its longer row's tile count; the units of an XCD
go longest first (ties by unit index) to slots slot * 8 + x. With split rows
a pair of cost c is cut into min(max(ceil(c / tau), 1), n_split) ranges, tau
the smallest value for which the XCD's ranges fit one round of its 32 CUs
(never fewer than one range per pair), a range's size being ceil(c / n); the
slots left over are empty, and the ranges a pair leaves unused carry
(max, sum) = (-inf, 0) for the merge. The outputs of such a call are checked
elsewhere; this pins the schedule itself, which decides its speed."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import synth
from gpu_common import run_path, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
XCD, CUS = 8, 32


def xcd_range(x, n):
    q, r = divmod(n, XCD)
    return x * q + min(x, r), q + (1 if x < r else 0)


def pairs_of(lens, N):
    """per head: [(longer row, other row or -1)] by rank"""
    out = []
    for h in range(lens.shape[0]):
        order = sorted(range(N), key=lambda i: (-int(lens[h, i]), i))
        out.append([(order[2 * k], order[2 * k + 1] if 2 * k + 1 < N else -1) for k in range((N + 1) // 2)])
    return out


def expected_plan(lens, N, n_split):
    H = lens.shape[0]
    pairs = (N + 1) // 2
    P = H * pairs
    prs = pairs_of(lens, N)
    slots = (P + XCD - 1) // XCD * n_split if n_split > 1 else None
    plan, unused = {}, []
    for x in range(XCD):
        base, cnt = xcd_range(x, P)
        units = []   # (size, unit index, entry)
        if n_split == 1:
            for w in range(cnt):
                h, pr = divmod(base + w, pairs)
                a, b = prs[h][pr]
                units.append((int(lens[h, a]) + N, w, (h, a, b, 1 << 8)))
        else:
            cost = []
            for w in range(cnt):
                h, pr = divmod(base + w, pairs)
                a, b = prs[h][pr]
                cost.append(int(lens[h, a]) + N)
            umax = max(cnt, min(CUS, cnt * n_split))
            nr = lambda c, tau: min(max(-(-c // tau), 1), n_split)
            tau = next(t for t in range(1, max(cost + [1]) + 1) if sum(nr(c, t) for c in cost) <= umax)
            u = 0
            for w in range(cnt):
                h, pr = divmod(base + w, pairs)
                a, b = prs[h][pr]
                n = nr(cost[w], tau)
                for r in range(n):
                    units.append((-(-cost[w] // n), u, (h, a, b, r | (n << 8))))
                    u += 1
                for r in range(n, n_split):
                    unused.append((r, h, a, b))
        units.sort(key=lambda t: (-t[0], t[1]))
        for slot, (_, _, e) in enumerate(units):
            plan[slot * XCD + x] = e
        if slots is not None:
            for slot in range(len(units), slots):
                plan[slot * XCD + x] = (-1, -1, -1, 0)
    return plan, unused


@pytest.mark.parametrize("heads,n_split", [(40, 1), (5, 4), (5, 16), (3, 7)])
def test_unit_plan_matches_its_rules(heads, n_split):
    wl = synth.chunk48(heads=heads) if heads != 40 else synth.chunk48()
    say(f"unit plan: chunk48 x {heads} heads, n_split={n_split}")
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v)
    H, N = wl.H, wl.N
    lens = r["lens"].cpu().numpy()
    if n_split == 1:
        ws = velox.attn_workspace(q, r["ids"].shape[-1])
        ws.fill_(0xFF)
        velox.sparse_attn(q, k, v, r["ids"], r["lens"], wl.M, workspace=ws)
        torch.cuda.synchronize()
        plan_bytes = ws
        part_ml = None
    else:
        ws = velox.split_workspace(q, n_split)
        ws.fill_(0xFF)
        velox.sparse_attn(q, k, v, r["ids"], r["lens"], wl.M, n_split=n_split, workspace=ws)
        torch.cuda.synchronize()
        rows = n_split * H * N * 128
        plan_bytes = ws[rows * 130 * 4:]
        part_ml = ws[rows * 128 * 4: rows * 130 * 4].view(torch.float32).view(n_split, H, N * 128, 2).cpu().numpy()
    want, unused = expected_plan(lens, N, n_split)
    got = plan_bytes[: 16 * (max(want) + 1)].view(torch.int32).view(-1, 4).cpu().numpy()
    for b, e in sorted(want.items()):
        assert tuple(int(v) for v in got[b]) == e, f"workgroup {b}: {tuple(got[b])} != {e}"
    for rr, h, a, b in unused:
        for row in (a, b):
            if row < 0:
                continue
            ml = part_ml[rr, h, row * 128:(row + 1) * 128]
            assert np.all(np.isneginf(ml[:, 0])) and np.all(ml[:, 1] == 0), (rr, h, row)
