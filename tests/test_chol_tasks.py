"""Task numbering of the one-launch tiled Cholesky in the GPU's error-feedback
quantizer (host logic, no GPU).

The kernel numbers the tasks of the right-looking tiled factorization of
reverse(H) (64 x 64 tiles, nt per side) as: for k, factor tile (k, k), solve
tiles (i, k) for i > k, then update tiles (i, j) for k < j <= i, column by
column.  Workgroups take numbers from a counter and wait on per-tile counters
(updates applied, plus one when final).  The waits end only if every task
waits for tasks with smaller numbers; this file restates the kernel's decode
of a task number and checks that property, that the numbering covers every
task once, and that executing the tasks in number order is the Cholesky
factorization.  The GPU parity tests cover the kernel itself.
"""
from __future__ import annotations

import numpy as np
import pytest


def task_count(nt: int) -> int:
    return sum(1 + (nt - 1 - k) + (nt - 1 - k) * (nt - k) // 2 for k in range(nt))


def decode(t: int, nt: int):
    """(type, i, j, k) of task t: type 0 factor, 1 solve, 2 update."""
    k, base, m = 0, 0, nt - 1
    while True:
        sz = 1 + m + m * (m + 1) // 2
        if t < base + sz:
            break
        base += sz
        k += 1
        m -= 1
    o = t - base
    if o == 0:
        return 0, k, k, k
    if o <= m:
        return 1, k + o, k, k
    u, j = o - 1 - m, k + 1
    while u >= nt - j:
        u -= nt - j
        j += 1
    return 2, j + u, j, k


def waits(task):
    """(tile i, tile j, counter value) pairs the task waits for."""
    ty, i, j, k = task
    w = [(i, j, k)]
    if ty == 1:
        w.append((k, k, k + 1))
    if ty == 2:
        w += [(i, k, k + 1), (j, k, k + 1)]
    return w


@pytest.mark.parametrize("nt", [1, 2, 3, 5, 32, 64])
def test_numbering_covers_every_task_once_in_dependency_order(nt):
    tasks = [decode(t, nt) for t in range(task_count(nt))]
    want = []
    for k in range(nt):
        want.append((0, k, k, k))
        want += [(1, i, k, k) for i in range(k + 1, nt)]
        want += [(2, i, j, k) for j in range(k + 1, nt) for i in range(j, nt)]
    assert tasks == want
    # replaying in number order, every wait is already satisfied: each task
    # waits only for smaller numbers
    ver = np.zeros((nt, nt), dtype=np.int64)
    for t, task in enumerate(tasks):
        for a, b, target in waits(task):
            assert ver[a, b] >= target, (nt, t, task)
        _, i, j, k = task
        ver[i, j] = k + 1
    assert all(ver[i, j] == j + 1 for i in range(nt) for j in range(i + 1))


@pytest.mark.parametrize("K", [32, 64, 96, 200, 320])
def test_tasks_in_number_order_give_the_cholesky_factor(K):
    rng = np.random.default_rng(K)
    X = rng.standard_normal((K + 5, K))
    H = X.T @ X + K * np.eye(K)
    A = np.tril(H)
    nt = (K + 63) // 64
    for t in range(task_count(nt)):
        ty, i, j, k = decode(t, nt)
        ri = slice(64 * i, min(K, 64 * i + 64))
        cj = slice(64 * j, min(K, 64 * j + 64))
        kk = slice(64 * k, min(K, 64 * k + 64))
        if ty == 0:
            blk = np.tril(A[ri, ri])
            A[ri, ri] = np.linalg.cholesky(blk + np.tril(blk, -1).T)
        elif ty == 1:
            A[ri, kk] = np.linalg.solve(np.tril(A[kk, kk]), A[ri, kk].T).T
        else:
            upd = A[ri, kk] @ A[cj, kk].T
            A[ri, cj] -= np.tril(upd) if i == j else upd
    assert np.allclose(np.tril(A), np.linalg.cholesky(H), rtol=1e-12, atol=1e-9)
