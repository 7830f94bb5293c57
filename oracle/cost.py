"""Integer cost-table lookup C_est(rows, len) (test infrastructure only).

CoDec (CoDec: Prefix-Shared Decoding Kernel for LLMs), section 工作负载平衡,
profile-based cost estimation: the partial-attention kernel is profiled over
a grid of KV lengths n and query counts n_q on the target hardware, and an
interpolation function C_est(n_q, n) estimates the shapes in between.

The pages say only "interpolation".  Reading used here (all integers, in
nanoseconds, so two implementations agree bit for bit):

* rows axis (query rows = n_q x GQA group): the smallest grid point >= rows
  (a step, never an underestimate); above the last point, the last point;
* length axis: below the first point, the first point's value; between two
  points L0 <= len < L1, C0 + (C1 - C0) * (len - L0) // (L1 - L0); above the
  last point, linear extrapolation from the last two points;
* a valid table is >= 1 everywhere and non-decreasing along both axes, so
  every term is non-negative and ``//`` is plain truncation.
"""
from __future__ import annotations

import bisect

import numpy as np


class CostTable:
    def __init__(self, rows_grid, len_grid, table):
        self.rows_grid = [int(x) for x in rows_grid]
        self.len_grid = [int(x) for x in len_grid]
        self.table = [[int(c) for c in row] for row in np.asarray(table).tolist()]
        if len(self.len_grid) < 2 or len(self.rows_grid) < 1:
            raise ValueError("grids too small")
        if any(b <= a for a, b in zip(self.rows_grid, self.rows_grid[1:])):
            raise ValueError("rows grid not ascending")
        if any(b <= a for a, b in zip(self.len_grid, self.len_grid[1:])):
            raise ValueError("len grid not ascending")
        if self.rows_grid[0] < 1 or self.len_grid[0] < 1:
            raise ValueError("grid points must be >= 1")
        R, L = len(self.rows_grid), len(self.len_grid)
        if len(self.table) != R or any(len(r) != L for r in self.table):
            raise ValueError("table shape")
        for i in range(R):
            for j in range(L):
                c = self.table[i][j]
                if c < 1:
                    raise ValueError("cost < 1")
                if j and c < self.table[i][j - 1]:
                    raise ValueError("not non-decreasing in len")
                if i and c < self.table[i - 1][j]:
                    raise ValueError("not non-decreasing in rows")

    def lookup(self, rows: int, length: int) -> int:
        ri = bisect.bisect_left(self.rows_grid, rows)
        if ri == len(self.rows_grid):
            ri -= 1
        row = self.table[ri]
        lg = self.len_grid
        if length <= lg[0]:
            return row[0]
        if length >= lg[-1]:
            c0, c1 = row[-2], row[-1]
            return c1 + (c1 - c0) * (length - lg[-1]) // (lg[-1] - lg[-2])
        j = bisect.bisect_right(lg, length) - 1  # lg[j] <= length < lg[j+1]
        c0, c1 = row[j], row[j + 1]
        return c0 + (c1 - c0) * (length - lg[j]) // (lg[j + 1] - lg[j])
