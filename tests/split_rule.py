"""The persistent GEMM's split schedule, stated on its own (test helper).

For a launch of `tiles` output tiles on `grid` workgroups, `kb` K blocks
per tile and a workspace of `slots` partial tiles: whole rounds of one tile
per workgroup first; when the tiles do not fill the last round and the
leftover (tiles mod grid) fills at most half of it, each leftover tile is cut
into the fewest pieces that reach the shortest piece length (in whole 4-block
rounds) allowed by min(grid // leftover, 16, rounds), if that is at least 2
and the pieces fit the workspace.  Returns (split_tiles, pieces)."""


def split_rule(tiles, grid, kb, slots):
    rounds = (kb + 3) // 4
    if grid <= 0 or tiles <= grid or slots <= 0 or tiles % grid == 0:
        return 0, 1
    left = tiles % grid
    most = min(grid // left, 16, rounds)
    if most < 2:
        return 0, 1
    per = -(-rounds // most)
    pieces = -(-rounds // per)
    if pieces < 2 or left * pieces > slots:
        return 0, 1
    return left, pieces


def persistent_grid(tiles, cus):
    """Workgroups of the persistent launch: the CU count rounded down to a
    multiple of 8, or one per tile when there are fewer tiles."""
    return cus // 8 * 8 if (cus >= 8 and tiles > cus) else tiles
