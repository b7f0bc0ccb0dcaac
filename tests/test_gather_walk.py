"""The fused lookup-gate's walk over the tables, modelled on the host (no GPU).

In gate_gather_kernel a wave's 64 lanes each own one token row; k-step k's memory operand is
chunks 8k .. 8k+7 of every token's concatenated row, which the kernel finds as chunk gO + c of
the row in table gT (or chunk gO + c - cpr in table gT + 1), advancing (gT, gO) by 8 chunks per
k-step and rotating the lanes' two row numbers when it enters a table; load instruction i of
a wave takes the row numbers of token 8i + lane/8 from that token's lane.  This model runs the
same state machine and checks, for every chunks-per-row count the kernel accepts (>= 8), every
lane, k-step and instruction, that the (token, table, chunk) loaded is the one the
concatenation defines (chunk q of the row is chunk q mod cpr of table q div cpr).
"""
import pytest


def row_key(r):
    return (r & 7) ^ ((r >> 3) & 1)


def walk(cpr, n_tables, wave):
    """Yields (k, lane, i, token, table, chunk) as the kernel's state machine computes them."""
    d_mem_chunks = n_tables * cpr
    nk = d_mem_chunks // 8
    gT, gO = 0, 0
    # lane L of the wave holds (token, table) row numbers for tables gT and gT + 1
    own = {L: ((wave * 64 + L, 0), (wave * 64 + L, 1) if n_tables > 1 else None) for L in range(64)}
    for k in range(nk):
        o, tb = gO, gT
        rows0 = {L: own[L][0] for L in range(64)}
        rows1 = {L: own[L][1] for L in range(64)}
        for lane in range(64):
            for i in range(8):
                src = i * 8 + (lane >> 3)                 # the lane that owns the token
                r = wave * 64 + i * 8 + (lane >> 3)        # the token row the load fills
                q = o + ((lane & 7) ^ row_key(r))
                nxt = q >= cpr
                held = rows1[src] if nxt else rows0[src]
                table = tb + 1 if nxt else tb
                yield k, lane, i, r, held, table, q - cpr if nxt else q
        gO += 8
        if gO >= cpr:
            gO -= cpr
            gT += 1
            own = {L: (own[L][1], (wave * 64 + L, gT + 1) if gT + 1 < n_tables else None) for L in range(64)}


@pytest.mark.parametrize("cpr", [8, 9, 10, 12, 16, 25, 29])
def test_walk_loads_the_concatenated_rows(cpr):
    for n_tables in range(1, 12):
        if (n_tables * cpr) % 8:
            continue  # d_mem must be a multiple of 64 values (8 chunks)
        seen = set()
        for wave in (0, 3):
            for k, lane, i, r, held, table, chunk in walk(cpr, n_tables, wave):
                logical = (lane & 7) ^ row_key(r)
                want_table, want_chunk = divmod(8 * k + logical, cpr)
                assert held == (r, want_table), (cpr, n_tables, k, lane, i)
                assert (table, chunk) == (want_table, want_chunk), (cpr, n_tables, k, lane, i)
                assert table < n_tables and 0 <= chunk < cpr
                seen.add((r, 8 * k + logical))
        # every chunk of every token row of the two waves is loaded
        assert len(seen) == 2 * 64 * n_tables * cpr
