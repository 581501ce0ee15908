"""The mma.sync page's own lane maps, emulated on the CPU over the oracle's
packed words (mma.sync page: "Operand coordinates and ownership" lane-map
table, and the loads and stores of the worked example kernel).

This pins the reading that the second atom coordinate of A and B is a packed
word index (k/2 axis, even K in the low half): with it, the page's 32-lane
maps cover each word of the atoms exactly once, and the emulated warp
produces a @ b.T for the worked example. The NVIDIA lane maps are not used by
the HIP kernels; this only checks the packing against the page.
"""
import numpy as np

import oracle
from tests import util

G = util.golden("mma_sync_lane_maps.json")


def coord(expr: str, l: int, r: int) -> int:
    # the table's formulas use only l, r, //, %, * and +
    return int(eval(expr, {"__builtins__": {}}, {"l": l, "r": r}))


def gather(atom_rows, table, regs, atom):
    """Registers of every lane for one K16 atom: {(lane, reg): word}."""
    out = {}
    for l in range(G["lanes"]):
        for r in range(regs):
            out[(l, r)] = atom[coord(table["row"], l, r), coord(table["word"], l, r)]
    return out


def test_maps_cover_each_word_once():
    for name, regs, shape in (("A", 4, (16, 8)), ("B", 2, (8, 8))):
        t = G[name]
        seen = {(coord(t["row"], l, r), coord(t["word"], l, r))
                for l in range(G["lanes"]) for r in range(regs)}
        assert len(seen) == G["lanes"] * regs == shape[0] * shape[1], name
    t = G["D"]
    seen = {(coord(t["row"], l, r), coord(t["col"], l, r))
            for l in range(G["lanes"]) for r in range(t["regs_per_lane"])}
    assert seen == {(i, j) for i in range(16) for j in range(8)}


def test_emulated_worked_example():
    g = util.golden("mma_sync_worked_example.json")
    rec = g["recipe"]
    rng = np.random.default_rng(rec["seed"])
    a = (rng.integers(rec["integers_low"], rec["integers_high_exclusive"], rec["a_shape"])
         / rec["divide_by"]).astype(rec["dtype"])
    b = (rng.integers(rec["integers_low"], rec["integers_high_exclusive"], rec["b_shape"])
         / rec["divide_by"]).astype(rec["dtype"])
    A = oracle.pack(a.view(np.uint16), 16)[0, 0]   # (K_repeat, 16, 8) words
    B = oracle.pack(b.view(np.uint16), 8)[0, 0]    # (K_repeat, 8, 8) words

    def halves(word):
        return [np.uint32(word) & 0xFFFF, np.uint32(word) >> 16]

    D = np.zeros((16, 8), np.float64)   # the recurrence starts from scalar C = 0
    for kk in range(g["K_repeat"]):
        ar = gather(16, G["A"], 4, A[kk])
        br = gather(8, G["B"], 2, B[kk])
        # rebuild the logical 16x16 and 8x16 K16 slices from the lanes' registers
        a_atom = np.zeros((16, 16), np.float64)
        b_atom = np.zeros((8, 16), np.float64)
        for (l, r), w in ar.items():
            i, wd = coord(G["A"]["row"], l, r), coord(G["A"]["word"], l, r)
            for h, bits in enumerate(halves(w)):
                a_atom[i, 2 * wd + h] = util.decode(np.array([bits], np.uint16), "f16")[0]
        for (l, r), w in br.items():
            j, wd = coord(G["B"]["row"], l, r), coord(G["B"]["word"], l, r)
            for h, bits in enumerate(halves(w)):
                b_atom[j, 2 * wd + h] = util.decode(np.array([bits], np.uint16), "f16")[0]
        D = D + a_atom @ b_atom.T
    # each lane stores its 4 results at the D map's coordinates
    out = np.full((16, 8), np.nan)
    t = G["D"]
    for l in range(G["lanes"]):
        for r in range(t["regs_per_lane"]):
            i, j = coord(t["row"], l, r), coord(t["col"], l, r)
            out[i, j] = D[i, j]
    assert np.array_equal(out, a.astype(np.float64) @ b.astype(np.float64).T)
