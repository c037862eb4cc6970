"""Host-side models of the B-through-LDS 16x16x32 kernels' plans (no GPU).

csrc/gsr_interleave16d.hpp runs two tiles, 256x256 (configuration 28) and
128x256 (configuration 29), from one kernel template whose tile
configurations carry the slot plan: where in the 2 x FM*FN MFMA slots of a
K-step each operand read, copy, wait and barrier is issued.  A wrong slot or
address does not fail to compile; it races or reads the wrong element.
These tests rebuild both plans in Python from the constants in the header
and check them:

* the program-order model runs the kernel's loop conditions over several
  K-steps and checks that every MFMA sees the operands of its own K-step and
  substep, that a stage is read only after the barrier that publishes it and
  copied into only after the barrier that frees it, and that the vmcnt wait
  before each barrier leaves only the copies that are not read next;
* the address model places every copied element (A rows, B rows through the
  fb16 swizzle) and every fragment read (A^T by 128-bit reads, B^T by
  ds_read_b64_tr_b16 with its lane exchange: in each 16-lane group output
  lane i, element e comes from source lane 4e + i / 4, element i mod 4) and
  checks each fragment against the 16x16x32 operand layout, with both
  operands pairing the same k, and that the eight rows the LDS serves per
  cycle sit on distinct banks;
* for the copy-wave kernels (gsr_interleave16c.hpp: two A and three B
  stages, or one ring of A+B stages), a barrier-interval model of the two
  roles: every stage the MFMA waves read in an interval has landed by the
  barrier that opens it, and no copy writes a stage during an interval in
  which it is read.

Planted mistakes in the plan (a copy before the barrier, an operand read too
late) are caught by the model, so it is not vacuous.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_dense_gemm_scale_amd", "csrc")
HDR = os.path.join(CSRC, "gsr_interleave16d.hpp")
HDR_C = os.path.join(CSRC, "gsr_interleave16c.hpp")

# tile shapes of the instantiations (four MFMA waves of 2 x 2 in all)
TILES = {"Ilv16DCfg": (256, 256), "Ilv16HDCfg": (128, 256)}
COPY_WAVE_TILES = {"Ilv16CCfg": (128, 256), "Ilv16QCCfg": (128, 128)}
SLOT_KEYS = ("X7_0", "X7_1", "Y0_0", "Y0_1", "BAR", "BC0", "BCD", "AC0", "ACD")
COPY_WAVE_KEYS = ("X7_0", "X7_1", "Y0_0", "Y0_1", "YS", "BAR", "RING")


def _constants(header: str, struct: str, keys) -> dict:
    """Integer constants of one configuration struct; a value written as
    Other::KEY is looked up in struct Other (in this header or the
    B-through-LDS one)."""
    src = open(header).read()
    body = src[src.index(f"struct {struct}"):]
    body = body[: body.index("};")]
    c = {}
    for key in keys:
        m = re.search(rf"\b{key} = (\w+)(?:::(\w+))?", body)
        assert m, (struct, key)
        if m.group(2) is None:
            c[key] = int(m.group(1))
        else:
            other = header if f"struct {m.group(1)}" in src else HDR
            c[key] = _constants(other, m.group(1), (m.group(2),))[m.group(2)]
    return c


def plan(struct: str) -> dict:
    """The slot constants of one tile configuration, read from the header.
    For the copy-wave kernels the copies are placed where the copy waves
    issue them relative to the barriers: B(t+2) before any read of substep 0
    (right after b_{t-1}), A(t+2) right after b_t; with a ring of RING
    stages, both copies of step t+RING right after b_t."""
    if struct in COPY_WAVE_TILES:
        c = _constants(HDR_C, struct, COPY_WAVE_KEYS)
        bm, bn = COPY_WAVE_TILES[struct]
        c.update(BC0=0, BCD=1, AC0=c["BAR"], ACD=1)
    else:
        c = _constants(HDR, struct, SLOT_KEYS)
        c.update(YS=4, RING=0)
        bm, bn = TILES[struct]
    c["FM"], c["FN"] = bm // 2 // 16, bn // 2 // 16
    c["A_PER"], c["B_PER"] = bm * 64 * 2 // 1024 // 4, bn * 64 * 2 // 1024 // 4
    return c


# ---- program-order model -----------------------------------------------------

def program(c: dict, ksteps: int) -> list:
    """The kernel's issue order: prologue, then per K-step t (A stage t % 2,
    B stage t % 3; with a ring, both t % RING) substep 0 and substep 1, slot
    by slot, as the loops in gsr_interleave16d.hpp and gsr_interleave16c.hpp
    emit them."""
    FM, FN, ring = c["FM"], c["FN"], c["RING"]
    per = c["A_PER"] + c["B_PER"]
    slots = FM * FN
    ev = []
    for s in range(ring or 2):
        ev += [("copyA", s, s)] * c["A_PER"] + [("copyB", s, s)] * c["B_PER"]
    ev += [("wait", (ring - 1) * per if ring else per), ("barrier",)]
    for a in range(FN):
        ev += [("readX", a, 0, 0, 0, 0), ("readX", a, 1, 0, 0, 0)]
    ev += [("readY", b, 0, 0, 0) for b in range(FM)]

    def reads(i, sr, br, t, kr, y0, x7):
        if FM <= i <= FM * (FN - 1) + 1 and i % FM < 2:
            ev.append(("readX", i // FM - 1, i % FM, br, t, kr))
        if i in (x7, x7 + 1):
            ev.append(("readX", FN - 1, i - x7, br, t, kr))
        if y0 <= i < y0 + c["YS"] * FM and (i - y0) % c["YS"] == 0:
            ev.append(("readY", (i - y0) // c["YS"], sr, t, kr))

    for t in range(ksteps):
        sa, sb = (t % ring, t % ring) if ring else (t % 2, t % 3)
        san, sbn = ((t + 1) % ring, (t + 1) % ring) if ring else (sa ^ 1, (sb + 1) % 3)
        for i in range(slots):
            ev.append(("mma", i, t, 0))
            reads(i, sa, sb, t, 1, c["Y0_0"], c["X7_0"])
            if not ring and i >= c["BC0"] and (i - c["BC0"]) % c["BCD"] == 0 and (i - c["BC0"]) // c["BCD"] < c["B_PER"]:
                ev.append(("copyB", (t + 2) % 3, t + 2))
        for i in range(slots):
            ev.append(("mma", i, t, 1))
            if i == c["BAR"]:
                ev += [("wait", (ring - 2) * per if ring else c["B_PER"]), ("barrier",)]
                if ring:
                    ev += [("copyA", sa, t + ring)] * c["A_PER"] + [("copyB", sb, t + ring)] * c["B_PER"]
            if i >= c["BAR"]:
                reads(i, san, sbn, t + 1, 0, c["Y0_1"], c["X7_1"])
            if not ring and i >= c["AC0"] and (i - c["AC0"]) % c["ACD"] == 0 and (i - c["AC0"]) // c["ACD"] < c["A_PER"]:
                ev.append(("copyA", sa, t + 2))
    return ev


def check_program(c: dict, ksteps: int) -> None:
    FM, FN = c["FM"], c["FN"]
    ev = program(c, ksteps)
    ahead = c["RING"] or 2  # copies issued past the last K-step (they write zeros)
    assert sum(e[0] == "copyB" for e in ev) == c["B_PER"] * (ksteps + ahead), "every B copy issued once"
    assert sum(e[0] == "copyA" for e in ev) == c["A_PER"] * (ksteps + ahead), "every A copy issued once"
    X, half, X7, Y = {}, {}, {}, {}
    in_flight, landed = [], {"A": {}, "B": {}}
    published, last_read = {"A": {}, "B": {}}, {"A": {}, "B": {}}
    barriers = 0
    for e in ev:
        kind = e[0]
        if kind in ("copyA", "copyB"):
            op, stage, step = kind[-1], e[1], e[2]
            assert last_read[op].get(stage, -1) < barriers, f"copy into {op} stage {stage} read since the last barrier"
            in_flight.append((op, stage, step))
            published[op].pop(stage, None)
        elif kind == "wait":  # vmcnt: the oldest copies beyond the count have landed
            while len(in_flight) > e[1]:
                op, stage, step = in_flight.pop(0)
                landed[op][stage] = step
        elif kind == "barrier":
            barriers += 1
            for op in "AB":
                published[op].update(landed[op])
        elif kind == "readX":
            a, rd, stage, t, ks = e[1:]
            assert published["B"].get(stage) == t, f"B^T read of B stage {stage} before step {t} is published"
            last_read["B"][stage] = barriers
            if rd == 0:
                half[a] = (t, ks)
            else:
                assert half.get(a) == (t, ks), "the two transpose reads of a fragment belong together"
                (X7 if a == FN - 1 else X)[ks if a == FN - 1 else a] = (t, ks)
        elif kind == "readY":
            b, stage, t, ks = e[1:]
            assert published["A"].get(stage) == t, f"A^T read of A stage {stage} before step {t} is published"
            last_read["A"][stage] = barriers
            Y[(ks, b)] = (t, ks)
        else:
            i, t, ks = e[1:]
            a, b = i // FM, i % FM
            x = X7.get(ks) if a == FN - 1 else X.get(a)
            assert x == (t, ks), f"MFMA slot {i} of step {t} substep {ks} sees B^T fragment {x}"
            assert Y.get((ks, b)) == (t, ks), f"MFMA slot {i} of step {t} substep {ks} sees A^T fragment {Y.get((ks, b))}"


def _step_counts(struct):
    """The two-plus-three layout runs K-steps in pairs, a ring one by one."""
    return [1, 2, 3, 4, 5, 6, 7, 8, 14] if plan(struct)["RING"] else [2, 4, 6, 8, 14]


@pytest.mark.parametrize("struct,ksteps", [(s, k) for s in sorted(TILES) + sorted(COPY_WAVE_TILES) for k in _step_counts(s)])
def test_slot_plan_is_consistent(struct, ksteps):
    check_program(plan(struct), ksteps)


@pytest.mark.parametrize("mistake", [
    {"AC0": 3},            # A copies before the barrier that frees their stage
    {"Y0_1": 2},           # next step's A^T reads before the barrier publishes them
    {"BAR": 8},            # barrier after the first X refill
    {"X7_1": 2},           # X[7] for the next step placed before the barrier: never read
], ids=lambda m: ",".join(f"{k}={v}" for k, v in m.items()))
def test_slot_model_catches_planted_mistakes(mistake):
    c = plan("Ilv16HDCfg")
    c.update(mistake)
    with pytest.raises(AssertionError):
        check_program(c, 8)


# ---- address model -----------------------------------------------------------

def lch(g):
    return ((g & 1) << 1) | (g >> 1)


def fb16(k):
    c = (k >> 3) & 3
    return ((k & 3) + (((c ^ (c >> 1)) & 1) << 2)) << 1


def swz_a(r):
    return (r ^ (r >> 3)) & 7


@pytest.mark.parametrize("tile", [(256, 256), (128, 256), (128, 128)], ids=lambda t: f"{t[0]}x{t[1]}")
def test_copy_and_read_addresses(tile):
    """Copy waves or MFMA waves alike: copier w = 0..3 (the wave, or the copy
    wave's index) fills 1 KiB blocks w + 4i."""
    bm, bn = tile
    bk, nw, rowb = 64, 4, bn * 2
    wtm, wtn = bm // 2, bn // 2
    cpr, rpk, cpw = bn // 8, 1024 // rowb, wtn // 8  # chunks per B row, rows per copy, chunks per wave
    a_per, b_per = bm * bk * 2 // 1024 // nw, bn * bk * 2 // 1024 // nw
    # B copies: copy i of copier w fills chunk positions 64 (w + 4i) + lane
    blds = {}
    for w in range(nw):
        for i in range(b_per):
            for lane in range(64):
                k = rpk * (w + nw * i) + lane // cpr
                c = (lane % cpr) ^ fb16(k)
                base = 1024 * (w + nw * i) + 16 * lane
                assert base == k * rowb + (lane % cpr) * 16
                for e in range(8):
                    blds[base + 2 * e] = (k, 8 * c + e)
    assert sorted(blds.values()) == sorted((k, n) for k in range(bk) for n in range(bn))
    # A copies: copy i of wave w fills the 1 KiB block w + 4i, rows
    # 8 w + 32 i + lane / 8, logical chunk c0 (c0 ^ 4 for odd i)
    alds = {}
    for w in range(nw):
        for i in range(a_per):
            for lane in range(64):
                c0 = (lane & 7) ^ (lane >> 3) ^ w ^ (4 if i & 1 else 0)
                r = 8 * w + 32 * i + (lane >> 3)
                base = 1024 * (w + nw * i) + 16 * lane
                assert base == r * 128 + (lane & 7) * 16 and (lane & 7) == c0 ^ swz_a(r)
                for e in range(8):
                    alds[base + 2 * e] = (r, 8 * c0 + e)
    assert sorted(alds.values()) == sorted((r, k) for r in range(bm) for k in range(bk))
    extra_bank_cycles = 0
    for w in range(nw):
        wm, wn = w // 2, w % 2
        for ks in range(2):
            for a in range(wtn // 16):  # B^T fragments by two transpose reads
                frag = {}
                for rd in range(2):
                    addr = []
                    for lane in range(64):
                        g, li = lane >> 4, lane & 15
                        e, q = li >> 2, li & 3
                        krow0 = 8 * lch(g) + e
                        xa = krow0 * rowb + (((cpw * wn + 2 * a + (q >> 1)) ^ fb16(krow0)) << 4) + (q & 1) * 8
                        addr.append(xa + ks * 32 * rowb + rd * 4 * rowb)
                    for lane in range(64):
                        g, i = lane >> 4, lane & 15
                        for e in range(4):
                            frag[(lane, 4 * rd + e)] = blds[addr[16 * g + 4 * e + i // 4] + 2 * (i % 4)]
                    for half in (range(32), range(32, 64)):
                        banks = {}
                        for lane in half:
                            for dw in range(2):
                                banks.setdefault((addr[lane] // 4 + dw) % 64, set()).add(addr[lane] // 4 + dw)
                        extra_bank_cycles += max(len(v) for v in banks.values()) - 1
                for lane in range(64):
                    for j in range(8):
                        assert frag[(lane, j)] == (32 * ks + 8 * lch(lane >> 4) + j, wtn * wn + 16 * a + (lane & 15))
            for b in range(wtm // 16):  # A^T fragments by 128-bit reads
                for lane in range(64):
                    lrow, lq = lane & 15, lane >> 4
                    ry = wm * wtm + (b & 3) * 16 + lrow
                    off = (b >> 2) * 64 * 128 + ((ry * 128 + ((lch(lq) ^ swz_a(ry)) << 4)) ^ (64 if ks else 0))
                    for j in range(8):
                        assert alds[off + 2 * j] == (wm * wtm + 16 * b + lrow, 32 * ks + 8 * lch(lq) + j)
    assert extra_bank_cycles == 0


# ---- the copy-wave protocol (gsr_interleave16c.hpp) --------------------------

def copy_wave_program(ksteps: int, ring: int = 0, a_per: int = 4, b_per: int = 8,
                      a_before_barrier: bool = False, wait=None) -> list:
    """Copy waves' issue order.  Two A and three B stages (ring 0): stage 0
    and 1 copies, wait, prologue barrier; per K-step t the B(t+2) copies, the
    wait, barrier b_t and the A(t+2) copies.  A ring of `ring` stages: the
    copies of steps 0 .. ring-1, wait, prologue barrier; per K-step t the
    wait, b_t and the copies of step t+ring into stage t mod ring.  Both end
    with a full drain and the epilogue's barrier."""
    per = a_per + b_per
    ev = []
    if not ring:
        ev += [("copy", "A", 0, 0)] * a_per + [("copy", "B", 0, 0)] * b_per
        ev += [("copy", "A", 1, 1)] * a_per + [("copy", "B", 1, 1)] * b_per
        ev += [("wait", per), ("barrier",)]
        for t in range(ksteps):
            ev += [("copy", "B", (t + 2) % 3, t + 2)] * b_per
            if a_before_barrier:
                ev += [("copy", "A", t % 2, t + 2)] * a_per
            ev += [("wait", b_per if wait is None else wait), ("barrier",)]
            if not a_before_barrier:
                ev += [("copy", "A", t % 2, t + 2)] * a_per
    else:
        for st in range(ring):
            ev += [("copy", "A", st, st)] * a_per + [("copy", "B", st, st)] * b_per
        ev += [("wait", (ring - 1) * per), ("barrier",)]
        for t in range(ksteps):
            copies = [("copy", "A", t % ring, t + ring)] * a_per + [("copy", "B", t % ring, t + ring)] * b_per
            if a_before_barrier:
                ev += copies
            ev += [("wait", (ring - 2) * per if wait is None else wait), ("barrier",)]
            if not a_before_barrier:
                ev += copies
    return ev + [("wait", 0), ("barrier",)]


def mfma_wave_reads(ksteps: int, ring: int = 0) -> list:
    """MFMA waves' stage reads per barrier interval: (interval, operand,
    stage, K-step of the data).  Interval j follows the j-th barrier of the
    kernel (the prologue's is the first, b_t the (t+2)-th)."""
    sa = (lambda t: t % ring) if ring else (lambda t: t % 2)
    sb = (lambda t: t % ring) if ring else (lambda t: t % 3)
    reads = [(1, "A", 0, 0), (1, "B", 0, 0)]  # step 0's substep-0 operands
    for t in range(ksteps):
        reads += [(t + 1, "A", sa(t), t), (t + 1, "B", sb(t), t)]                  # substep 0, for substep 1
        reads += [(t + 2, "A", sa(t + 1), t + 1), (t + 2, "B", sb(t + 1), t + 1)]  # after b_t
    return reads


def check_copy_waves(ksteps: int, ring: int = 0, **kw) -> None:
    ev = copy_wave_program(ksteps, ring=ring, **kw)
    interval, in_flight = 0, []
    landed = {}           # (operand, stage) -> K-step whose copies have landed
    landed_at = {}        # barrier index -> snapshot of landed data at that barrier
    written_in = {}       # interval -> set of (operand, stage) copied into during it
    for e in ev:
        if e[0] == "copy":
            in_flight.append(e[1:])
            written_in.setdefault(interval, set()).add((e[1], e[2]))
            landed.pop((e[1], e[2]), None)
        elif e[0] == "wait":
            while len(in_flight) > e[1]:
                op, st, step = in_flight.pop(0)
                landed[(op, st)] = step
        else:
            interval += 1
            landed_at[interval] = dict(landed)
    assert interval == ksteps + 2, "copy and MFMA waves pass the same number of barriers"
    for j, op, st, step in mfma_wave_reads(ksteps, ring):
        assert landed_at[j].get((op, st)) == step, f"{op} stage {st} read in interval {j} before step {step} landed"
        assert (op, st) not in written_in.get(j, set()), f"{op} stage {st} copied into while it is read (interval {j})"


def copy_wave_geometry(struct: str) -> dict:
    c = plan(struct)
    return {"ring": c["RING"], "a_per": c["A_PER"], "b_per": c["B_PER"]}


@pytest.mark.parametrize("struct,ksteps", [(s, k) for s in sorted(COPY_WAVE_TILES) for k in _step_counts(s)])
def test_copy_wave_protocol(struct, ksteps):
    check_copy_waves(ksteps, **copy_wave_geometry(struct))


@pytest.mark.parametrize("struct", sorted(COPY_WAVE_TILES))
@pytest.mark.parametrize("mistake", ["A-copies-before-the-barrier", "wait-too-loose"])
def test_copy_wave_model_catches_planted_mistakes(struct, mistake):
    g = copy_wave_geometry(struct)
    per = g["a_per"] + g["b_per"]
    if mistake == "A-copies-before-the-barrier":
        kw = {"a_before_barrier": True}
    else:  # one step more in flight than the barrier allows
        kw = {"wait": (g["ring"] - 1) * per if g["ring"] else per}
    with pytest.raises(AssertionError):
        check_copy_waves(8, **g, **kw)


def test_ring_depth_is_read_from_the_header():
    assert copy_wave_geometry("Ilv16CCfg")["ring"] == 0
    assert copy_wave_geometry("Ilv16QCCfg")["ring"] >= 3
