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
* for configuration 31 (gsr_interleave16c.hpp), whose copies run on waves of
  their own, a barrier-interval model of the two roles: every stage the MFMA
  waves read in an interval has landed by the barrier that opens it, and no
  copy writes a stage during an interval in which it is read.

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
COPY_WAVE_KEYS = ("X7_0", "X7_1", "Y0_0", "Y0_1", "YS", "BAR")


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
    (right after b_{t-1}), A(t+2) right after b_t."""
    if struct in COPY_WAVE_TILES:
        c = _constants(HDR_C, struct, COPY_WAVE_KEYS)
        bm, bn = COPY_WAVE_TILES[struct]
        c.update(BC0=0, BCD=1, AC0=c["BAR"], ACD=1)
    else:
        c = _constants(HDR, struct, SLOT_KEYS)
        c["YS"] = 4
        bm, bn = TILES[struct]
    c["FM"], c["FN"] = bm // 2 // 16, bn // 2 // 16
    c["A_PER"], c["B_PER"] = bm * 64 * 2 // 1024 // 4, bn * 64 * 2 // 1024 // 4
    return c


# ---- program-order model -----------------------------------------------------

def program(c: dict, ksteps: int) -> list:
    """The kernel's issue order: prologue, then per K-step t (A stage t % 2,
    B stage t % 3) substep 0 and substep 1, slot by slot, as the loops in
    gsr_interleave16d.hpp emit them."""
    FM, FN = c["FM"], c["FN"]
    slots = FM * FN
    ev = [("copyA", 0, 0)] * c["A_PER"] + [("copyB", 0, 0)] * c["B_PER"]
    ev += [("copyA", 1, 1)] * c["A_PER"] + [("copyB", 1, 1)] * c["B_PER"]
    ev += [("wait", c["A_PER"] + c["B_PER"]), ("barrier",)]
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
        sa, sb = t % 2, t % 3
        for i in range(slots):
            ev.append(("mma", i, t, 0))
            reads(i, sa, sb, t, 1, c["Y0_0"], c["X7_0"])
            if i >= c["BC0"] and (i - c["BC0"]) % c["BCD"] == 0 and (i - c["BC0"]) // c["BCD"] < c["B_PER"]:
                ev.append(("copyB", (t + 2) % 3, t + 2))
        for i in range(slots):
            ev.append(("mma", i, t, 1))
            if i == c["BAR"]:
                ev += [("wait", c["B_PER"]), ("barrier",)]
            if i >= c["BAR"]:
                reads(i, sa ^ 1, (sb + 1) % 3, t + 1, 0, c["Y0_1"], c["X7_1"])
            if i >= c["AC0"] and (i - c["AC0"]) % c["ACD"] == 0 and (i - c["AC0"]) // c["ACD"] < c["A_PER"]:
                ev.append(("copyA", sa, t + 2))
    return ev


def check_program(c: dict, ksteps: int) -> None:
    FM, FN = c["FM"], c["FN"]
    ev = program(c, ksteps)
    assert sum(e[0] == "copyB" for e in ev) == c["B_PER"] * (ksteps + 2), "every B copy issued once"
    assert sum(e[0] == "copyA" for e in ev) == c["A_PER"] * (ksteps + 2), "every A copy issued once"
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


@pytest.mark.parametrize("struct", sorted(TILES) + sorted(COPY_WAVE_TILES))
@pytest.mark.parametrize("ksteps", [2, 4, 6, 8, 14])
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


# ---- the copy-wave protocol (configuration 31, gsr_interleave16c.hpp) -----------

def copy_wave_program(ksteps: int, a_before_barrier: bool = False, wait=8) -> list:
    """Copy waves' issue order: stage 0 and 1 copies, wait, prologue barrier;
    per K-step t the B(t+2) copies, the wait, barrier b_t and the A(t+2)
    copies; then a full drain and the epilogue's barrier."""
    ev = [("copy", "A", 0, 0)] * 4 + [("copy", "B", 0, 0)] * 8 + [("copy", "A", 1, 1)] * 4 + [("copy", "B", 1, 1)] * 8
    ev += [("wait", 12), ("barrier",)]
    for t in range(ksteps):
        ev += [("copy", "B", (t + 2) % 3, t + 2)] * 8
        if a_before_barrier:
            ev += [("copy", "A", t % 2, t + 2)] * 4
        ev += [("wait", wait), ("barrier",)]
        if not a_before_barrier:
            ev += [("copy", "A", t % 2, t + 2)] * 4
    return ev + [("wait", 0), ("barrier",)]


def mfma_wave_reads(ksteps: int) -> list:
    """MFMA waves' stage reads per barrier interval: (interval, operand,
    stage, K-step of the data).  Interval j follows the j-th barrier of the
    kernel (the prologue's is the first, b_t the (t+2)-th)."""
    reads = [(1, "A", 0, 0), (1, "B", 0, 0)]  # step 0's substep-0 operands
    for t in range(ksteps):
        reads += [(t + 1, "A", t % 2, t), (t + 1, "B", t % 3, t)]                    # substep 0, for substep 1
        reads += [(t + 2, "A", (t + 1) % 2, t + 1), (t + 2, "B", (t + 1) % 3, t + 1)]  # after b_t
    return reads


def check_copy_waves(ksteps: int, **kw) -> None:
    ev = copy_wave_program(ksteps, **kw)
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
    for j, op, st, step in mfma_wave_reads(ksteps):
        assert landed_at[j].get((op, st)) == step, f"{op} stage {st} read in interval {j} before step {step} landed"
        assert (op, st) not in written_in.get(j, set()), f"{op} stage {st} copied into while it is read (interval {j})"


@pytest.mark.parametrize("ksteps", [2, 4, 6, 8, 14])
def test_copy_wave_protocol(ksteps):
    check_copy_waves(ksteps)


@pytest.mark.parametrize("mistake", [{"a_before_barrier": True}, {"wait": 12}],
                         ids=["A-copies-before-the-barrier", "wait-too-loose"])
def test_copy_wave_model_catches_planted_mistakes(mistake):
    with pytest.raises(AssertionError):
        check_copy_waves(8, **mistake)
