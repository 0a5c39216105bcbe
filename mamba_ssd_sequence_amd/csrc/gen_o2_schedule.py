"""Slot schedule of the order-2 state scan's MFMA work (fwd_o2_state.hip).

    python gen_o2_schedule.py            # rewrite the two generated blocks
    python gen_o2_schedule.py --print    # print them

A wave issues in order, so the kernel interleaves its VALU work with its
MFMA chains by hand: slot s holds one MFMA, up to two VALU units (four
instructions each) and up to one or two 16-byte LDS operand reads, and
scheduling barriers keep the compiler from regrouping slots.  This script
places the work of one step (two 64-token blocks) with earliest-deadline-
first list scheduling, from the dependencies below, and writes the slot
lines between the markers in fwd_o2_state.hip.

Chains (4 MFMAs each, k-steps kk = 0..3):
  out(at, t, kk)       output product of a-tile at over token tile t
  upd(at, bt, hb, kk)  update of a-tile at, b-tile bt with block hb
VALU units:
  cvt(SA, at, kk)  fp16 copy of the state (the first a-tile's copy for the
                   next step is made after its last update)
  mul(at, bt, g)   decay, before the tile's first update
  fy(at, t, m)     row scalings, three or more slots after the chain, and
                   always before the outputs are written
  bu(at, hb, kk)   update operand, three slots after its reads
LDS reads: rdQ(t, kk), rdK(bt, hb, kk), rdX(hb, kk), a few slots before use.
One a-tile per wave (NAT = 1) uses these chains; two a-tiles per wave use
schedule_sym (three state tiles, the state being symmetric in (a, b)).
"""
import heapq
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL = os.path.join(HERE, "fwd_o2_state.hip")


def edf(items, ns, cap0, lo, maxcap):
    """Earliest-deadline-first placement of (name, release, deadline, prio)
    items into slots lo..ns-1; slot capacities grow (up to maxcap) where a
    deadline would be missed.  Returns ({slot: [names]}, [names after the last slot])."""
    cap = dict(cap0)
    while True:
        placed = {s: [] for s in range(lo, ns)}
        pend, order, ui, miss = [], sorted(items, key=lambda u: u[1]), 0, None
        for s in range(lo, ns):
            while ui < len(order) and order[ui][1] <= s:
                heapq.heappush(pend, (order[ui][2], order[ui][3], ui, order[ui]))
                ui += 1
            for _ in range(cap.get(s, 1)):
                if pend:
                    d, _, _, u = heapq.heappop(pend)
                    placed[s].append(u[0])
                    if d < s:
                        miss = u
                        break
            if miss:
                break
        if miss is None:
            while ui < len(order):
                heapq.heappush(pend, (order[ui][2], order[ui][3], ui, order[ui]))
                ui += 1
            tail = [heapq.heappop(pend)[3] for _ in range(len(pend))]
            late = [u for u in tail if u[2] < ns]
            if not late:
                return placed, [u[0] for u in tail]
            miss = late[0]
        cand = [x for x in range(max(miss[1], 0), min(miss[2], ns - 1) + 1) if cap.get(x, 1) < maxcap]
        if not cand:
            raise SystemExit(f"no feasible schedule for {miss}")
        low = min(cap.get(x, 1) for x in cand)
        x = [x for x in cand if cap.get(x, 1) == low][-1]
        cap[x] = cap.get(x, 1) + 1


def schedule(nat, order, lq=3, lk=4, fd=7, front=True):
    chains = []
    if order == "split":  # all output chains, then all updates
        for t in range(4):
            chains += [("C", at, t) for at in range(nat)]
        for hb in range(2):
            chains += [("U", at, bt, hb) for at in range(nat) for bt in range(2)]
    else:  # per block: its two token tiles, then its updates
        for hb in range(2):
            for t in (2 * hb, 2 * hb + 1):
                chains += [("C", at, t) for at in range(nat)]
            chains += [("U", at, bt, hb) for at in range(nat) for bt in range(2)]
    ns = 4 * len(chains)
    start = {c: 4 * i for i, c in enumerate(chains)}
    mf = [f"out({c[1]}, {c[2]}, {kk});" if c[0] == "C" else f"upd({c[1]}, {c[2]}, {c[3]}, {kk});"
          for c in chains for kk in range(4)]
    first_u = {hb: min(start[("U", at, bt, hb)] for at in range(nat) for bt in range(2)) for hb in range(2)}
    reads = []
    for t in range(1, 4):
        for kk in range(4):
            need = start[("C", 0, t)] + kk
            reads.append((f"rdQ({t}, {kk});", need - lq - 6, need - lq, 0))
    for hb in range(2):
        for kk in range(4):
            d = first_u[hb] - lk + kk
            reads += [(f"rdK({bt}, {hb}, {kk});", d - 8, d, 1) for bt in range(2)]
            reads.append((f"rdX({hb}, {kk});", d - 8, d, 1))
    rplaced, rtail = edf(reads, ns, {-1: 4}, -1, 2)
    assert not rtail
    rslot = {n: s for s, v in rplaced.items() for n in v}
    units = []
    if nat == 2:
        units += [(f"cvt(SA1, 1, {kk});", -1, start[("C", 1, 0)] - 1, 2) for kk in range(4)]
    for at in range(nat):
        for t in range(4):
            r = start[("C", at, t)] + 6
            units += [(f"fy({at}, {t}, {m});", r, min(r + fd, ns - 2), 0) for m in range(4)]
    for at in range(nat):
        for bt in range(2):
            r = 0 if at == 0 else start[("C", 1, 0)] - 2
            units += [(f"mul({at}, {bt}, {g});", r, start[("U", at, bt, 0)] - 1, 1) for g in range(4)]
    for hb in range(2):
        for at in range(nat):
            for kk in range(4):
                r = max(rslot[f"rdK({at}, {hb}, {kk});"], rslot[f"rdX({hb}, {kk});"]) + 3
                units.append((f"bu({at}, {hb}, {kk});", r, start[("U", at, 0, hb)] + kk - 1, 3))
    for kk in range(4):
        units.append((f"cvt(SA0, 0, {kk});", start[("U", 0, kk >> 1, 1)] + 6, 10 ** 6, 4))
    cap = {-1: 2}
    if front:
        for x in range(0, ns // 2, 2):
            cap[x + 1] = 2
    placed, tail = edf(units, ns, cap, -1, 3)
    assert all(u.startswith("cvt(SA0") for u in tail), tail
    lastfy = max(s for s, v in placed.items() if any(u.startswith("fy(") for u in v))
    assert lastfy < ns - 1
    lines = ["rdQ(0, 0); rdQ(0, 1); rdQ(0, 2); rdQ(0, 3); " + " ".join(rplaced.get(-1, []) + placed[-1]) + " SB();"]
    for s in range(ns):
        w = ["wr();"] if s == lastfy + 1 else []
        lines.append(" ".join([mf[s]] + placed[s] + rplaced.get(s, []) + w) + " SB();")
    if tail:
        lines.append(" ".join(tail) + " SB();")
    return ["      " + re.sub(r"\s+", " ", l).strip() for l in lines]


def schedule_sym(lq=3, lk=4, fd=7):
    """Two a-tiles per wave with the state's symmetry: the tiles (b-tile 0,
    a-tile 0), (0, 1) and (1, 1) are held; (1, 0) is the transpose of (0, 1).
    Output chains: out(0, t, kk) over kk = 0, 1 (tile (0, 0)); outp(t, j),
    j = 0..5, the hi and lo parts of twice tile (0, 1) over kk = 0, 1, then
    tile (1, 1) over kk = 2, 3.  Updates: upd(at, bt, hb, kk) for the three
    tiles.  VALU units: cvh(kk, p), the hi / lo parts of twice tile (0, 1)
    (two of the eight values of k-step kk per unit); cvt(SA1, 1, kk), kk =
    2, 3; mul for the three tiles; fy and bu as above; cvt(SA0, 0, kk), kk =
    0, 1, after the last update of tile (0, 0)."""
    chains = []
    for t2 in (0, 2):
        chains += [("C0", t2), ("C0", t2 + 1), ("C1", t2), ("C1", t2 + 1)]
    for hb in range(2):
        chains += [("U", 0, 0, hb), ("U", 1, 0, hb), ("U", 1, 1, hb)]
    length = {"C0": 2, "C1": 6, "U": 4}
    start, s0 = {}, 0
    for c in chains:
        start[c] = s0
        s0 += length[c[0]]
    ns = s0
    mf = []
    for c in chains:
        if c[0] == "C0":
            mf += [f"out(0, {c[1]}, {kk});" for kk in range(2)]
        elif c[0] == "C1":
            mf += [f"outp({c[1]}, {j});" for j in range(6)]
        else:
            mf += [f"upd({c[1]}, {c[2]}, {c[3]}, {kk});" for kk in range(4)]
    # first use of Q fragment (t, kk): kk 0, 1 by out(0, t, kk), kk 2, 3 by outp(t, 4 + kk - 2)
    first_u = {hb: start[("U", 0, 0, hb)] for hb in range(2)}
    reads = []
    for t in range(1, 4):
        for kk in range(4):
            need = start[("C0", t)] + kk if kk < 2 else start[("C1", t)] + 4 + kk - 2
            reads.append((f"rdQ({t}, {kk});", need - lq - 6, need - lq, 0))
    for hb in range(2):
        for kk in range(4):
            d = first_u[hb] - lk + kk
            reads += [(f"rdK({bt}, {hb}, {kk});", d - 8, d, 1) for bt in range(2)]
            reads.append((f"rdX({hb}, {kk});", d - 8, d, 1))
    rplaced, rtail = edf(reads, ns, {-1: 4}, -1, 2)
    assert not rtail
    rslot = {n: s for s, v in rplaced.items() for n in v}
    c1 = start[("C1", 0)]
    units = []
    units += [(f"cvh({kk}, {p});", -1, c1 + kk - 1, 2) for kk in range(2) for p in range(4)]
    units += [(f"cvt(SA1, 1, {kk});", -1, c1 + 4 + kk - 2 - 1, 2) for kk in (2, 3)]
    for t in range(4):
        r = start[("C0", t)] + length["C0"] + 2
        units += [(f"fy(0, {t}, {m});", r, min(r + fd, ns - 2), 0) for m in range(4)]
        r = start[("C1", t)] + length["C1"] + 2
        units += [(f"fy(1, {t}, {m});", r, min(r + fd, ns - 2), 0) for m in range(4)]
    for (at, bt, r) in ((0, 0, 0), (1, 0, c1), (1, 1, c1 + 6)):
        units += [(f"mul({at}, {bt}, {g});", r, start[("U", at, bt, 0)] - 1, 1) for g in range(4)]
    for hb in range(2):
        for at in range(2):
            for kk in range(4):
                r = max(rslot[f"rdK({at}, {hb}, {kk});"], rslot[f"rdX({hb}, {kk});"]) + 3
                units.append((f"bu({at}, {hb}, {kk});", r, start[("U", at, 0, hb)] + kk - 1, 3))
    for kk in range(2):
        units.append((f"cvt(SA0, 0, {kk});", start[("U", 0, 0, 1)] + 6, 10 ** 6, 4))
    cap = {-1: 2}
    for x in range(0, ns // 2, 2):
        cap[x + 1] = 2
    placed, tail = edf(units, ns, cap, -1, 3)
    assert all(u.startswith("cvt(SA0") for u in tail), tail
    lastfy = max(s for s, v in placed.items() if any(u.startswith("fy(") for u in v))
    assert lastfy < ns - 1
    lines = ["rdQ(0, 0); rdQ(0, 1); rdQ(0, 2); rdQ(0, 3); " + " ".join(rplaced.get(-1, []) + placed[-1]) + " SB();"]
    for s in range(ns):
        w = ["wr();"] if s == lastfy + 1 else []
        lines.append(" ".join([mf[s]] + placed[s] + rplaced.get(s, []) + w) + " SB();")
    if tail:
        lines.append(" ".join(tail) + " SB();")
    return ["      " + re.sub(r"\s+", " ", l).strip() for l in lines]


def main():
    blocks = {2: schedule_sym(), 1: schedule(1, "inter", front=False)}
    if "--print" in sys.argv:
        for nat, lines in blocks.items():
            print(f"// {nat} a-tile(s)\n" + "\n".join(lines))
        return
    src = open(KERNEL).read()
    for nat, lines in blocks.items():
        pat = re.compile(rf"(      // -- generated schedule, {nat} a-tiles? per wave --\n)(.*?)(      // -- end of generated schedule --\n)", re.S)
        src, n = pat.subn(lambda m: m.group(1) + "\n".join(lines) + "\n" + m.group(3), src)
        assert n == 1, nat
    open(KERNEL, "w").write(src)


if __name__ == "__main__":
    main()
