"""The scheduled assembly of the bf16 wide attention sweep (gen_wide_substep.py), checked on the
CPU by a symbolic simulation of its instruction streams.

Every register is tagged with what it holds (the K operand of contraction step st of the
scores of sub-step u, the V^T operand of key half t and d block db of sub-step u, a raw /
scaled / exponentiated score of sub-step u, a bf16 weight pair, a partial row sum).  Over a
chain of pipelined sub-steps -- a first one, several more and the flush, as the kernel runs
them -- the simulation checks that each score product takes the K operand and Q operand of
its own contraction step, that each value product pairs the V^T operand and the weights of
the same sub-step and key half, that every (sub-step, key half, d block) product happens
exactly once, that every score is scaled and exponentiated once before its bf16 conversion,
that every weight enters the row sum exactly once, and that no register is read before it
is written.  The softmax these instructions compute is the windowed one of the ReHyAt blog
(maplevalley.com.cn), section 2.2.1; its values are checked against the oracle on the GPU.
"""
import os
import re
import sys

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "hybrid_softmax_linear_chunked_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_wide_substep as g  # noqa: E402


def regs(spec):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return list(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", spec)
    return [int(m.group(1))] if m else []


class Sim:
    def __init__(self, L):
        self.L = L
        R = L["reg"]
        self.R = R
        self.tag = {}
        for st in range(L["NS"]):
            for j in range(4):
                self.tag[R["Q"] + 4 * st + j] = ("Q", st)
        self.products = []
        self.sums = {}        # sub-step -> list of score indices added to l
        self.partial = {}     # T register -> (u, set of score indices)

    def run(self, lines, u, vextra, kextra):
        L, R = self.L, self.R
        VLD, KLD, NDB = L["VLD"], L["KLD"], L["NDB"]
        for line in lines:
            op, _, rest = line.partition(" ")
            args = [a.strip() for a in rest.split(",")] if rest else []
            if op == "ds_read_b64_tr_b16":
                off = int(re.search(r"offset:(\d+)", line).group(1)) - vextra
                hi = 0
                if off >= 8 * VLD * 2 and (off - 8 * VLD * 2) % 2 == 0 and ((off - 8 * VLD * 2) // 2) // (16 * VLD) * 16 * VLD + ((off - 8 * VLD * 2) // 2) % (16 * VLD) == (off - 8 * VLD * 2) // 2:
                    pass
                # decode (t, db, half) from the element offset 16 t VLD + db 32 (+ 8 VLD)
                e = off // 2
                t = e // (16 * VLD)
                rem = e - t * 16 * VLD
                if rem >= 8 * VLD:
                    hi, rem = 1, rem - 8 * VLD
                assert rem % 32 == 0, line
                db = rem // 32
                for r in regs(args[0]):
                    self.tag[r] = ("V", u, t, db, hi)
            elif op == "ds_read_b128":
                off = int(re.search(r"offset:(\d+)", line).group(1)) - kextra
                assert off % 32 == 0
                for r in regs(args[0]):
                    self.tag[r] = ("K", u + 2, off // 32)
            elif op == "v_mfma_f32_32x32x16_bf16":
                d, a, b, c = args
                dr, ar, br = regs(d), regs(a), regs(b)
                for r in ar + br:
                    assert r in self.tag, f"{line}: v{r} read before written"
                if R["SA"] <= dr[0] < R["O"]:
                    # score product: K operand of step st of sub-step (u+1) with Q step st
                    ka, qa = self.tag[ar[0]], self.tag[br[0]]
                    assert ka[0] == "K" and ka[1] == u + 1, (line, ka)
                    assert qa == ("Q", ka[2]), (line, qa)
                    assert all(self.tag[r] == ka for r in ar) and all(self.tag[r] == qa for r in br)
                    if c == "0":
                        acc = {"u": u + 1, "steps": {ka[2]}}
                    else:
                        prev = self.tag[dr[0]]
                        assert prev[0] == "Sacc" and prev[1] == u + 1, (line, prev)
                        acc = {"u": u + 1, "steps": set(prev[2]) | {ka[2]}}
                        assert ka[2] not in prev[2]
                    full = acc["steps"] == set(range(L["NS"]))
                    for i, r in enumerate(dr):
                        self.tag[r] = ("S", u + 1, i, "raw") if full else ("Sacc", u + 1, frozenset(acc["steps"]))
                else:
                    # value product into O block db: V^T (u', t, db) with weights (u', t)
                    vt = [self.tag[r] for r in ar]
                    pt = [self.tag[r] for r in br]
                    assert vt[0][0] == "V" and [x[4] for x in vt] == [0, 0, 1, 1], (line, vt)
                    uu, t, db = vt[0][1:4]
                    assert all(x[1:4] == (uu, t, db) for x in vt), (line, vt)
                    assert dr[0] == R["O"] + 16 * db and c == d, line
                    for j, x in enumerate(pt):
                        assert x == ("P", uu, t, j), (line, pt)
                    self.products.append((uu, t, db))
            elif op == "v_fma_f32":
                (r,) = regs(args[0])
                x = self.tag.get(r)
                assert x and x[0] == "S" and x[3] == "raw" and x[1] == u, (line, x)
                assert args[2] == "%[sc]" and args[3] == "-%[m]"
                self.tag[r] = ("S", u, x[2], "scaled")
            elif op == "v_exp_f32":
                (r,) = regs(args[0])
                x = self.tag.get(r)
                assert x and x[3] == "scaled" and x[1] == u, (line, x)
                self.tag[r] = ("S", u, x[2], "p")
            elif op == "v_cvt_pk_bf16_f32":
                (p,) = regs(args[0])
                x0, x1 = self.tag[regs(args[1])[0]], self.tag[regs(args[2])[0]]
                assert x0[3] == x1[3] == "p" and x0[1] == x1[1] == u, (line, x0, x1)
                # register r of the C tile is contraction slot r of the weight operand
                assert x1[2] == x0[2] + 1 and x0[2] % 2 == 0
                t, j = x0[2] // 8, (x0[2] % 8) // 2
                assert p == R["P"] + 4 * t + j, line
                self.tag[p] = ("P", u, t, j)
            elif op == "v_add_f32":
                dst = args[0]
                srcs = args[1:]
                if dst == "%[l]":
                    (tr,) = regs(srcs[1])
                    uu, idx = self.partial.pop(tr)
                    self.sums.setdefault(uu, []).extend(idx)
                    continue
                (dr,) = regs(dst)
                parts = []
                for sreg in srcs:
                    (sr,) = regs(sreg)
                    x = self.tag.get(sr)
                    if x and x[0] == "S":
                        assert x[3] == "p", (line, x)
                        parts.append((x[1], [x[2]]))
                    else:
                        parts.append(self.partial.pop(sr))
                uu = {p[0] for p in parts}
                assert len(uu) == 1, line
                self.partial[dr] = (uu.pop(), sum((p[1] for p in parts), []))
                self.tag[dr] = ("T",)
            elif op in ("s_waitcnt", "s_nop", "s_mov_b32", "s_add_u32", "s_mov_b64", "global_load_lds_dwordx4"):
                continue
            else:
                raise AssertionError(f"unexpected instruction {line}")


@pytest.mark.parametrize("D", [32, 64, 128])
def test_pipelined_sweep_dataflow(D):
    L = g.layout(D)
    sim = Sim(L)
    VX, KX = 32 * L["VLD"] * 2, 32 * L["KLD"] * 2
    # scores of sub-step 0 and the K operands of sub-step 1, as the kernel's prologue leaves them
    for i in range(16):
        sim.tag[L["reg"]["SA"] + i] = ("S", 0, i, "raw")
    for st in range(L["NS"]):
        for j in range(4):
            sim.tag[L["reg"]["K"] + 4 * st + j] = ("K", 1, st)
    n = 6
    for u in range(n):
        b = g.Block()
        g.pipe_substep(b, L, u % 2, "va", "ka", VX * (u % 2), KX * (u % 2), first=(u == 0))
        sim.run(b.lines, u, VX * (u % 2), KX * (u % 2))
    b = g.Block()
    g.pipe_flush(b, L)
    sim.run(b.lines, n - 1, 0, 0)
    want = sorted((u, t, db) for u in range(n) for t in (0, 1) for db in range(L["NDB"]))
    assert sorted(sim.products) == want
    for u in range(n):
        assert sorted(sim.sums.get(u, [])) == list(range(16)), (u, sim.sums.get(u))


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("stream", [False, True])
def test_loop_copies_slots_and_waits(D, stream):
    # The loop body holds the four ring phases of a sweep position (slots counted from the
    # workgroup's first position p0; the loop starts at p0 + 1, phase 1).  Each position issues
    # this wave's share of one K and one V tile copy, into slots (ph + 3) & 3 and (ph + 2) & 3,
    # reads V^T of slot ph and K of slot (ph + 1) & 3, waits for the previous position's copies
    # with the count of the wave with the fewest, waits for every LDS read, and meets the
    # barrier once.
    L = g.layout(D)
    text = g.cxx_loop(D, stream)
    body = re.search(r'asm volatile\("(.*?)"\n', text, re.S).group(1).split("\\n\\t")
    start = body.index("1:")
    bars = [i for i, l in enumerate(body) if l == "s_barrier"]
    assert len(bars) == 4
    KB, VB = L["K_BYTES"], L["V_BYTES"]
    VX, KX = 32 * L["VLD"] * 2, 32 * L["KLD"] * 2
    R = L["reg"]
    VA0, VA2, KA = R["T"] + 4, R["T"] + 5, R["T"] + 6
    prev = start
    for ph, bar in zip((1, 2, 3, 0), bars):
        pos = body[prev:bar]
        m0 = [l for l in pos if l.startswith("s_add_u32 m0")]
        assert len(m0) == L["PWK"] + L["PWV"]
        assert all(l.endswith(f", {((ph + 3) & 3) * KB}") for l in m0[:L["PWK"]]), m0
        assert all(l.endswith(f", {((ph + 2) & 3) * VB}") for l in m0[L["PWK"]:]), m0
        vreads = [l for l in pos if l.startswith("ds_read_b64_tr_b16")]
        base = f"v{VA0}" if ph < 2 else f"v{VA2}"
        for l in vreads:
            off = int(l.rsplit("offset:", 1)[1])
            assert f", {base} " in l and (ph % 2) * VB <= off < (ph % 2) * VB + VB, l
        kreads = [l for l in pos if l.startswith("ds_read_b128")]
        for l in kreads:
            off = int(l.rsplit("offset:", 1)[1])
            k0 = ((ph + 1) & 3) * KB
            assert f", v{KA} " in l and k0 <= off < k0 + KB, l
        assert len(vreads) == 2 * 2 * L["NV"] and len(kreads) == 2 * L["NS"]
        tail = body[max(i for i, l in enumerate(body[:bar]) if l.startswith("ds_read")):bar]
        assert "s_waitcnt lgkmcnt(0)" in tail
        assert body[bar - 1] == f"s_waitcnt vmcnt({L['NIK'] // g.NW + L['NIV'] // g.NW})"
        prev = bar


def test_generated_file_is_current():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(CSRC, "gen_wide_substep.py"), "--check"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
