"""Writes wide_substep.inc: the sweep of the bf16 wide attention kernel as scheduled gfx950
assembly (ReHyAt blog, maplevalley.com.cn, 2.2.1: the windowed softmax part of the hybrid).

One sub-step u of a wave (32 queries, 32 keys) is:
  phase A: the score products of sub-step u+1 (S_next = K_{u+1} Q^T, D/16 MFMAs) with the
           softmax of S_cur interleaved (p = exp2(s * scale - m), bf16 pairs for the value
           product, fp32 row sums as pairwise trees), and the 2 * D/16 transposing LDS reads
           of the V^T operands of u;
  phase B: the value products O^T += V_u^T P^T (D/16 MFMAs) with the LDS reads of the K
           operands of sub-step u+2 and this wave's share of one tile copy (LDS-DMA).
Every LDS read completes inside the sub-step.  Two forms are generated:
  wide_substep<D, PAR, 0>  one sub-step without a copy (the first sweep position, whose copies
                           the caller issues);
  wide_loop<D, STREAM>     sweep positions i0 .. iend-1: per position the copy addresses (K of
                           tile i+3, V of tile i+2, clamped to the last tile; in a streaming
                           window the segment holding the tile), sub-steps 2i (with the K copy)
                           and 2i+1 (with the V copy), the wait for the copies issued one
                           position earlier, and the workgroup barrier.
Registers are pinned (S_a, S_b, O, Q, K as operands; V, P and temporaries as clobbers, and
the 64-bit scalar pointers) so that each instruction names its registers.  The generator
checks the gfx950 dependency distances it relies on: a transcendental result is not read by
the next instruction, a VALU result is read by an MFMA at least three instructions later,
and an LDS read is waited for before its first use.

Run by the build; the output is committed beside the kernel.
"""
from __future__ import annotations

import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "wide_substep.inc")
NW = 8  # waves per workgroup (two per SIMD)
SP = 80  # first pinned scalar register: k1, v1, k2, v2 (inputs), kb, vb (copy sources)


def layout(D):
    NS = D // 16            # score products (contraction steps of 16 over d)
    NDB = D // 32           # 32-wide d blocks of O
    NV = 2 * NDB            # value products: 2 steps of 16 keys x NDB d blocks
    r = {"SA": 0, "SB": 16, "O": 32}
    r["Q"] = r["O"] + 16 * NDB
    r["K"] = r["Q"] + 4 * NS
    r["V"] = r["K"] + 4 * NS
    r["P"] = r["V"] + 4 * NV
    r["T"] = r["P"] + 8      # T..T+3 row-sum tree, T+4 V^T address, T+5 K address
    r["END"] = r["T"] + 8
    KLD = D + 8
    VLD = {128: 160, 64: 96, 32: 32}[D]
    CPK, CPV = KLD // 8, VLD // 8
    NIK, NIV = CPK, CPV       # DMA instructions per 64-token tile
    PWK, PWV = -(-NIK // NW), -(-NIV // NW)
    return dict(D=D, NS=NS, NDB=NDB, NV=NV, reg=r, KLD=KLD, VLD=VLD, NIK=NIK, NIV=NIV, PWK=PWK, PWV=PWV,
                K_BYTES=64 * KLD * 2, V_BYTES=64 * VLD * 2)


XDL_WAIT = 16  # wait states between an MFMA and a VALU access of its result (no interlock)


class Block:
    """Instruction list with the dependency checks."""

    def __init__(self):
        self.lines = []
        self.trans_last = {}    # vgpr -> index of the transcendental that wrote it
        self.valu_last = {}     # vgpr -> index of the VALU that wrote it
        self.xdl_last = {}      # vgpr -> index of the MFMA that wrote it
        self.lds_pending = []   # vgprs of LDS reads issued and not yet waited for, in order
        self.n = 0

    def emit(self, text):
        self.lines.append(text)
        self.n += 1

    def valu(self, dst, srcs, trans=False, text=None):
        for s in list(srcs) + [dst]:
            if s in self.xdl_last:
                gap = self.n - 1 - self.xdl_last[s]
                if gap < XDL_WAIT:
                    self.emit(f"s_nop {XDL_WAIT - 1 - gap}")
        for s in srcs:
            if s in self.trans_last and self.trans_last[s] == self.n - 1:
                self.emit("s_nop 0")
            self._check_lds(s)
        self.emit(text)
        if trans:
            self.trans_last[dst] = self.n - 1
        self.valu_last[dst] = self.n - 1

    def mfma(self, text, srcs, dsts=()):
        for s in srcs:
            self._check_lds(s)
            if s in self.valu_last:
                gap = self.n - 1 - self.valu_last[s]
                if gap < 3:
                    self.emit(f"s_nop {2 - gap}")
        self.emit(text)
        for d in dsts:
            self.xdl_last[d] = self.n - 1

    def settle_xdl(self):
        # pad so that compiler code after the block may access every MFMA result
        if self.xdl_last:
            gap = self.n - 1 - max(self.xdl_last.values())
            if gap < XDL_WAIT:
                self.emit(f"s_nop {XDL_WAIT - 1 - gap}")

    def lds(self, text, dsts, addr=None):
        if addr is not None and addr in self.valu_last and self.valu_last[addr] == self.n - 1:
            self.emit("s_nop 0")
        self.emit(text)
        self.lds_pending.append(set(dsts))

    def _check_lds(self, reg):
        for i, s in enumerate(self.lds_pending):
            if reg in s:
                keep = len(self.lds_pending) - i - 1
                self.emit(f"s_waitcnt lgkmcnt({min(keep, 15)})")
                self.lds_pending = self.lds_pending[i + 1:]
                return

    def wait_all_lds(self):
        if self.lds_pending:
            self.emit("s_waitcnt lgkmcnt(0)")
            self.lds_pending = []


def v(i):
    return f"v{i}"


def vr(a, n):
    return f"v[{a}:{a + n - 1}]"


def row_sum_pair(b, L, par, j):
    # pair j of S_cur (already exponentiated) into the running row sum: pair sums, then per
    # 8 values ((a0 + a1) + (a2 + a3)) added to the sum
    R = L["reg"]
    T = R["T"]
    sc_base = R["SA"] if par == 0 else R["SB"]
    x0, x1 = sc_base + 2 * j, sc_base + 2 * j + 1
    a = T + (j % 4)
    b.valu(a, [x0, x1], text=f"v_add_f32 {v(a)}, {v(x0)}, {v(x1)}")
    if j % 4 == 3:
        b.valu(T, [T, T + 1], text=f"v_add_f32 {v(T)}, {v(T)}, {v(T + 1)}")
        b.valu(T + 2, [T + 2, T + 3], text=f"v_add_f32 {v(T + 2)}, {v(T + 2)}, {v(T + 3)}")
        b.valu(T, [T, T + 2], text=f"v_add_f32 {v(T)}, {v(T)}, {v(T + 2)}")
        b.valu("l", [T], text=f"v_add_f32 %[l], %[l], {v(T)}")


def pipe_substep(b, L, par, vaddr, kaddr, vextra=0, kextra=0, dma=None, first=False, defer=True):
    """One sub-step u in the pipelined order.  The value products of u are split by key half
    t: t = 0 runs in this sub-step, t = 1 (its V^T operands read in this sub-step) runs in the
    next one (first: none pending from a previous sub-step; defer=False: run it at the end
    instead).  MFMA order, NDB = D/32:
        S_0 D_0 S_1 D_1 .. S_(NDB-1) D_(NDB-1) | S_NDB P_0 .. S_(2NDB-1) P_(NDB-1)
    S_st: score product st of u+1 (its K operand register is reloaded for u+2 right after);
    D_j: value product (t = 1, d block j) of u-1 (its V^T register is reloaded with t = 1 of u
    right after); P_j: value product (t = 0, d block j) of u.  The softmax of u is spread over
    the products: value r next to product r (16 // products per product), its bf16 pair and row
    sum one product later; P (t = 0) of u is complete before P_0, and P (t = 1) of u is written
    after the last D_j read the previous one.  dma: copy instructions after the last products."""
    R = L["reg"]
    NS, NDB, NV, VLD = L["NS"], L["NDB"], L["NV"], L["VLD"]
    sc_base = R["SA"] if par == 0 else R["SB"]
    sn_base = R["SB"] if par == 0 else R["SA"]
    P = R["P"]
    dma = dma or []
    order = []
    for st in range(NDB):
        order.append(("S", st))
        if not first:
            order.append(("D", st))
    for st in range(NDB, NS):
        order.append(("S", st))
        order.append(("P", st - NDB))
    if not defer:
        for j in range(NDB):
            order.append(("Q", j))   # t = 1 value products of u, at the end
    nslots = len(order)
    # softmax values per slot: values 0..7 (the t = 0 weights) over the slots before the first
    # t = 0 product, values 8..15 over the rest
    first_p = next(k for k, (kind, _) in enumerate(order) if kind == "P")
    plan = [[] for _ in range(nslots)]
    for r in range(8):
        plan[r * first_p // 8].append(r)
    for r in range(8, 16):
        plan[first_p + (r - 8) * (nslots - first_p) // 8].append(r)

    def vread(i, t):
        # V^T operand frag (t, db = i % NDB) of u into register block V + 4 * (t * NDB + db)
        db = i
        base = R["V"] + 4 * (t * NDB + db)
        off = (16 * t * VLD + db * 32) * 2 + vextra
        b.lds(f"ds_read_b64_tr_b16 {vr(base, 2)}, {vaddr} offset:{off}", [base, base + 1], addr=vaddr)
        b.lds(f"ds_read_b64_tr_b16 {vr(base + 2, 2)}, {vaddr} offset:{off + 8 * VLD * 2}", [base + 2, base + 3], addr=vaddr)

    def finish_pair(j):
        # weights 2j, 2j+1: bf16 pair into P (operand t = j // 4, register j % 4), row sum
        x0, x1 = sc_base + 2 * j, sc_base + 2 * j + 1
        p = P + 4 * (j // 4) + (j % 4)
        b.valu(p, [x0, x1], text=f"v_cvt_pk_bf16_f32 {v(p)}, {v(x0)}, {v(x1)}")
        row_sum_pair(b, L, par, j)

    pending_pairs = []
    done_vals = []
    t0_reads = list(range(NDB))   # t = 0 frags of u, read early
    # t = 1 frags of u: after the deferred product D_j frees their registers; a first sub-step
    # (no deferred products) reads them in its score slots after the t = 0 frags
    t1_reads = list(range(NDB)) if first else []
    dma_left = list(dma)
    for k, (kind, idx) in enumerate(order):
        if kind == "S":
            kreg, qreg = R["K"] + 4 * idx, R["Q"] + 4 * idx
            c = "0" if idx == 0 else vr(sn_base, 16)
            b.mfma(f"v_mfma_f32_32x32x16_bf16 {vr(sn_base, 16)}, {vr(kreg, 4)}, {vr(qreg, 4)}, {c}", [kreg, qreg],
                   range(sn_base, sn_base + 16))
            base = R["K"] + 4 * idx
            b.lds(f"ds_read_b128 {vr(base, 4)}, {kaddr} offset:{idx * 32 + kextra}", [base, base + 1, base + 2, base + 3], addr=kaddr)
        elif kind in ("D", "P", "Q"):
            t = 1 if kind in ("D", "Q") else 0
            if kind == "P":
                # the t = 0 weights of u are complete before their first product
                for j in [j for j in pending_pairs if j < 4]:
                    finish_pair(j)
                    pending_pairs.remove(j)
            vreg, oreg, preg = R["V"] + 4 * (t * NDB + idx), R["O"] + 16 * idx, P + 4 * t
            b.mfma(f"v_mfma_f32_32x32x16_bf16 {vr(oreg, 16)}, {vr(vreg, 4)}, {vr(preg, 4)}, {vr(oreg, 16)}",
                   [vreg, preg, preg + 1, preg + 2, preg + 3], range(oreg, oreg + 16))
            if kind == "D":
                vread(idx, 1)
        if kind == "S":
            if t0_reads:
                vread(t0_reads.pop(0), 0)
            elif t1_reads:
                vread(t1_reads.pop(0), 1)
        # softmax work of this slot: the pairs finished one slot ago, then new values
        for j in pending_pairs:
            finish_pair(j)
        rs = plan[k]
        for r in rs:
            x = sc_base + r
            b.valu(x, [x], text=f"v_fma_f32 {v(x)}, {v(x)}, %[sc], -%[m]")
        for r in rs:
            x = sc_base + r
            b.valu(x, [x], trans=True, text=f"v_exp_f32 {v(x)}, {v(x)}")
        done_vals += rs
        pending_pairs = []
        while len(done_vals) >= 2 and done_vals[0] % 2 == 0 and done_vals[1] == done_vals[0] + 1:
            pending_pairs.append(done_vals[0] // 2)
            done_vals = done_vals[2:]
        if dma_left and k >= nslots - len(dma_left):
            for line in dma_left.pop(0)():
                b.emit(line)
    while t0_reads:
        vread(t0_reads.pop(0), 0)
    while t1_reads:
        vread(t1_reads.pop(0), 1)
    for j in pending_pairs:
        finish_pair(j)
    while dma_left:
        for line in dma_left.pop(0)():
            b.emit(line)


def pipe_flush(b, L):
    """The deferred value products (t = 1) of the last sub-step."""
    R = L["reg"]
    NDB, P = L["NDB"], L["reg"]["P"]
    for j in range(NDB):
        vreg, oreg, preg = R["V"] + 4 * (NDB + j), R["O"] + 16 * j, P + 4
        b.mfma(f"v_mfma_f32_32x32x16_bf16 {vr(oreg, 16)}, {vr(vreg, 4)}, {vr(preg, 4)}, {vr(oreg, 16)}",
               [vreg, preg, preg + 1, preg + 2, preg + 3], range(oreg, oreg + 16))


def pinned_outs(L):
    R = L["reg"]
    outs = [f'[sa] "+{{v[{R["SA"]}:{R["SA"] + 15}]}}"(sa)', f'[sb] "+{{v[{R["SB"]}:{R["SB"] + 15}]}}"(sb)']
    for db in range(L["NDB"]):
        a = R["O"] + 16 * db
        outs.append(f'[o{db}] "+{{v[{a}:{a + 15}]}}"(o[{db}][0])')
    for st in range(L["NS"]):
        a = R["K"] + 4 * st
        outs.append(f'[kf{st}] "+{{v[{a}:{a + 3}]}}"(k[{st}])')
    outs.append('[l] "+v"(lsum)')
    return outs


def pinned_ins(L):
    R = L["reg"]
    ins = []
    for st in range(L["NS"]):
        a = R["Q"] + 4 * st
        ins.append(f'[q{st}] "{{v[{a}:{a + 3}]}}"(q[0][{st}])')
    ins += ['[m] "v"(m)', '[sc] "s"(sc)']
    return ins


def pinned_vp(L):
    R = L["reg"]
    ops = []
    for i in range(L["NV"]):
        a = R["V"] + 4 * i
        ops.append(f'[vf{i}] "+{{v[{a}:{a + 3}]}}"(vf[{i}])')
    for t in range(2):
        a = R["P"] + 4 * t
        ops.append(f'[pf{t}] "+{{v[{a}:{a + 3}]}}"(pf[{t}])')
    return ops


def tclobbers(L):
    R = L["reg"]
    return [f'"v{i}"' for i in range(R["T"], R["END"])]


def asm_stmt(lines, outs, ins, clob, end=None, scalars=False):
    # first line: a comment naming the compiler-assigned operands and the pinned range (the
    # scalar range only where the block pins it), which a test checks in the compiled
    # kernel (no such operand may land in a pinned register)
    free = []
    for op in outs + ins:
        m = re.match(r'\[(\w+)\] "[=+&]*([vs])"', op)
        if m:
            free.append(f"{m.group(1)}=%[{m.group(1)}]")
    if end is not None:
        srange = f" s{SP}-s{SP + 11}" if scalars else ""
        lines = [f"; pinned v0-v{end - 1}{srange}; free " + " ".join(free)] + lines
    body = "\\n\\t".join(lines)
    return (f'    asm volatile("{body}"\n        : ' + ",\n          ".join(outs)
            + "\n        : " + ",\n          ".join(ins)
            + "\n        : " + ", ".join(clob) + ");\n")


def cxx_pipe(D, par, first):
    L = layout(D)
    b = Block()
    if not first:
        b.emit("s_nop 2")  # the P operands of the deferred products may have just been written
    pipe_substep(b, L, par, "%[vaddr]", "%[kaddr]", first=first)
    b.wait_all_lds()
    b.settle_xdl()
    ins = pinned_ins(L) + ['[vaddr] "v"(vaddr)', '[kaddr] "v"(kaddr)']
    return (f"template <> __device__ inline void wide_pipe<{D}, {par}, {str(first).lower()}>(WIDE_PIPE_ARGS({D})) {{\n"
            + asm_stmt(b.lines, pinned_outs(L) + pinned_vp(L), ins, tclobbers(L) + ['"memory"'], L["reg"]["END"]) + "}\n")


def cxx_flush(D):
    L = layout(D)
    b = Block()
    b.emit("s_nop 2")  # the P operands of the deferred products may have just been written
    pipe_flush(b, L)
    b.settle_xdl()
    outs = [o for o in pinned_outs(L) if not o.startswith("[l]")] + pinned_vp(L)
    return (f"template <> __device__ inline void wide_flush<{D}>(WIDE_FLUSH_ARGS({D})) {{\n"
            + asm_stmt(b.lines, outs, [], ['"memory"'], L["reg"]["END"]) + "}\n")


def cxx_loop(D, stream, no_barrier=False, no_dma=False):
    """The steady-state loop over sweep positions i0 .. iend-1, unrolled by the four ring slots.
    Slots count from the workgroup's first position p0 = i0 - 1 (position i uses V^T slot
    (i - p0) & 3, reads K of the next tile from slot (i - p0 + 1) & 3, and copies K of tile i+3
    into slot (i - p0 + 3) & 3 and V of tile i+2 into (i - p0 + 2) & 3), so the four unrolled
    positions have fixed slot offsets.  The copy sources run as token counters kt, vt (first
    tokens of the tiles to copy, 64 more per position, held at the last tile `ktl`); a
    streaming window's tile lies below token len1 in segment 1, else in segment 2.  Pipelined
    sub-steps: the deferred value products of sub-step 2*i0 - 1 are pending on entry, those of
    the last sub-step on exit.  no_barrier / no_dma: variants for timing the loop's parts."""
    L = layout(D)
    R = L["reg"]
    b = Block()
    K1, V1, K2, V2, KB, VB = SP, SP + 2, SP + 4, SP + 6, SP + 8, SP + 10
    s = lambda i: f"s{i}"
    VA0, VA2, KA = R["T"] + 4, R["T"] + 5, R["T"] + 6
    tok_shift = {128: 8, 64: 7, 32: 6}[D]   # bytes per token row = 2 D = 1 << tok_shift
    KB_, VB_ = L["K_BYTES"], L["V_BYTES"]

    def tile_src(which, dst):
        tok = "%[kt]" if which == "k" else "%[vt]"
        src1, src2 = (K1, K2) if which == "k" else (V1, V2)
        if stream:
            # (the selects read SCC of the compare; the shift after them writes SCC)
            b.emit(f"s_sub_i32 %[t1], {tok}, %[len1]")
            b.emit(f"s_cmp_lt_i32 {tok}, %[len1]")
            b.emit(f"s_cselect_b32 %[t1], {tok}, %[t1]")
            b.emit(f"s_cselect_b32 {s(dst)}, {s(src1)}, {s(src2)}")
            b.emit(f"s_cselect_b32 {s(dst + 1)}, {s(src1 + 1)}, {s(src2 + 1)}")
            b.emit(f"s_lshl_b32 %[t1], %[t1], {tok_shift}")
            b.emit(f"s_add_u32 {s(dst)}, {s(dst)}, %[t1]")
            b.emit(f"s_addc_u32 {s(dst + 1)}, {s(dst + 1)}, 0")
        else:
            b.emit(f"s_lshl_b32 %[t1], {tok}, {tok_shift}")
            b.emit(f"s_add_u32 {s(dst)}, {s(src1)}, %[t1]")
            b.emit(f"s_addc_u32 {s(dst + 1)}, {s(src1 + 1)}, 0")

    def copy_ops(which, slot):
        if no_dma:
            return []
        pw = L["PWK"] if which == "k" else L["PWV"]
        ni = L["NIK"] if which == "k" else L["NIV"]
        src = KB if which == "k" else VB
        off = slot * (KB_ if which == "k" else VB_)
        ops = []
        for j in range(pw):
            masked = (ni % NW != 0) and j == pw - 1

            def op(j=j, masked=masked):
                out = []
                if masked:
                    out += ["s_mov_b64 %[es], exec", f"s_mov_b64 exec, %[{which}mask]"]
                out += [f"s_add_u32 m0, %[{which}cr{j}], {off}", "s_nop 0",
                        f"global_load_lds_dwordx4 %[{which}off{j}], s[{src}:{src + 1}]"]
                if masked:
                    out += ["s_mov_b64 exec, %[es]"]
                return out
            ops.append(op)
        return ops

    b.emit("s_mov_b32 %[m0s], m0")
    b.emit("s_mov_b32 %[i], %[i0]")
    b.emit("s_mov_b32 %[kt], %[kt0]")
    b.emit("s_mov_b32 %[vt], %[vt0]")
    # operand read bases: V^T slots 0-1 and 2-3 (offsets stay below 64 KB), K
    b.valu(VA0, [], text=f"v_add_u32 {v(VA0)}, %[vring], %[vlane]")
    b.emit(f"s_add_u32 %[t0], %[vring], {2 * VB_}")
    b.valu(VA2, [], text=f"v_add_u32 {v(VA2)}, %[t0], %[vlane]")
    b.valu(KA, [], text=f"v_add_u32 {v(KA)}, %[kring], %[klane]")
    b.emit("s_nop 1")
    vx, kx = 32 * L["VLD"] * 2, 32 * L["KLD"] * 2
    b.emit("1:")
    for ph in (1, 2, 3, 0):
        # position i with (i - p0) & 3 = ph
        tile_src("k", KB)
        tile_src("v", VB)
        va = v(VA0) if ph < 2 else v(VA2)
        vo = (ph % 2) * VB_
        ko = ((ph + 1) & 3) * KB_
        pipe_substep(b, L, 0, va, v(KA), vo, ko, copy_ops("k", (ph + 3) & 3))
        pipe_substep(b, L, 1, va, v(KA), vo + vx, ko + kx, copy_ops("v", (ph + 2) & 3))
        b.wait_all_lds()
        # the copies issued one position earlier are complete in every wave
        nmin = 0 if no_dma else L["NIK"] // NW + L["NIV"] // NW
        b.emit(f"s_waitcnt vmcnt({nmin})")
        if not no_barrier:
            b.emit("s_barrier")
        b.emit("s_add_i32 %[kt], %[kt], 64")
        b.emit("s_min_i32 %[kt], %[kt], %[ktl]")
        b.emit("s_add_i32 %[vt], %[vt], 64")
        b.emit("s_min_i32 %[vt], %[vt], %[ktl]")
        b.emit("s_add_i32 %[i], %[i], 1")
        b.emit("s_cmp_lt_i32 %[i], %[iend]")
        b.emit("s_cbranch_scc0 2f" if ph != 0 else "s_cbranch_scc1 1b")
    b.emit("2:")
    b.emit("s_mov_b32 m0, %[m0s]")

    outs = pinned_outs(L) + pinned_vp(L) + ['[m0s] "=&s"(m0s)', '[i] "=&s"(it)', '[t0] "=&s"(t0)', '[t1] "=&s"(t1)',
                                            '[kt] "=&s"(kt)', '[vt] "=&s"(vt)', '[es] "=&s"(es)']
    ins = pinned_ins(L) + [
        '[i0] "s"(i0)', '[iend] "s"(iend)', '[kt0] "s"(kt0)', '[vt0] "s"(vt0)', '[ktl] "s"(ktl)', '[len1] "s"(len1)',
        f'[k1] "{{s[{K1}:{K1 + 1}]}}"(k1)', f'[v1] "{{s[{V1}:{V1 + 1}]}}"(v1)',
        f'[k2] "{{s[{K2}:{K2 + 1}]}}"(k2)', f'[v2] "{{s[{V2}:{V2 + 1}]}}"(v2)',
        '[kring] "s"(kring)', '[vring] "s"(vring)', '[klane] "v"(klane)', '[vlane] "v"(vlane)',
        '[kcr0] "s"(kcr[0])', '[kcr1] "s"(kcr[1])', '[kcr2] "s"(kcr[2])',
        '[vcr0] "s"(vcr[0])', '[vcr1] "s"(vcr[1])', '[vcr2] "s"(vcr[2])',
        '[koff0] "v"(koff[0])', '[koff1] "v"(koff[1])', '[koff2] "v"(koff[2])',
        '[voff0] "v"(voff[0])', '[voff1] "v"(voff[1])', '[voff2] "v"(voff[2])',
        '[kmask] "s"(kmask)', '[vmask] "s"(vmask)']
    clob = tclobbers(L) + [f'"s{i}"' for i in range(KB, KB + 4)] + ['"scc"', '"memory"']
    return (f"template <> __device__ inline void wide_loop<{D}, {str(stream).lower()}>(WIDE_LOOP_ARGS({D})) {{\n"
            "    uint32_t m0s, it, t0, t1, kt, vt;\n    uint64_t es;\n"
            + asm_stmt(b.lines, outs, ins, clob, L["reg"]["END"], scalars=True) + "}\n")


def guard(D):
    # wait states after the last product of a sweep before compiler code touches S or O
    L = layout(D)
    R = L["reg"]
    ops = [f'"+{{v[{R["SA"]}:{R["SA"] + 15}]}}"(sa)', f'"+{{v[{R["SB"]}:{R["SB"] + 15}]}}"(sb)']
    for db in range(L["NDB"]):
        a = R["O"] + 16 * db
        ops.append(f'"+{{v[{a}:{a + 15}]}}"(o[{db}][0])')
    return (f"template <> __device__ inline void wide_guard<{D}>(f32x16& sa, f32x16& sb, f32x16 (&o)[{D // 32}][1]) {{\n"
            f'    asm volatile("s_nop 7\\n\\ts_nop 7\\n\\ts_nop 7" : ' + ", ".join(ops) + ");\n}\n")


def generate():
    parts = ["// Generated by gen_wide_substep.py -- do not edit.  The sweep of the bf16 wide attention\n"
             "// kernel as scheduled gfx950 assembly: one sub-step, the steady-state loop, and the wait\n"
             "// states after it, per head dim.\n"
             "#pragma once\n\n"]
    for D in (32, 64, 128):
        L = layout(D)
        R = L["reg"]
        parts.append(f"// D = {D}: pinned v0..v{R['END'] - 1} "
                     f"(S_a v0-15, S_b v16-31, O from v{R['O']}, Q from v{R['Q']}, K from v{R['K']}, "
                     f"V from v{R['V']}, P from v{R['P']}, temporaries from v{R['T']}); "
                     f"s{SP}..s{SP + 11} for the 64-bit copy pointers\n")
        for par in (0, 1):
            for first in (True, False):
                parts.append(cxx_pipe(D, par, first))
        parts.append(cxx_flush(D))
        for stream in (False, True):
            parts.append(cxx_loop(D, stream))
        parts.append(guard(D))
        parts.append("\n")
    return "".join(parts)


def main(argv):
    text = generate()
    if len(argv) > 1 and argv[1] == "--check":
        cur = open(OUT).read() if os.path.exists(OUT) else ""
        if cur != text:
            print("wide_substep.inc is out of date", file=sys.stderr)
            return 1
        return 0
    with open(OUT, "w") as f:
        f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
