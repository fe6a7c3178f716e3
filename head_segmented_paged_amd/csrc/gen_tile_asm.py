#!/usr/bin/env python3
"""Writes segkv_tile_asm.inc: the register-allocated tile bodies of the
two-block prefill kernel (attn_prefill_w2_kernel in segkv_attn.hip).

    python gen_tile_asm.py [--check]

The build runs it before compiling; --check only compares the committed file
with what it would write (exit status 1 on a difference).

Why generated inline assembly: each wavefront owns 64 query columns (two
32-column MFMA blocks), so every K or V^T operand read from LDS feeds two
MFMAs. At head dim 128 the state of such a wave is
    O^T accumulators  2 blocks x 128 dims x 32 columns fp32   128 registers
    Q^T operands      2 blocks x 128 dims x 32 columns bf16    64 registers
    scores S^T        2 blocks x 64 keys, for two tiles        128 registers
which fits one wave per SIMD (512 registers) only if O^T and Q^T live in
AGPRs (the MFMA's C/D and B operands may be AGPRs) and the scores in VGPRs.
That state lives in registers the compiler may not allocate: the kernel is
limited to 64 VGPRs and 64 AGPRs of its own (amdgpu_num_vgpr(64)), every
generated block names the registers it uses explicitly and lists the whole
upper range as clobbered (so the kernel descriptor counts it), and only
scalars (running maximum and sum, addresses, the scale) pass through
operands. The state therefore survives any code the compiler places between
the blocks. The blocks issue the tile in a fixed interleave:

  * tile j's scores become probabilities (exp2 against the running maximum,
    bf16 packing, row sums) and are multiplied into O^T (32 MFMAs) while the
    scores of tile j+1 are computed (32 MFMAs); once those are done, the
    same body masks them (edge tiles only), takes their maximum and applies
    the running-maximum refresh, so the next body starts on its
    exponentials at once, with no branch among its MFMAs;
  * LDS operand reads run a few operands ahead through a small register ring,
    with counted lgkmcnt waits;
  * the K and V^T tiles are staged in a three-slot LDS ring: each tile body
    issues the DMA of the K tile three ahead and the V^T tile two ahead
    (eight buffer_load ... lds instructions, spread between its first MFMAs,
    the source page and destination slot passed in) and ends with a wait for
    the previous tile's DMA only (vmcnt(8)) and the workgroup barrier, so the
    copies have more than a tile's time to land and their issue hides
    behind the matrix cores;
  * the running-maximum refresh (rare: only when a tile's maximum exceeds the
    running one by more than the slack) is a wave-uniform branch at the end
    of the body, just before the barrier.

Register map (fixed; v0..v63 and a0..a63 belong to the compiler):
  a[64:191]   O^T: block qb, 32-dim block db at a[64 + 64 qb + 16 db : +15]
  a[192:255]  Q^T: block qb, k-step s at a[192 + 32 qb + 4 s : +3]
  v[128:191]  score set X, v[192:255] score set Y: block qb, 32-key block kb
              at base + 32 qb + 16 kb; after the softmax, the bf16
              probabilities of 16-key step t sit at base + 32 qb + 16 (t/2) +
              8 (t%2) : +3 (written in place)
  v[64:87]    operand ring (six 4-register slots)
  v[88:99]    this tile's LDS operand addresses (K slot + lane offset per
              k-step, V^T slot + lane offset per 16-key step)
  v[116:127]  temporaries

Hazards handled here (the compiler's hazard recognizer does not look inside
inline assembly): MFMA results are read by VALU code only a tile later or
after at least HAZ_MFMA_VALU other instructions; VALU-written probabilities
reach an MFMA only after at least two other instructions; a transcendental
result is never read by the next instruction; v_permlane32_swap is padded on
both sides; M0 is written one instruction before the DMA that reads it.
"""

import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "segkv_tile_asm.inc")

XB, YB = 128, 192           # score sets
OA, QA = 64, 192            # O^T and Q^T in AGPRs
OWN = 64                    # registers below this index are the compiler's
RING0, NRING = 64, 6        # operand ring v[64:87]
TMP0 = 116                  # temporaries v116..v127
LOOKAHEAD = 4               # operand reads issued this many operands ahead
KADDR, VADDR = 88, 96       # per-tile LDS operand addresses
DMA_AFTER = (1, 3, 5, 7, 9, 11, 13, 15, 19)   # the tile's DMA groups follow these MFMAs (a ninth: scalar work)
KB_BYTES = 32 * 256         # 32 K rows of 128 bf16
DB_BYTES = 32 * 128         # 32 V^T rows of 64 bf16
NEG_INF = "0xff800000"
SLACK_LOG2 = "0x41000000"   # 8.0: refresh the running maximum only beyond this
# K operands (two S MFMAs each) issued before each group of P.V operands
# (t = 0..3); the 16 K operands in total.
S_SPLIT = (9, 3, 4, 0)
HAZ_MFMA_VALU = 12          # instructions between an MFMA and a VALU read of its result
WAIT_GROUP = 2              # one counted LDS wait covers this many operands
CAP = 6                     # issue slots that hide beside one 32x32x16 MFMA (v_exp_f32 takes two)


def weight(line):
    """Issue slots of one instruction line."""
    op = line.split()[0] if line else ""
    if op == "v_exp_f32":
        return 2
    if op == "s_nop":
        return int(line.split()[1]) + 1
    return 0 if (not op or op.endswith(":")) else 1
VMEM_SGPR_WAIT = 5          # wait states between a VALU write of an SGPR and a VMEM read of it
PAD2 = "@pad2 "             # post item prefix: two wait states after the previous post item


def T(i):
    return f"v{TMP0 + i}"


def vblk(base, n):
    return f"v[{base}:{base + n - 1}]"


def ablk(base, n):
    return f"a[{base}:{base + n - 1}]"


def sreg(base, qb, kb, e):
    return base + 32 * qb + 16 * kb + e


def key_const(kb, e):
    """Key offset (within the tile, before the 8 * half lane offset) of
    accumulator element e of 32-key block kb. MFMA row r = 8 (e/4) + 4 half +
    e%4 is fed K row r with bits 2 and 3 swapped."""
    jj, ii = e >> 2, e & 3
    return 32 * kb + 16 * (jj >> 1) + 4 * (jj & 1) + ii


class Operand:
    def __init__(self, kind, a, b):
        self.kind, self.a, self.b = kind, a, b   # ("K", kb, s) or ("V", db, t)

    @property
    def exp_t(self):
        return self.b if self.kind == "V" else None


def read_text(op, slot, koff=0, voff=0):
    """LDS read of operand op into ring slot `slot`; koff / voff: byte offset
    of the K / V^T ring slot from the address registers."""
    r = RING0 + 4 * slot
    if op.kind == "K":
        kb, s = op.a, op.b
        return f"ds_read_b128 {vblk(r, 4)}, v{KADDR + s} offset:{koff + kb * KB_BYTES}"
    db, t = op.a, op.b
    return f"ds_read_b128 {vblk(r, 4)}, v{VADDR + t} offset:{voff + db * DB_BYTES}"


def addr_lines(k=True, v=True):
    """This tile's operand addresses: lane offsets plus the slot's LDS address."""
    out = []
    if k:
        out += [f"v_add_u32 v{KADDR + s}, %[kslot], %[ka{s}]" for s in range(8)]
    if v:
        out += [f"v_add_u32 v{VADDR + t}, %[vslot], %[va{t}]" for t in range(4)]
    return out


def dma_lines(i):
    """DMA instruction i of the tile (0-3: the K tile, 4-7: the V^T tile), 1 KB
    per wave instruction: lane l's 16 bytes land at M0 + 1024 (i % 4) + 16 l.
    The instruction offset moves both the source and the LDS address, so M0
    is written once per tile (K, then V^T) and the lane offsets kd / vd hold
    the source offset minus 1024 (i % 4)."""
    j = i % 4
    if i < 4:
        load = f"buffer_load_dwordx4 %[kd{j}], %[rk], %[sok] offen offset:{1024 * j} lds"
        return ["s_mov_b32 m0, %[m0k]", "s_nop 0", load] if j == 0 else [load]
    load = f"buffer_load_dwordx4 %[vd{j}], %[rv], %[sov] offen offset:{1024 * j} lds"
    return ["s_mov_b32 m0, %[m0v]", "s_nop 0", load] if j == 0 else [load]


def mfma_texts(op, slot, cur, nxt):
    r = vblk(RING0 + 4 * slot, 4)
    out = []
    if op.kind == "K":
        kb, s = op.a, op.b
        for qb in range(2):
            d = vblk(sreg(nxt, qb, kb, 0), 16)
            q = ablk(QA + 32 * qb + 4 * s, 4)
            out.append(f"v_mfma_f32_32x32x16_bf16 {d}, {r}, {q}, {0 if s == 0 else d}")
    else:
        db, t = op.a, op.b
        for qb in range(2):
            o = ablk(OA + 64 * qb + 16 * db, 16)
            p = vblk(sreg(cur, qb, t >> 1, 8 * (t & 1)), 4)
            out.append(f"v_mfma_f32_32x32x16_bf16 {o}, {r}, {p}, {o}")
    return out


def mask_block(s_set):
    """Scores of keys outside [lo_i, pos_i] of their query become -inf:
    element (kb, e) of block qb holds key c + 8 half + tile start, visible iff
    c - a_qb <= span_qb (unsigned), a_qb = lo_i - tile start - 8 half.
    Skipped as a whole when the wave-uniform flag `full` is set (every key of
    the tile visible to every row of the wave)."""
    lines = ["s_cmp_lg_u32 %[full], 0",
             "s_cbranch_scc1 .Lw2full_%=",
             f"v_mov_b32 {T(8)}, {NEG_INF}"]
    k = 0
    for qb in range(2):
        for kb in range(2):
            for e in range(16):
                t = T(9 + (k & 1))
                r = f"v{sreg(s_set, qb, kb, e)}"
                lines += [f"v_sub_u32 {t}, {key_const(kb, e)}, %[a{qb}]",
                          f"v_cmp_le_u32 vcc, {t}, %[s{qb}]",
                          f"v_cndmask_b32 {r}, {T(8)}, {r}, vcc"]
                k += 1
    lines.append(".Lw2full_%=:")
    return "\n".join(lines)


def max_items(s_set):
    """Maxima of both blocks of a tile's scores: per block two chains of
    three-operand maxima (NaN-propagating), the exchange between the two
    32-lane halves, and the scale into the log2 domain (T4, T5)."""
    items = []
    for qb in range(2):
        ta, tb = T(2 * qb), T(2 * qb + 1)
        chains = []
        for kb, dst in ((0, ta), (1, tb)):
            regs = [f"v{sreg(s_set, qb, kb, e)}" for e in range(16)]
            ops = [f"v_maximum3_f32 {dst}, {regs[0]}, {regs[1]}, {regs[2]}"]
            i = 3
            while i < 16:
                a = regs[i]
                b = regs[i + 1] if i + 1 < 16 else regs[i]
                ops.append(f"v_maximum3_f32 {dst}, {dst}, {a}, {b}")
                i += 2
            chains.append(ops)
        for a, b in zip(*chains):
            items += [(a, 1), (b, 1)]
        items += [(f"v_maximum3_f32 {ta}, {ta}, {tb}, {tb}", 1),
                  (f"v_mov_b32 {tb}, {ta}", 1),
                  (f"{PAD2}v_permlane32_swap_b32 {ta}, {tb}", 1),
                  (f"{PAD2}v_maximum3_f32 {ta}, {ta}, {tb}, {tb}", 1),
                  (f"v_mul_f32 {T(4 + qb)}, %[scale], {ta}", 1)]
    return items


def refresh_block(with_o=True):
    """When some lane's tile maximum (T4, T5) exceeds its running maximum by
    more than the slack: m = max(m, mt), alpha = 2^(m_old - m), l and O^T
    scaled by alpha. Wave-uniform branch; O^T may still be being written by
    the body's last P.V MFMAs, hence the padding before reading it. A unit's
    first tile (with_o False) only sets m: l and O^T are still zero."""
    lines = [f"v_sub_f32 {T(6)}, {T(4)}, %[m0]",
             f"v_sub_f32 {T(7)}, {T(5)}, %[m1]",
             f"v_max_f32 {T(6)}, {T(6)}, {T(7)}",
             f"v_cmp_lt_f32 vcc, {SLACK_LOG2}, {T(6)}",
             "s_cbranch_vccz .Lw2keep_%="]
    if not with_o:
        lines += [f"v_max_f32 %[m0], %[m0], {T(4)}",
                  f"v_max_f32 %[m1], %[m1], {T(5)}",
                  ".Lw2keep_%=:"]
        return "\n".join(lines)
    lines += ["s_nop 7", "s_nop 7", "s_nop 7",
             f"v_max_f32 {T(0)}, %[m0], {T(4)}",
             f"v_max_f32 {T(1)}, %[m1], {T(5)}",
             f"v_sub_f32 {T(6)}, %[m0], {T(0)}",
             f"v_sub_f32 {T(7)}, %[m1], {T(1)}",
             f"v_exp_f32 {T(6)}, {T(6)}",
             f"v_exp_f32 {T(7)}, {T(7)}",
             f"v_mov_b32 %[m0], {T(0)}",
             f"v_mov_b32 %[m1], {T(1)}",
             f"v_mul_f32 %[l0], %[l0], {T(6)}",
             f"v_mul_f32 %[l1], %[l1], {T(7)}"]
    tmp = [T(0), T(1), T(2), T(3), T(8), T(9), T(10), T(11)]
    for g in range(0, 128, 8):
        alpha = T(6) if g < 64 else T(7)
        lines += [f"v_accvgpr_read_b32 {tmp[i]}, a{OA + g + i}" for i in range(8)]
        lines += [f"v_mul_f32 {tmp[i]}, {tmp[i]}, {alpha}" for i in range(8)]
        lines += [f"v_accvgpr_write_b32 a{OA + g + i}, {tmp[i]}" for i in range(8)]
    lines.append(".Lw2keep_%=:")
    return "\n".join(lines)


def exp_items(s_set, qb, t):
    """p = 2^(s * scale - m) for the 8 scores of 16-key step t of block qb,
    added to the row sum in fp32 and packed in place to the bf16 P^T operand."""
    base = sreg(s_set, qb, t >> 1, 8 * (t & 1))
    f = [(f"v_fma_f32 v{base + i}, v{base + i}, %[scale], -%[m{qb}]", 1) for i in range(8)]
    e = [(f"v_exp_f32 v{base + i}, v{base + i}", 2) for i in range(8)]
    a = [(f"v_add_f32 %[l{qb}], %[l{qb}], v{base + i}", 1) for i in range(8)]
    cvt = [(f"v_cvt_pk_bf16_f32 v{base + k}, v{base + 2 * k}, v{base + 2 * k + 1}", 1) for k in range(4)]
    # no result of a transcendental is read by the next instruction
    order = [f[0], f[1], f[2], f[3], e[0], f[4], e[1], f[5], e[2], f[6], e[3], f[7], e[4], a[0], e[5], a[1],
             e[6], a[2], e[7], a[3], a[4], a[5], a[6], a[7], cvt[0], cvt[1], cvt[2], cvt[3]]
    return order


def schedule(ops, exp_q, post_q, final, cur, nxt, dma, tail, head=(), koff=0, voff=0):
    """Interleave the MFMA operand stream `ops` with
      exp_q:  (text, weight, t) items, all of step t due before its first P.V MFMA;
      post_q: (text, weight) items that read the scores of the next tile, so
              only once every S MFMA of the body is HAZ_MFMA_VALU instructions
              old;
      final:  lines after the last MFMA and the queues (the refresh);
    plus the LDS operand reads (LOOKAHEAD operands ahead; `head` goes right
    after the first of them), the DMA line groups `dma` after the MFMAs listed
    in DMA_AFTER, and `tail`. Beside each
    MFMA goes an even share of the remaining VALU weight, exponentials first
    whenever their deadline needs them."""
    lines = []
    n = len(ops)
    slots = [i % NRING for i in range(n)]
    s_idx = [i for i, o in enumerate(ops) if o.kind == "K"]
    last_s = s_idx[-1] if s_idx else -1
    done_at = {}
    for i, v in enumerate(exp_q):
        done_at[v[2]] = i + 1
    ei = pi = 0                # next exp / post item
    s_end_at = None            # line count after the last S MFMA
    p_written = {}             # P operand base register -> line index of its last write
    mfma_no = 0
    pending_dma = list(dma)

    def post_ready():
        return s_end_at is not None and len(lines) - s_end_at >= HAZ_MFMA_VALU

    def take_exp():
        nonlocal ei
        text, wt, t = exp_q[ei]
        lines.extend(text.split("\n"))
        if text.startswith("v_cvt_pk_bf16_f32"):
            reg = int(text.split()[1].lstrip("v").rstrip(","))
            p_written[reg - (reg - cur) % 4] = len(lines)
        ei += 1
        return wt

    last_post = [-10]          # line index of the previous post item's last line

    def take_post():
        nonlocal pi
        text, wt = post_q[pi]
        if text.startswith(PAD2):
            text = text[len(PAD2):]
            gap = len(lines) - 1 - last_post[0]     # instructions since the previous item
            if gap < 2:
                lines.append(f"s_nop {1 - gap}")
        lines.extend(text.split("\n"))
        last_post[0] = len(lines) - 1
        pi += 1
        return wt

    issued = 0
    covered = -1               # operand reads known complete
    for i in range(min(LOOKAHEAD, n)):
        lines.append(read_text(ops[i], slots[i], koff, voff))
        issued += 1
    lines.extend(head)
    for i, op in enumerate(ops):
        if op.exp_t is not None:
            while ei < done_at.get(op.exp_t, 0):
                take_exp()
            for qb in range(2):
                base = sreg(cur, qb, op.exp_t >> 1, 8 * (op.exp_t & 1))
                if len(lines) - p_written.get(base, -10) < 2:
                    lines.append("s_nop 1")
                    break
        if covered < i:
            covered = min(i + WAIT_GROUP - 1, issued - 1)
            lines.append(f"s_waitcnt lgkmcnt({min(issued - 1 - covered, 15)})")
        for k, mt in enumerate(mfma_texts(op, slots[i], cur, nxt)):
            lines.append(mt)
            mark = len(lines)
            mfma_no += 1
            if k == 0 and i + LOOKAHEAD < n:
                j = i + LOOKAHEAD
                lines.append(read_text(ops[j], slots[j], koff, voff))
                issued += 1
            if k == 1 and i == last_s:
                s_end_at = len(lines)
            if pending_dma and mfma_no - 1 >= DMA_AFTER[len(dma) - len(pending_dma)]:
                lines.extend(pending_dma.pop(0))
            # issue slots left beside this MFMA: CAP less what is already
            # placed after it (read, DMA) and the next operand's wait
            used = sum(weight(ln) for ln in lines[mark:])
            if k == 1 and i + 1 < n and covered < i + 1:
                used += 1
            share = max(0, CAP - used)
            # exponentials the next deadline needs by now
            need = 0
            nxt_t = next((o.exp_t for o in ops[i + 1:] if o.exp_t is not None and ei < done_at[o.exp_t]), None)
            if nxt_t is not None:
                dl = next(j for j in range(i + 1, n) if ops[j].exp_t == nxt_t)
                # finished an MFMA early: no padding between the last bf16
                # pack and the MFMA that reads it
                slots_left = 2 * (dl - i) - (1 if k == 0 else 0) - 2
                due = sum(v[1] for v in exp_q[ei:done_at[nxt_t]])
                need = math.ceil(due / max(slots_left, 1))
            w = 0
            while w < need and ei < len(exp_q):
                w += take_exp()
            while True:
                if pi < len(post_q) and post_ready():
                    if w + post_q[pi][1] > share:
                        break
                    w += take_post()
                elif ei < len(exp_q):
                    if w + exp_q[ei][1] > share:
                        break
                    w += take_exp()
                else:
                    break
    while ei < len(exp_q):
        take_exp()
    while pi < len(post_q):
        if not post_ready():
            lines.append("s_nop 7")
            continue
        take_post()
    assert not pending_dma
    lines.extend(final)
    lines.extend(tail)
    return lines


def s_ops():
    return [Operand("K", kb, s) for s in range(8) for kb in range(2)]


def tile_body(cur, nxt):
    """One tile: softmax and P.V of the scores in set `cur`; with nxt, the
    next tile's scores into set `nxt` (then masked, their maximum taken and
    the running maximum refreshed), the DMA of later tiles, and the wait +
    barrier that end the tile."""
    ks = s_ops() if nxt is not None else []
    pv = [[Operand("V", db, t) for db in range(4)] for t in range(4)]
    ops = []
    pos = 0
    for t in range(4):
        take = S_SPLIT[t] if ks else 0
        ops += ks[pos:pos + take]
        pos += take
        ops += pv[t]
    assert pos == len(ks) and len(ops) == len(ks) + 16
    exp_q = []
    for t in range(4):
        for qb in range(2):
            exp_q += [(x, w, t) for x, w in exp_items(cur, qb, t)]
    post_q, final, tail = [], [], []
    if nxt is not None:
        post_q = [(mask_block(nxt), 2)] + max_items(nxt)
        final = refresh_block().split("\n")
        # the previous tile's K/V DMA has landed (this tile's eight may be in
        # flight) and every wave is done with the slots the next DMA refills
        tail = ["s_waitcnt vmcnt(8)", "s_barrier"]
    lines = addr_lines(k=nxt is not None)
    dma = [dma_lines(i) for i in range(8)] if nxt is not None else []
    return lines + schedule(ops, exp_q, post_q, final, cur, nxt, dma, tail)


def scores_body(nxt):
    """A unit's first tile: its scores into set nxt, masked, their maximum
    and the first running-maximum refresh (no softmax yet)."""
    post_q = [(mask_block(nxt), 2)] + max_items(nxt)
    lines = ["s_nop 3"]   # Q^T and O^T were just written to AGPRs
    lines += addr_lines(v=False)
    return lines + schedule(s_ops(), [], post_q, refresh_block(with_o=False).split("\n"), None, nxt, [], [])


# Steady-state run (w2_run): six tile bodies unrolled, one per phase of the
# three-slot ring and the two score sets, in one hardware loop. Only tiles
# every row of the unit sees whole run here (no mask, no V^T fix-up), and the
# per-tile scalars are computed inside the bodies, among the MFMAs:
#   s[88:91]  K buffer resource (tile j+3), s[92:95] V^T resource (tile j+2)
#   s84 / s83 their byte offsets within the page, s81 the pool's page count
#   (capped at 2^31 - 1), s80 a temporary, s82 the page id of tile j+4
#   (scalar load, waited for at the body's end).
RUN_SGPRS = [f"s{i}" for i in range(80, 96)]
KQ, VQ = "s[88:91]", "s[92:95]"
RSRC_WORD3 = "0x20000"


def run_dma(u):
    """The eight DMA groups of run body u (K tile into K slot u % 3, V^T tile
    into V slot (u + 2) % 3, M0 written before the first of each four, the
    instruction offset moving source and destination as in dma_lines), with
    the scalar work of the next page-id load and the loop count beside them."""
    fill = [["s_add_u32 s80, %[kk], 64"],          # first key of tile j+4
            ["s_lshr_b32 s80, s80, %[log2p]"],     # its page-list index
            ["s_min_u32 s80, s80, %[lastlp]"],
            ["s_lshl_b32 s80, s80, 2"],
            ["s_load_dword s82, %[pages], s80"],
            ["s_add_u32 %[kk], %[kk], 64"],
            ["s_sub_u32 %[cnt], %[cnt], 1"],
            []]
    # once the last V^T DMA has read s[92:95] and s83: the next body's V^T
    # tile is this body's K tile (resource moved to the V^T pool)
    after_v = ["s_add_u32 s92, s88, %[vdlo]",
               "s_addc_u32 s93, s89, %[vdhi]",
               "s_mov_b32 s94, s90",
               "s_lshr_b32 s83, s84, 7",
               "s_mov_b32 %[idv], %[idk]"]
    groups = []
    for i in range(4):
        load = f"buffer_load_dwordx4 %[kd{i}], {KQ}, s84 offen offset:{1024 * i} lds"
        groups.append(([f"s_add_u32 m0, %[m0k], {(u % 3) * 16384}"] + fill[i] + [load]) if i == 0 else
                      (fill[i] + [load]))
    for i in range(4):
        load = f"buffer_load_dwordx4 %[vd{i}], {VQ}, s83 offen offset:{1024 * i} lds"
        groups.append(([f"s_add_u32 m0, %[m0v], {((u + 2) % 3) * 16384}"] + fill[4 + i] + [load]) if i == 0 else
                      (fill[4 + i] + [load]))
    groups.append(after_v)
    return groups


def run_body(u):
    """Run body u: the tile whose position in the unit is u mod 6."""
    cur, nxt = (XB, YB) if u % 2 == 0 else (YB, XB)
    ks = s_ops()
    pv = [[Operand("V", db, t) for db in range(4)] for t in range(4)]
    ops, pos = [], 0
    for t in range(4):
        ops += ks[pos:pos + S_SPLIT[t]]
        pos += S_SPLIT[t]
        ops += pv[t]
    exp_q = []
    for t in range(4):
        for qb in range(2):
            exp_q += [(x, w, t) for x, w in exp_items(cur, qb, t)]
    # K resource of tile j+3 and its offset in the page, before the first DMA
    head = ["s_mul_i32 s88, %[idk], %[pbytes]",
            "s_mul_hi_u32 s89, %[idk], %[pbytes]",
            "s_add_u32 s88, s88, %[kplo]",
            "s_addc_u32 s89, s89, %[kphi]",
            "s_cmp_lt_u32 %[idk], s81",
            "s_cselect_b32 s90, %[pbytes], 0",
            "s_and_b32 s84, %[kk], %[pmask]",
            "s_lshl_b32 s84, s84, 8"]
    post = max_items(nxt) + [(f"v_sub_f32 {T(6)}, {T(4)}, %[m0]", 1),
                             (f"v_sub_f32 {T(7)}, {T(5)}, %[m1]", 1),
                             (f"v_max_f32 {T(6)}, {T(6)}, {T(7)}", 1),
                             (f"v_cmp_lt_f32 vcc, {SLACK_LOG2}, {T(6)}", 1)]
    final = [f"s_cbranch_vccnz .Lw2r{u}_%=",
             f".Lw2k{u}_%=:"]
    # next body's ids and V^T resource (this tile's K resource, moved to the
    # V^T pool), then the usual wait + barrier, and the exit test
    tail = ["s_waitcnt lgkmcnt(0)",
            "s_mov_b32 %[idk], s82",
            "s_cmp_eq_u32 %[cnt], 0",
            "s_waitcnt vmcnt(8)",
            "s_barrier",
            "s_cbranch_scc1 .Lw2end_%="]
    lines = [f".Lw2b{u}_%=:"]
    return lines + schedule(ops, exp_q, post, final, cur, nxt, run_dma(u), tail, head=head,
                            koff=((u + 1) % 3) * 16384, voff=(u % 3) * 16384)


def run_block():
    lines = [f"v_add_u32 v{KADDR + s}, %[kbase], %[ka{s}]" for s in range(8)]
    lines += [f"v_mov_b32 v{VADDR + t}, %[va{t}]" for t in range(4)]
    lines += ["s_mov_b64 s[80:81], %[npg]",
              "s_cmp_lg_u32 s81, 0",
              "s_cselect_b32 s80, 0x7fffffff, s80",
              "s_min_u32 s81, s80, 0x7fffffff",
              f"s_mov_b32 s91, {RSRC_WORD3}",
              f"s_mov_b32 s95, {RSRC_WORD3}",
              # V^T resource of tile j+2 and its offset in the page
              "s_mul_i32 s92, %[idv], %[pbytes]",
              "s_mul_hi_u32 s93, %[idv], %[pbytes]",
              "s_add_u32 s92, s92, %[kplo]",
              "s_addc_u32 s93, s93, %[kphi]",
              "s_add_u32 s92, s92, %[vdlo]",
              "s_addc_u32 s93, s93, %[vdhi]",
              "s_cmp_lt_u32 %[idv], s81",
              "s_cselect_b32 s94, %[pbytes], 0",
              "s_sub_u32 s83, %[kk], 64",
              "s_and_b32 s83, s83, %[pmask]",
              "s_lshl_b32 s83, s83, 1"]
    for u in range(1, 6):
        lines += [f"s_cmp_eq_u32 %[ph], {u}", f"s_cbranch_scc1 .Lw2b{u}_%="]
    for u in range(6):
        lines += run_body(u)
    lines.append("s_branch .Lw2b0_%=")
    # running-maximum refresh, out of line, shared by the six bodies
    for u in range(6):
        lines += [f".Lw2r{u}_%=:", f"s_mov_b32 s80, {u}", "s_branch .Lw2ref_%="]
    ref = refresh_block().split("\n")
    # drop the in-line form's test and skip label: the bodies did the test
    start = ref.index("s_cbranch_vccz .Lw2keep_%=")
    ref = ref[start + 1:-1]
    lines.append(".Lw2ref_%=:")
    lines += ref
    for u in range(5):
        lines += [f"s_cmp_eq_u32 s80, {u}", f"s_cbranch_scc1 .Lw2k{u}_%="]
    lines.append("s_branch .Lw2k5_%=")
    lines.append(".Lw2end_%=:")
    return lines


CLOBBER = (", ".join(f'"v{i}"' for i in range(OWN, 256)) + ", " + ", ".join(f'"a{i}"' for i in range(OWN, 256)) +
           ', "vcc", "scc", "m0", "memory"')
TILE_OUT = '[m0] "+v"(m0), [m1] "+v"(m1), [l0] "+v"(l0), [l1] "+v"(l1)'
ADDR_IN = ('[ka0] "v"(ad.ka[0]), [ka1] "v"(ad.ka[1]), [ka2] "v"(ad.ka[2]), [ka3] "v"(ad.ka[3]), '
           '[ka4] "v"(ad.ka[4]), [ka5] "v"(ad.ka[5]), [ka6] "v"(ad.ka[6]), [ka7] "v"(ad.ka[7]), '
           '[va0] "v"(ad.va[0]), [va1] "v"(ad.va[1]), [va2] "v"(ad.va[2]), [va3] "v"(ad.va[3]), '
           '[scale] "s"(scale), [kslot] "s"(st.kslot), [vslot] "s"(st.vslot)')
DMA_IN = ('[rk] "s"(st.rk), [rv] "s"(st.rv), [sok] "s"(st.sok), [sov] "s"(st.sov), [m0k] "s"(st.m0k), '
          '[m0v] "s"(st.m0v), [kd0] "v"(ad.kd[0]), [kd1] "v"(ad.kd[1]), [kd2] "v"(ad.kd[2]), [kd3] "v"(ad.kd[3]), '
          '[vd0] "v"(ad.vd[0]), [vd1] "v"(ad.vd[1]), [vd2] "v"(ad.vd[2]), [vd3] "v"(ad.vd[3])')
MASK_IN = '[a0] "v"(mk.a0), [s0] "v"(mk.s0), [a1] "v"(mk.a1), [s1] "v"(mk.s1), [full] "s"(mk.full)'
TILE_IN = ADDR_IN + ", " + DMA_IN + ", " + MASK_IN
TILE_PARAMS = ("float &m0, float &m1, float &l0, float &l1, const W2Addr &ad, const W2Step &st, const W2Mask &mk, "
               "float scale")


def c_string(lines, indent="        "):
    return "\n".join(f'{indent}"{ln}\\n"' for ln in lines)


def vmem_operand_pad(lines):
    """A vector-memory instruction reading an SGPR that a VALU instruction
    wrote needs VMEM_SGPR_WAIT wait states in between. The compiler may
    write an operand's SGPRs with VALU code (v_readlane, reloading a spilled
    value) right before a block and cannot see into it, so a block whose
    first VMEM instruction with operands comes sooner opens with s_nop."""
    n = 0
    for ln in lines:
        op = ln.split()[0] if ln.split() else ""
        if not op or op.endswith(":"):
            continue
        if op.startswith(("buffer_", "global_")) and "%[" in ln:
            break
        n += weight(ln) if op == "s_nop" else 1
        if n >= VMEM_SGPR_WAIT:
            return lines
    else:
        return lines
    return [f"s_nop {VMEM_SGPR_WAIT - n - 1}"] + lines


def function(name, doc, lines, outs, ins, params, clobbers=CLOBBER, template=""):
    lines = vmem_operand_pad(lines)
    return (f"// {doc}\n{template}"
            f"__device__ __forceinline__ void {name}({params})\n{{\n"
            f"    asm volatile(\n{c_string(lines)}\n"
            f"        : {outs}\n        : {ins}\n        : {clobbers});\n}}\n")


def generate():
    parts = ["// Generated by gen_tile_asm.py from the same directory; do not edit by hand.\n"
             "// Register-allocated tile bodies of the two-block prefill kernel (see the\n"
             "// generator's header for the register map and the hazard rules).\n"]
    # O^T = 0
    parts.append(function("w2_zero_o", "O^T accumulators to zero.",
                          [f"v_accvgpr_write_b32 a{OA + i}, 0" for i in range(128)], "", "", ""))
    # Q^T from the wave's LDS staging rows (row r = 32 qb + column at r * 256,
    # 16-byte chunk c at chunk position c ^ (r & 15)): qa_s holds the lane's
    # address for k-step s of block 0; block 1 lies 8 KB further on.
    lines = [f"ds_read_b128 {ablk(QA + 32 * qb + 4 * st, 4)}, %[qa{st}] offset:{8192 * qb}"
             for qb in range(2) for st in range(8)]
    lines.append("s_waitcnt lgkmcnt(0)")
    parts.append(function("w2_q_from_lds", "Q^T of both blocks into its AGPRs from the wave's staging rows in LDS "
                          "(qa_s: the lane's address of k-step s in block 0; block 1 at +8 KB).",
                          lines, "", ", ".join(f'[qa{st}] "v"(qa[{st}])' for st in range(8)),
                          "const unsigned (&qa)[8]"))
    parts.append(function("w2_scores_first", "A unit's first tile (K slot st.kslot): scores into set X, masked, "
                          "their maximum, the first running-maximum refresh.",
                          scores_body(XB), TILE_OUT, ADDR_IN + ", " + MASK_IN, TILE_PARAMS))
    for name, cur, nxt in (("w2_tile_xy", XB, YB), ("w2_tile_yx", YB, XB)):
        doc = (f"Tile with scores in set {'X' if cur == XB else 'Y'}; next tile's scores into set "
               f"{'Y' if nxt == YB else 'X'} (masked with mk, maximum, refresh); DMA of later tiles; wait + barrier.")
        parts.append(function(name, doc, tile_body(cur, nxt), TILE_OUT, TILE_IN, TILE_PARAMS))
    run_out = TILE_OUT + ', [cnt] "+s"(cnt), [kk] "+s"(kk), [idk] "+s"(idk), [idv] "+s"(idv)'
    run_in = ('[ka0] "v"(ad.ka[0]), [ka1] "v"(ad.ka[1]), [ka2] "v"(ad.ka[2]), [ka3] "v"(ad.ka[3]), '
              '[ka4] "v"(ad.ka[4]), [ka5] "v"(ad.ka[5]), [ka6] "v"(ad.ka[6]), [ka7] "v"(ad.ka[7]), '
              '[va0] "v"(ad.va[0]), [va1] "v"(ad.va[1]), [va2] "v"(ad.va[2]), [va3] "v"(ad.va[3]), '
              '[kd0] "v"(ad.kd[0]), [kd1] "v"(ad.kd[1]), [kd2] "v"(ad.kd[2]), [kd3] "v"(ad.kd[3]), '
              '[vd0] "v"(ad.vd[0]), [vd1] "v"(ad.vd[1]), [vd2] "v"(ad.vd[2]), [vd3] "v"(ad.vd[3]), '
              '[scale] "s"(scale), [kbase] "s"(rn.kbase), [m0k] "s"(rn.m0k), [m0v] "s"(rn.m0v), '
              '[pages] "s"(rn.pages), [kplo] "s"(rn.kplo), [kphi] "s"(rn.kphi), [vdlo] "s"(rn.vdlo), '
              '[vdhi] "s"(rn.vdhi), [pbytes] "s"(rn.pbytes), [npg] "s"(rn.npg), [lastlp] "s"(rn.lastlp), '
              '[log2p] "s"(rn.log2p), [pmask] "s"(rn.pmask), [ph] "s"(phase)')
    run_clob = CLOBBER + ", " + ", ".join(f'"{r}"' for r in RUN_SGPRS)
    parts.append(function("w2_run", "Run of cnt tile bodies over tiles every row of the unit sees whole, entered "
                          "at ring phase `phase` (tile position in the unit mod 6); kk = first key of tile j+3 "
                          "within the segment, idk / idv = page ids of tiles j+3 / j+2 (all updated on exit).",
                          run_block(), run_out, run_in,
                          "float &m0, float &m1, float &l0, float &l1, const W2Addr &ad, const W2Run &rn, "
                          "unsigned phase, unsigned &cnt, unsigned &kk, int &idk, int &idv, float scale",
                          clobbers=run_clob))
    for name, cur in (("w2_last_x", XB), ("w2_last_y", YB)):
        doc = f"A unit's last tile, scores in set {'X' if cur == XB else 'Y'} (no DMA, no barrier)."
        parts.append(function(name, doc, tile_body(cur, None), TILE_OUT, ADDR_IN,
                              "float &m0, float &m1, float &l0, float &l1, const W2Addr &ad, const W2Step &st, "
                              "float scale"))
    parts.append(function("w2_drain", "Wait until the last MFMAs writing O^T have finished.",
                          ["s_nop 7", "s_nop 7", "s_nop 7"], "", "", ""))
    # O^T read-out: four consecutive accumulator registers of (block QB, dim block DB, group J)
    body = []
    first = True
    for qb in range(2):
        for db in range(4):
            for j in range(4):
                a = OA + 64 * qb + 16 * db + 4 * j
                lines = [f"v_accvgpr_read_b32 %[y{i}], a{a + i}" for i in range(4)]
                body.append(f"    {'if' if first else 'else if'} constexpr (QB == {qb} && DB == {db} && J == {j})\n"
                            f"        asm volatile(\n{c_string(lines, '            ')}\n"
                            f"            : [y0] \"=v\"(y0), [y1] \"=v\"(y1), [y2] \"=v\"(y2), [y3] \"=v\"(y3)\n"
                            f"            :\n            : \"memory\");\n")
                first = False
    parts.append("// O^T elements 4 J .. 4 J + 3 of block QB, dim block DB (dims 32 DB + 8 J + 4 half + i).\n"
                 "template <int QB, int DB, int J>\n"
                 "__device__ __forceinline__ void w2_get_o(float &y0, float &y1, float &y2, float &y3)\n{\n" +
                 "".join(body) + "}\n")
    return "\n".join(parts)


def main():
    text = generate()
    if "--check" in sys.argv:
        try:
            cur = open(OUT).read()
        except OSError:
            cur = None
        if cur != text:
            print(f"{OUT} is stale; run {os.path.basename(__file__)}", file=sys.stderr)
            sys.exit(1)
        return
    try:
        if open(OUT).read() == text:
            return
    except OSError:
        pass
    with open(OUT, "w") as f:
        f.write(text)


if __name__ == "__main__":
    main()
