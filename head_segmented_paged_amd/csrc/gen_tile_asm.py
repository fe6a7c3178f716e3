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

  * the scores of tile j+1 (32 MFMAs) are computed while tile j's scores
    become probabilities (running maximum, exp2, bf16 packing, row sums) and
    are multiplied into O^T (32 MFMAs);
  * LDS operand reads run a few operands ahead through a small register ring,
    with counted lgkmcnt waits;
  * the running-maximum refresh (rare: only when a tile's maximum exceeds the
    running one by more than the slack) is a wave-uniform branch inside the
    block.

Register map (fixed; v0..v63 and a0..a63 belong to the compiler):
  a[64:191]   O^T: block qb, 32-dim block db at a[64 + 64 qb + 16 db : +15]
  a[192:255]  Q^T: block qb, k-step s at a[192 + 32 qb + 4 s : +3]
  v[128:191]  score set X, v[192:255] score set Y: block qb, 32-key block kb
              at base + 32 qb + 16 kb; after the softmax, the bf16
              probabilities of 16-key step t sit at base + 32 qb + 16 (t/2) +
              8 (t%2) : +3 (written in place)
  v[64:87]    operand ring (six 4-register slots; v[88:115] unused)
  v[116:127]  temporaries

Hazards handled here (the compiler's hazard recognizer does not look inside
inline assembly): MFMA results are read by VALU code only a tile later or
after explicit s_nop padding; VALU-written probabilities reach an MFMA only
after at least two other instructions; a transcendental result is never read
by the next instruction; v_permlane32_swap is padded on both sides.
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
KBUF_BYTES = 16384          # one K or V^T tile in LDS
KB_BYTES = 32 * 256         # 32 K rows of 128 bf16
DB_BYTES = 32 * 128         # 32 V^T rows of 64 bf16
ONES_BF16X2 = "0x3f803f80"  # (1.0, 1.0) in bf16
NEG_INF = "0xff800000"
SLACK_LOG2 = "0x41000000"   # 8.0: refresh the running maximum only beyond this
# S MFMA operands issued before each group of P.V operands (t = 0..3); the
# rest of the 16 K operands go first.
S_SPLIT = (9, 3, 2, 2)


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


def read_text(op, slot, kbuf, vbuf):
    r = RING0 + 4 * slot
    if op.kind == "K":
        kb, s = op.a, op.b
        return f"ds_read_b128 {vblk(r, 4)}, %[ka{s}] offset:{kbuf * KBUF_BYTES + kb * KB_BYTES}"
    db, t = op.a, op.b
    return f"ds_read_b128 {vblk(r, 4)}, %[va{t}] offset:{vbuf * KBUF_BYTES + db * DB_BYTES}"


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


def max_items(cur):
    """Running maximum of both blocks: per block two chains of three-operand
    maxima, the cross-half exchange, the scale; then the refresh test."""
    items = []
    for qb in range(2):
        ta, tb = T(2 * qb), T(2 * qb + 1)
        chains = []
        for kb, dst in ((0, ta), (1, tb)):
            regs = [f"v{sreg(cur, qb, kb, e)}" for e in range(16)]
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
                  ("s_nop 1", 2),
                  (f"v_permlane32_swap_b32 {ta}, {tb}", 1),
                  ("s_nop 1", 2),
                  (f"v_maximum3_f32 {ta}, {ta}, {tb}, {tb}", 1),
                  (f"v_mul_f32 {T(4 + qb)}, %[scale], {ta}", 1)]
    return items


def rescale_block():
    """Taken when some lane's tile maximum exceeds its running maximum by
    more than the slack: m = max(m, mt), alpha = 2^(m_old - m), l and O^T
    scaled by alpha."""
    lines = [f"v_sub_f32 {T(6)}, {T(4)}, %[m0]",
             f"v_sub_f32 {T(7)}, {T(5)}, %[m1]",
             f"v_max_f32 {T(6)}, {T(6)}, {T(7)}",
             f"v_cmp_lt_f32 vcc, {SLACK_LOG2}, {T(6)}",
             "s_cbranch_vccz .Lw2keep_%=",
             # the previous tile's P.V MFMAs may still be writing O^T
             "s_nop 7", "s_nop 7", "s_nop 7",
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


def exp_items(cur, qb, t):
    """p = 2^(s * scale - m) for the 8 scores of 16-key step t of block qb,
    packed in place to the bf16 P^T operand, and added to the row sum."""
    base = sreg(cur, qb, t >> 1, 8 * (t & 1))
    f = [(f"v_fma_f32 v{base + i}, v{base + i}, %[scale], -%[m{qb}]", 1) for i in range(8)]
    e = [(f"v_exp_f32 v{base + i}, v{base + i}", 2) for i in range(8)]
    order = [f[0], f[1], f[2], f[3], e[0], f[4], e[1], f[5], e[2], f[6], e[3], f[7], e[4], e[5], e[6], e[7]]
    cvt = [(f"v_cvt_pk_bf16_f32 v{base + k}, v{base + 2 * k}, v{base + 2 * k + 1}", 1) for k in range(4)]
    dot = [(f"v_dot2c_f32_bf16 %[l{qb}], {ONES_BF16X2}, v{base + k}", 1) for k in range(4)]
    return order + cvt + dot


def tile_body(cur, nxt, kbuf, vbuf):
    """One tile: softmax and P.V of the scores in set `cur` (V^T from buffer
    vbuf); with nxt, the next tile's scores into set `nxt` from K buffer kbuf."""
    s_ops = [Operand("K", kb, s) for s in range(8) for kb in range(2)] if nxt is not None else []
    pv = [[Operand("V", db, t) for db in range(4)] for t in range(4)]
    ops = []
    pos = 0
    for t in range(4):
        take = S_SPLIT[t] if s_ops else 0
        ops += s_ops[pos:pos + take]
        pos += take
        ops += pv[t]
    ops += s_ops[pos:]
    assert len(ops) == len(s_ops) + 16

    # VALU stream: maximum, refresh test + branch, then exp of steps 0..3.
    valu = [(x, w, -1) for x, w in max_items(cur)]
    valu.append((rescale_block(), 6, -1))
    for t in range(4):
        for qb in range(2):
            valu += [(x, w, t) for x, w in exp_items(cur, qb, t)]
    # done_at[t]: VALU items that must precede the first P.V MFMA of step t
    done_at = {t: max(i for i, v in enumerate(valu) if v[2] == t) + 1 for t in range(4)}

    lines = []
    vi = 0          # next VALU item
    since_p = {}    # instruction count since the last write of each P operand

    def emit(text):
        lines.append(text)
        for k in since_p:
            since_p[k] += 1

    def emit_valu(n_weight):
        nonlocal vi
        w = 0
        while vi < len(valu) and w < n_weight:
            text, wt, t = valu[vi]
            for ln in text.split("\n"):
                emit(ln)
            if text.startswith("v_cvt_pk_bf16_f32"):
                since_p[text.split()[1].rstrip(",")] = 0
            w += wt
            vi += 1

    n = len(ops)
    slots = [i % NRING for i in range(n)]
    issued = 0
    for i in range(min(LOOKAHEAD, n)):
        emit(read_text(ops[i], slots[i], kbuf, vbuf))
        issued += 1
    for i, op in enumerate(ops):
        # VALU needed before this operand's MFMAs
        if op.exp_t is not None:
            need = done_at[op.exp_t]
            if vi < need:
                emit_valu(sum(v[1] for v in valu[vi:need]))
            # the P operand registers: two instructions after their last write
            for qb in range(2):
                preg = f"v{sreg(cur, qb, op.exp_t >> 1, 8 * (op.exp_t & 1) + 3)}"
                if preg in since_p and since_p[preg] < 2:
                    emit("s_nop 1")
        emit(f"s_waitcnt lgkmcnt({min(issued - 1 - i, 15)})")
        texts = mfma_texts(op, slots[i], cur, nxt)
        # VALU weight to place beside each MFMA: spread evenly up to the next deadline
        nxt_t = next((o.exp_t for o in ops[i:] if o.exp_t is not None and vi < done_at[o.exp_t]), None)
        if nxt_t is not None:
            dl = next(j for j in range(i, n) if ops[j].exp_t == nxt_t)
            mfmas = 2 * max(dl - i, 1)
            rest = sum(v[1] for v in valu[vi:done_at[nxt_t]])
            per = math.ceil(rest / mfmas)
        else:
            rest = sum(v[1] for v in valu[vi:])
            per = math.ceil(rest / (2 * (n - i))) if rest else 0
        for k, mt in enumerate(texts):
            emit(mt)
            if k == 0 and i + LOOKAHEAD < n:
                j = i + LOOKAHEAD
                emit(read_text(ops[j], slots[j], kbuf, vbuf))
                issued += 1
            emit_valu(per)
    emit_valu(10 ** 9)
    assert vi == len(valu)
    return lines


def scores_body(nxt, kbuf):
    """Scores of a unit's first tile into set nxt (no softmax), then padding
    so that the VALU reads of the next block see the finished MFMAs."""
    ops = [Operand("K", kb, s) for s in range(8) for kb in range(2)]
    lines = ["s_nop 3"]   # Q^T and O^T were just written to AGPRs
    n = len(ops)
    issued = 0
    for i in range(LOOKAHEAD):
        lines.append(read_text(ops[i], i % NRING, kbuf, 0))
        issued += 1
    for i, op in enumerate(ops):
        lines.append(f"s_waitcnt lgkmcnt({min(issued - 1 - i, 15)})")
        texts = mfma_texts(op, i % NRING, None, nxt)
        for k, mt in enumerate(texts):
            lines.append(mt)
            if k == 0 and i + LOOKAHEAD < n:
                j = i + LOOKAHEAD
                lines.append(read_text(ops[j], j % NRING, kbuf, 0))
                issued += 1
    lines += ["s_nop 7", "s_nop 7", "s_nop 7"]
    return lines


def mask_body(cur):
    """Scores of keys outside [lo_i, pos_i] of their query become -inf:
    element (kb, e) of block qb holds key c + 8 half + tile start, visible iff
    c - a_qb <= span_qb (unsigned), a_qb = lo_i - tile start - 8 half. Skipped
    as a whole when the wave-uniform flag `full` is set (every key of the
    tile visible to every row of the wave): a branch inside the block keeps
    the caller free of control flow around the pinned registers."""
    lines = ["s_cmp_lg_u32 %[full], 0",
             "s_cbranch_scc1 .Lw2full_%=",
             f"v_mov_b32 {T(8)}, {NEG_INF}"]
    k = 0
    for qb in range(2):
        for kb in range(2):
            for e in range(16):
                t = T(9 + (k & 1))
                r = f"v{sreg(cur, qb, kb, e)}"
                lines += [f"v_sub_u32 {t}, {key_const(kb, e)}, %[a{qb}]",
                          f"v_cmp_le_u32 vcc, {t}, %[s{qb}]",
                          f"v_cndmask_b32 {r}, {T(8)}, {r}, vcc"]
                k += 1
    lines.append(".Lw2full_%=:")
    return lines


CLOBBER = (", ".join(f'"v{i}"' for i in range(OWN, 256)) + ", " + ", ".join(f'"a{i}"' for i in range(OWN, 256)) +
           ', "vcc", "scc", "memory"')
TILE_OUT = '[m0] "+v"(m0), [m1] "+v"(m1), [l0] "+v"(l0), [l1] "+v"(l1)'
TILE_IN = ('[ka0] "v"(ad.ka[0]), [ka1] "v"(ad.ka[1]), [ka2] "v"(ad.ka[2]), [ka3] "v"(ad.ka[3]), '
           '[ka4] "v"(ad.ka[4]), [ka5] "v"(ad.ka[5]), [ka6] "v"(ad.ka[6]), [ka7] "v"(ad.ka[7]), '
           '[va0] "v"(ad.va[0]), [va1] "v"(ad.va[1]), [va2] "v"(ad.va[2]), [va3] "v"(ad.va[3]), '
           '[scale] "s"(scale)')
TILE_PARAMS = "float &m0, float &m1, float &l0, float &l1, const W2Addr &ad, float scale"


def c_string(lines, indent="        "):
    return "\n".join(f'{indent}"{ln}\\n"' for ln in lines)


def function(name, doc, lines, outs, ins, params, clobbers=CLOBBER, template=""):
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
    # Q^T, one 16-byte chunk (k-step s of block qb) at a time
    body = []
    for qb in range(2):
        for st in range(8):
            a = QA + 32 * qb + 4 * st
            lines = [f"v_accvgpr_write_b32 a{a + i}, %[x{i}]" for i in range(4)]
            body.append(f"    {'if' if qb + st == 0 else 'else if'} constexpr (QB == {qb} && S == {st})\n"
                        f"        asm volatile(\n{c_string(lines, '            ')}\n"
                        f"            :\n            : [x0] \"v\"(x0), [x1] \"v\"(x1), [x2] \"v\"(x2), [x3] \"v\"(x3)\n"
                        f"            : {CLOBBER});\n")
    parts.append("// One 16-byte chunk of Q^T (block QB, k-step S) into its AGPRs.\n"
                 "template <int QB, int S>\n"
                 "__device__ __forceinline__ void w2_set_q(unsigned x0, unsigned x1, unsigned x2, unsigned x3)\n{\n" +
                 "".join(body) + "}\n")
    parts.append(function("w2_scores_first", "Scores of the first tile (K buffer 0) into set X.",
                          scores_body(XB, 0), "", TILE_IN, "const W2Addr &ad, float scale"))
    for name, cur, nxt, kbuf, vbuf in (("w2_tile_xy", XB, YB, 1, 0), ("w2_tile_yx", YB, XB, 0, 1)):
        doc = (f"Tile with scores in set {'X' if cur == XB else 'Y'} (V^T buffer {vbuf}); next tile's "
               f"scores into set {'Y' if nxt == YB else 'X'} from K buffer {kbuf}.")
        parts.append(function(name, doc, tile_body(cur, nxt, kbuf, vbuf), TILE_OUT, TILE_IN, TILE_PARAMS))
    for name, cur, vbuf in (("w2_last_x", XB, 0), ("w2_last_y", YB, 1)):
        doc = f"A unit's last tile, scores in set {'X' if cur == XB else 'Y'} (V^T buffer {vbuf})."
        parts.append(function(name, doc, tile_body(cur, None, 0, vbuf), TILE_OUT, TILE_IN, TILE_PARAMS))
    mask_in = '[a0] "v"(a0), [s0] "v"(s0), [a1] "v"(a1), [s1] "v"(s1), [full] "s"(full)'
    for name, cur in (("w2_mask_x", XB), ("w2_mask_y", YB)):
        parts.append(function(name, f"Mask the scores in set {'X' if cur == XB else 'Y'}.", mask_body(cur), "",
                              mask_in, "int a0, unsigned s0, int a1, unsigned s1, unsigned full"))
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
