"""Generator of the inline-asm score blocks of attention_fp8.hip.

The FP8-cache attention kernel runs its score products as asm blocks with fixed
register tuples (the compiler, left to schedule them, moved the output
accumulator out of its AGPRs to hold the scores and waited for each step's
reads before its products).  The blocks follow a few regular patterns, so they
are written by this script rather than by hand:

  scores_{split,fp8q}       nine 64-dim steps of one tile half: per step two
                            16-byte key reads (two steps ahead, three tuples
                            v[232:255]) and the query terms' products;
  scores_{split,fp8q}_dma   the same with the next tile's nine direct loads,
                            one after each step's products;
  qk1_{split,fp8q}_{p16,p8} tile half 1's products with the half-0 softmax
                            between them (row maximum over the lane and its
                            partner lane, ceiling, probability groups 0..3
                            with their fp32 sum; p16 also the E5M2 remainder);
  qk01_{split,fp8q}_{p16,p8} both halves in one block: half 0 with the next
                            tile's row address (under the first three steps'
                            products) and then its loads, half 1 with the
                            half-0 softmax, the key reads two steps ahead
                            across the halves; the half-0 scores stay in
                            v[206:221];
  pv_{p16,p8}               the pending stage's p.v: 16 value blocks' scaled
                            products (transposing reads two blocks ahead in
                            v[232:255], P in v[206:221]) with the half-1
                            softmax and the reference logic between them.

python gen_score_blocks.py --write   rewrite those functions in attention_fp8.hip
python gen_score_blocks.py --check   exit 1 if the source differs from the generator
"""
import os
import re
import sys

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attention_fp8.hip")

T = ["v[240:247]", "v[248:255]", "v[232:239]"]          # key operand tuples, step % 3
R = [("v[240:243]", "v[244:247]"), ("v[248:251]", "v[252:255]"), ("v[232:235]", "v[236:239]")]
HALF = 18432        # bytes of a tile half
STEP = 2048         # bytes of a 64-dim step of a tile half
S0 = 206            # the merged block's half-0 accumulator v[206:221]
NEG_2_30 = "0xce800000"
ROW_STEPS = 3       # merged block: steps whose products cover the row address


def wrap(items, width=104):
    out, line = [], ""
    for i, it in enumerate(items):
        piece = it + (", " if i + 1 < len(items) else "")
        if len(line) + len(piece.rstrip()) > width and line.strip():
            out.append(line.rstrip())
            line = ""
        line += piece
    out.append(line.rstrip())
    return "\n        ".join(out)


def q_inputs(split):
    if split:
        return [f'[q{i}] "v"(q.v[{i}])' for i in range(16)] + ['[q16] "v"(rope.hi)', '[q17] "v"(rope.lo)']
    return [f'[q{i}] "v"(q.v[{i}])' for i in range(9)]


def signature(head, parts):
    lines, cur = [], head
    for i, p in enumerate(parts):
        piece = p + ("," if i + 1 < len(parts) else ") {")
        if len(cur) + len(piece) + 1 > 110 and cur.strip() != head.strip():
            lines.append(cur.rstrip())
            cur = " " * len(head)
        cur += piece + " "
    lines.append(cur.rstrip())
    return "\n".join(lines) + "\n"


def softmax_ops(p8, s=lambda i: f"%[s{i}]"):
    """Half-0 softmax: row maximum with the partner lane, ceiling ms0 (-2^30 if
    nothing is visible), then groups 0..3 of p' = 2^(s * sc2 - ms0 + 8)."""
    ops = [
        f"v_max3_f32 v224, {s(0)}, {s(1)}, {s(2)}",
        f"v_max3_f32 v225, {s(3)}, {s(4)}, {s(5)}",
        f"v_max3_f32 v226, {s(6)}, {s(7)}, {s(8)}",
        f"v_max3_f32 v227, {s(9)}, {s(10)}, {s(11)}",
        f"v_max3_f32 v228, {s(12)}, {s(13)}, {s(14)}",
        "v_max3_f32 v224, v224, v225, v226",
        f"v_max3_f32 v227, v227, v228, {s(15)}",
        "v_max_f32 v224, v224, v227",
        "v_mov_b32 v225, v224",
        "s_nop 1",                                   # VALU write -> permlane read
        "v_permlane32_swap_b32 v224, v225",          # one of the two now holds the partner's
        "v_max_f32 v224, v224, v225",
        "v_mul_f32 v224, v224, %[sc2]",
        "v_ceil_f32 v224, v224",
        f"v_max_f32 %[ms0], {NEG_2_30}, v224",
        "v_sub_f32 v222, 0x41000000, %[ms0]",        # 8 - ms0
    ]
    for g in range(4):
        for i in range(4):
            ops.append(f"v_fma_f32 v{224 + i}, {s(4 * g + i)}, %[sc2], v222")
        for i in range(4):
            ops.append(f"v_exp_f32 v{224 + i}, v{224 + i}")
        ops += ["s_nop 0",                           # exponential -> VALU read
                "v_add_f32 v228, v224, v225",
                "v_add_f32 v229, v226, v227",
                f"v_cvt_pk_fp8_f32 %[hi{g}], v224, v225",
                f"v_cvt_pk_fp8_f32 %[hi{g}], v226, v227 op_sel:[0,0,1]",
                "v_add_f32 v228, v228, v229",
                "v_add_f32 %[sf], %[sf], v228"]
        if not p8:
            ops += [f"v_cvt_pk_f32_fp8 v[228:229], %[hi{g}]",
                    f"v_cvt_pk_f32_fp8_sdwa v[230:231], %[hi{g}] src0_sel:WORD_1",
                    "v_sub_f32 v228, v224, v228",
                    "v_sub_f32 v229, v225, v229",
                    "v_sub_f32 v230, v226, v230",
                    "v_sub_f32 v231, v227, v231",
                    f"v_cvt_pk_bf8_f32 %[lo{g}], v228, v229",
                    f"v_cvt_pk_bf8_f32 %[lo{g}], v230, v231 op_sel:[0,0,1]"]
    return ops


def q(line):
    return f'"{line}\\n\\t"'


def one_half(terms, dma_steps=(), softmax=None):
    """Body of a one-half block.  dma_steps: steps after whose products a load
    is issued (load operands g0..); softmax: VALU ops spread over the products."""
    out = []
    e = out.append
    ops = list(softmax or [])
    per = -(-len(ops) // (9 * terms)) if ops else 0
    if dma_steps:
        e(q("s_mov_b32 %[m0s], m0"))
        e(q("s_mov_b32 m0, %[dst]"))
    e(q("s_waitcnt lgkmcnt(0)"))

    def reads(st):
        a, b = R[st % 3]
        e(q(f"ds_read_b128 {a}, %[a0] offset:{STEP * st}"))
        e(q(f"ds_read_b128 {b}, %[a1] offset:{STEP * st}"))
    reads(0)
    reads(1)
    g, k = 0, 0
    for st in range(9):
        e(q("s_waitcnt lgkmcnt(2)") if st < 8 else q("s_waitcnt lgkmcnt(0)"))
        for tm in range(terms):
            src = "0" if (st == 0 and tm == 0) else "%[acc]"
            e(q(f"v_mfma_f32_32x32x64_f8f6f4 %[acc], {T[st % 3]}, %[q{terms * st + tm}], {src}"))
            n = len(ops) - k if (st == 8 and tm == terms - 1) else per
            for _ in range(n):
                if k < len(ops):
                    e(q(ops[k]))
                    k += 1
        if st in dma_steps:
            e(q(f"global_load_lds_dwordx4 %[g{g}], off"))
            g += 1
            if g < len(dma_steps):
                e(q("s_add_u32 m0, m0, 2048"))
        if st + 2 < 9:
            reads(st + 2)
    if dma_steps:
        e(q("s_mov_b32 m0, %[m0s]"))
    e(q("s_nop 15"))          # XDL result -> VALU read
    e(q("s_nop 3"))
    return out


def row_ops():
    """The next tile's row address for this lane's loads, into v[230:231],
    spread over the first steps' products (v224..v231 are free until the
    half-0 softmax).  The lane loads token t = ts + tok_slot(slot) of the
    next unit, slot = (l & 15) ^ 8 l4 (ts: that unit's stage start plus the
    wave's half and slot-block offset), 16 bytes at 16 (l >> 4) of its row:
    row (page << shift) + (t & mask) of the pool, or the zero row when t is
    past the row length (lmax) or the page is outside the pool (also reported
    in badm).  On the way, the load of this lane's page id of the unit after
    next, as fetch_page does: entry (ts2 + tok_slot(slot)) >> shift of the
    table row at pt2, entry 0 past lmax2."""
    return [
        "v_mbcnt_lo_u32_b32 v224, -1, 0",
        "v_mbcnt_hi_u32_b32 v224, -1, v224",
        "v_lshrrev_b32 v225, 1, v224",
        "v_and_b32 v225, 8, v225",
        "v_and_b32 v226, 15, v224",
        "v_xor_b32 v225, v225, v226",             # slot
        "v_lshrrev_b32 v226, 1, v225",            # tok_slot: swap slot bits 2 and 3
        "v_xor_b32 v226, v226, v225",
        "v_and_b32 v226, 4, v226",
        "v_mul_u32_u24 v226, 3, v226",
        "v_xor_b32 v225, v225, v226",
        # the page id of the unit after next for the same slot (its table row
        # at pt2), loaded before the tile loads so vmcnt(9) waits for it alone
        "v_add_u32 v226, %[ts2], v225",
        "v_cmp_gt_i32 vcc, %[lmax2], v226",
        "v_lshrrev_b32 v226, %[shift], v226",
        "v_cndmask_b32 v226, 0, v226, vcc",
        "v_mov_b32 v227, 0",
        "v_lshl_add_u64 v[228:229], v[226:227], 2, %[pt2]",
        "global_load_dword %[pnext], v[228:229], off",
        "v_add_u32 v225, %[ts], v225",            # t
        "v_cmp_gt_i32 %[inm], %[lmax], v225",     # t < lmax
        "v_and_b32 v226, %[mask], v225",
        "v_lshl_add_u32 v227, %[page], %[shift], v226",
        "v_and_b32 v224, 0x30, v224",             # 16 (l >> 4)
        "v_mov_b32 v225, 0",
        "v_lshl_add_u64 v[228:229], v[224:225], 0, %[pool]",
        "v_mov_b32 v226, 0x240",                  # 576 bytes a row
        "v_mad_u64_u32 v[230:231], vcc, v227, v226, v[228:229]",
        "v_lshl_add_u64 v[228:229], v[224:225], 0, %[zero]",
        "v_cmp_gt_u32 vcc, %[np], %[page]",       # page inside the pool
        "s_andn2_b64 %[badm], %[inm], vcc",
        "s_and_b64 vcc, %[inm], vcc",
        "v_cndmask_b32 v230, v228, v230, vcc",
        "v_cndmask_b32 v231, v229, v231, vcc",
    ]


def both_halves(terms, p8):
    out = []
    e = out.append
    ops = softmax_ops(p8, lambda i: f"v{S0 + i}")
    per = -(-len(ops) // (9 * terms - 1))
    e(q("s_mov_b32 %[m0s], m0"))
    e(q("s_mov_b32 m0, %[dst]"))
    e(q("s_waitcnt lgkmcnt(0)"))

    def reads(gs):
        a, b = R[gs % 3]
        off = (gs // 9) * HALF + (gs % 9) * STEP
        e(q(f"ds_read_b128 {a}, %[a0] offset:{off}"))
        e(q(f"ds_read_b128 {b}, %[a1] offset:{off}"))
    reads(0)
    reads(1)
    # the row address under the first ROW_STEPS steps' products, then the nine
    # loads over the remaining half-0 steps
    rops = row_ops()
    rper = -(-len(rops) // (ROW_STEPS * terms))
    nload = 9 - ROW_STEPS
    per_step = [9 // nload + (1 if i < 9 % nload else 0) for i in range(nload)]
    load_at = {ROW_STEPS + i: n for i, n in enumerate(per_step)}
    ld = 0
    k = 0
    for gs in range(18):
        half, st = divmod(gs, 9)
        acc = f"v[{S0}:{S0 + 15}]" if half == 0 else "%[s1]"
        e(q("s_waitcnt lgkmcnt(2)") if gs < 17 else q("s_waitcnt lgkmcnt(0)"))
        for tm in range(terms):
            src = "0" if (st == 0 and tm == 0) else acc
            e(q(f"v_mfma_f32_32x32x64_f8f6f4 {acc}, {T[gs % 3]}, %[q{terms * st + tm}], {src}"))
            if gs < ROW_STEPS:
                for op in rops[:rper]:
                    e(q(op))
                rops = rops[rper:]
            if half == 1:
                if gs == 9 and tm == 0:
                    e(q("s_nop 15"))      # XDL result -> VALU read of the half-0 scores
                    e(q("s_nop 3"))
                    continue
                n = len(ops) - k if (st == 8 and tm == terms - 1) else per
                for _ in range(n):
                    if k < len(ops):
                        e(q(ops[k]))
                        k += 1
        for _ in range(load_at.get(gs, 0)):
            # load ld: row bytes 64 ld on; the offset also moves the LDS
            # destination, so M0 steps by 2048 - 64
            e(q("global_load_lds_dwordx4 v[230:231], off" + (f" offset:{64 * ld}" if ld else "")))
            if ld < 8:
                e(q(f"s_add_u32 m0, m0, {STEP - 64}"))
            ld += 1
        if gs + 2 < 18:
            reads(gs + 2)
    assert k == len(ops) and ld == 9 and not rops
    e(q("s_mov_b32 m0, %[m0s]"))
    e(q("s_waitcnt vmcnt(9)"))       # the page id (the tile loads may still run)
    e(q("s_nop 15"))
    e(q("s_nop 3"))
    return out


VT = ["v[232:239]", "v[240:247]", "v[248:255]"]   # value operand tuples, block % 3
PP_HI, PP_LO = "v[206:213]", "v[214:221]"        # the pending stage's P operand


def half1_ops(p8):
    """The half-1 softmax of the p.v block: row maximum of s1 over the lane and
    its partner, ceiling ms1, the reference logic (mref starts with the first
    visible half; d0, d1 the halves' ceilings above it and their E8M0
    exponents di, clamped to [-127, 64]), then groups 4..7 of
    p' = 2^(s1 * sc2 - ms1 + 8).  Temps v222, v224..v231."""
    ops = [
        "v_max3_f32 v224, %[s0], %[s1], %[s2]",
        "v_max3_f32 v225, %[s3], %[s4], %[s5]",
        "v_max3_f32 v226, %[s6], %[s7], %[s8]",
        "v_max3_f32 v227, %[s9], %[s10], %[s11]",
        "v_max3_f32 v228, %[s12], %[s13], %[s14]",
        "v_max3_f32 v224, v224, v225, v226",
        "v_max3_f32 v227, v227, v228, %[s15]",
        "v_max_f32 v224, v224, v227",
        "v_mov_b32 v225, v224",
        "s_nop 1",
        "v_permlane32_swap_b32 v224, v225",
        "v_max_f32 v224, v224, v225",
        "v_mul_f32 v224, v224, %[sc2]",
        "v_ceil_f32 v224, v224",
        f"v_max_f32 %[ms1], {NEG_2_30}, v224",
        "v_sub_f32 v222, 0x41000000, %[ms1]",       # 8 - ms1
        "v_max_f32 %[msx], %[ms0], %[ms1]",
        f"v_cmp_lt_f32 vcc, {NEG_2_30}, %[msx]",
        "v_mov_b32 v225, 0xff800000",                    # (a literal and vcc both need the constant bus)
        "v_cndmask_b32 v225, v225, %[msx], vcc",         # a visible half: msx, else -inf
        "v_cmp_lt_f32 vcc, 0xff800000, %[mref]",
        "v_cndmask_b32 %[mref], v225, %[mref], vcc",     # keep a started reference
        "v_cmp_lt_f32 vcc, 0xff800000, %[mref]",
        "v_sub_f32 v226, %[ms0], %[mref]",
        "v_cndmask_b32 v226, 0, v226, vcc",              # d0
        "v_sub_f32 v227, %[ms1], %[mref]",
        "v_cndmask_b32 v227, 0, v227, vcc",              # d1
        "v_max_f32 %[delta], v226, v227",
        "v_min_f32 v226, 0x42800000, v226",
        "v_min_f32 v227, 0x42800000, v227",
        "v_max_f32 v226, 0xc2fe0000, v226",
        "v_max_f32 v227, 0xc2fe0000, v227",
        "v_cvt_i32_f32 %[di0], v226",
        "v_cvt_i32_f32 %[di1], v227",
    ]
    for g in range(4, 8):
        for i in range(4):
            ops.append(f"v_fma_f32 v{224 + i}, %[s{4 * (g - 4) + i}], %[sc2], v222")
        for i in range(4):
            ops.append(f"v_exp_f32 v{224 + i}, v{224 + i}")
        ops += ["s_nop 0",
                "v_add_f32 v228, v224, v225",
                "v_add_f32 v229, v226, v227",
                f"v_cvt_pk_fp8_f32 %[hi{g}], v224, v225",
                f"v_cvt_pk_fp8_f32 %[hi{g}], v226, v227 op_sel:[0,0,1]",
                "v_add_f32 v228, v228, v229",
                "v_add_f32 %[sf1], %[sf1], v228"]
        if not p8:
            ops += [f"v_cvt_pk_f32_fp8 v[228:229], %[hi{g}]",
                    f"v_cvt_pk_f32_fp8_sdwa v[230:231], %[hi{g}] src0_sel:WORD_1",
                    "v_sub_f32 v228, v224, v228",
                    "v_sub_f32 v229, v225, v229",
                    "v_sub_f32 v230, v226, v230",
                    "v_sub_f32 v231, v227, v231",
                    f"v_cvt_pk_bf8_f32 %[lo{g}], v228, v229",
                    f"v_cvt_pk_bf8_f32 %[lo{g}], v230, v231 op_sel:[0,0,1]"]
    return ops


def v_reads(e, d):
    base = (d >> 1) * STEP + (d & 1) * 512
    lo = int(VT[d % 3][2:].split(":")[0])
    for i, off in enumerate((0, 1024, HALF, HALF + 1024)):
        o = base + off
        e(q(f"ds_read_b64_tr_b8 v[{lo + 2 * i}:{lo + 2 * i + 1}], %[va]" + (f" offset:{o}" if o else "")))


def pv_body(p8):
    """The pending stage's p.v (16 value blocks of the tile at vtb, the P
    operand from the wave's staging area at pab, scale epo) with the half-1
    softmax and the reference logic between the products."""
    out = []
    e = out.append
    e(q("v_mbcnt_lo_u32_b32 v224, -1, 0"))
    e(q("v_mbcnt_hi_u32_b32 v224, -1, v224"))
    e(q("v_lshl_add_u32 %[pa], v224, 4, %[pab]"))
    # value block 0 offset of lane l = (l0, k = l1..l3, l4, l5): 8 l0 + 16 k + 128 (l4 ^ l5) + 256 l4
    for op in ["v_lshlrev_b32 %[va], 3, v224",
               "v_and_b32 %[va], 0x78, %[va]",
               "v_bfe_u32 v225, v224, 4, 1",
               "v_lshl_or_b32 %[va], v225, 8, %[va]",
               "v_bfe_u32 v226, v224, 5, 1",
               "v_xor_b32 v225, v225, v226",
               "v_lshl_or_b32 %[va], v225, 7, %[va]",
               "v_add_u32 %[va], %[vtb], %[va]"]:
        e(q(op))
    e(q(f"ds_read_b128 v[206:209], %[pa]"))
    e(q(f"ds_read_b128 v[210:213], %[pa] offset:1024"))
    if not p8:
        e(q(f"ds_read_b128 v[214:217], %[pa] offset:2048"))
        e(q(f"ds_read_b128 v[218:221], %[pa] offset:3072"))
    v_reads(e, 0)
    v_reads(e, 1)
    ops = half1_ops(p8)
    # the maximum and the reference logic run under the reads' latency
    head = next(i for i, op in enumerate(ops) if op.startswith("v_fma_f32"))
    for op in ops[:head]:
        e(q(op))
    ops = ops[head:]
    terms = 1 if p8 else 2
    per = -(-len(ops) // (16 * terms - 1))
    k = 0
    for d in range(16):
        e(q("s_waitcnt lgkmcnt(4)") if d < 15 else q("s_waitcnt lgkmcnt(0)"))
        e(q(f"v_mfma_scale_f32_32x32x64_f8f6f4 %[o{d}], {VT[d % 3]}, {PP_HI}, %[o{d}], %[one], %[epo] op_sel_hi:[0,0,0]"))
        n = per if (d, 0) != (15, terms - 1) else len(ops) - k
        for op in ops[k:k + n]:
            e(q(op))
        k += n
        if not p8:
            e(q(f"v_mfma_scale_f32_32x32x64_f8f6f4 %[o{d}], {VT[d % 3]}, {PP_LO}, %[o{d}], %[one], %[epo] op_sel_hi:[0,0,0] blgp:1"))
            n = per if d < 15 else len(ops) - k
            for op in ops[k:k + n]:
                e(q(op))
            k += n
        if d + 2 < 16:
            v_reads(e, d + 2)
    assert k == len(ops)
    return out


def pv_function(p8):
    name = f"pv_{'p8' if p8 else 'p16'}"
    parts = ["floatx16 (&o)[16]", "const floatx16 &s1", "float ms0", "float sc2", "int epo", "uint32_t pab",
             "uint32_t vtb", f"PvOut<{'true' if p8 else 'false'}> &r"]
    outs = [f'[o{d}] "+a"(o[{d}])' for d in range(16)]
    outs += [f'[hi{g}] "=&v"(r.hi[{g - 4}])' for g in range(4, 8)]
    if not p8:
        outs += [f'[lo{g}] "=&v"(r.lo[{g - 4}])' for g in range(4, 8)]
    outs += ['[sf1] "+v"(r.sf1)', '[ms1] "=&v"(r.ms1)', '[msx] "=&v"(r.msx)', '[delta] "=&v"(r.delta)',
             '[di0] "=&v"(r.di0)', '[di1] "=&v"(r.di1)', '[mref] "+v"(r.mref)', '[pa] "=&v"(pa)',
             '[va] "=&v"(va)']
    ins = [f'[s{i}] "v"(s1[{i}])' for i in range(16)]
    ins += ['[ms0] "v"(ms0)', '[sc2] "v"(sc2)', '[epo] "v"(epo)', '[one] "v"(kScaleOne)', '[pab] "s"(pab)',
            '[vtb] "s"(vtb)']
    clob = [f'"v{r}"' for r in list(range(206, 223)) + list(range(224, 256))] + ['"memory"', '"vcc"']
    s = signature(f"__device__ inline void {name}(", parts)
    s += "  uint32_t pa, va;\n"
    s += "  asm volatile(\n" + "\n".join("      " + l for l in pv_body(p8)) + "\n"
    s += "      : " + wrap(outs) + "\n"
    s += "      : " + wrap(ins) + "\n"
    s += "      : " + wrap(clob) + ");\n"
    s += "}\n"
    return name, s


def function(kind, split, p8=False):
    terms = 2 if split else 1
    qname = "split" if split else "fp8q"
    base = ["KAddr ka", "const QOp<false> &q", "const Rope &rope"] if split else ["KAddr ka", "const QOp<true> &q"]
    ins = ['[a0] "v"(ka.a0)', '[a1] "v"(ka.a1)'] + q_inputs(split)
    clob_regs = list(range(232, 256))
    flags = ['"memory"']
    if kind == "scores":
        name, ret = f"scores_{qname}", "floatx16"
        parts, outs, body = base, ['[acc] "=&v"(acc)'], one_half(terms)
    elif kind == "scores_dma":
        name, ret = f"scores_{qname}_dma", "floatx16"
        parts = base + ["const uint8_t *row", "uint32_t dst"]
        outs = ['[acc] "=&v"(acc)', '[m0s] "=&s"(saved)']
        ins += [f'[g{k}] "v"(row + {64 * k})' for k in range(9)] + ['[dst] "s"(dst)']
        body = one_half(terms, dma_steps=tuple(range(9)))
        flags.append('"scc"')
    elif kind == "qk1":
        name, ret = f"qk1_{qname}_{'p8' if p8 else 'p16'}", "void"
        parts = base + ["const floatx16 &s0", "float sc2", f"Half0<{'true' if p8 else 'false'}> &o"]
        outs = ['[acc] "=&v"(o.s1)', '[ms0] "=&v"(o.ms0)', '[sf] "+v"(o.sf0)']
        outs += [f'[hi{g}] "=&v"(o.hi[{g}])' for g in range(4)]
        if not p8:
            outs += [f'[lo{g}] "=&v"(o.lo[{g}])' for g in range(4)]
        ins += [f'[s{i}] "v"(s0[{i}])' for i in range(16)] + ['[sc2] "v"(sc2)']
        body = one_half(terms, softmax=softmax_ops(p8))
        clob_regs = [222] + list(range(224, 256))
    else:   # qk01
        name, ret = f"qk01_{qname}_{'p8' if p8 else 'p16'}", "void"
        parts = base + ["const NextRow &nr", "uint32_t dst", "float sc2", f"Half0<{'true' if p8 else 'false'}> &o"]
        outs = ['[s1] "=&v"(o.s1)', '[ms0] "=&v"(o.ms0)', '[sf] "+v"(o.sf0)']
        outs += [f'[hi{g}] "=&v"(o.hi[{g}])' for g in range(4)]
        if not p8:
            outs += [f'[lo{g}] "=&v"(o.lo[{g}])' for g in range(4)]
        outs += ['[m0s] "=&s"(saved)', '[inm] "=&s"(inm)', '[badm] "=&s"(o.badm)']
        outs.append('[pnext] "=&v"(o.pnext)')
        ins += ['[page] "v"(nr.page)', '[ts] "s"(nr.ts)', '[lmax] "s"(nr.lmax)', '[mask] "s"(nr.mask)',
                '[shift] "s"(nr.shift)', '[np] "s"(nr.np)', '[pool] "s"(nr.pool)', '[zero] "s"(nr.zero)',
                '[ts2] "s"(nr.ts2)', '[lmax2] "s"(nr.lmax2)', '[pt2] "s"(nr.pt2)', '[dst] "s"(dst)',
                '[sc2] "v"(sc2)']
        body = both_halves(terms, p8)
        clob_regs = list(range(S0, S0 + 16)) + [222] + list(range(224, 256))
        flags.append('"scc"')
        flags.append('"vcc"')
    clob = [f'"v{r}"' for r in clob_regs] + flags
    s = signature(f"__device__ inline {ret} {name}(", parts)
    if ret == "floatx16":
        s += "  floatx16 acc;\n"
    if kind in ("scores_dma", "qk01"):
        s += "  uint32_t saved;\n"
    if kind == "qk01":
        s += "  uint64_t inm;\n"
    s += "  asm volatile(\n" + "\n".join("      " + l for l in body) + "\n"
    s += "      : " + wrap(outs) + "\n"
    s += "      : " + wrap(ins) + "\n"
    s += "      : " + wrap(clob) + ");\n"
    if ret == "floatx16":
        s += "  return acc;\n"
    s += "}\n"
    return name, s


def all_functions():
    out = [pv_function(False), pv_function(True)]
    for split in (True, False):
        out.append(function("scores", split))
        out.append(function("scores_dma", split))
        for p8 in (False, True):
            out.append(function("qk1", split, p8))
            out.append(function("qk01", split, p8))
    return out


def locate(src, name):
    m = re.search(r"^__device__ inline (?:floatx16|void) " + re.escape(name) + r"\(", src, re.M)
    if not m:
        raise KeyError(name)
    end = src.index("\n}\n", m.start()) + 3
    return m.start(), end


def main():
    src = open(SRC).read()
    new = src
    for name, text in all_functions():
        i, j = locate(new, name)
        new = new[:i] + text + new[j:]
    if "--write" in sys.argv:
        if new != src:
            open(SRC, "w").write(new)
        print("written" if new != src else "unchanged")
        return 0
    if new != src:
        print("attention_fp8.hip differs from gen_score_blocks.py; run it with --write")
        return 1
    print("attention_fp8.hip matches gen_score_blocks.py")
    return 0


if __name__ == "__main__":
    sys.exit(main())
