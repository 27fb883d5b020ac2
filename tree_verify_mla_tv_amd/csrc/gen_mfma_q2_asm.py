#!/usr/bin/env python3
"""Generate attn_mfma_q2_asm.h: the step block of attn_mfma_q2.hip.

    python tree_verify_mla_tv_amd/csrc/gen_mfma_q2_asm.py   # rewrites attn_mfma_q2_asm.h

attn_mfma_q2.hip is the bf16-cache kernel that keeps the queries' precision:
each scaled query x is carried as two bf16 terms, hi = bf16(x) and lo =
bf16(x - hi), whose sum is x to 2^-17.  A wave owns 16 query rows; the B
operand of its score product S^T = K Q^T has 32 columns, hi of the 16 rows in
columns 0..15 and lo in columns 16..31, so one v_mfma_f32_32x32x16_bf16 gives
both terms of 32 keys x 16 rows and a lane-row swap adds them.

TV_Q2_STEP_ASM -- per wave, for tile t (scores) and tile t-1 (values):
  1. Scores: 36 x v_mfma_f32_32x32x16_bf16 into S (v[224:239]); k-step ks < 32
     takes its K fragment at %[lat] + 32 ks and the query operand %[q<ks>],
     ks >= 32 takes K at %[rope] + 256 (ks - 32) and %[qr<ks - 32>].  Lane l
     then holds column l % 32 (hi of row l % 16 if l % 32 < 16, else its lo)
     for keys 8 (i/4) + 4 (l/32) + i % 4 in score i.
     Woven in: this wave's copy of tile t+1 (the TV_STAGE_ASM loads of
     attn_mfma_asm.h, one group per op) and the LDS reads of the value
     fragments of tile t-1, read well ahead: the weights into the AGPR pool,
     the latent (value) fragments into v[192:223], fragment f at
     v[192 + 4 f], and there converted from bf16 to fp16 in place, CVT_DELAY
     matrix ops after their read (per dword: widen both halves to fp32, then
     one v_cvt_pk_f16_f32; exact for magnitudes from 2^-17 to 65504).
  2. Values O^T[rb][db] (%[o<4 rb + db>], rb = 0, 1: rows 32 rb .. 32 rb + 31)
     += V(db, h) x P(rb, h): 16 x v_mfma_f32_32x32x16_f16, n = 8 h + 2 db + rb.
     V(db, h) (fragment f = 2 h ... as n >> 1) is read from the row-major
     tile with two ds_read_b64_tr_b16 at %[tb] + 16640 h + 16 db (+ 8320 for
     keys 8..15 of the half), P(rb, h) with ds_read_b128 at %[pb] + 1024
     (2 rb + h).
     Woven in, for tile t (VALU):
       combine  v_permlane16_swap of scores i and i + 8, then their sum: lane
                l (row l % 16, rho = l / 16) keeps 8 scores, of keys
                16 (rho & 1) + 8 (i/4) + 4 (rho >> 1) + i % 4, i = 0..7;
       mask     (only when %[nm] != 0, out of line): score i becomes -inf
                unless bit i of %[mask] is set;
       max      over the 8 scores, then the row's four lanes (l, l ^ 16,
                l ^ 32, l ^ 48: v_permlane16_swap and v_permlane32_swap);
       state    %[mseen], %[mref] (set on the first visible tile), %[exc],
                reference max(%[mref], -FLT_MAX), as in attn_mfma.hip;
       weights  exp2(s - ref), packed to fp16 in v[240:243] and stored with
                one ds_write_b128 at %[pw] (the B operand of the value product
                for the lane's row block, key half and key group);
       row sum  %[l] adds the packed (rounded) weights, widened back to fp32.
     These ops are list-scheduled into the gaps after value ops (dependencies
     from their register operands; plain VALU results are forwarded, so a
     consumer may share its producer's gap unless the producer is a
     transcendental or the consumer a v_permlane*_swap; the mask is a
     pseudo-op between the combine and everything after it).
The K and weight fragments of the matrix ops go through a pool of 32 AGPR
quads a[128:255]; a quad is reused one matrix op after its last reader.  Waits
are exact lgkmcnt counts from the wave's in-order LDS queue.

Hazards handled: LDS data waits; the matrix result S before its first VALU
read (>= S_HAZARD wait states); the copy's M0 and offset writes a matrix op
before the loads that read them; v_permlane*_swap two wait states after the
VALU write of a source and a transcendental's result one wait state before
its first reader (both kept a matrix op apart, or by s_nop in the last gap);
a converted value fragment at least one matrix op before its first reader;
the accumulators before anything outside the sweep
reads them (TV_MFMA_DRAIN_ASM of attn_mfma_asm.h after the last step).
"""
import os
import re

import gen_mfma_asm as G

S_BASE = 224                                  # v[224:239]: scores
P_PACK = 240                                  # v[240:243]: packed weights
TMP = list(range(244, 252))                   # v[244:251]: VALU temporaries
V_BASE = 192                                  # v[192:223]: value fragments V0..V7, four dwords each
CVT_TMP = 190                                 # v190: temporary of the bf16 -> fp16 conversion
CLOBBERED_V = list(range(CVT_TMP, 224)) + list(range(S_BASE, 252))
POOL = [128 + 4 * i for i in range(32)]       # a[128:255]: LDS fragment quads
AHEAD_K = 8           # a K fragment is read at most this many matrix ops before its use
AHEAD_VP = 24         # value-phase fragments may be read this far ahead (during the scores)
CVT_DELAY = 6         # a value fragment is converted this many matrix ops after its read
LOADS_PER_GAP = 2     # LDS fragment reads issued before one matrix op, at most
COPY_GROUPS = 18      # copy groups, one after each of the first score ops
GAP_BUDGET = 6        # VALU instructions between two value ops
TRANS_PER_GAP = 3
S_HAZARD = 12
NEG_INF = G.NEG_INF

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "attn_mfma_q2_asm.h")


def S(i):
    return f"v{S_BASE + i}"


def aquad(r):
    return f"a[{r}:{r + 3}]"


def rw(text):
    """(registers read, registers written) of one VALU / LDS-store op."""
    text = re.sub(r"\s+src0_sel:\S+", "", text)
    if text.startswith("v_permlane16_swap") or text.startswith("v_permlane32_swap"):
        _, _, rest = text.partition(" ")
        regs = [G._regs(o) for o in rest.split(",")]
        return regs[0] + regs[1], regs[0] + regs[1]
    return G._reads_writes(text)


MASK = "MASK"
MASK_READS = [S(i) for i in range(8)] + ["%[mask]"]
MASK_WRITES = [S(i) for i in range(8)] + ["vcc", f"v{TMP[0]}", f"v{TMP[1]}"]


def softmax_valu():
    """Tile t's VALU work in program order: (text, lds_name or None, deps)."""
    t = [f"v{r}" for r in TMP]
    ops = []
    last_w, last_r = {}, {}

    def op(text, lds=None):
        rd, wr = (MASK_READS, MASK_WRITES) if text == MASK else rw(text)
        deps = set()
        for r in rd:
            if r in last_w:
                deps.add(last_w[r])
        for r in wr:
            deps.update(last_r.get(r, ()))
            if r in last_w:
                deps.add(last_w[r])
        i = len(ops)
        ops.append((text, lds, tuple(sorted(deps))))
        for r in rd:
            last_r.setdefault(r, set()).add(i)
        for r in wr:
            last_w[r] = i
            last_r[r] = set()
        return i

    # hi + lo: swap rows so that each lane pairs its column with the
    # matching one, then add (scores i and i + 8 of the same lane combine
    # into score i of the lanes of rows rho = 0, 2, and score i + 8 of
    # rho = 1, 3 -- all kept in register i).
    for i in range(8):
        op(f"v_permlane16_swap_b32 {S(i)}, {S(i + 8)}")
        op(f"v_add_f32 {S(i)}, {S(i)}, {S(i + 8)}")
    op(MASK)
    op(f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]")
    op(f"v_max3_f32 {t[0]}, {S(0)}, {S(1)}, {S(2)}")
    op(f"v_max3_f32 {t[1]}, {S(3)}, {S(4)}, {S(5)}")
    op(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {S(6)}")
    op(f"v_max_f32 {t[0]}, {t[0]}, {S(7)}")
    op(f"v_mov_b32 {t[1]}, {t[0]}")
    op(f"v_permlane16_swap_b32 {t[0]}, {t[1]}")
    op(f"v_max_f32 {t[0]}, {t[0]}, {t[1]}")
    op(f"v_mov_b32 {t[1]}, {t[0]}")
    op(f"v_permlane32_swap_b32 {t[0]}, {t[1]}")
    op(f"v_max_f32 {t[0]}, {t[0]}, {t[1]}")
    op(f"v_max_f32 %[mseen], %[mseen], {t[0]}")
    op(f"v_cndmask_b32 %[mref], %[mref], {t[0]}, vcc")
    op(f"v_sub_f32 {t[2]}, {t[0]}, %[mref]")
    op(f"v_max_f32 %[exc], %[exc], {t[2]}")
    op(f"v_max_f32 {t[3]}, 0xff7fffff, %[mref]")
    for i in range(8):
        op(f"v_sub_f32 {S(i)}, {S(i)}, {t[3]}")
        op(f"v_exp_f32 {S(i)}, {S(i)}")
    pk = [f"v{P_PACK + k}" for k in range(4)]
    for k in range(4):
        op(f"v_cvt_pk_f16_f32 {pk[k]}, {S(2 * k)}, {S(2 * k + 1)}")
    op(f"ds_write_b128 %[pw], v[{P_PACK}:{P_PACK + 3}]", lds="w")
    op(f"v_mov_b32 {t[4]}, 0")
    for k in range(4):
        acc = "%[l]" if k % 2 == 0 else t[4]
        lo, hi = (t[5], t[6]) if k % 2 == 0 else (t[7], t[1])
        op(f"v_cvt_f32_f16 {lo}, {pk[k]}")
        op(f"v_cvt_f32_f16_sdwa {hi}, {pk[k]} src0_sel:WORD_1")
        op(f"v_add_f32 {acc}, {acc}, {lo}")
        op(f"v_add_f32 {acc}, {acc}, {hi}")
    op(f"v_add_f32 %[l], %[l], {t[4]}")
    return ops


def mask_block():
    """Out-of-line mask code: combined score i becomes -inf unless bit i of
    %[mask] is set; then back into the block."""
    t0, t1 = f"v{TMP[0]}", f"v{TMP[1]}"
    lines = [".Ltv_q2_mask_%=:", f"v_mov_b32 {t0}, {NEG_INF}"]
    for i in range(8):
        lines += [f"v_bfe_u32 {t1}, %[mask], {i}, 1", f"v_cmp_ne_u32 vcc, 0, {t1}",
                  f"v_cndmask_b32 {S(i)}, {t0}, {S(i)}, vcc"]
    lines.append("s_branch .Ltv_q2_masked_%=")
    return lines


def step_asm() -> str:
    mfma, needs = [], []
    for ks in range(36):
        mfma.append(("qk", ks))
        needs.append([f"K{ks}"])
    for n in range(16):
        f, rb = n >> 1, n & 1
        mfma.append(("pv", n))
        needs.append([f"V{f}", f"P{rb}{f >> 2}"])
    first_use, last_use, order = {}, {}, []
    for m, frs in enumerate(needs):
        for fr in frs:
            if fr not in first_use:
                first_use[fr] = m
                order.append(fr)
            last_use[fr] = m
    release = {}
    for fr, m in last_use.items():
        release.setdefault(m + 2, []).append(fr)

    def ahead(fr):
        return AHEAD_K if fr[0] == "K" else AHEAD_VP

    # Pass 1: which fragments are read before each matrix op (first-use
    # order among the eligible ones, while the pool has quads).
    free = list(POOL)
    where = {}
    loads_before = [[] for _ in mfma]
    pending = list(order)
    for m in range(len(mfma)):
        for fr in release.get(m, []):
            if fr[0] != "V":
                free.append(where[fr])
        issued = 0
        for fr in list(pending):
            if not free and fr[0] != "V":
                continue
            must = first_use[fr] <= m
            # before the first op, every K fragment within reach (the step
            # starts with the pipeline of reads empty)
            cap = AHEAD_K + 1 if m == 0 else LOADS_PER_GAP
            if first_use[fr] <= m + ahead(fr) and (issued < cap or must):
                where[fr] = V_BASE + 4 * int(fr[1:]) if fr[0] == "V" else free.pop(0)
                loads_before[m].append(fr)
                pending.remove(fr)
                issued += 1
        assert all(first_use[fr] > m for fr in pending), f"pool too small at op {m}"
    assert not pending

    lines = ["s_mov_b32 %[ms], m0"]
    q = G.LdsQueue(lines)
    cur_m = [0]
    read_at = {}
    ws = [None]   # wait states since the last score op

    def emit(text, lds_name=None):
        if lds_name:
            q.issue(text, lds_name)
        else:
            lines.append(text)
        if ws[0] is not None:
            ws[0] += sum(int(x.split()[1]) + 1 if x.strip().startswith("s_nop") else 1
                         for x in text.split("\\n") if x.strip() and not x.strip().endswith(":"))

    def load(fr):
        r = where[fr]
        kind, idx = fr[0], fr[1:]
        if kind == "K":
            ks = int(idx)
            src = f"%[lat] offset:{32 * ks}" if ks < 32 else f"%[rope] offset:{256 * (ks - 32)}"
            emit(f"ds_read_b128 {aquad(r)}, {src}", fr)
        elif kind == "V":
            f = int(idx)
            off = 16640 * (f >> 2) + 16 * (f & 3)
            emit(f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[tb] offset:{off}", fr + "lo")
            emit(f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[tb] offset:{off + 8320}", fr)
            read_at[f] = cur_m[0]
        else:  # P<rb><h>
            rb, h = int(idx[0]), int(idx[1])
            emit(f"ds_read_b128 {aquad(r)}, %[pb] offset:{1024 * (2 * rb + h)}", fr)

    stage = G.stage_ops()
    assert len(stage) == COPY_GROUPS
    valu = softmax_valu()
    s_regs = {S(i) for i in range(16)}
    reads_s = [text != MASK and any(r in s_regs for r in rw(text)[0]) for text, _, _ in valu]
    pending_v = list(range(len(valu)))
    gap_of = {}
    first_read = [False]

    def same_gap_ok(i, d):
        """May op i sit in the same gap as its producer d?  Plain VALU results
        are forwarded without wait states; a transcendental's result and a
        v_permlane*_swap source written by VALU are not."""
        return not valu[d][0].startswith("v_exp") and not valu[i][0].startswith("v_permlane")

    def place(i, n):
        text, lds_name, _ = valu[i]
        if reads_s[i] and not first_read[0]:
            pad = max(S_HAZARD - ws[0], 0)
            if pad:
                emit(f"s_nop {pad - 1}")
            assert ws[0] >= S_HAZARD
            first_read[0] = True
        if text == MASK:
            for x in G.mask_branch():
                emit(x.replace(".Ltv_", ".Ltv_q2_"))
        else:
            emit(text, lds_name)
        gap_of[i] = n
        pending_v.remove(i)

    def fill_gap(n, budget, last):
        """List-schedule VALU ops into the gap after value op n: at most
        budget instructions and TRANS_PER_GAP transcendentals; an op whose
        producer sits in this gap only if same_gap_ok.  The last gap takes
        everything left, in program order, with s_nop where a producer in
        the same gap needs wait states."""
        if last:
            for i in list(pending_v):
                if any(gap_of.get(d) == n and not same_gap_ok(i, d) for d in valu[i][2]):
                    emit("s_nop 1")
                place(i, n)
            return
        placed = trans = 0
        for i in list(pending_v):
            text, _, deps = valu[i]
            is_trans = text.startswith("v_exp")
            need = 2 if text == MASK else 1
            if placed + need > budget:
                break
            if is_trans and trans == TRANS_PER_GAP:
                continue
            if not all(d in gap_of and (gap_of[d] < n or same_gap_ok(i, d)) for d in deps):
                continue
            place(i, n)
            placed += need
            trans += is_trans

    def convert_half(f, h):
        """bf16 -> fp16 in place, dwords 2h, 2h + 1 of value fragment f
        (exact for magnitudes from 2^-17 to 65504; below that rounded to
        fp16's 2^-24 spacing)."""
        base = V_BASE + 4 * f
        for d in (base + 2 * h, base + 2 * h + 1):
            emit(f"v_lshlrev_b32 v{CVT_TMP}, 16, v{d}")
            emit(f"v_and_b32 v{d}, 0xffff0000, v{d}")
            emit(f"v_cvt_pk_f16_f32 v{d}, v{CVT_TMP}, v{d}")

    cvt_todo = []      # (fragment, half) in order; one half per gap once due
    cvt_done_at = {}   # fragment -> matrix-op index after which it was converted

    def convert_due(m):
        if cvt_todo:
            f, h = cvt_todo[0]
            if read_at[f] + CVT_DELAY <= m or first_use[f"V{f}"] <= m + 2:
                cvt_todo.pop(0)
                if h == 0:
                    q.wait_for(f"V{f}")
                convert_half(f, h)
                if h == 1:
                    cvt_done_at[f] = m

    for m, (kind, idx) in enumerate(mfma):
        cur_m[0] = m
        for fr in loads_before[m]:
            load(fr)
            if fr[0] == "V":
                cvt_todo.extend([(int(fr[1:]), 0), (int(fr[1:]), 1)])
        q.wait_for(*needs[m])
        if kind == "pv":
            f_need = idx >> 1
            assert cvt_done_at.get(f_need, m) < m - 1, f"value fragment {f_need} converted too late for op {m}"
        if kind == "qk":
            ks = idx
            b = f"%[q{ks}]" if ks < 32 else f"%[qr{ks - 32}]"
            c = "0" if ks == 0 else f"v[{S_BASE}:{S_BASE + 15}]"
            emit(f"v_mfma_f32_32x32x16_bf16 v[{S_BASE}:{S_BASE + 15}], {aquad(where[f'K{ks}'])}, {b}, {c}")
            if ks < len(stage):
                for x in stage[ks]:
                    emit(x)
            convert_due(m)
            if ks == 35:
                ws[0] = 0
        else:
            n = idx
            f, rb = n >> 1, n & 1
            o = f"%[o{4 * rb + (f & 3)}]"
            vq = where[f"V{f}"]
            emit(f"v_mfma_f32_32x32x16_f16 {o}, v[{vq}:{vq + 3}], {aquad(where[f'P{rb}{f >> 2}'])}, {o}")
            convert_due(m)
            fill_gap(n, GAP_BUDGET, n == 15)
            if n == 0:
                assert first_read[0], "the first gap must start the softmax"
    assert not pending_v, "softmax does not fit between the value ops"
    assert not cvt_todo and len(cvt_done_at) == 8, "value fragments left unconverted"
    lines.append("s_mov_b32 m0, %[ms]")
    lines.append("s_waitcnt lgkmcnt(0)")
    lines.append("s_branch .Ltv_q2_end_%=")
    lines.extend(mask_block())
    lines.append(".Ltv_q2_end_%=:")
    return "\\n".join(lines) + "\\n"


def main():
    clob = [f'"v{r}"' for r in CLOBBERED_V] + [f'"a{r}"' for r in range(128, 256)]
    text = f"""// Generated by gen_mfma_q2_asm.py -- do not edit by hand.
// Inline-asm step block of attn_mfma_q2.hip (see the generator's docstring).
#pragma once

#define TV_Q2_STEP_ASM "{step_asm()}"

// Registers the step block uses by number (clobbered).
#define TV_Q2_STEP_CLOBBERS {", ".join(clob)}
"""
    with open(OUT, "w") as f:
        f.write(text)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
