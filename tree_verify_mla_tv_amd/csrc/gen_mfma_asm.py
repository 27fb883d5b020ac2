#!/usr/bin/env python3
"""Generate attn_mfma_asm.h: the inline-asm blocks of attn_mfma.hip.

    python tree_verify_mla_tv_amd/csrc/gen_mfma_asm.py   # rewrites attn_mfma_asm.h

One step of the kv sweep is one asm block, written out instruction by
instruction, so that the matrix core never waits on anything the schedule can
hide: every LDS fragment is read several matrix ops ahead of its use, the
value product of the previous tile starts right behind the last score op, and
the mask, row max and softmax of this tile run between value ops.  (Left to
the compiler, short of registers next to 256 accumulators and 128 query
registers, each read lands right before its consumer and the VALU work runs
between the two products.)

TV_STEP_ASM -- per wave, for tile t (scores) and tile t-1 (values):
  1. Scores S^T = K Q^T: 36 x v_mfma_f32_32x32x16_bf16 into S (v[176:191]).
     k-step ks < 32 takes its K fragment at %[lat] + 32 ks and the query
     fragment %[q<ks>]; ks >= 32 takes K at %[rope] + 256 (ks - 32) and the
     query fragment at %[qr] + 4096 (ks - 32) (rope part, LDS).
     Woven in: this wave's copy of tile t+1 (the TV_STAGE_ASM loads, one every
     second op), so that the four waves never queue 36 LDS-DMA loads at once.
  2. Values O^T[rb][db] (%[o<4 rb + db>]) += V(db, h) x P(rb, h) for tile t-1:
     32 MFMAs, n = 16 h + 4 db + rb.  V(db, h) is read from the row-major tile
     with two ds_read_b64_tr_b16 at %[tb] + 16640 h + 16 db (+ 8320 for keys
     8..15 of the half); P(rb, h), tile t-1's bf16 weights, with ds_read_b128
     at %[pb] + 1024 (2 rb + h).
     Woven in, for tile t (all VALU, lane = one query row, 16 of its scores):
       mask   (only when %[nm] != 0, out of line behind a branch): score i
              becomes -inf unless bit i of %[mask] is set;
       max    over the 16 scores and the other half of the wave (the lane
              l ^ 32 holds the same row: v_permlane32_swap);
       state  %[mseen] = max(%[mseen], max); %[mref] takes the max if it was
              -inf (first visible tile); %[exc] = max(%[exc], max - %[mref]);
              the reference used is max(%[mref], -FLT_MAX) (equal to %[mref]
              unless every score so far is -inf, when exp2(-inf - ref) = 0);
       weights  s <- exp2(s - ref), packed to bf16 pairs in v[240:247] and
              stored with ds_write_b128 at %[pw] (keys 0..15) and %[pw] + 1024;
              the row sum %[l] adds the packed (rounded) weights, unpacked
              with a shift and a mask, in two fp32 chains.
     These ops form a dependency graph (derived from their register
     operands) that is list-scheduled into the gaps between value ops: at
     most GAP_BUDGET instructions per gap counting the LDS loads and waits
     there (one wave per SIMD issues about one instruction per 4 cycles; a
     matrix op lasts 32), TRANS_PER_GAP transcendentals, and never in the
     same gap as an op whose result they read.  The first read of S comes
     S_HAZARD wait states after the last score op, right behind the mask
     branch; ops that touch VCC or the mask's temporaries also follow it.
All LDS fragments go through a pool of register quads v[192:239] assigned here
(an MFMA operand must be one register quad, and an asm operand cannot be
split); a quad is reused one matrix op after its last reader.  Waits are
exact lgkmcnt counts from a simulation of the wave's in-order LDS queue.

TV_STAGE_ASM -- the copy alone: wave w's nine buffer_load_dwordx4 ... lds of a
  tile.  Latent row r = 0..7 (key min(%[kb] + r, %[km])) lands at LDS
  %[mb] + 1040 r from buffer %[rl] at byte key * 1024 + %[l16]; the rope rows
  land at %[mr] from buffer %[rr] at per-lane byte %[ro].  M0 (the LDS
  destination of a DMA load) is saved in %[ms] and restored at the end, and
  %[t] holds each row's buffer offset.

Hazards handled inside the blocks: LDS data waits; the matrix-core result S
before the first VALU read (>= S_HAZARD wait states); the M0 and offset writes a
matrix op before the DMA load that reads them; v_permlane32_swap two wait
states after the VALU write of its operand; every transcendental result used
a matrix op or more later; the accumulators before anything outside the
sweep reads them (TV_MFMA_DRAIN_ASM after the last step).
"""
import os
import re

S_BASE = 176                                  # v[176:191]: the 16 scores (MFMA accumulator)
POOL = [192 + 4 * i for i in range(12)]       # v[192:239]: LDS fragment quads
P_QUADS = [240, 244]                          # v[240:247]: packed weights, key half 0 and 1
TMP = list(range(248, 256))                   # v[248:255]: VALU temporaries
CLOBBERED = list(range(S_BASE, 256))
AHEAD = 6        # a fragment is read at most this many matrix ops before its first use
QK_COPY_GROUPS = 18   # copy groups issued among the score ops; the rest go among the value ops
GAP_BUDGET = 5        # instructions between two value MFMAs (one wave per SIMD issues ~1 per 4 cycles; an MFMA is 32)
TRANS_PER_GAP = 3     # of which v_exp_f32
S_HAZARD = 12         # wait states from the last score MFMA to the first VALU read of S
STORES_AT_END = False # weights stored after the last value op instead of between them
NOP_AFTER = "s_nop 7\\n s_nop 7\\n s_nop 7\\n"   # >= 19 wait states after the last MFMA
NEG_INF = "0xff800000"
ONE_ONE_BF16 = "0x3f803f80"

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "attn_mfma_asm.h")


def S(i):
    return f"v{S_BASE + i}"


def quad(r):
    return f"v[{r}:{r + 3}]"


class LdsQueue:
    """Issue order of LDS instructions; a wait for one of them is the number
    issued after it (LDS instructions of one wave complete in order)."""

    def __init__(self, lines):
        self.lines = lines
        self.issued = []

    def issue(self, text, name):
        self.lines.append(text)
        self.issued.append(name)

    def wait_for(self, *names):
        idx = max(self.issued.index(n) for n in names)
        self.lines.append(f"s_waitcnt lgkmcnt({min(len(self.issued) - idx - 1, 15)})")


def stage_ops():
    """The tile copy as groups of instructions; a group is issued after one
    matrix op.  The address group of a row and its load sit one op apart, so
    the M0 / offset writes are a few wait states before the load reads them."""
    groups = []
    for r in range(8):
        m0 = "s_mov_b32 m0, %[mb]" if r == 0 else f"s_add_u32 m0, %[mb], {1040 * r}"
        groups.append([m0, f"s_add_i32 %[t], %[kb], {r}", "s_min_i32 %[t], %[t], %[km]",
                       "s_lshl_b32 %[t], %[t], 10"])
        groups.append(["buffer_load_dwordx4 %[l16], %[rl], %[t] offen lds"])
    groups.append(["s_mov_b32 m0, %[mr]"])
    groups.append(["buffer_load_dwordx4 %[ro], %[rr], 0 offen lds"])
    return groups


def stage_asm() -> str:
    lines = ["s_mov_b32 %[ms], m0"]
    for g in stage_ops():
        lines.extend(g)
        lines.append("s_nop 1")
    lines.append("s_mov_b32 m0, %[ms]")
    return "\\n".join(lines) + "\\n"


def _regs(tok):
    """Registers named by one operand token: v12, v[12:15], %[name], vcc."""
    tok = tok.strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return [f"v{r}" for r in range(int(m.group(1)), int(m.group(2)) + 1)]
    if re.fullmatch(r"v\d+", tok) or tok.startswith("%[") or tok == "vcc":
        return [tok]
    return []


def _reads_writes(text):
    mnem, _, rest = text.partition(" ")
    ops = [o for o in rest.split(",")]
    ops = [o.split(" offset")[0] for o in ops]
    regs = [_regs(o) for o in ops]
    if mnem.startswith("v_cmp"):
        return sum(regs[1:], []), ["vcc"]
    if mnem.startswith("v_cndmask"):
        return sum(regs[1:], []), regs[0]
    if mnem.startswith("v_permlane32_swap"):
        return regs[0] + regs[1], regs[0] + regs[1]
    if mnem.startswith("ds_write"):
        return sum(regs, []), []
    if mnem.startswith("v_"):
        return sum(regs[1:], []), regs[0]
    return [], []


def softmax_valu():
    """Tile t's VALU work in program order: list of (text, lds_name or None,
    deps), deps being the earlier ops this one must follow (it reads their
    results, or overwrites a register they read or write).  The mask is
    separate (a branch, before all of this)."""
    t = [f"v{r}" for r in TMP]
    ops = []
    last_w, last_r = {}, {}

    def op(text, lds=None):
        rd, wr = _reads_writes(text)
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

    # VCC = (m_ref == -inf), taken before m_ref changes.
    op(f"v_cmp_eq_f32 vcc, {NEG_INF}, %[mref]")
    # Row max: a tree of v_max3 over the 16 scores, then the other half-wave.
    for k in range(5):
        op(f"v_max3_f32 {t[k]}, {S(3 * k)}, {S(3 * k + 1)}, {S(3 * k + 2)}")
    op(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {t[2]}")
    op(f"v_max3_f32 {t[3]}, {t[3]}, {t[4]}, {S(15)}")
    op(f"v_max_f32 {t[0]}, {t[0]}, {t[3]}")
    op(f"v_mov_b32 {t[1]}, {t[0]}")
    op(f"v_permlane32_swap_b32 {t[0]}, {t[1]}")
    op(f"v_max_f32 {t[0]}, {t[0]}, {t[1]}")
    # Row state.  m_ref takes the max on the first visible tile; the
    # reference of this tile's exponentials is max(m_ref, -FLT_MAX): it equals
    # m_ref unless every score so far is -inf, and then exp2(-inf - ref) = 0.
    op(f"v_max_f32 %[mseen], %[mseen], {t[0]}")
    op(f"v_cndmask_b32 %[mref], %[mref], {t[0]}, vcc")
    op(f"v_sub_f32 {t[2]}, {t[0]}, %[mref]")
    op(f"v_max_f32 %[exc], %[exc], {t[2]}")
    op(f"v_max_f32 {t[3]}, 0xff7fffff, %[mref]")
    # Weights: s <- exp2(s - ref), packed pairs.
    for i in range(16):
        op(f"v_sub_f32 {S(i)}, {S(i)}, {t[3]}")
        op(f"v_exp_f32 {S(i)}, {S(i)}")

    def pk(k):  # packed pair k: scores 2k, 2k+1 (key half k // 4)
        return f"v{P_QUADS[k // 4] + k % 4}"

    for k in range(8):
        op(f"v_cvt_pk_bf16_f32 {pk(k)}, {S(2 * k)}, {S(2 * k + 1)}")
        if k % 4 == 3 and not STORES_AT_END:
            # Store each half as soon as it is packed (listed early, so the
            # scheduler issues it early and its latency hides behind the
            # remaining value ops).
            h = k // 4
            op(f"ds_write_b128 %[pw], {quad(P_QUADS[h])} offset:{1024 * h}", lds=f"w{h}")
    # The row sum takes the rounded weights the value product uses: a bf16
    # value is its bits in the top half of an fp32 word, so each packed pair
    # unpacks with one shift and one mask, then plain fp32 adds in two chains
    # (even pairs into l, odd pairs into t[4]).  (v_dot2c_f32_bf16 would add
    # two at once but holds back the next matrix op by ~16 cycles.)
    op(f"v_mov_b32 {t[4]}, 0")
    for k in range(8):
        acc = "%[l]" if k % 2 == 0 else t[4]
        lo, hi = (t[5], t[6]) if k % 2 == 0 else (t[7], t[1])
        op(f"v_lshlrev_b32 {lo}, 16, {pk(k)}")
        op(f"v_and_b32 {hi}, 0xffff0000, {pk(k)}")
        op(f"v_add_f32 {acc}, {acc}, {lo}")
        op(f"v_add_f32 {acc}, {acc}, {hi}")
    op(f"v_add_f32 %[l], %[l], {t[4]}")
    return ops


def schedule_valu(ops, n_slots, first_slot, per_slot, trans_per_slot=3):
    """Greedy list schedule of the VALU graph into the gaps after matrix ops:
    at most per_slot ops (and trans_per_slot transcendentals) per gap, and an
    op never shares a gap with an op it reads (a matrix op, >= 32 cycles, sits
    between producer and consumer)."""
    slot_of = {}
    out = [[] for _ in range(n_slots)]
    pending = list(range(len(ops)))
    for sl in range(first_slot, n_slots):
        placed = trans = 0
        for i in list(pending):
            if placed == per_slot:
                break
            is_trans = ops[i][0].startswith("v_exp")
            if is_trans and trans == trans_per_slot:
                continue
            if all(d in slot_of and slot_of[d] < sl for d in ops[i][2]):
                slot_of[i] = sl
                out[sl].append(ops[i])
                pending.remove(i)
                placed += 1
                trans += is_trans
        if not pending:
            break
    assert not pending, "softmax does not fit between the value ops"
    return out


def mask_branch():
    """Entry to the mask: a branch taken only when %[nm] != 0 (tiles holding
    tree keys or the unit's range end).  The mask code itself sits out of line
    after the block's last instruction (mask_block), so the common path runs
    straight through: a taken branch here would stall instruction fetch right
    behind the first value MFMA on every step."""
    return ["s_cmp_lg_u32 %[nm], 0", "s_cbranch_scc1 .Ltv_mask_%=", ".Ltv_masked_%=:"]


def mask_block():
    """Out-of-line mask code: score i becomes -inf unless bit i of %[mask] is
    set; then back into the block."""
    # -inf in a register: v_cndmask with VCC has no constant-bus slot left
    # for a literal.
    t0, t1 = f"v{TMP[0]}", f"v{TMP[1]}"
    lines = [".Ltv_mask_%=:", f"v_mov_b32 {t0}, {NEG_INF}"]
    for i in range(16):
        lines += [f"v_bfe_u32 {t1}, %[mask], {i}, 1", f"v_cmp_ne_u32 vcc, 0, {t1}",
                  f"v_cndmask_b32 {S(i)}, {t0}, {S(i)}, vcc"]
    lines.append("s_branch .Ltv_masked_%=")
    return lines


def step_asm() -> str:
    # Matrix ops in issue order and the fragments each reads.
    mfma, needs = [], []
    for ks in range(36):
        mfma.append(("qk", ks))
        needs.append([f"K{ks}"] if ks < 32 else [f"K{ks}", f"R{ks - 32}"])
    for n in range(32):
        f, rb = n >> 2, n & 3
        mfma.append(("pv", n))
        needs.append([f"V{f}", f"P{rb}{f >> 2}"])
    first_use, last_use, order = {}, {}, []
    for m, frs in enumerate(needs):
        for fr in frs:
            if fr not in first_use:
                first_use[fr] = m
                order.append(fr)
            last_use[fr] = m
    # A quad whose last reader is op m goes back to the pool once op m + 1 has
    # been issued (release[m + 2] is handed back before op m + 2).
    release = {}
    for fr, m in last_use.items():
        release.setdefault(m + 2, []).append(fr)

    # Pass 1: the LDS fragment loads.  Before matrix op m, every fragment whose
    # first use is at most AHEAD ops away is loaded, while the pool has quads.
    free = list(POOL)
    where = {}
    loads_before = [[] for _ in mfma]
    nxt = 0
    for m in range(len(mfma)):
        for fr in release.get(m, []):
            free.append(where[fr])
        while nxt < len(order) and first_use[order[nxt]] <= m + AHEAD and free:
            where[order[nxt]] = free.pop(0)
            loads_before[m].append(order[nxt])
            nxt += 1
    assert nxt == len(order)

    lines = ["s_mov_b32 %[ms], m0"]
    q = LdsQueue(lines)
    ws = [None]   # wait states (instructions) since the last score MFMA

    def emit(text, lds_name=None):
        if lds_name:
            q.issue(text, lds_name)
        else:
            lines.append(text)
        if ws[0] is not None:
            ws[0] += sum(int(t.split()[1]) + 1 if t.strip().startswith("s_nop") else 1
                         for t in text.split("\\n") if t.strip() and not t.strip().endswith(":"))

    def load(fr):
        r = where[fr]
        kind, idx = fr[0], fr[1:]
        if kind == "K":
            ks = int(idx)
            src = f"%[lat] offset:{32 * ks}" if ks < 32 else f"%[rope] offset:{256 * (ks - 32)}"
            emit(f"ds_read_b128 {quad(r)}, {src}", fr)
        elif kind == "R":
            emit(f"ds_read_b128 {quad(r)}, %[qr] offset:{4096 * int(idx)}", fr)
        elif kind == "V":
            f = int(idx)
            off = 16640 * (f >> 2) + 16 * (f & 3)
            emit(f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[tb] offset:{off}", fr + "lo")
            emit(f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[tb] offset:{off + 8320}", fr)
        else:  # P<rb><h>
            rb, h = int(idx[0]), int(idx[1])
            emit(f"ds_read_b128 {quad(r)}, %[pb] offset:{1024 * (2 * rb + h)}", fr)

    def n_instr(fr):
        return 2 if fr[0] == "V" else 1

    stage = stage_ops()
    stage_qk, stage_pv = stage[:QK_COPY_GROUPS], stage[QK_COPY_GROUPS:]
    valu = softmax_valu()
    s_regs = {S(i) for i in range(16)}
    reads_s = [any(r in s_regs for r in _reads_writes(t)[0]) for t, _, _ in valu]
    # The mask code overwrites VCC and two temporaries: an op that touches
    # them, like one that reads S, must come after the mask branch.
    mask_regs = {"vcc", f"v{TMP[0]}", f"v{TMP[1]}"}
    after_mask = [reads_s[i] or any(r in mask_regs for rw in _reads_writes(t) for r in rw)
                  for i, (t, _, _) in enumerate(valu)]
    pending = list(range(len(valu)))
    gap_of = {}
    masked = [False]

    def fill_gap(n, budget, last):
        """List-schedule VALU ops into the gap after value op n: at most budget
        instructions, TRANS_PER_GAP transcendentals, and no op in the same gap
        as an op it depends on, so a matrix op (32 cycles) covers each
        producer's latency and hazard.  The first read of S comes
        >= S_HAZARD wait states after the last score MFMA, padded with s_nop
        if nothing else fills them, right behind the mask branch."""
        placed = trans = 0
        for i in list(pending):
            text, lds_name, deps = valu[i]
            is_trans = text.startswith("v_exp")
            first_s = after_mask[i] and not masked[0]
            pad = max(S_HAZARD - ws[0] - 2, 0) if first_s else 0
            need = 1 + (2 + (pad > 0) if first_s else 0)
            if placed + need > budget:
                if first_s:
                    continue
                break
            if is_trans and trans == TRANS_PER_GAP and not last:
                continue
            # Within the last gap a chain may run back to back, except where
            # the hardware does not interlock: a transcendental's result (one
            # wait state) and a VGPR that v_permlane32_swap reads (two).
            if not all(d in gap_of and (gap_of[d] < n or (last and not valu[d][0].startswith("v_exp")
                                                          and not text.startswith("v_permlane")))
                       for d in deps):
                continue
            if first_s:
                if pad:
                    emit(f"s_nop {pad - 1}")
                for t in mask_branch():
                    emit(t)
                masked[0] = True
            elif reads_s[i]:
                assert ws[0] >= S_HAZARD
            emit(text, lds_name)
            gap_of[i] = n
            pending.remove(i)
            placed += need
            trans += is_trans

    for m, (kind, idx) in enumerate(mfma):
        for fr in loads_before[m]:
            load(fr)
        q.wait_for(*needs[m])
        if kind == "qk":
            ks = idx
            a = quad(where[f"K{ks}"])
            b = f"%[q{ks}]" if ks < 32 else quad(where[f"R{ks - 32}"])
            c = "0" if ks == 0 else f"v[{S_BASE}:{S_BASE + 15}]"
            emit(f"v_mfma_f32_32x32x16_bf16 v[{S_BASE}:{S_BASE + 15}], {a}, {b}, {c}")
            if ks < len(stage_qk):
                for t in stage_qk[ks]:
                    emit(t)
            if ks == 35:
                ws[0] = 0
        else:
            n = idx
            f, rb = n >> 2, n & 3
            o = f"%[o{4 * rb + (f & 3)}]"
            emit(f"v_mfma_f32_32x32x16_bf16 {o}, {quad(where[f'V{f}'])}, "
                 f"{quad(where[f'P{rb}{f >> 2}'])}, {o}")
            if n < len(stage_pv):
                for t in stage_pv[n]:
                    emit(t)
            nxt_loads = sum(n_instr(fr) for fr in loads_before[m + 1]) if m + 1 < len(mfma) else 0
            budget = GAP_BUDGET - nxt_loads - (1 if m + 1 < len(mfma) else 0)
            last = n == len(mfma) - 37   # the last gap takes whatever is left
            fill_gap(n, 10 ** 6 if last else max(budget, 1), last)
    assert not pending, "softmax does not fit between the value ops"
    if STORES_AT_END:
        for h in range(2):
            q.issue(f"ds_write_b128 %[pw], {quad(P_QUADS[h])} offset:{1024 * h}", f"w{h}")
    lines.append("s_mov_b32 m0, %[ms]")
    lines.append("s_waitcnt lgkmcnt(0)")
    # The out-of-line mask code, jumped over (the only taken branch on the
    # common path, behind the last MFMA).  No padding: nothing reads the
    # accumulators until after the sweep (TV_MFMA_DRAIN_ASM there).
    lines.append("s_branch .Ltv_end_%=")
    lines.extend(mask_block())
    lines.append(".Ltv_end_%=:")
    return "\\n".join(lines) + "\\n"


def main():
    text = f"""// Generated by gen_mfma_asm.py -- do not edit by hand.
// Inline-asm blocks of attn_mfma.hip (see the generator's docstring).
#pragma once

#define TV_STAGE_ASM "{stage_asm()}"

#define TV_STEP_ASM "{step_asm()}"

// After the last step: >= 19 wait states before the accumulators are read.
#define TV_MFMA_DRAIN_ASM "{NOP_AFTER}"

// Registers the step block uses by number (clobbered).
#define TV_STEP_CLOBBERS {", ".join(f'"v{r}"' for r in CLOBBERED)}
"""
    with open(OUT, "w") as f:
        f.write(text)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
