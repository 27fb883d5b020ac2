#!/usr/bin/env python3
"""Generate attn_mfma_asm.h: the two inline-asm blocks of attn_mfma.hip.

    python tree_verify_mla_tv_amd/csrc/gen_mfma_asm.py   # rewrites attn_mfma_asm.h

The blocks are written out instruction by instruction so that every LDS read
is issued well ahead of the matrix op that consumes it and the softmax VALU
work sits between matrix ops (the compiler, short of registers next to 256
accumulators and 128 query registers, otherwise places each read right before
its consumer, waits for it, and runs the softmax between the two products).
Register choice stays with the compiler through named operands, except for the
four value-fragment slots (see below); only order and waits are fixed here.

TV_QK_ASM -- scores of one tile, per wave: 36 x v_mfma_f32_32x32x16_bf16 into
  %[s].  k-step ks < 32 reads its K fragment at %[lat] + 32 ks, ks >= 32 at
  %[rope] + 256 (ks - 32); its Q fragment is %[qN] for ks < 32, and for
  ks >= 32 an LDS fragment at %[qr] + 4096 (ks - 32), read first into %[rN].

TV_PVS_ASM -- value product of the previous tile with this tile's softmax woven
  in.  Value part: 32 MFMAs, n = 16 h + 4 db + rb, accumulate
  O[rb][db] (%[o<4 rb + db>]) += V(db, h) x P(rb, h), where
    V(db, h)  this wave's d-block db (32 latent columns) of key half h, read
              from the row-major tile with two ds_read_b64_tr_b16 at
              %[tb] + 16640 h + 64 db (+ 8320 for keys 8..15 of the half) into
              one of four fixed register quads v[240:255] (an MFMA operand
              must be one quad, and an operand of the asm cannot be split);
    P(rb, h)  the previous tile's bf16 weights of row block rb, key half h,
              read with ds_read_b128 at %[pb] + 1024 (2 rb + h) into %[pi<2 rb + h>].
  Softmax part: for this tile's 16 scores %[s0..15] of the lane's row,
  s <- exp2(s - %[mref]), packed to bf16 pairs %[pk0..7], summed into %[l]
  with a bf16 dot product against (1, 1), and stored at %[pw0] (keys of half 0)
  and %[pw1] (half 1).

Hazards handled inside the blocks: LDS data waits (s_waitcnt lgkmcnt, counted
by simulating the in-order LDS queue of the block's own reads and writes),
the distance between a transcendental result and its first use, and the
matrix-core results before anything outside a block reads them (s_nop padding
at the end of each block).
"""
import os

DEPTH = 4   # score chain: K reads in flight ahead of the matrix op that consumes them
SLOTS = 6   # score chain: rotating K fragment registers
NOP_AFTER = "s_nop 7\\n s_nop 7\\n s_nop 7\\n"   # >= 19 wait states after the last MFMA
V_QUADS = [240, 244, 248, 252]   # value-fragment register quads of TV_PVS_ASM
V_AHEAD = 2                      # value fragments loaded ahead of the one in use

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "attn_mfma_asm.h")


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


def qk_asm() -> str:
    lines = []
    q = LdsQueue(lines)
    for r in range(4):
        q.issue(f"ds_read_b128 %[r{r}], %[qr] offset:{4096 * r}", f"r{r}")

    def k_read(ks):
        slot = ks % SLOTS
        if ks < 32:
            q.issue(f"ds_read_b128 %[k{slot}], %[lat] offset:{32 * ks}", f"k{ks}")
        else:
            q.issue(f"ds_read_b128 %[k{slot}], %[rope] offset:{256 * (ks - 32)}", f"k{ks}")

    for ks in range(DEPTH):
        k_read(ks)
    for ks in range(36):
        if ks < 32:
            q.wait_for(f"k{ks}")
            src_b = f"%[q{ks}]"
        else:
            q.wait_for(f"k{ks}", f"r{ks - 32}")
            src_b = f"%[r{ks - 32}]"
        src_c = "0" if ks == 0 else "%[s]"
        lines.append(f"v_mfma_f32_32x32x16_bf16 %[s], %[k{ks % SLOTS}], {src_b}, {src_c}")
        if ks + DEPTH < 36:
            k_read(ks + DEPTH)
    return "\\n".join(lines) + "\\n" + NOP_AFTER


def softmax_ops():
    """The softmax VALU/LDS work in dependency order, as (text, lds_name or None)."""
    ops = []
    for i in range(16):
        ops.append((f"v_sub_f32 %[s{i}], %[s{i}], %[mref]", None))
        ops.append((f"v_exp_f32 %[s{i}], %[s{i}]", None))
    for k in range(8):
        ops.append((f"v_cvt_pk_bf16_f32 %[pk{k}], %[s{2 * k}], %[s{2 * k + 1}]", None))
        if k >= 1:
            ops.append((f"v_dot2c_f32_bf16 %[l], 0x3f803f80, %[pk{k - 1}]", None))
    ops.append(("v_dot2c_f32_bf16 %[l], 0x3f803f80, %[pk7]", None))
    for h in range(2):
        for pair in range(2):
            a, b = 4 * h + 2 * pair, 4 * h + 2 * pair + 1
            ops.append((f"ds_write2_b32 %[pw{h}], %[pk{a}], %[pk{b}] offset0:{2 * pair} offset1:{2 * pair + 1}",
                        f"w{h}{pair}"))
    return ops


def pvs_asm() -> str:
    lines = []
    q = LdsQueue(lines)

    def quad(f):
        return V_QUADS[f % len(V_QUADS)]

    def v_read(f):
        h, db = f >> 2, f & 3
        r = quad(f)
        off = 16640 * h + 64 * db
        q.issue(f"ds_read_b64_tr_b16 v[{r}:{r + 1}], %[tb] offset:{off}", f"vlo{f}")
        q.issue(f"ds_read_b64_tr_b16 v[{r + 2}:{r + 3}], %[tb] offset:{off + 8320}", f"vhi{f}")

    def p_read(rb, h):
        q.issue(f"ds_read_b128 %[pi{2 * rb + h}], %[pb] offset:{1024 * (2 * rb + h)}", f"p{rb}{h}")

    # Weights of key half 0, the first value fragments, then weights of half 1.
    for rb in range(4):
        p_read(rb, 0)
    for f in range(V_AHEAD):
        v_read(f)
    for rb in range(4):
        p_read(rb, 1)

    # Spread the softmax over the 32 matrix ops: two per op while exponentials
    # remain (they are quarter-rate), then the packing, sums and stores.
    sm = softmax_ops()
    per_slot, i = [], 0
    for n in range(32):
        take = 2 if n < 24 else 1
        per_slot.append(sm[i:i + take])
        i += take
    per_slot[-1].extend(sm[i:])

    for f in range(8):
        h, db = f >> 2, f & 3
        r = quad(f)
        for rb in range(4):
            n = 4 * f + rb
            q.wait_for(f"vhi{f}", f"p{rb}{h}")
            lines.append(f"v_mfma_f32_32x32x16_bf16 %[o{4 * rb + db}], v[{r}:{r + 3}], %[pi{2 * rb + h}], "
                         f"%[o{4 * rb + db}]")
            if rb == 0 and f + V_AHEAD < 8:
                v_read(f + V_AHEAD)
            for text, lds_name in per_slot[n]:
                if lds_name:
                    q.issue(text, lds_name)
                else:
                    lines.append(text)
    lines.append("s_waitcnt lgkmcnt(0)")
    return "\\n".join(lines) + "\\n" + NOP_AFTER


def main():
    qk = qk_asm()
    pvs = pvs_asm()
    text = f"""// Generated by gen_mfma_asm.py -- do not edit by hand.
// Inline-asm blocks of attn_mfma.hip (see the generator's docstring).
#pragma once

#define TV_QK_ASM "{qk}"

#define TV_PVS_ASM "{pvs}"
"""
    with open(OUT, "w") as f:
        f.write(text)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
