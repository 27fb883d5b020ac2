#!/usr/bin/env python3
"""Generate attn_mfma_asm.h: the two inline-asm MFMA chains of attn_mfma.hip.

    python tree_verify_mla_tv_amd/csrc/gen_mfma_asm.py   # rewrites attn_mfma_asm.h

The chains are written out instruction by instruction so that every LDS read
is issued DEPTH matrix ops ahead of its use (the compiler, short of registers
next to 256 accumulators and 128 query registers, otherwise places each read
right before its consumer and waits for it).  Register choice stays with the
compiler through named operands; only the order and the waits are fixed here.

Score chain (per tile, per wave): 36 x v_mfma_f32_32x32x16_bf16 into %[s].
  k-step ks < 32 reads its K fragment at %[lat] + 32 ks, ks >= 32 at
  %[rope] + 256 (ks - 32); its Q fragment is %[qN] for ks < 32, and for
  ks >= 32 an LDS fragment at %[qr] + 4096 (ks - 32), read first into %[rN].
Value chain: 32 x MFMA, n = 2 db + h accumulates into %[o<db>] with the V^T
  fragment at %[a<h>] + 2048 db and the weights %[p<h>].

Hazards handled inside the blocks: LDS data waits (s_waitcnt lgkmcnt, counted
from the reads the block itself issued, in order), the VALU-written weights
before the first value MFMA, and the matrix-core results before any VALU or
memory instruction outside the block reads them (s_nop padding).
"""
import os

DEPTH = 4   # reads in flight ahead of the matrix op that consumes them
SLOTS = 6   # rotating fragment registers (a slot is rewritten 2 ops after its last use)
NOP_AFTER = "s_nop 7\\n s_nop 7\\n s_nop 7\\n"   # >= 19 wait states after the last MFMA
NOP_BEFORE = "s_nop 4\\n"   # VALU-written weights -> first value MFMA
CONSERVATIVE_PVT = False
TBUFS = 8  # transpose staging registers: one set per unit, never reused within a block

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "attn_mfma_asm.h")


def qk_asm() -> str:
    lines = []
    # Q rope fragments first (oldest in the LDS queue).
    for r in range(4):
        lines.append(f"ds_read_b128 %[r{r}], %[qr] offset:{4096 * r}")

    def k_read(ks):
        slot = ks % SLOTS
        if ks < 32:
            return f"ds_read_b128 %[k{slot}], %[lat] offset:{32 * ks}"
        return f"ds_read_b128 %[k{slot}], %[rope] offset:{256 * (ks - 32)}"

    for ks in range(DEPTH):
        lines.append(k_read(ks))
    for ks in range(36):
        newest = min(ks + DEPTH - 1, 35)
        lines.append(f"s_waitcnt lgkmcnt({newest - ks})")
        q = f"%[q{ks}]" if ks < 32 else f"%[r{ks - 32}]"
        src_c = "0" if ks == 0 else "%[s]"
        lines.append(f"v_mfma_f32_32x32x16_bf16 %[s], %[k{ks % SLOTS}], {q}, {src_c}")
        if ks + DEPTH < 36:
            lines.append(k_read(ks + DEPTH))
    return "\\n".join(lines) + "\\n" + NOP_AFTER


def pv_asm() -> str:
    lines = [NOP_BEFORE.rstrip("\\n")]

    def v_read(n):
        return f"ds_read_b128 %[v{n % SLOTS}], %[a{n & 1}] offset:{2048 * (n >> 1)}"

    for n in range(DEPTH):
        lines.append(v_read(n))
    for n in range(32):
        newest = min(n + DEPTH - 1, 31)
        lines.append(f"s_waitcnt lgkmcnt({newest - n})")
        db = n >> 1
        lines.append(f"v_mfma_f32_32x32x16_bf16 %[o{db}], %[v{n % SLOTS}], %[p{n & 1}], %[o{db}]")
        if n + DEPTH < 32:
            lines.append(v_read(n + DEPTH))
    return "\\n".join(lines) + "\\n" + NOP_AFTER


def pv_transpose_asm() -> str:
    """Value chain with one wave's quarter of the next tile's transpose woven in.

    Transpose unit u (0..7) reads two ds_read_b64_tr_b16 halves at
    %[tb] + 16640 (u & 1) + 64 (u >> 1) (+ 8320 for the second) into %[t<u%2>lo/hi]
    at value step 4u, and writes them (two 8-byte stores) to %[wb<u&1>] +
    2048 (u >> 1) at step 4u + 2.  Wait counts come from simulating the in-order
    LDS queue.
    """
    lines = [NOP_BEFORE.rstrip("\\n")]
    issued = []  # names of LDS ops in issue order

    def issue(text, name):
        lines.append(text)
        issued.append(name)

    def wait_for(name):
        if CONSERVATIVE_PVT:
            lines.append("s_waitcnt lgkmcnt(0)")
            return
        idx = issued.index(name)
        lines.append(f"s_waitcnt lgkmcnt({len(issued) - idx - 1})")

    def v_read(n):
        issue(f"ds_read_b128 %[v{n % SLOTS}], %[a{n & 1}] offset:{2048 * (n >> 1)}", f"v{n}")

    for n in range(DEPTH):
        v_read(n)
    for n in range(32):
        wait_for(f"v{n}")
        db = n >> 1
        lines.append(f"v_mfma_f32_32x32x16_bf16 %[o{db}], %[v{n % SLOTS}], %[p{n & 1}], %[o{db}]")
        if n + DEPTH < 32:
            v_read(n + DEPTH)
        u, phase = divmod(n, 4)
        if phase == 0:
            off = 16640 * (u & 1) + 64 * (u >> 1)
            b = u % TBUFS
            issue(f"ds_read_b64_tr_b16 %[t{b}lo], %[tb] offset:{off}", f"tlo{u}")
            issue(f"ds_read_b64_tr_b16 %[t{b}hi], %[tb] offset:{off + 8320}", f"thi{u}")
        elif phase == 2:
            b = u % TBUFS
            wait_for(f"thi{u}")
            woff = 2048 * (u >> 1)
            issue(f"ds_write_b64 %[wb{u & 1}], %[t{b}lo] offset:{woff}", f"wlo{u}")
            issue(f"ds_write_b64 %[wb{u & 1}], %[t{b}hi] offset:{woff + 8}", f"whi{u}")
    lines.append("s_waitcnt lgkmcnt(0)")
    return "\\n".join(lines) + "\\n" + NOP_AFTER


def main():
    qk = qk_asm()
    pv = pv_asm()
    pvt = pv_transpose_asm()
    text = f"""// Generated by gen_mfma_asm.py -- do not edit by hand.
// Inline-asm MFMA chains of attn_mfma.hip (see the generator's docstring).
#pragma once

#define TV_QK_ASM "{qk}"

#define TV_PV_ASM "{pv}"

#define TV_PV_TRANSPOSE_ASM "{pvt}"
"""
    with open(OUT, "w") as f:
        f.write(text)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
