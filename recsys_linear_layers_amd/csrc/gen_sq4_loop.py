"""Writes gemm_sq4_loop.inc: the instruction stream of the 256x256 GEMM kind
with four waves of 128x128 (KIND_SQ4_HO), ordered by hand.

    python gen_sq4_loop.py            # rewrites gemm_sq4_loop.inc next to this file

The k-loop of one work item is a single inline-asm statement, so that where
every wait, LDS fragment read, direct-to-LDS load and barrier sits relative to
the 16 MFMAs of a k16 step is fixed here rather than by the compiler's
scheduler.  Registers (per wave, one wave per SIMD):

* a[0:255]: the 128x128 fp32 accumulators; block (i, j) (32x32, i rows,
  j columns) is a[16*(4i+j) : 16*(4i+j)+15].
* v[192:223] / v[224:255]: two fragment buffers F0 / F1, each 4 A fragments
  (4 VGPRs each: 32 rows x 16 k, bf16/fp16) then 4 B fragments.
* s[88:91] / s[92:95]: private copies of the A / B buffer descriptors, whose
  base advances by one k-slice per issued slice (64-bit SALU add).

Ring: two LDS slots of 64 KB (A tile [256][64] K-contiguous, then B tile
[64][256] N-contiguous, both swizzled as the loaders write them).  Slice j is
in slot j%2.  Per slice, k16 steps 0..2 each wait for their fragments, then
issue 16 MFMAs with the next step's 12 fragment reads spread between them.
Step 3 waits for its fragments (every read of slot j%2 is then done), issues
a few MFMAs, waits until this wave's loads of slice j+1 have landed and meets
the other waves at the barrier; after it, slice j+1 is in LDS for every wave
and slot j%2 is free, so the rest of step 3's MFMAs are interleaved with the
reads of slice j+1's first step and the 16 loads of slice j+2 into slot j%2.
The last slice has no barrier; the one before it issues no loads.

Operands the statement expects (names as in gemm_sq4.hpp):
  n (+s)                slices of the work item, >= 1
  a0..a3, b0..b3 (s)    descriptors based at slice 0 of the work item
  incb (s)              bytes of B per slice (64 k-rows)
  ldsw (s)              LDS byte address of slot 0 plus 1024 * wave
  m0 (+{m0})            M0, rewritten by the loads
  va0..va7, vb0..vb7 (v) per-lane offsets of the wave's 8 A and 8 B loads
  fa_S_K_P (v)          LDS address of A fragments of slot S, k16 step K,
                        32-row block parity P (block i+2 at +8192)
  fb_S_J (v)            LDS address of B fragment J of slot S at step 0
                        (step K at +8192*K, the second half at +2048)
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "gemm_sq4_loop.inc")

FBASE = 192         # first fragment VGPR
READ_SPAN = 10      # MFMAs of steps 0..2 over which the next step's 12 reads are spread
BAR_AFTER = 0       # MFMAs of step 3 issued before the load wait and barrier
L3 = 6              # loads of slice j+2 issued in step 3 of slice j; the rest go to steps 0..2 of slice j+1
CARRY_STEPS = 2     # how many of steps 0..2 of slice j+1 share the rest
CARRY_SPAN = 14     # MFMAs over which a step's reads and carried loads are spread
B_FIRST = 0         # load order within a slice: 0 A0, B0, A1, B1, ...; 1 B0, A0, B1, A1, ...
CARRY_BLOCKS = 0    # 0: step k takes every CARRY_STEPS-th carried load; 1: contiguous runs of them
SLOT = 65536
B_OFF = 32768


def fa(buf, i):
    return FBASE + 32 * buf + 4 * i


def fb(buf, j):
    return FBASE + 32 * buf + 16 + 4 * j


def acc(i, j):
    return 16 * (4 * i + j)


def mfmas(op, buf):
    out = []
    for i in range(4):
        for j in range(4):
            a = acc(i, j)
            out.append(f"{op} a[{a}:{a + 15}], v[{fa(buf, i)}:{fa(buf, i) + 3}], "
                       f"v[{fb(buf, j)}:{fb(buf, j) + 3}], a[{a}:{a + 15}]")
    return out


def reads(slot, kk, buf):
    """The 12 fragment reads of k16 step kk from `slot` into buffer `buf`."""
    out = []
    for i in range(4):
        off = (i >> 1) * 8192
        o = f" offset:{off}" if off else ""
        out.append([f"ds_read_b128 v[{fa(buf, i)}:{fa(buf, i) + 3}], %[fa_{slot}_{kk}_{i & 1}]{o}"])
    for j in range(4):
        lo, hi = kk * 8192, kk * 8192 + 2048
        o = f" offset:{lo}" if lo else ""
        out.append([f"ds_read_b64_tr_b16 v[{fb(buf, j)}:{fb(buf, j) + 1}], %[fb_{slot}_{j}]{o}"])
        out.append([f"ds_read_b64_tr_b16 v[{fb(buf, j) + 2}:{fb(buf, j) + 3}], %[fb_{slot}_{j}] offset:{hi}"])
    return out


def loads(slot):
    """The wave's 16 direct-to-LDS loads of one slice into `slot` (M0 set per
    load), A and B alternating, the first of each pair per B_FIRST."""
    out = []
    for i in range(8):
        a = [f"s_add_u32 m0, %[ldsw], {slot * SLOT + i * 4096}", "s_nop 0",
             f"buffer_load_dwordx4 %[va{i}], s[88:91], 0 offen lds"]
        b = [f"s_add_u32 m0, %[ldsw], {slot * SLOT + B_OFF + i * 4096}", "s_nop 0",
             f"buffer_load_dwordx4 %[vb{i}], s[92:95], 0 offen lds"]
        out += [b, a] if B_FIRST else [a, b]
    return out


# Move both descriptors on by one slice: the 64-bit base up, num_records (the
# operand's bytes from the base; the plan keeps every operand this kind reads
# below 2 GB, so it is exact) down by the same amount, floored at 0 - a base
# moved past the operand then reads zeros instead of memory beyond it.
ADVANCE = ["s_add_u32 s88, s88, 128", "s_addc_u32 s89, s89, 0",
           "s_sub_u32 s90, s90, 128", "s_cselect_b32 s90, 0, s90",
           "s_add_u32 s92, s92, %[incb]", "s_addc_u32 s93, s93, 0",
           "s_sub_u32 s94, s94, %[incb]", "s_cselect_b32 s94, 0, s94"]


def interleave(mf, ops, span):
    """MFMAs in order, with op k placed after MFMA floor(k * span / len(ops))."""
    after = {}
    for k, op in enumerate(ops):
        after.setdefault(min(len(mf) - 1, k * span // max(1, len(ops))), []).extend(op)
    out = []
    for m, line in enumerate(mf):
        out.append(line)
        out.extend(after.get(m, []))
    return out


def carried(slot, kk):
    """Loads of the next slice (into the other slot) issued in step kk (0..2):
    the 16 - L3 that step 3 of the previous slice left, spread over the first
    CARRY_STEPS steps; the descriptors advance once, right after the last of
    them (every path through a slice advances them exactly once)."""
    rest = loads(1 - slot)[L3:]
    assert rest and 1 <= CARRY_STEPS <= 3
    if CARRY_BLOCKS:
        cut = [len(rest) * k // CARRY_STEPS for k in range(CARRY_STEPS + 1)]
        per = [rest[cut[k]:cut[k + 1]] for k in range(CARRY_STEPS)] + [[]] * (3 - CARRY_STEPS)
    else:
        per = [rest[k::CARRY_STEPS] for k in range(CARRY_STEPS)] + [[]] * (3 - CARRY_STEPS)
    last = max(k for k in range(3) if per[k])
    return per[kk] + ([ADVANCE] if kk == last else [])


def step(op, slot, kk, buf, carry):
    """k16 step kk (0..2) of a slice in `slot`: MFMAs on `buf`, reads of step kk+1,
    and (carry) this step's share of the next slice's remaining loads."""
    rd = reads(slot, kk + 1, 1 - buf)
    ops = rd
    if carry:
        ld = carried(slot, kk)
        ops = []
        for k in range(max(len(rd), len(ld))):
            if k < len(rd):
                ops.append(rd[k])
            if k < len(ld):
                ops.append(ld[k])
    return ["s_waitcnt lgkmcnt(0)"] + interleave(mfmas(op, buf), ops, READ_SPAN if not carry else CARRY_SPAN)


def step3(op, slot, kind):
    """Step 3 (fragments in F1).  kind: "last" (no next slice), "noload" (next
    slice, nothing more to load), "load" (next slice, and load slice j+2)."""
    mf = mfmas(op, 1)
    if kind == "last":
        return ["s_waitcnt lgkmcnt(0)"] + mf
    out = ["s_waitcnt lgkmcnt(0)"] + mf[:BAR_AFTER] + ["s_waitcnt vmcnt(0)", "s_barrier"]
    rd = reads(1 - slot, 0, 0)
    ops = []
    if kind == "load":
        ld = loads(slot)[:L3]
        # alternate fragment reads (needed first) with loads (longest latency)
        for k in range(max(len(rd), len(ld))):
            if k < len(rd):
                ops.append(rd[k])
            if k < len(ld):
                ops.append(ld[k])
        if L3 == 16:
            ops.append(ADVANCE)
    else:
        ops = rd
    out += interleave(mf[BAR_AFTER:], ops, len(mf) - BAR_AFTER - 2)
    return out


def loop(op):
    L = []
    # private descriptor copies, advanced from slice 0 (the operands) to
    # slice 2, the first slice the loop loads
    L += ["s_mov_b32 s88, %[a0]", "s_mov_b32 s89, %[a1]", "s_mov_b32 s90, %[a2]", "s_mov_b32 s91, %[a3]",
          "s_mov_b32 s92, %[b0]", "s_mov_b32 s93, %[b1]", "s_mov_b32 s94, %[b2]", "s_mov_b32 s95, %[b3]"]
    # with every load of a slice in step 3 the loop's first load is of slice
    # 2; otherwise the rest of slice 1 (whose first L3 loads the prologue
    # issued) comes first, in the first slice's steps 0..2
    L += ADVANCE + ADVANCE if L3 == 16 else ADVANCE
    L += [f"v_accvgpr_write_b32 a{r}, 0" for r in range(256)]
    L += ["s_nop 4"]
    L += [x for r in reads(0, 0, 0) for x in r]
    for slot in (0, 1):
        L += [f"L_top{slot}_%=:"]
        if L3 < 16:
            L += ["s_cmp_lt_u32 %[n], 2", f"s_cbranch_scc1 L_noc{slot}_%="]
            for kk in range(3):
                L += step(op, slot, kk, kk % 2, True)
            L += [f"s_branch L_st3{slot}_%=", f"L_noc{slot}_%=:"]
        for kk in range(3):
            L += step(op, slot, kk, kk % 2, False)
        L += [f"L_st3{slot}_%=:"]
        L += ["s_cmp_eq_u32 %[n], 1", f"s_cbranch_scc1 L_last{slot}_%=",
              "s_cmp_eq_u32 %[n], 2", f"s_cbranch_scc1 L_nold{slot}_%="]
        L += step3(op, slot, "load")
        L += ["s_sub_u32 %[n], %[n], 1", f"s_branch L_top{1 - slot}_%="]
        L += [f"L_nold{slot}_%=:"]
        L += step3(op, slot, "noload")
        L += ["s_sub_u32 %[n], %[n], 1", f"s_branch L_top{1 - slot}_%="]
        L += [f"L_last{slot}_%=:"]
        L += step3(op, slot, "last")
        L += ["s_branch L_done_%="]
    # the accumulators are read with v_accvgpr_read after this statement:
    # at least 18 wait states after the last 32x32 MFMA that writes them
    L += ["L_done_%=:", "s_nop 7", "s_nop 7", "s_nop 7"]
    return L


def cstring(lines):
    return " \\\n".join(f'  "{ln}\\n\\t"' for ln in lines)


def read_acc(i, j):
    a = acc(i, j)
    return cstring([f"v_accvgpr_read_b32 %{r}, a{a + r}" for r in range(16)])


def clobbers():
    regs = [f'"v{r}"' for r in range(FBASE, 256)] + [f'"a{r}"' for r in range(256)] + \
           [f'"s{r}"' for r in range(88, 96)] + ['"scc"', '"memory"']
    return ", ".join(regs)


def main():
    parts = ["// Generated by gen_sq4_loop.py; do not edit.  The k-loop of the 256x256 GEMM",
             "// kind with four 128x128 waves as one hand-ordered instruction stream",
             "// (see gen_sq4_loop.py for the register plan and the order).",
             "#pragma once", ""]
    parts.append("#define LL_SQ4_LOOP_BF16 \\\n" + cstring(loop("v_mfma_f32_32x32x16_bf16")) + "\n")
    parts.append("#define LL_SQ4_LOOP_F16 \\\n" + cstring(loop("v_mfma_f32_32x32x16_f16")) + "\n")
    for i in range(4):
        for j in range(4):
            parts.append(f"#define LL_SQ4_READ_ACC_{i}_{j} \\\n" + read_acc(i, j) + "\n")
    parts.append(f"// loads of a slice issued after the barrier of the slice two before; the\n"
                 f"// prologue issues this many of slice 1\n#define LL_SQ4_L3 {L3}\n"
                 f"// the loads of a slice alternate A and B, B first if 1\n#define LL_SQ4_B_FIRST {B_FIRST}\n")
    parts.append("#define LL_SQ4_CLOBBERS " + clobbers() + "\n")
    text = "\n".join(parts)
    with open(OUT, "w") as f:
        f.write(text)
    return text


if __name__ == "__main__":
    main()
    print(OUT)
