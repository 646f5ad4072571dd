"""Writes gemm_sq4_loop.inc: the instruction stream of the 256x256 GEMM kind
with four waves of 128x128 (KIND_SQ4_HO), ordered by hand.

    python gen_sq4_loop.py            # rewrites gemm_sq4_loop.inc next to this file

The k-loop of one work item is a single inline-asm statement, so that where
every wait, LDS fragment read, direct-to-LDS load and barrier sits relative to
the 64 MFMAs of a k32 step is fixed here rather than by the compiler's
scheduler.  The MFMA is the 16x16x32 one: for the same flops it moves half
the accumulator bytes of the 32x32x16 one, and under the chip's power limit
it holds a higher clock.  Registers (per wave, one wave per SIMD):

* a[0:255]: the 128x128 fp32 accumulators; block (i, j) (16x16, i rows,
  j columns, 0..7 each) is a[4*(8i+j) : 4*(8i+j)+3].
* v[128:191] / v[192:255]: two fragment buffers F0 / F1, each 8 A fragments
  (4 VGPRs each: 16 rows x 32 k, bf16/fp16) then 8 B fragments (32 k x 16
  columns).
* s[88:91] / s[92:95]: private copies of the A / B buffer descriptors, whose
  base advances by one k-slice per issued slice (64-bit SALU add).

Ring: two LDS slots of 64 KB (A tile [256][64] K-contiguous, then B tile
[64][256] N-contiguous, both swizzled as the loaders write them).  Slice j is
in slot j%2.  Per slice, k32 step 0 waits for its fragments, then issues 64
MFMAs with step 1's 24 fragment reads spread between them.  Step 1 waits for
its fragments (every read of slot j%2 is then done), issues a few MFMAs,
waits until this wave's loads of slice j+1 have landed and meets the other
waves at the barrier; after it, slice j+1 is in LDS for every wave and slot
j%2 is free, so the rest of step 1's MFMAs are interleaved with the reads of
slice j+1's first step and the first loads of slice j+2 into slot j%2; the
rest of slice j+2's loads go between step 0's MFMAs of slice j+1.  The last
slice has no barrier; the one before it issues no loads.

Operands the statement expects (names as in gemm_sq4.hpp):
  n (+s)                slices of the work item, >= 1
  a0..a3, b0..b3 (s)    descriptors based at slice 0 of the work item
  incb (s)              bytes of B per slice (64 k-rows)
  ldsw (s)              LDS byte address of slot 0 plus 1024 * wave
  m0 (+{m0})            M0, rewritten by the loads
  va0..va7, vb0..vb7 (v) per-lane offsets of the wave's 8 A and 8 B loads
  fa_S_K_P (v)          LDS address of A fragments of slot S, k32 step K,
                        16-row block i with i % 4 == P (block i+4 at +8192)
  fb_S_J (v)            LDS address of B fragment J of slot S at step 0
                        (step K at +16384*K, the second half at +2048)

The _BK variant of the loop takes B K-contiguous instead (the usual layout of
a linear layer's weight, C = X W^T): its LDS tile is [256 columns][64 k]
like A's, each B fragment one ds_read_b128 like an A fragment (16 reads per
step instead of 24), and it expects fbk_S_K_P in place of fb_S_J (B blocks j
and j+4 at +8192, as for A) and incb = 128.

The _AM variants take A M-contiguous (C = X^T Y, a layer's weight gradient):
its LDS tile is [64 k][256 rows] like an N-contiguous B's, each A fragment two
ds_read_b64_tr_b16 like a B fragment, read at fat_S_I (step K at +16384*K,
the second half at +2048), and A's descriptor moves by inca bytes per slice.
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "gemm_sq4_loop.inc")

STEPS = 2           # k32 steps per 64-deep slice
MFMAS = 64          # MFMAs per step (8 x 8 blocks of 16x16)
READS = 24          # fragment reads per step: 8 A (ds_read_b128), 16 B (two ds_read_b64_tr_b16 each)
READS_BK = 16       # the same with B K-contiguous: 8 A and 8 B, all ds_read_b128
READS_AM = 8        # more with A M-contiguous (two ds_read_b64_tr_b16 per A fragment)
B_STEP = 16384      # LDS bytes between a B fragment's steps (32 k-rows of 512 bytes)
FBASE = 128         # first fragment VGPR
FBUF = 64           # VGPRs per fragment buffer
READ_SPAN = 40      # MFMAs of step 0 over which step 1's reads are spread
BAR_AFTER = 8       # MFMAs of step 1 issued before the load wait and barrier
L3 = 10             # loads of slice j+2 issued in step 1 of slice j; the rest go to step 0 of slice j+1
CARRY_STEPS = 1     # how many of the steps before the last of slice j+1 share the rest
CARRY_SPAN = 52     # MFMAs over which a step's reads and carried loads are spread
B_FIRST = 0         # load order within a slice: 0 A0, B0, A1, B1, ...; 1 B0, A0, B1, A1, ...
CARRY_BLOCKS = 0    # 0: step k takes every CARRY_STEPS-th carried load; 1: contiguous runs of them
PREFETCH = 1        # L2 prefetch of the slice after the next, right after the descriptors advance: bit 0 B, bit 1 A
SLOT = 65536
B_OFF = 32768


def fa(buf, i):
    return FBASE + FBUF * buf + 4 * i


def fb(buf, j):
    return FBASE + FBUF * buf + 32 + 4 * j


def acc(i, j):
    return 4 * (8 * i + j)


def mfmas(op, buf):
    out = []
    for i in range(8):
        for j in range(8):
            a = acc(i, j)
            out.append(f"{op} a[{a}:{a + 3}], v[{fa(buf, i)}:{fa(buf, i) + 3}], "
                       f"v[{fb(buf, j)}:{fb(buf, j) + 3}], a[{a}:{a + 3}]")
    return out


def reads(slot, kk, buf, bk=False, am=False):
    """The 24 fragment reads of k32 step kk from `slot` into buffer `buf` (16
    with B K-contiguous; 8 more with A M-contiguous)."""
    out = []
    for i in range(8):
        if am:
            lo, hi = kk * B_STEP, kk * B_STEP + 2048
            o = f" offset:{lo}" if lo else ""
            out.append([f"ds_read_b64_tr_b16 v[{fa(buf, i)}:{fa(buf, i) + 1}], %[fat_{slot}_{i}]{o}"])
            out.append([f"ds_read_b64_tr_b16 v[{fa(buf, i) + 2}:{fa(buf, i) + 3}], %[fat_{slot}_{i}] offset:{hi}"])
            continue
        off = (i >> 2) * 8192
        o = f" offset:{off}" if off else ""
        out.append([f"ds_read_b128 v[{fa(buf, i)}:{fa(buf, i) + 3}], %[fa_{slot}_{kk}_{i & 3}]{o}"])
    if bk:
        for j in range(8):
            off = (j >> 2) * 8192
            o = f" offset:{off}" if off else ""
            out.append([f"ds_read_b128 v[{fb(buf, j)}:{fb(buf, j) + 3}], %[fbk_{slot}_{kk}_{j & 3}]{o}"])
        return out
    for j in range(8):
        lo, hi = kk * B_STEP, kk * B_STEP + 2048
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
# the same with A M-contiguous: A moves 64 k-rows (inca bytes) per slice
ADVANCE_AM = [x.replace("s88, s88, 128", "s88, s88, %[inca]").replace("s90, s90, 128", "s90, s90, %[inca]")
              for x in ADVANCE]


def prefetch():
    """One dword per 128-byte line of this wave's share of the slice the
    descriptors now point at (the one after the slice being loaded), into a
    dummy LDS area, so that the real loads of that slice find it in L2.  The
    per-lane offsets (vpa, vpb) are range-checked against num_records, so a
    slice past the operand's end reads nothing."""
    out = []
    if PREFETCH & 1:
        out.append(["s_add_u32 m0, %[ldsp], 0", "s_nop 0", "buffer_load_dword %[vpb], s[92:95], 0 offen lds"])
    if PREFETCH & 2:
        out.append(["s_add_u32 m0, %[ldsp], 0", "s_nop 0", "buffer_load_dword %[vpa], s[88:91], 0 offen lds"])
    return out


def npf():
    return bin(PREFETCH & 3).count("1")


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


def carried(slot, kk, am=False):
    """Loads of the next slice (into the other slot) issued in step kk (one of
    the STEPS - 1 steps before the last): the 16 - L3 that the last step of
    the previous slice left, spread over the first CARRY_STEPS steps; the
    descriptors advance once, right after the last of them (every path
    through a slice advances them exactly once)."""
    rest = loads(1 - slot)[L3:]
    early = STEPS - 1
    assert rest and 1 <= CARRY_STEPS <= early
    if CARRY_BLOCKS:
        cut = [len(rest) * k // CARRY_STEPS for k in range(CARRY_STEPS + 1)]
        per = [rest[cut[k]:cut[k + 1]] for k in range(CARRY_STEPS)] + [[]] * (early - CARRY_STEPS)
    else:
        per = [rest[k::CARRY_STEPS] for k in range(CARRY_STEPS)] + [[]] * (early - CARRY_STEPS)
    last = max(k for k in range(early) if per[k])
    return per[kk] + ([ADVANCE_AM if am else ADVANCE] + prefetch() if kk == last else [])


def step(op, slot, kk, buf, carry, bk=False, am=False):
    """Step kk (before the last) of a slice in `slot`: MFMAs on `buf`, reads of
    step kk+1, and (carry) this step's share of the next slice's remaining
    loads."""
    rd = reads(slot, kk + 1, 1 - buf, bk, am)
    ops = rd
    if carry:
        ld = carried(slot, kk, am)
        ops = []
        for k in range(max(len(rd), len(ld))):
            if k < len(rd):
                ops.append(rd[k])
            if k < len(ld):
                ops.append(ld[k])
    return ["s_waitcnt lgkmcnt(0)"] + interleave(mfmas(op, buf), ops, READ_SPAN if not carry else CARRY_SPAN)


def step_last(op, slot, kind, bk=False, am=False):
    """The last step of a slice (fragments in buffer (STEPS - 1) % 2).  kind:
    "last" (no next slice), "noload" (next slice, nothing more to load),
    "load" (next slice, and load slice j+2)."""
    mf = mfmas(op, (STEPS - 1) % 2)
    if kind == "last":
        return ["s_waitcnt lgkmcnt(0)"] + mf
    out = ["s_waitcnt lgkmcnt(0)"] + mf[:BAR_AFTER] + [f"s_waitcnt vmcnt({npf()})", "s_barrier"]
    rd = reads(1 - slot, 0, 0, bk, am)
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
            ops.append(ADVANCE_AM if am else ADVANCE)
            ops += prefetch()
    else:
        ops = rd
    out += interleave(mf[BAR_AFTER:], ops, len(mf) - BAR_AFTER - 2)
    return out


def loop(op, bk=False, am=False):
    L = []
    # private descriptor copies, advanced from slice 0 (the operands) to
    # slice 2, the first slice the loop loads
    L += ["s_mov_b32 s88, %[a0]", "s_mov_b32 s89, %[a1]", "s_mov_b32 s90, %[a2]", "s_mov_b32 s91, %[a3]",
          "s_mov_b32 s92, %[b0]", "s_mov_b32 s93, %[b1]", "s_mov_b32 s94, %[b2]", "s_mov_b32 s95, %[b3]"]
    # with every load of a slice in the last step the loop's first load is of
    # slice 2; otherwise the rest of slice 1 (whose first L3 loads the
    # prologue issued) comes first, in the first slice's earlier steps
    adv = ADVANCE_AM if am else ADVANCE
    L += adv + adv if L3 == 16 else adv
    L += [f"v_accvgpr_write_b32 a{r}, 0" for r in range(256)]
    L += ["s_nop 4"]
    L += [x for r in reads(0, 0, 0, bk, am) for x in r]
    for slot in (0, 1):
        L += [f"L_top{slot}_%=:"]
        if L3 < 16:
            L += ["s_cmp_lt_u32 %[n], 2", f"s_cbranch_scc1 L_noc{slot}_%="]
            for kk in range(STEPS - 1):
                L += step(op, slot, kk, kk % 2, True, bk, am)
            L += [f"s_branch L_st3{slot}_%=", f"L_noc{slot}_%=:"]
        for kk in range(STEPS - 1):
            L += step(op, slot, kk, kk % 2, False, bk, am)
        L += [f"L_st3{slot}_%=:"]
        L += ["s_cmp_eq_u32 %[n], 1", f"s_cbranch_scc1 L_last{slot}_%=",
              "s_cmp_eq_u32 %[n], 2", f"s_cbranch_scc1 L_nold{slot}_%="]
        L += step_last(op, slot, "load", bk, am)
        L += ["s_sub_u32 %[n], %[n], 1", f"s_branch L_top{1 - slot}_%="]
        L += [f"L_nold{slot}_%=:"]
        L += step_last(op, slot, "noload", bk, am)
        L += ["s_sub_u32 %[n], %[n], 1", f"s_branch L_top{1 - slot}_%="]
        L += [f"L_last{slot}_%=:"]
        L += step_last(op, slot, "last", bk, am)
        L += ["s_branch L_done_%="]
    # the accumulators are read with v_accvgpr_read after this statement:
    # more wait states after the last MFMA that writes them than any MFMA
    # needs (24 against at most 18)
    L += ["L_done_%=:", "s_nop 7", "s_nop 7", "s_nop 7"]
    return L


def cstring(lines):
    return " \\\n".join(f'  "{ln}\\n\\t"' for ln in lines)


def read_acc(n):
    """Accumulator block n = 8i + j into the statement's outputs %0..%3."""
    return cstring([f"v_accvgpr_read_b32 %{r}, a{4 * n + r}" for r in range(4)])


def clobbers():
    regs = [f'"v{r}"' for r in range(FBASE, 256)] + [f'"a{r}"' for r in range(256)] + \
           [f'"s{r}"' for r in range(88, 96)] + ['"scc"', '"memory"']
    return ", ".join(regs)


def main():
    parts = ["// Generated by gen_sq4_loop.py; do not edit.  The k-loop of the 256x256 GEMM",
             "// kind with four 128x128 waves as one hand-ordered instruction stream",
             "// (see gen_sq4_loop.py for the register plan and the order).",
             "#pragma once", ""]
    parts.append("#define LL_SQ4_LOOP_BF16 \\\n" + cstring(loop("v_mfma_f32_16x16x32_bf16")) + "\n")
    parts.append("#define LL_SQ4_LOOP_F16 \\\n" + cstring(loop("v_mfma_f32_16x16x32_f16")) + "\n")
    parts.append("// the same with B K-contiguous\n#define LL_SQ4_LOOP_BF16_BK \\\n" +
                 cstring(loop("v_mfma_f32_16x16x32_bf16", True)) + "\n")
    parts.append("#define LL_SQ4_LOOP_F16_BK \\\n" + cstring(loop("v_mfma_f32_16x16x32_f16", True)) + "\n")
    for bk in (False, True):
        suf = "_AM_BK" if bk else "_AM"
        parts.append(f"// A M-contiguous{', B K-contiguous' if bk else ''}\n#define LL_SQ4_LOOP_BF16{suf} \\\n" +
                     cstring(loop("v_mfma_f32_16x16x32_bf16", bk, True)) + "\n")
        parts.append(f"#define LL_SQ4_LOOP_F16{suf} \\\n" + cstring(loop("v_mfma_f32_16x16x32_f16", bk, True)) + "\n")
    for n in range(64):
        parts.append(f"#define LL_SQ4_READ_ACC_{n} \\\n" + read_acc(n) + "\n")
    parts.append("// X(n) for every accumulator block n = 8 * row block + column block\n#define LL_SQ4_BLOCKS(X) " +
                 " ".join(f"X({n})" for n in range(64)) + "\n")
    parts.append(f"// L2 prefetch of the slice after the next: bit 0 B, bit 1 A\n#define LL_SQ4_PREFETCH {PREFETCH}\n")
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
