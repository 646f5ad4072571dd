"""CPU checks of the hand-ordered GEMM k-loop (gemm_sq4_loop.inc).

The committed include is what gen_sq4_loop.py writes, and an emulation of the
generated instruction stream (its scalar control flow, descriptor moves, M0
values, waits and barriers; one wave stands for all four, which run the same
stream) shows for every slice count and every load split that:

* each slice's 16 loads (8 of A, 8 of B) are issued exactly once, counting
  the ones the prologue issues, never for a slice past the last, with both
  descriptors at that slice and M0 at that load's place in the slice's slot;
* a load into a slot is issued only after every fragment read of the slice
  that slot held has completed and a barrier has followed;
* a fragment read finds every load of its slice completed and published by a
  barrier, reads the slot its slice went to, and the reads come in the order
  slice 0 step 0, 1, slice 1 step 0, ... (two k32 steps per slice);
* the descriptors move by exactly one slice per slice, so num_records stays
  the operand's bytes from the base;
* there is one barrier per slice but the last, 128 MFMAs per slice (two k32
  steps of 64), and no load is still outstanding at the end.
"""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "recsys_linear_layers_amd", "csrc", "gen_sq4_loop.py")
INC = os.path.join(ROOT, "recsys_linear_layers_amd", "csrc", "gemm_sq4_loop.inc")
OP = "v_mfma_f32_16x16x32_bf16"


def _gen(**params):
    spec = importlib.util.spec_from_file_location("gen_sq4_loop_t", GEN)
    g = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(g)
    for k, v in params.items():
        setattr(g, k, v)
    return g


def test_committed_include_is_the_generators_output(tmp_path):
    g = _gen(OUT=str(tmp_path / "out.inc"))
    assert g.main() == open(INC).read()


PIECES = [("A", i) for i in range(8)] + [("B", i) for i in range(8)]


def emulate(g, n, inc_b=4096 * 64 * 2, ext_a=10 ** 9, ext_b=10 ** 9, bk=False, am=False, inc_a=128):
    lines = g.loop(OP, bk, am)
    nreads = (g.READS_BK if bk else g.READS) + (g.READS_AM if am else 0)
    labels = {ln[:-1]: k for k, ln in enumerate(lines) if ln.endswith(":")}
    issued = {}          # slice -> set of pieces
    pending, completed, visible = [], set(), set()   # pending: issue order, prefetches as ("PF", slice)
    prefetches = 0
    # prologue (C++): slice 0 whole and the first L3 loads of slice 1 (order
    # A0, B0, A1, B1, ...), then a wait for all of them and a barrier
    order = [("A" if (k % 2 == 0) != bool(g.B_FIRST) else "B", k // 2) for k in range(16)]
    issued[0] = set(PIECES)
    if n > 1:
        issued[1] = set(order[:g.L3])
    completed |= {(s, p) for s in issued for p in issued[s]}
    visible |= completed
    reads_issued = reads_done = released = 0
    barriers = mfmas = 0
    a_adv, b_adv, m0, scc, nreg = 0, 0, None, False, n
    nrec_a = nrec_b = None
    pc = 0
    while pc < len(lines):
        ln = lines[pc]
        pc += 1
        if ln.endswith(":"):
            continue
        m = re.match(r"s_mov_b32 s(\d+), %\[([ab])(\d)\]", ln)
        if m:
            if m.group(1) == "90":
                nrec_a = ext_a
            if m.group(1) == "94":
                nrec_b = ext_b
            continue
        if ln == ("s_add_u32 s88, s88, %[inca]" if am else "s_add_u32 s88, s88, 128"):
            a_adv += 1
        elif ln == "s_add_u32 s92, s92, %[incb]":
            b_adv += 1
        elif ln == ("s_sub_u32 s90, s90, %[inca]" if am else "s_sub_u32 s90, s90, 128"):
            nrec_a = max(0, nrec_a - inc_a)
        elif ln == "s_sub_u32 s94, s94, %[incb]":
            nrec_b = max(0, nrec_b - inc_b)
        elif ln.startswith(("s_addc_u32", "s_cselect_b32", "s_nop", "v_accvgpr_write")):
            pass
        elif ln.startswith("s_add_u32 m0, %[ldsw], "):
            m0 = int(ln.split(", ")[-1])
        elif ln == "s_add_u32 m0, %[ldsp], 0":
            m0 = "pf"
        elif ln.startswith("buffer_load_dword "):
            m = re.match(r"buffer_load_dword %\[vp([ab])\], s\[(\d+):\d+\], 0 offen lds", ln)
            assert m and m0 == "pf", ln
            which = m.group(1).upper()
            assert m.group(2) == ("88" if which == "A" else "92"), ln
            s = a_adv if which == "A" else b_adv
            # the descriptors point at the slice after the one whose loads were issued last
            assert all(s > t for t in issued), f"prefetch of slice {s} after its loads"
            pending.append(("PF", s))
            prefetches += 1
        elif ln.startswith("buffer_load_dwordx4"):
            m = re.match(r"buffer_load_dwordx4 %\[v([ab])(\d)\], s\[(\d+):\d+\], 0 offen lds", ln)
            assert m, ln
            which, i = m.group(1).upper(), int(m.group(2))
            assert m.group(3) == ("88" if which == "A" else "92"), ln
            s = a_adv if which == "A" else b_adv
            assert 0 <= s < n, f"load of slice {s} with n = {n}"
            assert (which, i) not in issued.setdefault(s, set()), f"slice {s} {which}{i} loaded twice"
            want_m0 = (s % 2) * g.SLOT + (g.B_OFF if which == "B" else 0) + i * 4096
            assert m0 == want_m0, (s, which, i, m0, want_m0)
            if s >= 2:
                assert released >= g.STEPS * (s - 1), f"slot of slice {s - 2} refilled before its reads were released"
            issued[s].add((which, i))
            pending.append((s, (which, i)))
        elif (m := re.match(r"s_waitcnt vmcnt\((\d+)\)", ln)):
            keep = int(m.group(1))
            done = pending[:len(pending) - keep] if keep else pending
            completed |= {x for x in done if x[0] != "PF"}
            pending = pending[len(done):]
        elif ln == "s_waitcnt lgkmcnt(0)":
            reads_done = reads_issued
        elif ln == "s_barrier":
            barriers += 1
            visible |= completed
            released = reads_done // nreads
        elif ln.startswith("ds_read"):
            grp = reads_issued // nreads
            s, kk = grp // g.STEPS, grp % g.STEPS
            m = re.search(r"%\[f(a|b|bk|at)_(\d)_(\d)(?:_(\d))?\](?: offset:(\d+))?", ln)
            assert m, ln
            assert ln.startswith("ds_read_b128") == (m.group(1) in ("a", "bk")), ln
            assert m.group(1) in (("at",) if am else ("a",)) + (("bk",) if bk else ("b",)), ln
            slot = int(m.group(2))
            off = int(m.group(5) or 0)
            if m.group(1) in ("a", "bk"):
                assert int(m.group(3)) == kk, (ln, kk)
            else:
                assert off // g.B_STEP == kk, (ln, kk)
            assert slot == s % 2, (ln, s)
            missing = [p for p in PIECES if (s, p) not in visible]
            assert not missing, f"read of slice {s} step {kk} before {missing} were published"
            reads_issued += 1
        elif ln.startswith(OP):
            mfmas += 1
        elif (m := re.match(r"s_cmp_(eq|lt)_u32 %\[n\], (\d+)", ln)):
            scc = nreg == int(m.group(2)) if m.group(1) == "eq" else nreg < int(m.group(2))
        elif (m := re.match(r"s_cbranch_scc1 (\S+)", ln)):
            if scc:
                pc = labels[m.group(1)]
        elif (m := re.match(r"s_branch (\S+)", ln)):
            pc = labels[m.group(1)]
        elif ln == "s_sub_u32 %[n], %[n], 1":
            nreg -= 1
        else:
            raise AssertionError(f"instruction the emulation does not know: {ln}")
        if ln.startswith("buffer_load_dwordx4"):
            assert nrec_a == max(0, ext_a - a_adv * inc_a) and nrec_b == max(0, ext_b - b_adv * inc_b)
    assert nrec_a == max(0, ext_a - a_adv * inc_a) and nrec_b == max(0, ext_b - b_adv * inc_b)
    for s in range(n):
        assert issued.get(s) == set(PIECES), f"slice {s}: {sorted(set(PIECES) - issued.get(s, set()))} never loaded"
    assert not [x for x in pending if x[0] != "PF"], "loads still outstanding at the end"
    # each descriptor advance inside the loop (not the one or two before it) is followed by the prefetches
    in_loop = a_adv - (2 if g.L3 == 16 else 1)
    assert prefetches == g.npf() * in_loop, (prefetches, in_loop)
    assert reads_issued == nreads * g.STEPS * n and mfmas == g.MFMAS * g.STEPS * n and barriers == n - 1
    # the descriptors end at most one slice past the last loaded one
    assert a_adv == b_adv and b_adv in (n, n + 1) or n <= 2


SPLITS = [dict(L3=16)] + [dict(L3=l3) for l3 in (14, 12, 10, 8, 6, 4, 2)] + \
         [dict(L3=l3, B_FIRST=1) for l3 in (8, 6, 4)] + \
         [dict(L3=6, READ_SPAN=r, CARRY_SPAN=c) for r, c in ((16, 24), (63, 63), (1, 1))] + \
         [dict(L3=l3, PREFETCH=pf) for l3 in (10, 16) for pf in (1, 2, 3)]


@pytest.mark.parametrize("params", SPLITS, ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()))
@pytest.mark.parametrize("n", range(1, 10))
def test_emulated_loop(params, n):
    emulate(_gen(**params), n)


@pytest.mark.parametrize("params", [dict(), dict(L3=16), dict(L3=4), dict(L3=10, PREFETCH=3)],
                         ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()) or "committed")
@pytest.mark.parametrize("n", range(1, 10))
def test_emulated_loop_b_k_contiguous(params, n):
    """The variant for a K-contiguous B (B fragments read like A's, 16 reads
    per step), with B moving 128 bytes per slice like A."""
    emulate(_gen(**params), n, inc_b=128, bk=True)


@pytest.mark.parametrize("params", [dict(), dict(L3=16), dict(L3=4), dict(L3=10, PREFETCH=3)],
                         ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()) or "committed")
@pytest.mark.parametrize("bk", [False, True])
@pytest.mark.parametrize("n", range(1, 10))
def test_emulated_loop_a_m_contiguous(params, bk, n):
    """The variants for an M-contiguous A (A fragments read like an
    N-contiguous B's, A moving 64 k-rows per slice), with B either way."""
    emulate(_gen(**params), n, inc_b=128 if bk else 4096 * 64 * 2, bk=bk, am=True, inc_a=3000 * 64 * 2)


def test_committed_parameters_emulate():
    g = _gen()
    for n in range(1, 12):
        emulate(g, n)
        emulate(g, n, inc_b=128, bk=True)
        emulate(g, n, am=True, inc_a=3000 * 64 * 2)
        emulate(g, n, inc_b=128, bk=True, am=True, inc_a=3000 * 64 * 2)


def test_emulation_catches_a_double_advance():
    """The emulation rejects a stream whose descriptors move twice in a slice."""
    g = _gen(L3=8)
    real = g.carried
    g.carried = lambda slot, kk, am=False: real(slot, kk, am) + ([g.ADVANCE] if kk == 0 else [])
    with pytest.raises(AssertionError):
        emulate(g, 6)
