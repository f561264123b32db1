"""Wait states after MFMAs in the compiled kernels (host-side, no GPU).

A VALU, LDS or memory instruction that reads the result of an MFMA must be
issued enough cycles after it; the compiler inserts the wait states (s_nop)
for the MFMAs it emits.  A build of an eight-wavefront variant of the
<= 16-row kernel showed that it does not always do so when a branch follows
the MFMA: the logits were read at the branch target one instruction after
the last Q.K^T MFMA, some reads saw a partial sum, and the parity tests
caught the wrong log-sum-exps.  The kernels here place explicit waits where
they read MFMA results they accumulate themselves (inline-asm chains), and
this test compiles the device code and checks every path after every MFMA:
no instruction other than a dependent MFMA (which may take the result as its
accumulator at once) reads the result within the wait states the compiler
itself gives straight-line code (12 issue slots after a 32x32 MFMA, 8 after
a 16x16 one), following fall-through and branch targets."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_mla_kv_decode_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _functions(asm):
    out = []
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        out.append((m.group(1), asm[m.end():end]))
    return out


_LOADS = ("ds_read", "ds_bpermute", "ds_permute", "buffer_load", "global_load", "scratch_load", "flat_load")


def early_reads(body):
    """(mfma index, reader index, slots between, reader) for every read of an
    MFMA result that comes too early on some path."""
    labels, ins = {}, []
    for line in body.split("\n"):
        t = line.strip()
        m = re.match(r"(\.LBB\d+_\d+):", t)
        if m:
            labels[m.group(1)] = len(ins)
            continue
        if not t or t.startswith((";", ".")):
            continue
        ins.append(t.split(";")[0].strip())
    bad = []
    for i, t in enumerate(ins):
        if not t.startswith("v_mfma"):
            continue
        dst = _regs(t.split(None, 1)[1].split(",")[0].strip())
        need = 12 if "32x32" in t else 8
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, slots = stack.pop()
            while j < len(ins) and slots < need and (j, slots) not in seen:
                seen.add((j, slots))
                u = ins[j]
                op = u.split()[0]
                ops = [x.strip() for x in u.split(None, 1)[1].split(",")] if " " in u else []
                if op == "s_nop":
                    slots += int(ops[0]) + 1
                    j += 1
                    continue
                if op.startswith("v_mfma"):
                    if (_regs(ops[1]) | _regs(ops[2])) & dst:   # srcA / srcB (srcC may follow at once)
                        bad.append((i, j, slots, u))
                elif op.startswith(("v_", "ds_", "buffer_", "global_", "scratch_", "flat_")):
                    srcs = ops[1:] if op.startswith("v_") or op.startswith(_LOADS) else ops
                    if set().union(*[_regs(x) for x in srcs]) & dst if srcs else False:
                        bad.append((i, j, slots, u))
                        break
                if op.startswith("s_cbranch") or op == "s_branch":
                    if ops and ops[0] in labels:
                        stack.append((labels[ops[0]], slots + 1))
                    if op == "s_branch":
                        break
                if op == "s_endpgm":
                    break
                slots += 1
                j += 1
    return bad


def test_checker_sees_a_read_behind_a_branch():
    hazard = """
\tv_mfma_f32_16x16x32_bf16 v[14:17], v[22:25], v[40:43], v[14:17]
\ts_cbranch_scc1 .LBB0_2
\tv_cndmask_b32_e64 v17, v240, v17, s[18:19]
.LBB0_2:
\tv_max_f32_e32 v2, v17, v17
\ts_endpgm
"""
    found = {(u.split()[0], slots) for _, _, slots, u in early_reads(hazard)}
    # both paths read too early: the fall-through and the branch target
    assert found == {("v_cndmask_b32_e64", 1), ("v_max_f32_e32", 1)}
    safe = """
\tv_mfma_f32_16x16x32_bf16 v[14:17], v[22:25], v[40:43], v[14:17]
\tv_mfma_f32_16x16x32_bf16 v[14:17], v[26:29], v[40:43], v[14:17]
\ts_nop 7
\ts_cbranch_scc1 .LBB0_2
\tv_cndmask_b32_e64 v17, v240, v17, s[18:19]
.LBB0_2:
\tv_max_f32_e32 v2, v17, v17
\tv_accvgpr_read_b32 v3, a5
\ts_endpgm
"""
    assert early_reads(safe) == []
    agpr = "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n\ts_nop 7\n\tv_accvgpr_read_b32 v1, a3\n"
    assert len(early_reads(agpr)) == 1   # 9 slots after a 32x32 MFMA: too early


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["decode.hip", "proj.hip"])
def test_no_early_read_of_an_mfma_result(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-S", "--offload-device-only", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    funcs = _functions(out.read_text())
    assert funcs
    report = []
    for name, body in funcs:
        for i, j, slots, u in early_reads(body):
            report.append("%s: MFMA #%d read %d slots later by %s" % (name, i, slots, u))
    assert not report, "\n".join(report[:20])
