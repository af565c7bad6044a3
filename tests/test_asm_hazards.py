"""Wait states after the hand-placed MFMAs, checked in the gfx950 assembly.

Some kernels keep long-lived accumulators in AGPRs through MFMAs written as
inline asm (``mfma32_agpr``).  The compiler does not
know the latency of those instructions, so it cannot insert the wait states
a later instruction needs before it reads, copies or overwrites such an
accumulator: a 16-pass 32x32x16 MFMA needs 18 (CDNA3/CDNA4 ISA, "Dependency
Resolution: Required Independent Instructions").  The kernels cover this
with explicit ``s_nop`` drains.  This test compiles every source for the
device and follows every path (fall-through and branch targets) from each
MFMA whose destination is an AGPR range: no non-MFMA instruction may touch
those registers within 18 wait states.  MFMAs with VGPR destinations come
from the compiler's builtins, whose hazards the compiler resolves itself.

CPU only (hipcc cross-compiles); skipped when hipcc is absent.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sparse_attention_long_attn_amd import build  # noqa: E402

WAIT_STATES = 18
_REG = re.compile(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b")
_LABEL = re.compile(r"^(\.LBB[0-9_]+):")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _kernels(asm: str):
    """(name, instructions, labels) per kernel body of a device .s file."""
    lines = asm.split("\n")
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S*kernel\S*):", lines[i])
        if not m:
            i += 1
            continue
        name = m.group(1)
        insts, labels = [], {}
        i += 1
        while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
            raw = lines[i]
            lm = _LABEL.match(raw)
            if lm:
                labels[lm.group(1)] = len(insts)
            else:
                text = raw.split(";")[0].strip()
                if text and not text.startswith(".") and not text.endswith(":"):
                    insts.append((text.split()[0], text))
            i += 1
        yield name, insts, labels


def _violations(insts, labels):
    """Instructions that touch an AGPR-destination MFMA's registers too soon."""
    found = []

    def scan(i, ws, dst, src, seen):
        while i < len(insts):
            op, text = insts[i]
            if op == "s_nop":
                ws += int(text.split()[1]) + 1
                if ws >= WAIT_STATES:
                    return
                i += 1
                continue
            ws += 1
            if ws > WAIT_STATES:
                return
            if not op.startswith("v_mfma") and _regs(text) & dst:
                found.append((src, text, ws))
            if op.startswith("s_cbranch") or op == "s_branch":
                target = text.split()[1]
                if target in labels and (target, ws) not in seen:
                    seen.add((target, ws))
                    scan(labels[target], ws, dst, src, seen)
                if op == "s_branch":
                    return
            if op in ("s_endpgm", "s_setpc_b64"):
                return
            i += 1

    for i, (op, text) in enumerate(insts):
        if op.startswith("v_mfma") and " a[" in text.split(",")[0]:
            scan(i + 1, 0, _regs(text.split(",")[0]), text, set())
    return found


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src)[:-4] + ".s")
    cmd = [build.hipcc(), *build.HIPCC_FLAGS,
           "-I", os.path.join(ROOT, "include"), "-I", build.CSRC,
           "--cuda-device-only", "-S", "-o", out, src]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL,
                   stderr=subprocess.DEVNULL)
    return out


def test_agpr_mfma_wait_states(tmp_path):
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    srcs = build.sources()
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        outs = list(ex.map(lambda s: _device_asm(s, str(tmp_path)), srcs))
    checked, bad = 0, []
    for path in outs:
        for name, insts, labels in _kernels(open(path).read()):
            checked += sum(1 for op, t in insts
                           if op.startswith("v_mfma") and " a[" in t.split(",")[0])
            bad += [(name[:60], v) for v in _violations(insts, labels)]
    assert checked > 0, "no AGPR-destination MFMA found: the scan is not looking"
    assert not bad, bad[:10]


def test_scan_flags_a_planted_hazard():
    """The scan itself: a copy 3 wait states after an AGPR MFMA, on the path
    through a branch, is found; the same copy after an 18-state drain is not."""
    body = [
        ("v_mfma_f32_32x32x16_bf16", "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]"),
        ("s_cbranch_scc1", "s_cbranch_scc1 .LBB0_2"),
        ("s_endpgm", "s_endpgm"),
        ("s_nop", "s_nop 0"),
        ("v_accvgpr_mov_b32", "v_accvgpr_mov_b32 a20, a3"),
    ]
    assert len(_violations(body, {".LBB0_2": 3})) == 1
    drained = body[:1] + [("s_nop", "s_nop 7")] * 3 + body[1:]
    assert _violations(drained, {".LBB0_2": 6}) == []
