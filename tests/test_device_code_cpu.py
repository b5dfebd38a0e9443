"""Checks on the gfx950 assembly of the kernels (hipcc cross-compiles without a
GPU): properties the sources rely on but the compiler could silently break.

* no packed fp32 arithmetic (the build disables it; its results are not
  trusted on this hardware),
* no round-toward-zero fp16 conversion (every fp32 -> fp16 rounding in the
  kernels is round-to-nearest-even),
* no scalar-cache writes (scalar stores, scalar atomics, scalar cache
  write-back or discard),
* no scratch memory (register spills would put stack traffic in the loop),
* M0 is written only by the kernels' own LDS-DMA sequences and read by nothing
  else: those sequences set M0 in inline assembly, which is sound only while
  the compiler keeps no value of its own in M0,
* every vector instruction inside inline assembly that reads a matrix
  product's result comes at least 19 wait states after the product: the
  compiler's hazard recognizer does not look into inline assembly, so the
  sources keep such reads apart (by the products between them, or by an
  explicit fence),
* every buffer load inside inline assembly (the LDS-DMA sequences) comes at
  least 5 wait states after a vector instruction that writes one of its
  scalar operands (v_readlane / v_readfirstlane and the like), for the same
  reason,
* the head_dim-128 fp16 kernels keep their hand-placed matrix phase: four
  exponentials after each of eight consecutive S^T products, not bunched in
  front of them (the order the compiler chose on its own, 12 % slower with the
  key split).
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from precision_flashattention_numerics_amd import build as B  # noqa: E402

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None, reason="hipcc not available")

KERNEL_SOURCES = ("pasa_fwd_d64.hip", "pasa_fwd_d128.hip", "pasa_decode.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    for src in KERNEL_SOURCES:
        path = os.path.join(B.CSRC, src)
        dst = os.path.join(d, src + ".s")
        subprocess.run([HIPCC, *flags, *B.SOURCE_FLAGS.get(src, []), "-w", "--cuda-device-only",
                        "-S", "-o", dst, path], check=True)
        out[src] = [l.split(";")[0].strip() for l in open(dst)]
        out["raw:" + src] = [l.rstrip("\n") for l in open(dst)]
    return out


def instructions(lines):
    return [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_packed_fp32_math(asm, src):
    bad = [l for l in instructions(asm[src]) if re.match(r"v_pk_(add|mul|fma)_f32\b", l)]
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_round_toward_zero_conversion(asm, src):
    bad = [l for l in instructions(asm[src]) if l.startswith("v_cvt_pkrtz")]
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_scalar_cache_writes(asm, src):
    pat = re.compile(r"s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")
    bad = [l for l in instructions(asm[src]) if pat.match(l)]
    assert not bad, bad[:5]


def test_no_scratch(asm):
    for src in KERNEL_SOURCES:
        text = "\n".join(asm[src])
        sizes = re.findall(r"\.private_segment_fixed_size:\s*(\d+)", text)
        assert sizes, src
        assert all(int(x) == 0 for x in sizes), (src, sizes)


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_m0_only_in_lds_dma(asm, src):
    ins = instructions(asm[src])
    n_dma = 0
    for i, l in enumerate(ins):
        if "m0" not in l:
            continue
        if l.startswith("s_mov_b32 m0,"):
            # the next instruction past the s_nop is the LDS-DMA load that consumes it
            nxt = [x for x in ins[i + 1:i + 3] if not x.startswith("s_nop")]
            assert nxt and re.match(r"buffer_load_dword\w*\s.*\blds\b", nxt[0]), (l, ins[i + 1:i + 3])
            n_dma += 1
        else:
            raise AssertionError(f"M0 used outside the LDS-DMA sequences: {l}")
    assert n_dma > 0


MFMA_DST = re.compile(r"^v_mfma\S*\s+v\[(\d+):(\d+)\]")
VREG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")


def _vregs(operands):
    regs = set()
    for m in VREG.finditer(operands):
        if m.group(1) is not None:
            regs.add(int(m.group(1)))
        else:
            regs.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return regs


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_inline_asm_reads_of_products_wait(asm, src):
    """Walk back from each vector instruction inside an inline-asm block over
    the preceding instructions (in program text order, counting s_nop N as N+1
    wait states and any other instruction as one) and require 19 wait states
    after a product whose destination it reads."""
    raw = asm["raw:" + src]
    inside = False
    seq = []   # (text, in_asm)
    for line in raw:
        if "#ASMSTART" in line:
            inside = True
            continue
        if "#ASMEND" in line:
            inside = False
            continue
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        seq.append((t, inside))
    bad = []
    for i, (t, in_asm) in enumerate(seq):
        if not in_asm or not t.startswith("v_") or t.startswith("v_mfma"):
            continue
        parts = t.split(None, 1)
        ops = parts[1].split(",") if len(parts) > 1 else []
        srcs = _vregs(",".join(ops[1:]))
        # an SDWA op preserving the other half also reads its destination
        if "UNUSED_PRESERVE" in t:
            srcs |= _vregs(ops[0])
        waits = 0
        for j in range(i - 1, -1, -1):
            u = seq[j][0]
            m = MFMA_DST.match(u)
            if m and srcs & set(range(int(m.group(1)), int(m.group(2)) + 1)):
                if waits < 19:
                    bad.append((t, u, waits))
                break
            n = re.match(r"s_nop\s+(\d+)", u)
            waits += int(n.group(1)) + 1 if n else 1
            if waits >= 19:
                break
    assert not bad, bad[:5]


SREG = re.compile(r"\bs(\d+)\b|\bs\[(\d+):(\d+)\]")


def _sregs(operands):
    regs = set()
    for m in SREG.finditer(operands):
        if m.group(1) is not None:
            regs.add(int(m.group(1)))
        else:
            regs.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return regs


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_inline_asm_buffer_loads_after_valu_sgpr_writes(asm, src):
    raw = asm["raw:" + src]
    inside = False
    seq = []
    for line in raw:
        if "#ASMSTART" in line:
            inside = True
            continue
        if "#ASMEND" in line:
            inside = False
            continue
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        seq.append((t, inside))
    checked, bad = 0, []
    for i, (t, in_asm) in enumerate(seq):
        if not in_asm or not t.startswith("buffer_load"):
            continue
        checked += 1
        srcs = _sregs(t.split(None, 1)[1])
        waits = 0
        for j in range(i - 1, -1, -1):
            u = seq[j][0]
            if u.startswith("v_"):
                ops = u.split(None, 1)
                dst = ops[1].split(",")[0] if len(ops) > 1 else ""
                if _sregs(dst) & srcs:
                    if waits < 5:
                        bad.append((t, u, waits))
                    break
            n = re.match(r"s_nop\s+(\d+)", u)
            waits += int(n.group(1)) + 1 if n else 1
            if waits >= 5:
                break
    assert checked > 0
    assert not bad, bad[:5]


def kernel_body(lines, name_re):
    """Instructions of the one kernel whose symbol matches name_re."""
    body, inside = None, False
    for l in lines:
        if not inside and l.endswith(":") and re.search(name_re, l):
            inside, body = True, []
            continue
        if inside and l.startswith(".Lfunc_end"):
            break
        if inside and l and not l.startswith(".") and not l.endswith(":"):
            body.append(l)
    assert body, name_re
    return body


@pytest.mark.parametrize("causal,ks", [(1, 0), (0, 0), (0, 1), (1, 1)],
                         ids=["causal", "full", "key_split", "causal_key_split"])
@pytest.mark.parametrize("var", [0, 1, 2], ids=["pasa", "strict", "naive"])
def test_head_dim_128_matrix_phase_keeps_exponentials_between_products(asm, var, causal, ks):
    body = kernel_body(asm["pasa_fwd_d128.hip"], rf"fwd_kernelILi128ELb{causal}ELi{var}ELb{ks}E")
    seq = "".join("M" if l.startswith("v_mfma") else "e" if l.startswith("v_exp_f16") else ""
                  for l in body)
    assert re.search(r"(Meeee){8}M", seq), seq[:200]
