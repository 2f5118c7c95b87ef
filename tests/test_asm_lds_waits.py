"""The matrix-core kernels read V operands with ds_read_b64_tr_b16 written
as inline assembly, so the compiler does not know that the destination
registers are still being filled after the instruction issues; the code is
correct only if nothing touches those registers before an s_waitcnt
lgkmcnt(N) that covers the read (LDS reads complete in issue order, so
lgkmcnt(N) covers a read followed by at least N later LDS instructions).

This scans the gfx950 machine code of the built library (its own device
code, disassembled with the ROCm llvm-objdump) and fails on any instruction
that reads or writes a pending destination, and on any pending read that
crosses a branch or the end of a kernel (the scan is linear, so a read must
be waited for inside its basic block).  CPU only.
"""
import os
import re
import subprocess
import tempfile

import pytest

import tree_verification_attention_tsw_amd as tsw

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?![0-9]))")


def _tools_ok():
    return all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump"))


def _device_listings(lib_path):
    """objdump text of every gfx950 code object bundled into the library."""
    with tempfile.TemporaryDirectory(prefix="tsw_asm_") as d:
        fat = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fat, lib_path],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        offs = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
        out = []
        for n, (a, b) in enumerate(zip(offs, offs[1:])):
            part, obj = os.path.join(d, "b%d" % n), os.path.join(d, "o%d" % n)
            with open(part, "wb") as f:
                f.write(data[a:b])
            subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + part,
                            "--targets=" + TARGET, "--output=" + obj], check=True, capture_output=True)
            r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", obj],
                               check=True, capture_output=True, text=True)
            out.append(r.stdout)
        return out


def _regs(text):
    """Set of (file, index) registers named in an operand string."""
    s = set()
    for kind, lo, hi, one in REG.findall(text):
        if one:
            s.add((kind, int(one)))
        else:
            s.update((kind, i) for i in range(int(lo), int(hi) + 1))
    return s


def scan(listing):
    """Violations in one objdump listing: (function, instruction, reason)."""
    bad = []
    fn = None
    pending = []            # [dest registers, LDS instructions issued after it]
    for line in listing.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            if pending and fn:
                bad.append((fn, "end", "transposed read pending at the end of the function"))
            fn, pending = m.group(1), []
            continue
        if not line.startswith("\t") or fn is None:
            continue
        ins = line.split("//")[0].strip()
        if not ins:
            continue
        op, _, rest = ins.partition(" ")
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", rest)
            if m:
                n = int(m.group(1))
                pending = [p for p in pending if p[1] < n]
            continue
        if op.startswith("s_branch") or op.startswith("s_cbranch") or op in ("s_setpc_b64", "s_endpgm"):
            if pending:
                bad.append((fn, ins, "transposed read pending across a branch or the end of the kernel"))
                pending = []
            continue
        used = _regs(rest)
        for dest, _ in pending:
            if used & dest:
                bad.append((fn, ins, "touches a pending ds_read_b64_tr_b16 destination"))
                break
        if op.startswith("ds_"):
            for p in pending:
                p[1] += 1
        if op == "ds_read_b64_tr_b16":
            dest = _regs(rest.split(",")[0])
            pending.append([dest, 0])
    return bad


def test_scan_catches_planted_mistakes():
    """The scanner itself: a use before the wait, a wait that does not cover
    the read, and a read pending across a branch are caught; correct code
    passes."""
    ok = ("0000000000000000 <k>:\n"
          "\tds_read_b64_tr_b16 v[10:11], v2 offset:8192 // 0\n"
          "\tds_read_b64_tr_b16 v[12:13], v2 offset:12288 // 0\n"
          "\ts_waitcnt lgkmcnt(1) // 0\n"
          "\tv_mov_b32_e32 v20, v10 // 0\n"
          "\ts_waitcnt lgkmcnt(0) // 0\n"
          "\tv_mov_b32_e32 v21, v12 // 0\n"
          "\ts_endpgm // 0\n")
    assert scan(ok) == []
    early = ok.replace("\ts_waitcnt lgkmcnt(1) // 0\n", "")
    assert len(scan(early)) == 1
    short = ok.replace("lgkmcnt(1)", "lgkmcnt(2)")
    assert len(scan(short)) == 1
    branch = ok.replace("\ts_waitcnt lgkmcnt(1) // 0\n", "\ts_cbranch_scc1 12 // 0\n\ts_waitcnt lgkmcnt(1) // 0\n")
    assert any("branch" in r for _, _, r in scan(branch))
    overwrite = ok.replace("\ts_waitcnt lgkmcnt(1) // 0\n", "\tv_mov_b32_e32 v11, 0 // 0\n\ts_waitcnt lgkmcnt(1) // 0\n")
    assert len(scan(overwrite)) == 1


@pytest.mark.skipif(not _tools_ok(), reason="ROCm llvm tools not found")
def test_transposed_reads_are_waited_for():
    if not os.path.exists(tsw.LIB_PATH):
        pytest.skip("libtsw.so is not built")
    listings = _device_listings(tsw.LIB_PATH)
    n_reads = sum(l.count("ds_read_b64_tr_b16") for l in listings)
    assert n_reads > 1000, n_reads            # the matrix-core kernels are in the library
    bad = [v for l in listings for v in scan(l)]
    assert not bad, bad[:10]
