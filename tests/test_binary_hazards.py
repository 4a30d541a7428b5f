"""Static check of the built GPU code: no register written by a vector-memory
or LDS load is read or overwritten before a wait that covers the load.

Some kernels issue loads from inline assembly, which the compiler's own wait
tracking does not see; if register allocation then moves, spills or reuses a
destination register while the load is in flight, the late data lands on
whatever the register holds by then (an address, say) and the kernel faults
or computes garbage.  This test disassembles every gfx950 kernel of
libfd_attn.so and walks its control-flow graph from each load: on every
path, each instruction that names one of the load's destination registers
must come after a covering s_waitcnt.  Vector-memory loads complete in issue
order, so vmcnt(N) covers a load once N vector-memory instructions were
issued after it.  LDS loads also complete in order, but they share lgkmcnt
with scalar memory loads, which may complete out of order: lgkmcnt(N) covers
an LDS load once N LDS instructions were issued after it and no scalar load
was.  CPU only; needs the ROCm LLVM tools.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

import split_kv_asynchronous_amd as fd

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
VMEM = ("global_", "buffer_", "scratch_")
BRANCH = re.compile(r"^s_(c?branch\w*)\b")
TARGET = re.compile(r"<[^>+]+\+0x([0-9a-f]+)>")
VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _tools_present():
    return all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objdump", "clang-offload-bundler"))


def _code_objects(lib, tmp):
    """gfx950 code objects of every offload bundle in the library's fat binary."""
    # objcopy rewrites the file it reads: work on a private copy of the library
    copy = os.path.join(tmp, "lib.so")
    shutil.copyfile(lib, copy)
    fat = os.path.join(tmp, "fatbin")
    subprocess.run(["objcopy", "--dump-section", ".hip_fatbin=" + fat, copy], check=True)
    data = open(fat, "rb").read()
    offs = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
    out = []
    for i in range(len(offs) - 1):
        part = os.path.join(tmp, "bundle%d" % i)
        with open(part, "wb") as f:
            f.write(data[offs[i]:offs[i + 1]])
        co = os.path.join(tmp, "co%d" % i)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--input=" + part, "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        "--output=" + co], check=True)
        out.append(co)
    return out


def _kernels(co):
    dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                         check=True, stdout=subprocess.PIPE, text=True).stdout
    kernels, name = {}, None
    for line in dis.splitlines():
        m = re.match(r"^([0-9a-f]+) <(\S+)>:$", line)
        if m:
            name = m.group(2)
            kernels[name] = []
            continue
        if name and line.startswith("\t"):
            code, _, comment = line.partition("//")
            addr = re.match(r"\s*([0-9A-F]+):", comment)
            kernels[name].append((int(addr.group(1), 16) if addr else None, code.strip(), line))
    return kernels


def _regs(text):
    r = set()
    for a, b, c in VREG.findall(text):
        r |= set(range(int(a), int(b) + 1)) if a else {int(c)}
    return r


def _operands(ins):
    parts = ins.split(None, 1)
    return parts[1] if len(parts) > 1 else ""


def _wait(ins, counter):
    """The counter's value in an s_waitcnt, or None if it does not wait on it."""
    if not ins.startswith("s_waitcnt ") and ins != "s_waitcnt":
        return None
    m = re.search(counter + r"\((\d+)\)", ins)
    return int(m.group(1)) if m else None


def _hazards(body):
    """(load, offending instruction) pairs of one kernel."""
    index = {addr: i for i, (addr, _, _) in enumerate(body) if addr is not None}
    start = body[0][0] if body and body[0][0] is not None else 0

    def successors(i):
        ins = body[i][1]
        if ins.startswith("s_endpgm"):
            return []
        m = BRANCH.match(ins)
        if m:
            t = TARGET.search(body[i][2])
            tgt = [index[start + int(t.group(1), 16)]] if t and (start + int(t.group(1), 16)) in index else []
            return tgt if m.group(1) == "branch" else tgt + [i + 1]
        return [i + 1] if i + 1 < len(body) else []

    found = []
    for i, (_, ins, _) in enumerate(body):
        op = ins.split(None, 1)[0] if ins else ""
        vmem = op.startswith(VMEM) and "load" in op and "lds" not in op and not ins.endswith(" lds")
        lds = op.startswith("ds_read") or op.startswith("ds_load")
        if not (vmem or lds):
            continue
        dst = _regs(_operands(ins).split(",")[0])
        if not dst:
            continue
        counter = "vmcnt" if vmem else "lgkmcnt"
        seen = set()
        # state: (instruction, same-kind ops issued since, a scalar load issued since)
        stack = [(j, 0, False) for j in successors(i)]
        while stack:
            j, later, smem = stack.pop()
            if (j, later, smem) in seen:
                continue
            seen.add((j, later, smem))
            t = body[j][1]
            w = _wait(t, counter)
            if w is not None and (w == 0 or (w <= later and not smem)):
                continue                      # the load is complete on this path
            ops = _operands(t)
            top = t.split(None, 1)[0] if t else ""
            if _regs(ops) & dst:
                same_kind = (top.startswith(VMEM) and "load" in top) if vmem else top.startswith("ds_read")
                if same_kind and not _regs(",".join(ops.split(",")[1:])) & dst:
                    continue                  # a newer load takes the registers over (in-order completion)
                found.append((ins, t))
                break
            if vmem:
                nxt, nsmem = later + (1 if top.startswith(VMEM) else 0), smem
            else:
                nxt = later + (1 if top.startswith("ds_") else 0)
                nsmem = smem or top.startswith("s_load") or top.startswith("s_buffer_load")
            stack.extend((k, min(nxt, 64), nsmem) for k in successors(j))
    return found


@pytest.mark.skipif(not _tools_present() or shutil.which("objcopy") is None,
                    reason="ROCm LLVM tools not installed")
def test_no_register_is_touched_before_its_load_completes():
    lib = fd.library_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    with tempfile.TemporaryDirectory() as tmp:
        names, bad = [], []
        for co in _code_objects(lib, tmp):
            for name, body in _kernels(co).items():
                names.append(name)
                bad += [(name, a, b) for a, b in _hazards(body)]
    assert any("prefill_kernel" in n for n in names) and any("chunk_kernel" in n for n in names)
    assert not bad, "\n".join("%s: %s ... %s" % x for x in bad[:10])
