"""Structure of the compiled gfx950 kernels (host test: hipcc cross-compiles).

A workgroup barrier must sit in control flow that every wave of the workgroup
runs the same number of times.  The persistent attention kernel's item loop
starts with a block that only thread 0 runs, then two barriers; when thread-0
code also ran between an item's work and the loop's back edge, the compiler
turned the loop into two nested loops whose inner one (holding the barriers)
was left through the exec mask: thread 0 went round the outer loop while the
other lanes of wave 0, and waves 1-3, went back to the barriers without it,
and the kernel never finished.  This test compiles every HIP source to
assembly and fails if any loop that contains `s_barrier` can be left through
an exec-masked branch (`s_andn2_b64 exec, exec, ...` then `s_cbranch_execz` to
a block outside the loop).  Loops are read from the compiler's own
annotations of each block ("Loop Header", "in Loop: Header=", "Child Loop").
"""
import os
import re
import subprocess

import pytest

from chunked_prefill_mixed_hybrid_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.hipcc()), reason="hipcc not available")

_LABEL = re.compile(r"^(\.LBB\d+_\d+):")
_BB = re.compile(r"^; %bb\.(\d+):")


def _functions(asm: str) -> dict:
    funcs, cur = {}, None
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
        elif cur and line.startswith(".Lfunc_end"):
            cur = None
        elif cur:
            funcs[cur].append(line)
    return funcs


def divergent_barrier_loops(lines: list) -> list:
    """(loop header, block, exit target) for every exec-masked exit of a loop
    that contains a barrier, in one function's assembly."""
    blocks, order, name = {}, [], None
    for line in lines:
        m = _LABEL.match(line)
        b = _BB.match(line)
        if m or b:
            name = m.group(1) if m else "%bb." + b.group(1)
            blocks[name] = [line]
            order.append(name)
        elif name:
            blocks[name].append(line)
    innermost, children = {}, {}
    for b in order:
        head = " ".join(blocks[b][:16])
        if "Loop Header: Depth" in head:
            innermost[b] = b
            children[b] = [".LBB" + c for c in re.findall(r"Child Loop BB(\d+_\d+)", head)]
        else:
            m = re.search(r"Header=BB(\d+_\d+) Depth", blocks[b][0])
            if m:
                innermost[b] = ".LBB" + m.group(1)

    def members(h):
        s = {b for b, hh in innermost.items() if hh == h}
        for c in children.get(h, []):
            s |= members(c)
        return s

    found = []
    for h in children:
        loop = members(h)
        if not any("s_barrier" in l for b in loop for l in blocks[b]):
            continue
        for b in loop:
            body = blocks[b]
            for k, line in enumerate(body):
                if "s_andn2_b64 exec, exec" not in line:
                    continue
                m = re.search(r"s_cbranch_execz\s+(\.LBB\d+_\d+)", " ".join(body[k + 1:k + 3]))
                if m and m.group(1) not in loop:
                    found.append((h, b, m.group(1)))
    return found


def _device_asm(src, tmp_path):
    out = tmp_path / (src.stem + ".s")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC",) and not f.startswith("-W")]
    res = subprocess.run([build.hipcc(), *flags, f"-I{build.INCLUDE}", f"-I{build.CSRC}",
                          "--cuda-device-only", "-S", str(src), "-o", str(out)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.mark.parametrize("source", build.SOURCES)
def test_no_barrier_inside_a_divergent_loop(source, tmp_path):
    asm = _device_asm(build.CSRC / source, tmp_path)
    funcs = _functions(asm)
    if "__global__" in (build.CSRC / source).read_text():
        assert funcs, "no kernels found in the assembly"
    bad = {fn: f for fn, lines in funcs.items() if (f := divergent_barrier_loops(lines))}
    assert not bad, f"barrier inside an exec-masked loop: {bad}"


def test_detector_flags_thread0_code_before_the_back_edge(tmp_path):
    """The detector itself: a loop shaped like the item loop, with thread-0
    code after the work, is flagged in the same way as the kernel was."""
    src = tmp_path / "probe.hip"
    src.write_text(r"""
#include <hip/hip_runtime.h>
__global__ void probe(int* q, int* out, int n) {
  __shared__ int s_next, s_item;
  if (threadIdx.x == 0) s_next = atomicAdd(q, 1);
  __syncthreads();
  for (;;) {
    if (threadIdx.x == 0) s_item = s_next;
    __syncthreads();
    const int it = __builtin_amdgcn_readfirstlane(s_item);
    __syncthreads();
    if (it >= n) break;
    out[it * blockDim.x + threadIdx.x] += it;
    if (threadIdx.x == 0) s_next = atomicAdd(q, 1);
  }
}
""")
    asm = _device_asm(src, tmp_path)
    funcs = _functions(asm)
    assert any(divergent_barrier_loops(lines) for lines in funcs.values())


# ---------------------------------------------------------------- LDS-DMA wait states
# A pool-to-LDS load (buffer_load ... lds) reads M0 (its LDS address) and the
# buffer descriptor in SGPRs.  On gfx9-family chips it needs one wait state
# after an SALU write of M0, and five after a VALU write of any SGPR it reads.
# The compiler inserts them for the loads it emits itself; for loads written
# as inline asm it cannot, so the compiled code is checked here.
_SGPR = re.compile(r"^s\[(\d+):(\d+)\]$|^s(\d+)$")


def _sgprs(tok):
    tok = tok.strip(",")
    if tok == "m0":
        return {"m0"}
    m = _SGPR.match(tok)
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def lds_dma_hazards(lines: list) -> list:
    """(load, writer, wait states) for every LDS-DMA load that follows an SALU
    write of M0 by fewer than 1 wait state, or a VALU write of one of its SGPR
    operands by fewer than 5, in one function's assembly."""
    code = [l.strip() for l in lines]
    code = [l for l in code if l and not l.startswith((";", ".")) and not l.endswith(":")]
    found = []
    for i, line in enumerate(code):
        op = line.split()[0]
        if not (op.startswith("buffer_load") and line.endswith(" lds")):
            continue
        reads = {"m0"}
        for tok in line.split()[1:]:
            reads |= _sgprs(tok)
        waits = 0
        for k in range(i - 1, max(i - 12, -1), -1):
            prev = code[k].split()
            dst = _sgprs(prev[1]) if len(prev) > 1 else set()
            if prev[0].startswith("s_") and "m0" in dst and waits < 1:
                found.append((line, code[k], waits))
            if prev[0].startswith("v_") and dst & reads and waits < 5:
                found.append((line, code[k], waits))
            waits += int(prev[1]) + 1 if prev[0] == "s_nop" else 1
            if waits >= 5:
                break
    return found


@pytest.mark.parametrize("source", build.SOURCES)
def test_lds_dma_wait_states(source, tmp_path):
    asm = _device_asm(build.CSRC / source, tmp_path)
    bad = {fn: f for fn, lines in _functions(asm).items() if (f := lds_dma_hazards(lines))}
    assert not bad, f"LDS-DMA load too close to a write of its SGPR operands: {bad}"


def test_lds_dma_detector_flags_a_missing_wait_state(tmp_path):
    """The detector itself: an inline-asm LDS-DMA load right after the SALU
    write of M0 (the compiler sees no load there) is flagged."""
    src = tmp_path / "probe_dma.hip"
    src.write_text(r"""
#include <hip/hip_runtime.h>
__global__ void probe_dma(const unsigned* src, int n) {
  __shared__ __attribute__((aligned(16))) unsigned char st[4096];
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, n * 4, 0x00020000);
  const auto lp = (__attribute__((address_space(3))) unsigned char*)(st + (threadIdx.x >> 6) * 1024);
  const unsigned lds = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>(lp)));
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(threadIdx.x * 16), "s"(rs), "{m0}"(lds) : "memory");
}
""")
    asm = _device_asm(src, tmp_path)
    assert any(lds_dma_hazards(lines) for lines in _functions(asm).values())
