"""Wait states after every MFMA in the generated gfx950 code (CPU only: hipcc cross-compiles).

A VALU, LDS or memory instruction that touches an MFMA's result registers before the MFMA has
written them reads or overwrites a stale value; the hardware does not stall for it, the compiler
must leave enough independent instructions or s_nop wait states in between.  hipcc does so in
straight-line code, but it has been seen to leave too few where the reader sits after a branch
join (one arm held the MFMA).  The walkers put MFMAs under wave-uniform branches on purpose, so
this test compiles every library source to device assembly and follows every control-flow path
from each MFMA to the first non-accumulating instruction that touches its destination registers.
Each path must have at least the wait states that hipcc itself inserts in straight-line code
for the same MFMA (measured on a two-kernel probe compiled here).  Every fp32 MFMA must also
keep its explicit 16-state guard (the accumulator input of an 8-pass MFMA is read late, and the
compiler has been seen to overwrite it right after issue).
"""
import concurrent.futures
import heapq
import os
import re
import shutil
import subprocess

import pytest

from causal_prefix_scan_hla2_amd import build as B

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")

_REG = re.compile(r"(?<![\w.])([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_LIMIT = 64  # paths longer than this many wait states are clear of every MFMA hazard

PROBE = r"""
#include <hip/hip_runtime.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
extern "C" __global__ void probe_bf16(const bf16x8 *a, const bf16x8 *b, float *o) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], b[threadIdx.x], c, 0, 0, 0);
  o[threadIdx.x] = c[0] * 3.f + c[3];
}
extern "C" __global__ void probe_f32(const float *a, const float *b, float *o) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[threadIdx.x], b[threadIdx.x], c, 0, 0, 0);
  o[threadIdx.x] = c[0] * 3.f + c[3];
}
"""


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            lo = hi = int(m.group(4))
        else:
            lo, hi = int(m.group(2)), int(m.group(3))
        out.update((m.group(1), r) for r in range(lo, hi + 1))
    return out


def _functions(asm):
    """name -> (instructions [(mnemonic, operands)], label -> instruction index)."""
    funcs, cur = {}, None
    for line in asm.splitlines():
        s = line.split(";")[0].rstrip()
        if not s:
            continue
        m = re.match(r"^([_A-Za-z][\w.$]*):", s)
        if m and not s.startswith("."):
            cur = funcs.setdefault(m.group(1), ([], {}))
            continue
        if cur is None:
            continue
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        m = re.match(r"^(\.LBB[\w]+):", s)
        if m:
            cur[1][m.group(1)] = len(cur[0])
            continue
        t = s.strip()
        if t.startswith("."):
            continue
        parts = t.split(None, 1)
        cur[0].append((parts[0], parts[1] if len(parts) > 1 else ""))
    return funcs


def _wait_states(ins):
    return int(ins[1].strip(), 0) + 1 if ins[0] == "s_nop" else 1


def _consumer_paths(code, labels, with_src_c=False):
    """For every MFMA: (opcode, index, fewest wait states to a consumer, whether that path
    crosses a branch or a join).  A consumer touches the MFMA's destination registers (and,
    with `with_src_c`, its accumulator input registers)."""
    targets = set(labels.values())

    def succ(i):
        op, ops = code[i]
        if op == "s_branch":
            return [labels[ops.strip()]]
        if op.startswith("s_cbranch"):
            return [i + 1, labels[ops.strip()]]
        if op in ("s_endpgm", "s_setpc_b64"):
            return []
        return [i + 1]

    out = []
    for i, (op, ops) in enumerate(code):
        if not op.startswith("v_mfma"):
            continue
        o = ops.split(",")
        dst = _regs(o[0]) | (_regs(o[3]) if with_src_c and len(o) >= 4 else set())
        heap, seen = [(0, False, i)], set()
        while heap:
            d, crossed, j = heapq.heappop(heap)
            if (j, crossed) in seen:
                continue
            seen.add((j, crossed))
            for k in succ(j):
                if k >= len(code):
                    continue
                c2 = crossed or k != j + 1 or code[j][0].startswith("s_cbranch") or k in targets
                op2, ops2 = code[k]
                if dst & _regs(ops2):
                    if not op2.startswith("v_mfma"):
                        out.append((op, i, d, c2))
                        continue
                    if dst & _regs(ops2.split(",")[0]):
                        continue  # rewritten by the next product: later readers are its own
                    # read as an MFMA operand (the MFMA-to-MFMA rules are not checked here)
                nd = d + _wait_states(code[k])
                if nd <= _LIMIT:
                    heapq.heappush(heap, (nd, c2, k))
    return out


def _compile_asm(src, out, extra=()):
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=" + B.ARCH, "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", B.INCLUDE, "-I", B.CSRC, "-Wno-unused-result", *extra, "-o", out, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def floors(tmp_path_factory):
    d = tmp_path_factory.mktemp("probe")
    src = os.path.join(d, "probe.hip")
    with open(src, "w") as f:
        f.write(PROBE)
    asm = _compile_asm(src, os.path.join(d, "probe.s"))
    fl = {}
    for name, (code, labels) in _functions(asm).items():
        for op, _, dist, _ in _consumer_paths(code, labels):
            fl[op] = min(fl.get(op, 1 << 30), dist)
    assert set(fl) == {"v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x4_f32"}, fl
    return fl


@pytest.fixture(scope="module")
def library_asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    srcs = [p for p in B.sources() if p.endswith(".hip")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {p: ex.submit(_compile_asm, p, os.path.join(d, os.path.basename(p) + ".s"))
                for p in srcs}
        return {os.path.basename(p): f.result() for p, f in futs.items()}


def test_probe_floors_are_positive(floors):
    # the probes read the result right away, so hipcc must have padded with wait states
    assert all(v >= 4 for v in floors.values()), floors


def test_every_path_from_an_mfma_has_the_straight_line_wait_states(floors, library_asm):
    bad, n_paths, n_crossing, n_mfma = [], 0, 0, 0
    for fname, asm in library_asm.items():
        for kname, (code, labels) in _functions(asm).items():
            for op, i, dist, crossed in _consumer_paths(code, labels):
                n_paths += 1
                n_crossing += crossed
                if dist < floors[op]:
                    bad.append((fname, kname[:80], i, op, dist, floors[op], crossed))
            n_mfma += sum(1 for ins in code if ins[0].startswith("v_mfma"))
    assert n_mfma > 10000 and n_paths > 100 and n_crossing > 50, (n_mfma, n_paths, n_crossing)
    assert not bad, bad[:10]


def test_every_fp32_mfma_keeps_its_guard(library_asm):
    # nothing touches an fp32 MFMA's accumulator input or output within 16 wait states
    n, bad = 0, []
    for fname, asm in library_asm.items():
        for kname, (code, labels) in _functions(asm).items():
            for op, i, dist, _ in _consumer_paths(code, labels, with_src_c=True):
                if op != "v_mfma_f32_16x16x4_f32":
                    continue
                n += 1
                if dist < 16:
                    bad.append((fname, kname[:80], i, dist))
    assert n > 1000 and not bad, (n, bad[:10])


def test_scanner_finds_a_short_path_across_a_join():
    # hand-written text (never assembled): the second product sits in one arm of a branch and
    # its result is read right after the join; the first one's result two states later
    asm = "\n".join([
        "kern:",
        "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
        "\ts_cbranch_execz .LBB0_2",
        "\tv_mfma_f32_16x16x32_bf16 v[12:15], v[4:7], v[8:11], 0",
        ".LBB0_2:",
        "\tv_add_f32_e32 v16, v12, v0",
        "\ts_nop 7",
        "\tv_add_f32_e32 v17, v13, v1",
        "\ts_endpgm",
        ".Lfunc_end0:",
    ])
    (code, labels), = _functions(asm).values()
    paths = sorted((i, d, c) for _, i, d, c in _consumer_paths(code, labels))
    # first product: via the taken branch after 1 state, via the other arm after 2 (the
    # reader of v0 is the same instruction on both paths); second product: at once, after the join
    assert (0, 1, True) in paths and (2, 0, True) in paths
    assert all(d <= 2 for _, d, _ in paths)
