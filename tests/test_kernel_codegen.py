"""Code-generation checks on the decode kernels (CPU only: decode.hip is compiled
to gfx950 assembly here and the assembly is read).

Some defects leave every result bit-exact and only cost time, so no parity test
sees them:
  * a wait for *all* outstanding vector-memory operations (vmcnt(0)) inside the
    tile loop of the dense bf16 kernel drains the two tiles of global->LDS copies
    it keeps in flight (a register spill whose reload the compiler cannot prove
    complete produces exactly that wait);
  * scratch (spill) traffic or generic (flat) accesses inside a tile loop;
  * a VALU write of a VGPR followed within two issue slots by a hand-written
    MFMA that reads it (the compiler does not pad inline assembly), which the
    CDNA3/CDNA4 ISA lists among the hazards software must cover with
    independent instructions or s_nop.
"""

from __future__ import annotations

import os
import re
import subprocess

import pytest

from paged_kv_head_amd import build as build_mod

HIPCC = build_mod.HIPCC
DECODE = os.path.join(build_mod.CSRC, "decode.hip")
INDEXER = os.path.join(build_mod.CSRC, "indexer.hip")
SCORE_KERNEL = "_ZN3mla12_GLOBAL__N_118index_score_kernelILi{}EEEvNS0_9IndexArgsE"
QUERY_KERNEL = "_ZN3mla12_GLOBAL__N_118index_query_kernelENS0_9IndexArgsE"
TOPK_KERNEL = "_ZN3mla12_GLOBAL__N_117index_topk_kernelENS0_9IndexArgsE"
KERNELS = {  # (cache format, sparse) -> mangled name
    (0, False): "_ZN3mla12_GLOBAL__N_113decode_kernelILi0ELb0EEEvNS_10DecodeArgsE",
    (1, False): "_ZN3mla12_GLOBAL__N_113decode_kernelILi1ELb0EEEvNS_10DecodeArgsE",
    (0, True): "_ZN3mla12_GLOBAL__N_113decode_kernelILi0ELb1EEEvNS_10DecodeArgsE",
    (1, True): "_ZN3mla12_GLOBAL__N_113decode_kernelILi1ELb1EEEvNS_10DecodeArgsE",
}
DENSE_IN_FLIGHT = 8  # copies the dense bf16 tile loop leaves outstanding at each of its two waits


def compile_asm(tmp_path_factory, src):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    out = str(tmp_path_factory.mktemp("asm") / (os.path.basename(src) + ".s"))
    flags = [f for f in build_mod.FLAGS if f not in ("-fPIC", "-shared")]
    subprocess.check_call([HIPCC, *flags, "-S", "--cuda-device-only", src, "-o", out])
    with open(out) as f:
        return f.read().split("\n")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return compile_asm(tmp_path_factory, DECODE)


@pytest.fixture(scope="module")
def asm_indexer(tmp_path_factory):
    return compile_asm(tmp_path_factory, INDEXER)


def function_body(lines, name):
    start = next(i for i, l in enumerate(lines) if l.startswith(name + ":"))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    return lines[start:end + 1]


def instructions(block_lines):
    out = []
    for l in block_lines:
        t = l.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            out.append(t)
    return out


def loop_blocks(body):
    """Loop depth LLVM gives each line's block."""
    depth_of = []
    depth = 0
    for i, l in enumerate(body):
        if l.startswith(".LBB") or l.startswith("; %bb"):
            # the label's comment, continued on comment-only lines: the
            # enclosing loops outermost first, then this block's own loop
            ctx = [l]
            k = i + 1
            while k < len(body) and body[k].lstrip().startswith(";") and not body[k].startswith(";"):
                ctx.append(body[k])
                k += 1
            m = re.findall(r"Depth=(\d+)", " ".join(ctx))
            depth = max(map(int, m)) if m else 0
        depth_of.append(depth)
    return depth_of


def innermost_loop(body):
    """Instructions of the blocks LLVM marks as lying in the deepest loop."""
    depth_of = loop_blocks(body)
    deepest = max(depth_of)
    assert deepest >= 1, "no loop found"
    return instructions([l for l, d in zip(body, depth_of) if d == deepest]), deepest


def vgprs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def test_dense_tile_loop_keeps_copies_in_flight(asm):
    loop, depth = innermost_loop(function_body(asm, KERNELS[(0, False)]))
    assert depth == 3  # work loop > restart pass > tile loop
    waits = [re.search(r"vmcnt\((\d+)\)", t) for t in loop if t.startswith("s_waitcnt")]
    counts = [int(w.group(1)) for w in waits if w]
    assert counts and all(c == DENSE_IN_FLIGHT for c in counts), counts
    # per wave and tile: 16 NoPE + 2 RoPE copies (a branch may duplicate some)
    assert sum(t.startswith("global_load_lds_dwordx4") for t in loop) >= 18


@pytest.mark.parametrize("key", list(KERNELS))
def test_tile_loops_have_no_spill_or_flat_access(asm, key):
    loop, _ = innermost_loop(function_body(asm, KERNELS[key]))
    assert not [t for t in loop if t.startswith("scratch_")]
    assert not [t for t in loop if t.startswith("flat_")]


@pytest.mark.parametrize("key", list(KERNELS))
def test_inline_mfma_operands_are_not_fresh_valu_results(asm, key):
    ins = instructions(function_body(asm, KERNELS[key]))
    checked = 0
    for i, t in enumerate(ins):
        if not t.startswith("v_mfma_") or " v[" not in t.split(",")[0] + " ":
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        if not ops[0].startswith("v["):
            continue  # AGPR accumulators: compiler-scheduled MFMAs, padded by the compiler
        checked += 1
        srcs = set().union(*(vgprs(o) for o in ops[1:4]))
        slots = []
        k = i - 1
        while k >= 0 and len(slots) < 2:
            p = ins[k]
            if p.startswith("s_nop"):
                slots.extend(["nop"] * (int(p.split()[1], 0) + 1))
            else:
                slots.append(p)
            k -= 1
        for p in slots[:2]:
            if p.startswith("v_") and not p.startswith("v_mfma"):
                assert not (vgprs(p.split(None, 1)[1].split(",")[0].strip()) & srcs), (p, t)
    if key == (0, False):
        assert checked > 0


def test_lds_fits_one_workgroup_per_cu(asm):
    sizes = {}
    for name in KERNELS.values():
        body_start = next(i for i, l in enumerate(asm) if l.strip() == ".amdhsa_kernel " + name)
        for l in asm[body_start:body_start + 80]:
            if ".amdhsa_group_segment_fixed_size" in l:
                sizes[name] = int(l.split()[-1])
                break
    assert len(sizes) == len(KERNELS)
    assert all(0 < v <= 160 * 1024 for v in sizes.values()), sizes


def test_indexer_page_loop_waits_only_for_its_copies(asm_indexer):
    """Each score kernel's page loop (outermost loop) waits on vector memory
    only through its three explicit waits (two pages ahead, one, none), and
    no indexer kernel spills or touches memory through flat pointers in a
    loop."""
    for tg in (1, 2, 3, 4):
        body = function_body(asm_indexer, SCORE_KERNEL.format(tg))
        depth = loop_blocks(body)
        page_loop = instructions([l for l, d in zip(body, depth) if d == 1])
        counts = sorted(int(re.search(r"vmcnt\((\d+)\)", t).group(1)) for t in page_loop
                        if t.startswith("s_waitcnt") and "vmcnt" in t)
        assert counts == [0, 4, 8], (tg, counts)
        assert sum("row_ror" in t for t in page_loop) == 8 * tg  # 2 rows x 4 rotations per token
    for name in [SCORE_KERNEL.format(t) for t in (1, 2, 3, 4)] + [TOPK_KERNEL, QUERY_KERNEL]:
        b = function_body(asm_indexer, name)
        d = loop_blocks(b)
        in_loops = instructions([l for l, x in zip(b, d) if x >= 1])
        assert not [t for t in in_loops if t.startswith("scratch_") or t.startswith("flat_")], name
    # the selection kernel keeps no spill at all (its 64 keys per thread fill
    # the 128 registers a 1024-thread workgroup leaves each lane)
    topk = instructions(function_body(asm_indexer, TOPK_KERNEL))
    assert not [t for t in topk if t.startswith("scratch_")]


MFMA_THEN_VALU = r'''
#include <hip/hip_runtime.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ void probe(const bf16x8* a, const bf16x8* b, float* out) {
  f32x16 acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], b[threadIdx.x], acc, 0, 0, 0);
  out[threadIdx.x] = acc[0] * 3.0f + acc[5];
}
'''


def test_score_chain_drain_covers_the_mfma_to_valu_hazard(tmp_path_factory):
    """The hand-written score chains end with a drain of s_nop wait states
    before any VALU instruction touches the accumulator.  The compiler pads
    the same dependency (v_mfma_f32_32x32x16_bf16 result read by a VALU
    instruction) in code it can see; the drain must give at least as many
    wait states as that padding."""
    d = tmp_path_factory.mktemp("probe")
    src = str(d / "probe.hip")
    with open(src, "w") as f:
        f.write(MFMA_THEN_VALU)
    lines = [t for t in instructions(compile_asm(tmp_path_factory, src)) if t]
    i = next(k for k, t in enumerate(lines) if t.startswith("v_mfma_f32_32x32x16_bf16"))
    j = next(k for k in range(i + 1, len(lines)) if lines[k].startswith("v_") and "mfma" not in lines[k])
    needed = sum(int(re.match(r"s_nop\s+(\d+)", t).group(1)) + 1 for t in lines[i + 1:j]
                 if t.startswith("s_nop"))
    assert needed > 0
    with open(DECODE) as f:
        text = f.read()
    body = re.search(r"void mfma_s_drain\(f32x16& acc\) \{\s*asm volatile\(\"([^\"]*)\"", text).group(1)
    drain = sum(int(n) + 1 for n in re.findall(r"s_nop (\d+)", body))
    assert drain >= needed, (drain, needed)
