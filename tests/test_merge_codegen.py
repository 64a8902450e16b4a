"""The instruction-level facts the in-kernel merges rely on, checked on the
gfx950 code objects inside the built libfi_bsr.so (CPU only; the
disassembly is of this repository's own build): the decode kernels' merge
trees (vector and matrix kernels, one wave per item) and the merges of cut
tiles in the latent-attention kernel (four waves per item) and the prefill
tile kernel (eight): the same facts, with a barrier between the waves' waits
and the arrival, and between the arrival and the election.

A wave that finished a chunk of a cut request stores its partial state and
then counts its arrival at a merge node with a relaxed agent-scope atomic
add; the wave whose add returns the last count merges the node's children.
That this is correct across the XCDs' private L2 caches rests on four facts
of the generated code, for every decode kernel variant:

1. the arrival add is issued after an ``s_waitcnt vmcnt(0)`` with no vector
   memory instruction and no branch target between them, so every partial
   store of the wave (write-through ``sc1`` stores) has completed when the
   add is issued, whatever path led there;
2. after the add, the wave waits for its result (``vmcnt(0)``) before the
   branch that decides whether it merges, and issues no vector load before
   that branch: the merging wave cannot read a partial before its election;
3. every vector load after the add (the children's partial states) carries
   ``sc1``: it reads the device-coherent level, not a stale L2 line;
4. the partial stores carry ``sc1`` (write-through to that level).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_kv_bsr_amd", "libfi_bsr.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
# kernels whose merges follow the protocol: the decode kernels (one wave per
# item) and the latent-attention tile kernel (four waves per item)
DECODE = ("decode_bsr_kernel", "decode_mma_kernel")
KERNELS = DECODE + ("mla_attend_kernel", "tile_attend_kernel")


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} is not installed")
    return path


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    """{kernel symbol: [(address, mnemonic, operands)]} for every decode
    kernel variant in the library's gfx950 code objects."""
    if not os.path.exists(LIB):
        pytest.skip("libfi_bsr.so is not built")
    tmp = tmp_path_factory.mktemp("codegen")
    fat = str(tmp / "fatbin")
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", LIB, str(tmp / "x")],
                   check=True, capture_output=True)
    data = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
    text = []
    for i in range(len(starts) - 1):
        piece, co = str(tmp / f"b{i}"), str(tmp / f"b{i}.co")
        open(piece, "wb").write(data[starts[i]:starts[i + 1]])
        r = subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={piece}",
                            f"--output={co}"], capture_output=True)
        if r.returncode != 0 or not os.path.getsize(co):
            continue
        r = subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", co],
                           capture_output=True, text=True, check=True)
        text.append(r.stdout)
    funcs, cur = {}, None
    for ln in "\n".join(text).split("\n"):
        m = re.match(r"^([0-9a-f]+) <(.*)>:$", ln)
        if m:
            cur = funcs.setdefault(m.group(2), []) if any(k in m.group(2) for k in KERNELS) else None
            if cur is not None:
                cur.append(("start", int(m.group(1), 16)))
            continue
        if cur is None:
            continue
        m = re.match(r"^\s+(\S+)\s*(.*?)\s*// ([0-9A-F]+):", ln)
        if m:
            cur.append((int(m.group(3), 16), m.group(1), m.group(2)))
    out = {}
    for name, rows in funcs.items():
        start = rows[0][1]
        out[name] = (start, rows[1:])
    assert out, "no decode kernel found in the library's code objects"
    return out


@pytest.fixture(scope="module")
def decode_kernels(kernels):
    return {k: v for k, v in kernels.items() if any(d in k for d in DECODE)}


@pytest.fixture(scope="module")
def mla_kernel(kernels):
    found = [v for k, v in kernels.items() if "mla_attend_kernel" in k]
    assert len(found) == 1
    return found[0]


@pytest.fixture(scope="module")
def prefill_kernels(kernels):
    """{head_dim: [...]} of the prefill variants of the tile kernel (bf16
    d 128 and 64, fp8, rotary); the shared-prefix variants merge nothing."""
    out = {}
    for k, v in kernels.items():
        m = re.search(r"tile_attend_kernelILi(\d+)ELb1E", k)
        if m:
            out.setdefault(int(m.group(1)), []).append((k, v))
    return out


def _branch_targets(start, ins):
    tg = set()
    for _, mn, ops in ins:
        if mn.startswith("s_cbranch") or mn == "s_branch":
            m = re.search(r"\+0x([0-9a-f]+)>", ops)
            if m:
                tg.add(start + int(m.group(1), 16))
    return tg


def _is_vmem(mn):
    return mn.startswith(("global_", "buffer_", "flat_", "scratch_"))


def _arrival(ins):
    return next(k for k, x in enumerate(ins) if x[1].startswith("global_atomic_add"))


def check_arrival_after_wait(start, ins):
    """Fact 1; returns a complaint or None."""
    targets = _branch_targets(start, ins)
    i = _arrival(ins)
    j = i - 1
    while not (ins[j][1] == "s_waitcnt" and "vmcnt(0)" in ins[j][2]):
        if j == 0:
            return "no full wait before the arrival"
        if _is_vmem(ins[j][1]):
            return f"{ins[j][1]} between the wait and the arrival"
        j -= 1
    if any(ins[j][0] < a <= ins[i][0] for a in targets):
        return "a branch lands between the wait and the arrival"
    return None


def check_no_load_before_election(start, ins):
    """Fact 2."""
    i = _arrival(ins)
    dst = ins[i][2].split(",")[0].strip()
    waited = False
    for _, mn, ops in ins[i + 1:]:
        if mn == "s_waitcnt" and "vmcnt(0)" in ops:
            waited = True
        if mn == "v_readfirstlane_b32" and ops.split(",")[1].strip() == dst and not waited:
            return "the count is read before the wait"
        if mn.startswith(("global_load", "buffer_load", "flat_load")):
            return f"{mn} before the election branch"
        if mn in ("s_cbranch_vccnz", "s_cbranch_vccz", "s_cbranch_scc0", "s_cbranch_scc1"):
            return None if waited else "no wait for the count"
    return "no election branch"


def check_coherent_partials(start, ins):
    """Facts 3 and 4."""
    i = _arrival(ins)
    loads = [x for x in ins[i:] if x[1].startswith("global_load")]
    if not loads or not all(" sc1" in " " + x[2] for x in loads):
        return "a load after the arrival without sc1"
    if len([x for x in ins if x[1].startswith("global_store") and "sc1" in x[2]]) < 2:
        return "no write-through partial stores"
    return None


CHECKS = [check_arrival_after_wait, check_no_load_before_election, check_coherent_partials]


def test_every_variant_has_a_merge_arrival(decode_kernels):
    # vector kernel: dtype (fp32, bf16, fp8) x head_dim x group x streaming x
    # page-size path x RoPE; matrix kernel: fp8 / bf16 x group x streaming x RoPE
    assert sum("decode_bsr_kernel" in k for k in decode_kernels) >= 40
    assert sum("decode_mma_kernel" in k for k in decode_kernels) == 32
    for name, (_, ins) in decode_kernels.items():
        adds = [x for x in ins if x[1].startswith("global_atomic_add")]
        assert len(adds) == 1, name
        assert "sc0" in adds[0][2], name  # the add returns the count it replaced


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_fact_holds_in_every_variant(decode_kernels, check):
    for name, (start, ins) in decode_kernels.items():
        assert check(start, ins) is None, (name, check(start, ins))


def test_checks_catch_planted_reorderings(decode_kernels):
    """Each check flags the reordering it is there for, planted into a copy of
    a real kernel's instruction list."""
    name = sorted(decode_kernels)[0]
    start, ins = decode_kernels[name]
    i = _arrival(ins)
    addr = ins[i][0]
    store = (addr - 2, "global_store_dwordx2", "v[0:1], v[2:3], off sc1")
    assert check_arrival_after_wait(start, ins[:i] + [store] + ins[i:]) is not None
    w = next(k for k in range(i - 1, 0, -1) if ins[k][1] == "s_waitcnt" and "vmcnt(0)" in ins[k][2])
    assert check_arrival_after_wait(start, ins[:w] + ins[w + 1:]) is not None
    load = (addr + 2, "global_load_dwordx2", "v[0:1], v[2:3], off sc1")
    assert check_no_load_before_election(start, ins[:i + 1] + [load] + ins[i + 1:]) is not None
    j = next(k for k in range(i + 1, len(ins)) if ins[k][1].startswith("global_load"))
    stale = ins[:j] + [(ins[j][0], ins[j][1], ins[j][2].replace(" sc1", ""))] + ins[j + 1:]
    assert check_coherent_partials(start, stale) is not None


# ---- the latent-attention tile kernel: four waves per item. Every wave
# stores its part of the chunk's partial state (write-through) and waits for
# its stores; a barrier then orders all of them before the arrival that one
# thread issues; the count reaches the other waves through LDS behind a
# second barrier, and the merge's loads follow the branch on it.

def _vec_loads(ins):
    return [x for x in ins if x[1].startswith(("global_load", "buffer_load", "flat_load"))]


def check_mla_arrival(start, ins):
    """Fact 1 for a work-group: a full vmcnt wait, then a barrier, then the
    arrival, with no vector memory instruction and no branch target between
    the wait and the arrival."""
    targets = _branch_targets(start, ins)
    i = _arrival(ins)
    j = i - 1
    barrier = False
    while not (ins[j][1] == "s_waitcnt" and "vmcnt(0)" in ins[j][2]):
        if j == 0:
            return "no full wait before the arrival"
        if _is_vmem(ins[j][1]):
            return f"{ins[j][1]} between the wait and the arrival"
        barrier |= ins[j][1] == "s_barrier"
        j -= 1
    if not barrier:
        return "no barrier between the wait and the arrival"
    if any(ins[j][0] < a <= ins[i][0] for a in targets):
        return "a branch lands between the wait and the arrival"
    return None


def check_mla_election(start, ins):
    """Fact 2 for a work-group: the count is read after a vmcnt wait; a
    barrier follows, then the election branch; no vector load in between."""
    i = _arrival(ins)
    dst = ins[i][2].split(",")[0].strip()
    waited = barrier = False
    for _, mn, ops in ins[i + 1:]:
        if mn == "s_waitcnt" and "vmcnt(0)" in ops:
            waited = True
        if mn == "v_readfirstlane_b32" and ops.split(",")[1].strip() == dst and not waited:
            return "the count is read before the wait"
        if mn.startswith(("global_load", "buffer_load", "flat_load")):
            return f"{mn} before the election branch"
        if mn == "s_barrier":
            if not waited:
                return "the barrier comes before the wait for the count"
            barrier = True
        if barrier and mn.startswith("s_cbranch"):
            return None
    return "no election branch"


def check_mla_coherent(start, ins, runs=32):
    """Facts 3 and 4: the merge's loads and the partial stores use sc1 (a
    lane stores its part of the state as `runs` float pairs: 32 for the
    latent kernel's 16 x 256 floats per wave and the prefill tile's 32 x 128,
    16 for 32 x 64)."""
    i = _arrival(ins)
    loads = _vec_loads(ins[i:])
    if not loads or not all(" sc1" in " " + x[2] for x in loads):
        return "a load after the arrival without sc1"
    stores = [x for x in ins[:i] if x[1].startswith("global_store") and "sc1" in x[2]]
    if len(stores) < runs:
        return "no write-through partial stores"
    return None


MLA_CHECKS = [check_mla_arrival, check_mla_election, check_mla_coherent]


def test_mla_kernel_has_one_arrival(mla_kernel):
    _, ins = mla_kernel
    adds = [x for x in ins if x[1].startswith("global_atomic_add")]
    assert len(adds) == 1 and "sc0" in adds[0][2]
    # the merge reads through buffer resources, two passes of four chunks x 16 runs
    assert len([x for x in _vec_loads(ins) if x[1].startswith("buffer_load")]) >= 64


@pytest.mark.parametrize("check", MLA_CHECKS, ids=lambda f: f.__name__)
def test_mla_fact_holds(mla_kernel, check):
    start, ins = mla_kernel
    assert check(start, ins) is None, check(start, ins)


def test_mla_checks_catch_planted_reorderings(mla_kernel):
    start, ins = mla_kernel
    i = _arrival(ins)
    addr = ins[i][0]
    # a store moved between the wait and the arrival
    store = (addr - 2, "global_store_dwordx2", "v[0:1], v[2:3], off sc1")
    assert check_mla_arrival(start, ins[:i] + [store] + ins[i:]) is not None
    # the barrier taken out
    b = max(k for k in range(i) if ins[k][1] == "s_barrier")
    assert check_mla_arrival(start, ins[:b] + ins[b + 1:]) is not None
    # a load hoisted above the election
    load = (addr + 2, "buffer_load_dwordx2", "v[0:1], v2, s[0:3], 0 offen sc1")
    assert check_mla_election(start, ins[:i + 1] + [load] + ins[i + 1:]) is not None
    # a merge load without sc1
    j = next(k for k in range(i + 1, len(ins)) if ins[k][1].startswith("buffer_load"))
    stale = ins[:j] + [(ins[j][0], ins[j][1], ins[j][2].replace(" sc1", ""))] + ins[j + 1:]
    assert check_mla_coherent(start, stale) is not None


# ---- the prefill / append tile kernel merges its cut tiles the same way
# (eight waves per item; in the rotary variant four of them hand their state
# to the other four and stay, idle, for the barriers).

def test_prefill_variants_have_one_arrival(prefill_kernels):
    assert sorted(prefill_kernels) == [64, 128] and len(prefill_kernels[128]) == 3
    for d, ks in prefill_kernels.items():
        for name, (_, ins) in ks:
            adds = [x for x in ins if x[1].startswith("global_atomic_add")]
            assert len(adds) == 1 and "sc0" in adds[0][2], name
            assert len([x for x in _vec_loads(ins) if x[1].startswith("buffer_load")]) >= d // 4, name


@pytest.mark.parametrize("check", MLA_CHECKS, ids=lambda f: f.__name__)
def test_prefill_fact_holds(prefill_kernels, check):
    for d, ks in prefill_kernels.items():
        for name, (start, ins) in ks:
            got = check(start, ins, runs=d // 4) if check is check_mla_coherent else check(start, ins)
            assert got is None, (name, got)
