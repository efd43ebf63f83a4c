"""Static checks of the gfx950 machine code that build() produced (the
disassembly of the library's own objects; no GPU): the GEMMs' load ring and
the cross-entropy's row loads.

The 16-bit GEMMs fill an LDS ring with buffer-to-LDS loads several stages
ahead and order their LDS reads against those loads themselves (each wave
waits for its own loads of a stage, then the block barrier).  The compiler
inserts a wait for every in-flight load (s_waitcnt vmcnt(0)) before an LDS
read that it cannot tell apart from the loads' LDS writes, as it did for
the transpose reads of the weight-gradient and dX kernels: that cuts the
ring to depth one and exposes a memory latency at every stage, and nothing
but the machine code shows it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decoder_only_transformer_02_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def _disassemble(src, d):
    """gfx950 disassembly of the device code in _build/<src>.o."""
    tools = [_tool(n) for n in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(tools):
        pytest.skip("ROCm LLVM tools not found")
    obj = os.path.join(ROOT, "_build", src.replace(".hip", ".o"))
    if not os.path.exists(obj):
        pytest.skip("no build: run __graft_entry__.build() first")
    newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
    if os.path.getmtime(obj) < newest:
        pytest.skip("the build is older than the sources: run __graft_entry__.build() again")
    objcopy, bundler, objdump = tools
    fat, co = str(d / (src + ".fatbin")), str(d / (src + ".co"))
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", obj], check=True)
    subprocess.run([bundler, "--unbundle", "--type=o", f"--input={fat}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True)
    r = subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True, capture_output=True, text=True)
    return r.stdout


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    return _disassemble("gemm.hip", tmp_path_factory.mktemp("gemm_isa"))


@pytest.fixture(scope="module")
def disassembly_attention(tmp_path_factory):
    return _disassemble("attention.hip", tmp_path_factory.mktemp("attention_isa"))


@pytest.fixture(scope="module")
def disassembly_elementwise(tmp_path_factory):
    return _disassemble("elementwise.hip", tmp_path_factory.mktemp("elementwise_isa"))


def kernels(text):
    """Kernel symbol -> its instructions (mnemonic and operands, without the
    address and encoding comment)."""
    out, cur = {}, None
    for line in text.split("\n"):
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            cur = out.setdefault(m.group(1), [])
            continue
        t = line.split("//")[0].strip()
        if cur is not None and t:
            cur.append(t)
    return out


def ring_drains(instrs):
    """Places where a full vector-memory wait directly precedes an LDS read
    (s_nop padding ignored)."""
    n, prev = 0, None
    for t in instrs:
        if t.startswith("s_nop"):
            continue
        if prev is not None and re.match(r"s_waitcnt\b.*\bvmcnt\(0\)", prev) and t.startswith("ds_read"):
            n += 1
        prev = t
    return n


def test_disassembly_has_the_ring_gemms(disassembly):
    ks = kernels(disassembly)
    tn = [k for k in ks if "k_gemm_tn" in k]
    bkn = [k for k in ks if "k_gemm_nt" in k and k.endswith("ELb1EEEvNS_2GPE")]
    assert len(tn) >= 3 and len(bkn) >= 6, (len(tn), len(bkn))


def test_no_load_ring_drain_before_lds_reads(disassembly):
    ks = kernels(disassembly)
    bad = {k: ring_drains(v) for k, v in ks.items() if re.search(r"k_gemm_(nt|tn)I", k)}
    bad = {k: n for k, n in bad.items() if n}
    assert not bad, bad


def test_the_check_sees_a_drain():
    """The detector itself, on the instruction pattern the compiler had
    emitted before the transpose reads carried alias-scope information."""
    assert ring_drains(["buffer_load_dwordx4 v1, s[4:7], 0 offen lds", "s_waitcnt vmcnt(0)",
                        "ds_read_b64_tr_b16 v[2:3], v4"]) == 1
    assert ring_drains(["s_waitcnt vmcnt(4)", "ds_read_b128 v[0:3], v4"]) == 0
    assert ring_drains(["s_waitcnt vmcnt(0)", "s_nop 0", "ds_read_b128 v[0:3], v4"]) == 1
    assert ring_drains(["s_waitcnt lgkmcnt(0)", "ds_read_b128 v[0:3], v4"]) == 0


def serialized_loads(instrs):
    """Global loads that wait for every earlier load (s_waitcnt vmcnt(0))
    with no other load between: the pattern of loads issued one at a time."""
    seq = []
    for t in instrs:
        if t.startswith("global_load") or (t.startswith("buffer_load") and " lds" not in t):
            seq.append("G")
        elif re.match(r"s_waitcnt\b.*\bvmcnt\(0\)", t):
            seq.append("W")
    s = "".join(seq)
    return sum(1 for i in range(len(s) - 2) if s[i:i + 3] == "GWG")


def test_cross_entropy_row_loads_are_in_flight_together(disassembly_elementwise):
    """The register-resident cross-entropy loads its whole row (up to 25
    chunks of 16 bytes per thread) before it waits.  With the loads under
    per-chunk branches, the compiler had issued them one at a time (a
    register copy at each branch join waited for the load), 25 memory
    latencies per row."""
    ks = kernels(disassembly_elementwise)
    xent = {k: v for k, v in ks.items() if re.search(r"k_xentI.*Li(2|4|8|16|25)E", k)}
    assert len(xent) >= 15, len(xent)
    bad = {k: serialized_loads(v) for k, v in xent.items()}
    # a prologue load or two (target id, loss scale) may wait; the row's
    # loads one at a time gave one per chunk (4 to 25 here)
    bad = {k: n for k, n in bad.items() if n > 2}
    assert not bad, bad


def test_the_serialization_check_sees_one():
    assert serialized_loads(["global_load_dwordx4 v[0:3], v8, s[2:3]", "s_waitcnt vmcnt(0)",
                             "v_mov_b32 v4, v0", "global_load_dwordx4 v[0:3], v9, s[2:3]",
                             "s_waitcnt vmcnt(0)", "global_load_dwordx4 v[0:3], v10, s[2:3]"]) == 2
    assert serialized_loads(["global_load_dwordx4 v[0:3], v8, s[2:3]",
                             "global_load_dwordx4 v[4:7], v9, s[2:3]", "s_waitcnt vmcnt(1)",
                             "s_waitcnt vmcnt(0)"]) == 0


def longest_store_run(instrs):
    """The longest run of global stores with no full vector-memory wait
    (vmcnt(0)) between them: a wait with a nonzero count leaves the later
    stores and loads in flight, a full one drains every earlier store."""
    best = run = 0
    for t in instrs:
        if t.startswith("global_store"):
            run += 1
            best = max(best, run)
        elif re.match(r"s_waitcnt\b.*\bvmcnt\(0\)", t):
            run = 0
    return best


@pytest.mark.parametrize("epi", [0, 2, 3, 4])
def test_epilogues_stream_their_stores(disassembly, epi):
    """The whole-tile epilogues (plain store with bias, GELU, residual,
    gelu'; the 256x192 and 256x256 tiles) have a body that issues all of a
    lane's stores with no full wait between them: the bias comes from LDS,
    the residual is already in the accumulators, and gelu' prefetches its u
    values several groups ahead.  Each bias, residual or u load had been
    waited for with vmcnt(0), which also drained every store issued before
    it (one to eight stores per wait)."""
    ks = kernels(disassembly)
    for tile, per_lane in (("Li256ELi192ELi2ELi2E", 48), ("Li256ELi256ELi4ELi2E", 32)):
        name = [k for k in ks if re.search(rf"k_gemm_ntIDF16b{tile}Li{epi}ELb0E", k)]
        assert len(name) == 1, (tile, epi)
        want = per_lane * (2 if epi == 2 else 1)   # GELU writes u and gelu(u)
        got = longest_store_run(ks[name[0]])
        assert got >= want, (name[0], got, want)


def test_the_store_run_check():
    assert longest_store_run(["global_store_dwordx2 v[0:1], v[2:3], off", "s_waitcnt vmcnt(0)",
                              "global_load_dwordx4 v[4:7], v[0:1], off", "global_store_dwordx2 v[0:1], v[2:3], off",
                              "global_store_dwordx2 v[0:1], v[2:3], off"]) == 2
    assert longest_store_run(["global_store_dwordx2 v[0:1], v[2:3], off", "s_waitcnt vmcnt(9)",
                              "global_store_dwordx2 v[0:1], v[2:3], off"]) == 2


def reads_ahead(instrs):
    """The most 16-byte LDS reads issued in a row before the next MFMA."""
    best = run = 0
    for t in instrs:
        if t.startswith("ds_read_b128"):
            run += 1
            best = max(best, run)
        elif t.startswith("v_mfma"):
            run = 0
    return best


@pytest.mark.parametrize("kernel,ahead", [("k_attn_fwd64", 8), ("k_attn_dkv64", 8), ("k_attn_dq64", 4)])
def test_attention_score_reads_run_ahead(disassembly_attention, kernel, ahead):
    """The score phase (S = K Q^T, and dP in the backward) reads its key or
    query fragments ahead of the MFMAs that use them: all eight in the
    forward and dK/dV, two k steps (four reads) in dQ, which would lose its
    third wave per SIMD otherwise.  The compiler had issued the forward's
    reads at most two ahead of their MFMAs and dK/dV's at most six.  (For
    dQ this bound does not separate the versions: its first four reads
    were already issued together; the change is that later reads stay two
    steps ahead instead of one.)"""
    ks = kernels(disassembly_attention)
    names = [k for k in ks if kernel in k and "IDF16" in k]
    assert names, kernel
    for k in names:
        assert reads_ahead(ks[k]) >= ahead, (k, reads_ahead(ks[k]))
