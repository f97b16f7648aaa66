"""The bf16 kernels' inline-assembly LDS reads are consumed only after their wait: the
compiled gfx950 assembly is checked statically (no GPU needed, hipcc cross-compiles)."""
import pytest

import asm_check
from orthogonalized_momentum_optimizer_amd import build

KERNEL_SOURCES = ["ns_apply_bf16.hip", "ns_gemm_bf16.hip", "ns_sym256_bf16.hip", "ns_quad_bf16.hip",
                  "ns_fused_bf16.hip"]


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_use_of_lds_read_results_before_their_wait(src):
    try:
        path = build.device_asm(src)
    except RuntimeError as e:  # no HIP toolchain on this host
        pytest.skip(str(e))
    text = open(path).read()
    assert "v_mfma" in text
    v = asm_check.violations(text)
    assert not v, "\n".join(v[:10])


def test_checker_flags_a_premature_copy():
    text = "\n".join([
        "ds_read_b128 v[4:7], v0 offset:0",
        "v_mov_b64_e32 v[20:21], v[4:5]",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b64_e32 v[22:23], v[6:7]",
    ])
    v = asm_check.violations(text)
    assert len(v) == 1 and "v[20:21]" in v[0]


def test_checker_honours_partial_waits():
    text = "\n".join([
        "ds_read_b128 v[4:7], v0",
        "ds_read_b128 v[8:11], v1",
        "s_waitcnt lgkmcnt(1)",
        "v_mov_b32_e32 v20, v4",    # first read complete: fine
        "v_mov_b32_e32 v21, v8",    # second still pending: flagged
    ])
    v = asm_check.violations(text)
    assert len(v) == 1 and "v21" in v[0]


def test_checker_follows_a_read_across_a_branch_join():
    """A read issued before a conditional branch is still pending where the paths join: a
    copy there, before the wait, is flagged (a checker that forgets pending reads at labels
    would miss it)."""
    text = "\n".join([
        "ds_read_b128 v[4:7], v0 offset:0",
        "s_cbranch_scc1 .LBB0_2",
        "v_mov_b32_e32 v9, v1",
        ".LBB0_2:",
        "v_mov_b32_e32 v20, v4",
        "s_waitcnt lgkmcnt(0)",
        "s_endpgm",
    ])
    v = asm_check.violations(text)
    assert len(v) == 1 and "v20, v4" in v[0]


def test_checker_flags_a_read_issued_on_one_path_only():
    """The shape of the bug once found in a kernel: a transposing read issued on one path
    only, its result copied at the join before the wait."""
    text = "\n".join([
        "s_cbranch_scc0 .LBB0_3",
        "ds_read_b64_tr_b16 v[8:9], v2",
        ".LBB0_3:",
        "v_mov_b32_e32 v30, v8",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32_e32 v31, v9",
        "s_endpgm",
    ])
    v = asm_check.violations(text)
    assert len(v) == 1 and "v30, v8" in v[0]


def test_checker_flags_a_wait_taken_on_one_path_only():
    text = "\n".join([
        "ds_read_b128 v[4:7], v0",
        "s_cbranch_scc1 .LBB0_2",
        "s_waitcnt lgkmcnt(0)",
        ".LBB0_2:",
        "v_add_f32_e32 v20, v4, v5",
        "s_endpgm",
    ])
    assert len(asm_check.violations(text)) == 1


def test_checker_follows_a_loop_back_edge():
    """A read issued at the end of a loop body reaches the top of the loop pending."""
    text = "\n".join([
        "ds_read_b128 v[4:7], v0",
        "s_waitcnt lgkmcnt(0)",
        ".LBB0_1:",
        "v_mov_b32_e32 v20, v4",
        "ds_read_b128 v[4:7], v0 offset:64",
        "s_cbranch_scc1 .LBB0_1",
        "s_waitcnt lgkmcnt(0)",
        "s_endpgm",
    ])
    v = asm_check.violations(text)
    assert len(v) >= 1 and "v20, v4" in v[0]


def test_checker_accepts_waits_on_every_path():
    text = "\n".join([
        "ds_read_b128 v[4:7], v0",
        "s_cbranch_scc1 .LBB0_2",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32_e32 v9, v4",
        "s_branch .LBB0_3",
        ".LBB0_2:",
        "ds_read_b128 v[12:15], v1",
        "s_waitcnt lgkmcnt(1)",
        ".LBB0_3:",
        "v_mov_b32_e32 v20, v4",
        "s_waitcnt lgkmcnt(0)",
        "v_mov_b32_e32 v21, v12",
        "s_endpgm",
    ])
    assert asm_check.violations(text) == []


def test_checker_completes_scalar_loads_only_at_zero():
    """Scalar loads may complete out of order: a partial wait does not cover them."""
    text = "\n".join([
        "s_load_dword s4, s[0:1], 0x0",
        "ds_read_b32 v4, v0",
        "s_waitcnt lgkmcnt(1)",
        "s_mov_b32 s5, s4",
        "s_waitcnt lgkmcnt(0)",
        "s_mov_b32 s6, s4",
        "s_endpgm",
    ])
    v = asm_check.violations(text)
    assert len(v) == 1 and "s5, s4" in v[0]


def _vm_sequence(func_text):
    """Vector-memory loads and vmcnt waits of one function, in program order: 'L' a
    direct-to-LDS load, 'P' an 8-byte global load, ('W', n) a wait for vmcnt <= n."""
    import re
    seq = []
    for ln in func_text.splitlines():
        t = ln.strip()
        if t.startswith("global_load_lds"):
            seq.append("L")
        elif t.startswith("global_load_dwordx2"):
            seq.append("P")
        elif t.startswith("s_waitcnt") and "vmcnt" in t:
            seq.append(("W", int(re.search(r"vmcnt\((\d+)\)", t).group(1))))
    return seq


def test_poly_b_a_loads_match_the_tail_waits():
    """The 128-tile polynomial kernel issues its 16 loads of the b A term right after the last
    refill and its three tail stages wait with those 16 still pending: the compiled code must
    hold exactly 16 such loads behind the refill's direct loads, followed by the waits
    2k + 16, k + 16, 16 (k = direct loads per wave per stage: 4, or 2 on a diagonal tile)."""
    import re
    try:
        path = build.device_asm("ns_gemm_bf16.hip")
    except RuntimeError as e:
        pytest.skip(str(e))
    text = open(path).read()
    funcs = re.split(r"\n(?=_Z\S+: ; @)", text)
    poly = [f for f in funcs if f.startswith("_ZN4muon12_GLOBAL__N_111ns_sym_bf16ILi1")]
    assert len(poly) == 2, [f.split(":")[0] for f in poly]   # single- and multi-group
    for f in poly:
        seq = _vm_sequence(f)
        runs = [i for i in range(len(seq)) if seq[i] == "P" and (i == 0 or seq[i - 1] != "P")]
        assert len(runs) == 2, "one run of b A loads per tile kind (diagonal, off-diagonal)"
        ks = []
        for i in runs:
            n = 0
            while seq[i + n] == "P":
                n += 1
            assert n == 16, n
            k = 0
            while seq[i - 1 - k] == "L":
                k += 1
            waits = [x[1] for x in seq[i + n:i + n + 3]]
            assert all(isinstance(x, tuple) for x in seq[i + n:i + n + 3]), seq[i + n:i + n + 3]
            assert waits == [2 * k + 16, k + 16, 16], (k, waits)
            ks.append(k)
        assert sorted(ks) == [2, 4], ks
    # the Gram kernels load no b A term
    gram = [f for f in funcs if f.startswith("_ZN4muon12_GLOBAL__N_111ns_sym_bf16ILi0")]
    assert gram and all("P" not in _vm_sequence(f) for f in gram)


def test_apply_tile_start_waits_count_the_previous_stores():
    """The persistent apply kernels prefetch a tile's first four stages before the previous
    tile's epilogue stores its output (32 stores per wave, 16 when the tile's right half lies
    outside the matrix, none when the wave's rows do). The vector-memory counter completes in
    issue order, so the wait for the new tile's first stage leaves 3 stages of loads plus
    those stores pending: the compiled kernels must hold the three variants 24, 40 and 56,
    with 32 conditional stores and the 32-load prefetch before them."""
    import re
    try:
        path = build.device_asm("ns_apply_bf16.hip")
    except RuntimeError as e:
        pytest.skip(str(e))
    text = open(path).read()
    funcs = re.split(r"\n(?=_Z\S+: ; @)", text)
    persistent = [f for f in funcs if re.match(r"_ZN4muon12_GLOBAL__N_1\d+ns_apply_bf16", f)]
    assert len(persistent) == 4, [f.split(":")[0] for f in persistent]
    for f in persistent:
        waits = [int(x) for x in re.findall(r"s_waitcnt[^\n]*vmcnt\((\d+)\)", f)]
        assert {24, 40, 56} <= set(waits) and max(waits) == 56, sorted(set(waits))
        assert len(re.findall(r"\n\s*global_store_dwordx4", f)) == 32
        body = "\n".join(ln.strip() for ln in f.splitlines())
        last_prefetch = body.rfind("global_load_lds")
        assert last_prefetch < body.find("global_store_dwordx4")


def test_apply_kernels_use_no_scratch_and_defer_their_stores():
    """Every apply kernel keeps its values in registers (no scratch: a spill would add vector-
    memory operations that the counted waits do not expect). The kernels that hold stores back
    issue 8 at a tile's end, 2 in each of the next tile's first 12 iterations and the held 24
    after the block's last tile: 56 store instructions, each behind its own condition."""
    import re
    try:
        path = build.device_asm("ns_apply_bf16.hip")
    except RuntimeError as e:
        pytest.skip(str(e))
    text = open(path).read()
    meta = dict(zip(re.findall(r"\.name:\s+(_Z\S+)", text),
                    re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)))
    assert meta and all(v == "0" for v in meta.values()), meta
    funcs = re.split(r"\n(?=_Z\S+: ; @)", text)
    defer = [f for f in funcs if re.match(r"_ZN4muon12_GLOBAL__N_1\d+ns_apply_defer_bf16", f)]
    assert len(defer) == 2
    for f in defer:
        assert len(re.findall(r"\n\s*global_store_dwordx4", f)) == 8 + 12 * 2 + 24
        assert "v_accvgpr_write" not in f     # the first K step starts from a zero operand
