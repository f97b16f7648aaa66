"""The bf16 kernels' inline-assembly LDS reads are consumed only after their wait: the
compiled gfx950 assembly is checked statically (no GPU needed, hipcc cross-compiles)."""
import pytest

from orthogonalized_momentum_optimizer_amd import asm_check, build

KERNEL_SOURCES = ["ns_apply_bf16.hip", "ns_gemm_bf16.hip", "ns_sym256_bf16.hip"]


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
