"""The wait-state checker used by the build flags the hazards it is meant to
catch around MFMAs the compiler cannot see, and accepts correctly spaced code."""
import pytest

from mla_latent_decode_absorbed_amd.isa_check import check_asm, check_function

pytestmark = pytest.mark.cpu


def run(src: str):
    return check_function(src.strip().splitlines(), "k")


def test_valu_write_then_mfma_read_needs_two_wait_states():
    bad = run("""
        v_mov_b32_e32 v3, v40
        v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
    """)
    assert len(bad) == 1 and "VALU write" in bad[0]
    assert run("""
        v_mov_b32_e32 v3, v40
        s_nop 1
        v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
    """) == []
    # an unrelated VALU write right before the MFMA is fine
    assert run("""
        v_mov_b32_e32 v30, v40
        v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
    """) == []


def test_accvgpr_write_then_mfma_accumulator_read():
    bad = run("""
        v_accvgpr_write_b32 a7, v1
        v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
    """)
    assert len(bad) == 1


def test_mfma_result_read_by_valu_needs_the_opcodes_wait_states():
    """12 wait states after the 8-pass bf16 MFMA, 20 after the 16-pass f8f6f4
    one (the counts the compiler inserts after its own MFMAs on gfx950)."""
    bad = run("""
        v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0
        s_nop 7
        s_nop 2
        v_add_f32_e32 v1, v10, v11
    """)
    assert len(bad) == 1 and "MFMA" in bad[0]
    bad = run("""
        v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
        s_nop 7
        v_accvgpr_read_b32 v1, a3
    """)
    assert len(bad) == 1
    assert run("""
        v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0
        s_nop 7
        s_nop 3
        v_add_f32_e32 v1, v10, v11
    """) == []
    # the f8f6f4 MFMA: 12 (or 19) wait states are not enough, 20 are
    for nops in ("s_nop 7\n s_nop 3", "s_nop 7\n s_nop 7\n s_nop 2"):
        bad = run(f"""
            v_mfma_f32_32x32x64_f8f6f4 v[10:25], v[30:37], v[40:47], 0
            {nops}
            v_add_f32_e32 v1, v10, v11
        """)
        assert len(bad) == 1 and "MFMA" in bad[0], nops
    assert run("""
        v_mfma_f32_32x32x64_f8f6f4 v[10:25], v[30:37], v[40:47], 0
        s_nop 7
        s_nop 7
        s_nop 3
        v_add_f32_e32 v1, v10, v11
    """) == []
    # a VALU write of the result counts like a read
    bad = run("""
        v_mfma_f32_32x32x16_bf16 v[10:25], v[2:5], v[6:9], 0
        s_nop 7
        v_mov_b32_e32 v12, 0
    """)
    assert len(bad) == 1 and "overwrites" in bad[0]


def test_every_kernel_of_a_listing_is_checked():
    """check_asm scans every kernel the listing declares, also one whose name
    extends another's, and reports the one with the hazard."""
    listing = """
_Z6decodev:
        v_mov_b32_e32 v30, v40
        v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
        s_endpgm
_Z9decode_abv:
        v_and_b32_e32 v6, 0x7f7f7f7f, v6
        v_mfma_f32_32x32x64_f8f6f4 v[10:25], v[2:9], v[6:13], v[10:25]
        s_endpgm
        .amdhsa_kernel _Z6decodev
        .end_amdhsa_kernel
        .amdhsa_kernel _Z9decode_abv
        .end_amdhsa_kernel
"""
    bad = check_asm(listing)
    assert len(bad) == 1 and bad[0].startswith("_Z9decode_abv") and "VALU write" in bad[0]
    assert check_asm(listing, kernels=("_Z6decodev",)) == []
