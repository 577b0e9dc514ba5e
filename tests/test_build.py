"""Host checks of the build's DPP hazard scan over generated assembly: a VALU
write of a VGPR read through DPP needs two wait states, a VALU write of EXEC
five; scalar EXEC writes are interlocked by the hardware."""
from volumetric_delay_sum_amd._build import scan_dpp_hazards

DPP = "v_fmac_f32_dpp v10, v1, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf"


def test_valu_write_then_dpp_read_is_flagged():
    asm = "\n".join(["v_mul_f32_e32 v1, v3, v4", DPP])
    assert scan_dpp_hazards(asm)


def test_two_wait_states_clear_the_vgpr_hazard():
    assert not scan_dpp_hazards("\n".join(["v_mul_f32_e32 v1, v3, v4", "s_nop 1", DPP]))
    assert not scan_dpp_hazards("\n".join(["v_mul_f32_e32 v1, v3, v4", "v_add_f32_e32 v7, v8, v9",
                                           "v_add_f32_e32 v5, v8, v9", DPP]))


def test_write_of_another_register_is_fine():
    assert not scan_dpp_hazards("\n".join(["v_mul_f32_e32 v2, v3, v4", DPP]))   # v2 is not the DPP source


def test_register_ranges_are_expanded():
    assert scan_dpp_hazards("\n".join(["v_mov_b64_e32 v[0:1], s[4:5]", DPP]))


def test_valu_exec_write_needs_five_wait_states():
    assert scan_dpp_hazards("\n".join(["v_cmpx_gt_u32_e32 vcc, 32, v0", "s_nop 2", DPP]))
    assert not scan_dpp_hazards("\n".join(["v_cmpx_gt_u32_e32 vcc, 32, v0", "s_nop 4", DPP]))


def test_scalar_exec_writes_are_interlocked():
    asm = "\n".join(["s_and_saveexec_b64 s[0:1], vcc", "s_cbranch_execz .LBB0_3", "s_or_b64 exec, exec, s[0:1]", DPP])
    assert not scan_dpp_hazards(asm)


def test_hazard_across_a_branch_is_found():
    # the write sits before a branch to the DPP's block
    asm = "\n".join(["v_mul_f32_e32 v1, v3, v4", "s_cbranch_scc1 .LBB0_4", "s_nop 4", "s_branch .LBB0_5",
                     ".LBB0_4:", DPP, ".LBB0_5:", "s_endpgm"])
    assert scan_dpp_hazards(asm)


def test_fall_through_predecessor_is_checked():
    assert scan_dpp_hazards("\n".join(["v_mul_f32_e32 v1, v3, v4", ".LBB0_4:", DPP]))
    assert not scan_dpp_hazards("\n".join(["v_mul_f32_e32 v1, v3, v4", "s_nop 1", ".LBB0_4:", DPP]))


def test_settled_predecessors_pass():
    asm = "\n".join(["v_mul_f32_e32 v1, v3, v4", "s_nop 1", "s_cbranch_scc1 .LBB0_4",
                     "buffer_load_dword v9, v8, s[0:3], 0 offen", ".LBB0_4:", DPP])
    assert not scan_dpp_hazards(asm)
