"""Host-side build logic: the resource-report parser that rejects kernels using scratch."""
from weight_only_quantized_mpgemm_amd import build

REPORT = """\
k.hip:27:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
k.hip:27:1: remark:     VGPRs: 27 [-Rpass-analysis=kernel-resource-usage]
k.hip:27:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.hip:43:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]
k.hip:43:1: remark:     ScratchSize [bytes/lane]: 488 [-Rpass-analysis=kernel-resource-usage]
k.hip:60:1: remark: Function Name: _Z3bazPf [-Rpass-analysis=kernel-resource-usage]
k.hip:60:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_scratch_users_names_only_spilling_kernels():
    assert build.scratch_users(REPORT) == [("_Z3barPf", 488)]


def test_scratch_users_empty_report():
    assert build.scratch_users("") == []


ASM = """\
    .text
_Z6kernelPf:                            ; @_Z6kernelPf
; %bb.0:
	v_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]
	v_mfma_f32_32x32x16_f16 a[16:31], v[0:3], v[4:7], a[16:31]
	v_accvgpr_read_b32 v8, a3
	s_endpgm
.Lfunc_end0:
_Z7kernel2Pf:                           ; @_Z7kernel2Pf
; %bb.0:
	v_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]
	s_nop 7
	s_nop 7
	s_nop 7
	s_nop 7
	v_accvgpr_read_b32 v8, a3
	v_accvgpr_read_b32 v9, a40
	s_endpgm
.Lfunc_end1:
"""


def test_acc_read_hazards_flags_early_reads_only():
    # kernel 1 reads a3 one instruction after the MFMA that writes a[0:15]; kernel 2 waits
    # 32 states (and its read of a40 belongs to no MFMA)
    assert build.acc_read_hazards(ASM) == [("_Z6kernelPf", 1)]


def _ring_path(wait_imm_stage0):
    """Prologue: DMA stages 0, 1, 2 (two loads each), two weight loads, barrier; then a
    stage barrier whose wait is given, needing stage 1."""
    dma = "buffer_load_dwordx4 v1, s[0:3], s4 offen lds"
    w = "buffer_load_dwordx4 v[2:5], v6, s[8:11], s4 offen"
    return ([dma, dma, dma, dma, dma, dma, w, w, "s_waitcnt vmcnt(4)", "s_barrier",
             f"s_waitcnt vmcnt({wait_imm_stage0})", "s_barrier"])


def test_stage_wait_check_accepts_waits_that_leave_only_later_loads():
    # after stage 1's last part: stage 2 (2 loads) and two weight loads are in flight
    assert build.stage_wait_violations(_ring_path(2), 2) == []
    assert build.stage_wait_violations(_ring_path(4), 2) == []


def test_stage_wait_check_flags_a_wait_that_can_pass_early():
    # vmcnt(5) would let stage 1's last DMA part still be in flight
    assert build.stage_wait_violations(_ring_path(5), 2) == [(1, 4, 5)]


def test_stage_wait_check_flags_a_stage_never_issued():
    seq = ["buffer_load_dwordx4 v1, s[0:3], s4 offen lds", "s_waitcnt vmcnt(0)", "s_barrier"]
    assert build.stage_wait_violations(seq, 2) == [(0, -1, 0)]


def _kernel_asm(tail_wait):
    """A ring kernel's skeleton as the compiler lays it out: prologue (three 2-load DMA
    stages, barrier), a branch over the loop, the loop body (four stages), the branch over
    the four-stage tail, the tail, and the block that skips the loop."""
    dma = "\tbuffer_load_dwordx4 v1, s[0:3], s4 offen lds"
    w = "\tbuffer_load_dwordx4 v[2:5], v6, s[8:11], s4 offen"

    def stage(wait):
        return [f"\ts_waitcnt vmcnt({wait})", "\ts_barrier", dma, dma, w]
    lines = ["_Z18prefill_x32_kernelv:", dma, dma, dma, dma, dma, dma, w,
             "\ts_waitcnt vmcnt(4)", "\ts_barrier", "\ts_cbranch_scc1 .LBB0_9", ".LBB0_2:"]
    for _ in range(4):
        lines += stage(2)
    lines += ["\ts_cbranch_scc1 .LBB0_2", "\ts_cbranch_scc1 .LBB0_7", ".LBB0_6:"]
    for _ in range(4):
        lines += stage(tail_wait)
    lines += [".LBB0_7:", "\ts_endpgm", ".LBB0_9:", "\ts_mov_b32 s5, 0",
              "\ts_cbranch_scc0 .LBB0_6", "\ts_branch .LBB0_7", ".Lfunc_end0:", ""]
    return "\n" + "\n".join(lines)


def _mangled(nws, sh, ma):
    """A tiled kernel's name with template arguments <ACT, SYM, G, NWS, SH, CODE, RAG, MA>."""
    return (f"_ZN6mpgemm12_GLOBAL__N_118prefill_x32_kernelILi0ELb0ELi128ELi{nws}ELi{sh}"
            f"ELi0ELb0ELi{ma}EEEvPKt")


def test_ring_shape_follows_the_template_arguments():
    # one row of tiles with fewer live row blocks than the tile, four weight sets: eight
    # stages holding the live rows; otherwise four stages of the whole tile
    assert build.ring_shape(_mangled(4, 1, 2)) == (8, 2)
    assert build.ring_shape(_mangled(4, 1, 4)) == (8, 4)
    assert build.ring_shape(_mangled(4, 2, 2)) == (8, 2)
    assert build.ring_shape(_mangled(4, 1, 8)) == (4, 8)
    assert build.ring_shape(_mangled(4, 2, 4)) == (4, 4)
    assert build.ring_shape(_mangled(4, 3, 8)) == (4, 8)
    assert build.ring_shape(_mangled(2, 1, 2)) == (4, 8)
    assert build.ring_shape(_mangled(2, 2, 2)) == (4, 4)
    assert build.ring_shape("_Z18prefill_x32_kernelv") == (4, None)


def _deep_kernel_asm(stage_waits):
    """An eight-stage ring kernel's skeleton (two DMA loads per stage, four weight loads in
    the even stages): prologue of seven DMA stages, then one pass of eight stages whose
    waits are given, then the end of the kernel."""
    dma = "\tbuffer_load_dwordx4 v1, s[0:3], s4 offen lds"
    w = "\tbuffer_load_dwordx4 v[2:5], v6, s[8:11], s4 offen"
    lines = ["_ZN6mpgemm12_GLOBAL__N_118prefill_x32_kernelILi0ELb0ELi128ELi4ELi1ELi0ELb0ELi2EEEv:"]
    lines += [dma] * 14 + [w] * 4 + ["\ts_waitcnt vmcnt(12)", "\ts_barrier",
                                     "\ts_cbranch_scc1 .LBB0_9", ".LBB0_2:"]
    for k, wait in enumerate(stage_waits):
        lines += [f"\ts_waitcnt vmcnt({wait})", "\ts_barrier", dma, dma]
        if k % 2 == 0:
            lines += [w] * 4
    lines += ["\ts_cbranch_scc1 .LBB0_2", "\ts_cbranch_scc1 .LBB0_7", ".LBB0_6:",
              "\ts_nop 0", ".LBB0_7:", "\ts_endpgm", ".LBB0_9:", "\ts_mov_b32 s5, 0",
              "\ts_branch .LBB0_7", ".Lfunc_end0:", ""]
    return "\n" + "\n".join(lines)


def test_ring_wait_check_counts_weight_loads_behind_the_dma_of_an_eight_stage_ring():
    # stage k (of a pass) needs the DMA issued six stages earlier, in stage k - 6; behind it
    # are the DMAs of five stages (10 loads) and the weight loads of the even stages from
    # k - 6 on, counted only within the pass (the first pass follows the prologue)
    good = [10 + 4 * sum(1 for j in range(max(0, k - 6), k) if j % 2 == 0) for k in range(8)]
    assert good == [10, 14, 14, 18, 18, 22, 22, 22]
    assert build.ring_wait_violations(_deep_kernel_asm(good)) == []
    # one more than the 22 loads behind the DMA stage 7 needs lets that wait pass early
    bad = build.ring_wait_violations(_deep_kernel_asm(good[:7] + [23]))
    assert {path for _, path, _ in bad} == {"loop once", "loop twice"}
    assert all(v[0] % 8 == 0 and v[1:] == (22, 23) for _, _, vs in bad for v in vs)


def test_ring_wait_check_walks_loop_and_tail_paths():
    assert build.ring_wait_violations(_kernel_asm(2)) == []
    bad = build.ring_wait_violations(_kernel_asm(5))     # tail waits leave too much in flight
    assert {path for _, path, _ in bad} == {"loop and tail", "tail only"}


VALU_ASM = """\
    .text
_Z7kernelAPf:                           ; @_Z7kernelAPf
; %bb.0:
	v_and_or_b32 v5, v1, s2, v3
	s_nop 0
	v_mfma_f32_16x16x32_bf16 v[10:13], v[4:7], v[0:3], 0
	s_endpgm
.Lfunc_end0:
_Z7kernelBPf:                           ; @_Z7kernelBPf
; %bb.0:
	v_and_or_b32 v5, v1, s2, v3
	s_nop 1
	v_mfma_f32_16x16x32_bf16 v[10:13], v[4:7], v[0:3], 0
	v_readfirstlane_b32 s0, v9
	v_mfma_f32_16x16x32_bf16 v[10:13], v[4:7], v[8:11], 0
	v_mov_b32 v20, v1
	v_mov_b32 v20, v2
	s_nop 1
	v_mfma_f32_16x16x32_bf16 v[10:13], v[20:23], v[0:3], 0
	s_endpgm
.Lfunc_end1:
_Z7kernelCPf:                           ; @_Z7kernelCPf
; %bb.0:
	v_accvgpr_write_b32 a2, v1
	s_cbranch_scc1 .LBB2_2
	s_nop 7
.LBB2_2:
	v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]
	s_endpgm
.Lfunc_end2:
"""


def test_valu_mfma_hazards_flags_reads_within_two_wait_states_on_any_path():
    # A: one wait state between the write of v5 and the MFMA reading v[4:7]; B: two, an SGPR
    # write, and a write overwritten before any MFMA reads it; C: the taken branch reaches
    # the MFMA reading a2 after one wait state (the branch), the fall-through after nine
    assert build.valu_mfma_hazards(VALU_ASM) == [
        ("_Z7kernelAPf", "v_and_or_b32 v5, v1, s2, v3", 1),
        ("_Z7kernelCPf", "v_accvgpr_write_b32 a2, v1", 1)]
