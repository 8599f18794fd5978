"""Host logic of the build and the benchmark (no GPU): loop-placement parsing and padding, and
the benchmark's refusal of more than one GPU."""
import os
import subprocess
import sys

from lm_head_log_lmhead_amd import _build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _fake_disassembly(symbol: str, base: int, loop_at: int, n_mfma: int = 64):
    """llvm-objdump -d style lines of one kernel: n_mfma MFMAs, then a backward branch to loop_at."""
    lines = [f"{base:016x} <{symbol}>:"]
    addr = base
    for _ in range(n_mfma):
        lines.append(f"\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\t// {addr:012X}: ")
        addr += 8
    simm = (loop_at - (addr + 4)) // 4
    lines.append(f"\ts_cbranch_scc1 {simm & 0xffff}\t// {addr:012X}: ")
    lines.append("\ts_endpgm")
    return lines


def test_kernel_ids_follow_the_template_arguments():
    fwd = "_ZN3lmh30fwd_partials_persistent_kernelINS_6FwdCfgINS_7PipeCfgILi2ELi4ELi4ELi2ELi64EEELi2EEENS_6RecOpt"
    assert B._kernel_id(fwd + "ILb1ELb0EEEEEvNS_7FwdArgsEii") == 2
    assert B._kernel_id(fwd + "ILb0ELb1EEEEEvNS_7FwdArgsEii") == 1
    dz = "_ZN3lmh13bwd_dz_kernelINS_7PipeCfgILi2ELi4ELi4ELi2ELi64EEELb1ELb1EEEvPKDF16b"
    assert B._kernel_id(dz) == 7
    assert B._kernel_id("_ZN3lmh29gemm_tn_f32_persistent_kernelINS_7PipeCfgILi2ELi4ELi4ELi2ELi64EEEEEv") == 8
    assert B._kernel_id("_ZN3lmh19fwd_finalize_kernelILb0ELi16EEEvNS_7FwdArgsEi") is None


def test_loop_head_is_the_backward_branch_target():
    sym = "_ZN3lmh13bwd_dz_kernelINS_7PipeCfgILi2ELi4ELi4ELi2ELi64EEELb0ELb1EEEv"
    lines = _fake_disassembly(sym, 0x1000, 0x1040)
    assert B.loop_heads(lines) == {5: 0x1040}
    # fewer than 64 MFMAs: no K loop recognised
    assert B.loop_heads(_fake_disassembly(sym, 0x1000, 0x1040, n_mfma=32)) == {}


def test_pads_move_every_head_to_the_target():
    at = {0: 0x1000, 4: 0x2014, 8: 0x3004}
    pads = B.pads_for(at)
    for kid, addr in at.items():
        assert (addr + 4 * pads[kid]) % B.LOOP_GRANULE == B.LOOP_TARGET
        assert 0 <= pads[kid] < B.LOOP_GRANULE // 4
    assert pads[1] == 0 and len(pads) == B.N_LOOP_KERNELS


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
