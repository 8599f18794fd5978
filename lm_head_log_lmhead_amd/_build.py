"""Build the HIP library in-tree: lm_head_log_lmhead_amd/_lib/liblmhead_logprob.so (gfx950 only).

Compiled with hipcc, no fast-math, no floating-point contraction (every fused multiply-add in the
kernels is written out explicitly, so all template instantiations compute the same bits), and
with the packed-fp32 instructions disabled.

Two passes.  The kernels that contain the ping-pong K loop start with a per-kernel count of
no-ops (LOOP_PAD in tile_gemm.hpp) that places the loop 4 bytes past a 32-byte boundary, its
fastest placement.  The first pass compiles the device code of fwd.hip and bwd.hip with no
padding, reads where each loop landed from the disassembly of that build, and the second pass
builds the library with the counts that move every loop to the target.  If the tools needed for
the first pass are missing, the library is built unpadded (same results, placement not tuned).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "liblmhead_logprob.so")
SOURCES = ["api.hip", "fwd.hip", "bwd.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The only atomics are the persistent kernels' tile claims, issued by one thread a tile ahead
    # of use (near the end of a range at its end), and the K-split's workgroup counter and flags,
    # one thread each.  The atomic optimizer rewrites them into a wavefront-wide scan that
    # consumes the result at once, i.e. waits (vmcnt 0) for it, and for the next tile's loads
    # just issued.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


# ---- loop placement ---------------------------------------------------------------------------

N_LOOP_KERNELS = 13
LOOP_TARGET = 4        # bytes past a LOOP_GRANULE boundary
LOOP_GRANULE = 32


def _kernel_id(symbol: str):
    """LOOP_PAD id of a kernel symbol (see tile_gemm.hpp), or None."""
    m = re.search(r"fwd_partials_persistent_kernel.*RecOptILb(\d)ELb(\d)E", symbol)
    if m:
        return 2 * int(m.group(1)) + int(m.group(2))
    m = re.search(r"bwd_dz_kernel.*ELb(\d)ELb(\d)E", symbol)
    if m:
        return 4 + 2 * int(m.group(1)) + int(m.group(2))
    if "gemm_tn_f32_persistent_kernel" in symbol:
        return 8
    m = re.search(r"fwd_partials_sk_kernel.*RecOptILb(\d)ELb(\d)E", symbol)
    if m:
        return 9 + 2 * int(m.group(1)) + int(m.group(2))
    return None


def _tool(name: str):
    for cand in (os.path.join("/opt/rocm/llvm/bin", name), shutil.which(name)):
        if cand and os.path.exists(cand):
            return cand
    return None


def _loop_offsets(elf: str) -> dict[int, int]:
    """Byte address of the K-loop head of every padded kernel in a device code object."""
    out = subprocess.run([_tool("llvm-objdump"), "-d", "--no-show-raw-insn", elf], capture_output=True,
                         text=True, check=True).stdout.splitlines()
    return loop_heads(out)


def loop_heads(out: list[str]) -> dict[int, int]:
    """From llvm-objdump -d lines: per padded kernel, the target of the first backward branch
    after the kernel's first run of 64 MFMAs (the head of its K loop)."""
    heads = [i for i, l in enumerate(out) if re.match(r"^[0-9a-f]+ <", l)]
    found = {}
    for k, st in enumerate(heads):
        kid = _kernel_id(out[st])
        if kid is None:
            continue
        end = heads[k + 1] if k + 1 < len(heads) else len(out)
        mfma = [i for i in range(st, end) if "v_mfma" in out[i]]
        if len(mfma) < 64:
            continue
        for line in out[mfma[63]:min(end, mfma[63] + 64)]:
            m = re.search(r"s_(?:c)?branch\w*\s+(\d+)\s.*//\s*([0-9A-Fa-f]+):", line)
            if not m:
                continue
            simm, addr = int(m.group(1)), int(m.group(2), 16)
            simm = simm - 65536 if simm > 32767 else simm
            if simm < 0:
                found[kid] = addr + 4 + 4 * simm
                break
    return found


def _device_object(src: str, defines: list[str], out_dir: str) -> str:
    """Device code object (unbundled ELF) of one source."""
    base = os.path.join(out_dir, os.path.basename(src))
    cmd = [hipcc(), *[f for f in FLAGS if f not in ("-fPIC", "-shared")], *defines, f"-I{INCLUDE}", f"-I{CSRC}",
           "--cuda-device-only", "-c", src, "-o", base + ".co"]
    subprocess.run(cmd, capture_output=True, text=True, check=True)
    subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o",
                    f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--input={base}.co", f"--output={base}.elf"],
                   capture_output=True, text=True, check=True)
    return base + ".elf"


def _measure(defines: list[str]) -> dict[int, int]:
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(2) as ex:
        elfs = list(ex.map(lambda s: _device_object(os.path.join(CSRC, s), defines, d), ("fwd.hip", "bwd.hip")))
        found = {}
        for e in elfs:
            found.update(_loop_offsets(e))
        return found


def pads_for(at: dict[int, int]) -> list[int]:
    """4-byte no-op counts that move each loop head at byte address at[kid] to LOOP_TARGET modulo
    LOOP_GRANULE (the pad sits before the loop, so it shifts the head by 4 bytes per no-op)."""
    pads = [0] * N_LOOP_KERNELS
    for kid, addr in at.items():
        pads[kid] = ((LOOP_TARGET - addr) % LOOP_GRANULE) // 4
    return pads


def loop_pads(verbose: bool = False):
    """No-op counts that put every padded kernel's K loop at LOOP_TARGET (None if not measurable)."""
    if not (_tool("llvm-objdump") and _tool("clang-offload-bundler")):
        return None
    try:
        at = _measure([])
    except (subprocess.CalledProcessError, OSError) as e:
        if verbose:
            print(f"loop placement not measured: {e}", file=sys.stderr)
        return None
    pads = pads_for(at)
    if verbose:
        print(f"loop heads {dict(sorted((k, hex(a)) for k, a in at.items()))} -> pads {pads}", flush=True)
    return pads


def build(verbose: bool = False, extra_flags: list[str] | None = None, place_loops: bool = True) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    pads = loop_pads(verbose) if place_loops else None
    defines = [f"-DLMH_LOOP_PADS={','.join(str(p) for p in pads)}"] if pads else []
    cmd = [hipcc(), *FLAGS, *defines, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
