"""Build libech.so (all HIP sources) for gfx950, in-tree.

    python -m indexer_top_kv_amd.build

Compiles every csrc/*.hip into one shared library next to this file. Packed
FP32 instructions are disabled for device code (their generation by the
compiler is turned off; the host pass warns that it does not know the
feature, which is harmless). MFMA results are kept in ordinary VGPRs rather
than accumulation registers, which saves the copies out of them (one VALU
instruction per result register) in the scoring kernels.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, 'libech.so')
ARCH = os.environ.get('ECH_OFFLOAD_ARCH', 'gfx950')


def sources():
    return sorted(glob.glob(os.path.join(HERE, 'csrc', '*.hip')))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')
    tmp = LIB + '.tmp'
    cmd = [hipcc, f'--offload-arch={ARCH}', '-O3', '-std=c++17', '-shared', '-fPIC',
           '-Wall', '-Wno-unused-function',
           '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
           '-mllvm', '-amdgpu-mfma-vgpr-form',
           '-I', os.path.join(ROOT, 'include'), '-I', os.path.join(HERE, 'csrc'),
           *sources(), '-o', tmp]
    if verbose:
        print(' '.join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        sys.stderr.write('\n'.join(msgs) + '\n')
        raise RuntimeError(f'hipcc failed with exit code {r.returncode}')
    if verbose and msgs:
        print('\n'.join(msgs))
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """The host code of every source (entry points, argument checks,
    workspace sizing), built with AddressSanitizer and UBSan on the host side
    only (each -fsanitize flag is passed to the host compiler; device code is
    built as usual) into _build/libech_san.so (not tracked). Loading it needs
    the sanitizer runtime preloaded; the checks run with it launch no kernel."""
    hipcc = os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')
    out_dir = os.path.join(ROOT, '_build')
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, 'libech_san.so')
    cmd = [hipcc, f'--offload-arch={ARCH}', '-O1', '-g', '-std=c++17', '-shared', '-fPIC',
           '-Xarch_host', '-fsanitize=address', '-Xarch_host', '-fsanitize=undefined',
           '-Xarch_host', '-fno-omit-frame-pointer', '-shared-libsan',
           '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
           '-I', os.path.join(ROOT, 'include'), '-I', os.path.join(HERE, 'csrc'),
           *sources(), '-o', out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f'hipcc (sanitized host build) failed with exit code {r.returncode}')
    if verbose:
        print(' '.join(cmd))
    return out


if __name__ == '__main__':
    print(build(verbose=True))
