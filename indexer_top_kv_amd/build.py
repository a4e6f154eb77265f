"""Build libech.so (all HIP sources) for gfx950, in-tree.

    python -m indexer_top_kv_amd.build

Compiles every csrc/*.hip into one shared library next to this file. Packed
FP32 instructions are disabled for device code (their generation by the
compiler is turned off; the host pass warns that it does not know the
feature, which is harmless). Each source becomes an object of its own, so
the flags can differ per file: MFMA results are kept in ordinary VGPRs rather
than accumulation registers, which saves the copies out of them (one VALU
instruction per result register) in the scoring kernels, except in the files
of ACC_REG_SOURCES.
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


# Sources built without -amdgpu-mfma-vgpr-form: their MFMA accumulators
# outgrow the 256 architectural VGPRs and must live in accumulation
# registers (the sparse attention keeps 32 heads x 512 values per wave).
ACC_REG_SOURCES = {'attn.hip'}


def _flags(src: str):
    f = [f'--offload-arch={ARCH}', '-O3', '-std=c++17', '-fPIC', '-Wall', '-Wno-unused-function',
         '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
         '-I', os.path.join(ROOT, 'include'), '-I', os.path.join(HERE, 'csrc')]
    if os.path.basename(src) not in ACC_REG_SOURCES:
        f += ['-mllvm', '-amdgpu-mfma-vgpr-form']
    return f


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libech.so."""
    hipcc = os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')
    obj_dir = os.path.join(ROOT, '_build', 'obj')
    os.makedirs(obj_dir, exist_ok=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    procs = []
    for src in sources():
        obj = os.path.join(obj_dir, os.path.basename(src)[:-4] + '.o')
        cmd = [hipcc, *_flags(src), '-c', src, '-o', obj]
        if verbose:
            print(' '.join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, obj, p in procs:
        out = p.communicate()[0]
        msgs = [ln for ln in out.splitlines() if noise not in ln]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write('\n'.join(msgs) + '\n')
        elif verbose and msgs:
            print('\n'.join(msgs))
    if failed:
        raise RuntimeError(f'hipcc failed on {", ".join(os.path.basename(f) for f in failed)}')
    tmp = LIB + '.tmp'
    cmd = [hipcc, f'--offload-arch={ARCH}', '-shared', '-fPIC', *[o for _, o, _ in procs], '-o', tmp]
    if verbose:
        print(' '.join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f'hipcc link failed with exit code {r.returncode}')
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
