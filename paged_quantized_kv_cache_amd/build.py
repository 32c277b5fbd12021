"""Build libkvq.so (hand-written HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import hashlib
import os
import struct
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
SOURCES = [os.path.join(CSRC, "kvq_api.hip")]
HEADERS = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hpp")] + \
    [os.path.join(INCLUDE, "kvq.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # IEEE fp32 division (the INT8 scale and x / scale are fp32 by definition)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # no packed-fp32 instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs (no AGPR copies around the
    # online-softmax rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _elf_sections(b: bytes, base: int = 0) -> dict:
    """name -> (offset, size, address) of the sections of the 64-bit ELF at
    b[base:]."""
    shoff, = struct.unpack_from("<Q", b, base + 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, base + 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", b, base + shoff + i * shentsize)
            for i in range(shnum)]
    names = base + hdrs[shstrndx][4]
    out = {}
    for h in hdrs:
        end = b.index(b"\0", names + h[0])
        out[b[names + h[0]:end].decode()] = (base + h[4], h[5], h[3])
    return out


def _functions(b: bytes, base: int) -> dict:
    """name -> machine code of every function symbol in the ELF at b[base:]."""
    secs = _elf_sections(b, base)
    to, _ts, taddr = secs[".text"]
    so, ss, _ = secs[".symtab"]
    stro = secs[".strtab"][0]
    out = {}
    for i in range(ss // 24):
        st_name, st_info, _oth, _shn, st_value, st_size = struct.unpack_from("<IBBHQQ", b, so + 24 * i)
        if st_info & 0xF != 2 or st_size == 0:  # STT_FUNC
            continue
        end = b.index(b"\0", stro + st_name)
        name = b[stro + st_name:end].decode()
        out[name] = b[to + st_value - taddr:to + st_value - taddr + st_size]
    return out


def device_code_hash(path: str = LIB, kernels=None) -> str:
    """Hash of the gfx950 machine code in the library's offload bundle: the
    whole .text, or (kernels: substrings of mangled names) only the
    functions whose names contain one of them, so a measurement taken on
    some kernels stays matched while other kernels change.  Comments or
    host-side edits leave it unchanged; any change to a hashed kernel's
    instructions changes it."""
    with open(path, "rb") as f:
        b = f.read()
    off, size, _ = _elf_sections(b)[".hip_fatbin"]
    fb = b[off:off + size]
    if not fb.startswith(b"__CLANG_OFFLOAD_BUNDLE__"):
        raise ValueError("no offload bundle in %s" % path)
    n, = struct.unpack_from("<Q", fb, 24)
    pos, h = 32, hashlib.sha256()
    for _ in range(n):
        eo, _es, tl = struct.unpack_from("<QQQ", fb, pos)
        triple = fb[pos + 24:pos + 24 + tl].decode()
        pos += 24 + tl
        if "gfx950" not in triple:
            continue
        if kernels is None:
            to, ts, _ = _elf_sections(fb, eo)[".text"]
            h.update(fb[to:to + ts])
        else:
            for name, code in sorted(_functions(fb, eo).items()):
                if any(k in name for k in kernels):
                    h.update(name.encode() + b"\0" + code)
    return h.hexdigest()[:16]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
