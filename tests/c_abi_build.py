"""Build tests/c_abi_fwd (the forward through the C ABI from plain C) with gcc,
linking libbsattn.so, liboracle.so and the HIP runtime; run paths are relative to
the binary, so the tree can move."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_fwd.c")
BIN = os.path.join(HERE, "c_abi_fwd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(force: bool = True) -> str:
    if not force and os.path.exists(BIN) and os.path.getmtime(BIN) >= os.path.getmtime(SRC):
        return BIN
    tmp = BIN + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "block_sparse_flash_mask_amd"), "-lbsattn",
           "-L", os.path.join(ROOT, "oracle"), "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../block_sparse_flash_mask_amd:$ORIGIN/../oracle:" + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, BIN)
    return BIN
