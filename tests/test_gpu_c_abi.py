"""One decode step driven from a plain C program through the C ABI (no
Python or torch in that process): tests/c_abi_decode.c reads the pools,
new tokens, queries and tables from a file, runs paged_kv_write and
paged_attn_decode, and writes the output, which must match the oracle's
decode (max-abs 2e-3, as every 16-bit parity test)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle.ref as ref
import workloads as wl

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "paged_kv_cache_30_amd")
ROCM = "/opt/rocm"


def build(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = tmp_path / "c_abi_decode"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c_abi_decode.c"), "-L", LIBDIR, "-lpagedattn",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{LIBDIR}",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", str(exe)], check=True)
    return exe


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_from_c(tmp_path, dtype):
    print(f"c abi decode {dtype}", flush=True)
    exe = build(tmp_path)
    w = wl.make_decode(lens=[1, 37, 600, 2000], num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                       dtype=dtype, seed=51, spare_blocks=3)
    kp, vp = ref.build_pools(w, include_step=False)
    seq_idx, pos, k_new, v_new = w.step_tokens()
    code = {"f16": 1, "bf16": 2}[dtype]
    hdr = np.array([w.num_blocks, w.block_size, w.num_heads, w.num_kv_heads, w.head_dim, code, w.num_seqs,
                    w.block_tables.shape[1], w.max_context_len, len(seq_idx)], np.int32)
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.float32(w.scale).tobytes())
        for a in (kp, vp, w.q, k_new, v_new):
            f.write(np.ascontiguousarray(a).tobytes())
        for a in (seq_idx, pos, w.block_tables, w.context_lens):
            f.write(np.ascontiguousarray(a, dtype=np.int32).tobytes())
    out_path = tmp_path / "out.bin"
    r = subprocess.run([str(exe), str(inp), str(out_path)], capture_output=True, text=True, timeout=120)
    print(r.stdout.strip(), r.stderr.strip(), flush=True)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(out_path, dtype=np.float32).reshape(w.num_seqs, w.num_heads, w.head_dim)
    kp2, vp2 = ref.build_pools(w)
    want, _ = ref.decode(w.q, kp2, vp2, w.block_tables, w.context_lens, block_size=w.block_size,
                         num_kv_heads=w.num_kv_heads, window=0, scale=w.scale, dtype=dtype)
    err = float(np.abs(got - want).max())
    print(f"c abi decode {dtype}: max abs err {err:.3g}", flush=True)
    assert np.isfinite(got).all() and err <= 2e-3
