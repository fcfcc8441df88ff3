"""paged_attn_decode_noalloc (the decode call with the library's fixed
per-GPU scratch in place of a caller's workspace) against paged_attn_decode,
through the C ABI: two calls in a row, the second on a smaller batch, both
bit-identical to the workspace call (same kernels, same split), and within
the 16-bit bar of the fp64 oracle; a call whose workspace would exceed the
scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

import oracle.ref as ref
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_30_amd as pkv
    return pkv


def _device(w):
    from paged_kv_cache_30_amd import session
    d = session.DeviceWorkload(w)
    d.write_step()
    torch.cuda.synchronize()
    return d


def _both(pkv, d, w):
    kw = dict(window=w.window, sinks=w.sinks, scale=w.scale)
    H = w.num_heads
    ref_out = torch.full((w.num_seqs, H, w.head_dim), 3.0, dtype=torch.float32, device="cuda")
    ref_lse = torch.full((w.num_seqs, H), 3.0, dtype=torch.float32, device="cuda")
    ws = pkv.decode_workspace(d.k_pool, H, w.num_seqs, w.max_context_len, window=w.window, sinks=w.sinks)
    pkv.paged_attn_decode(ref_out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, w.max_context_len, lse=ref_lse,
                          workspace=ws, **kw)
    out = torch.full_like(ref_out, 5.0)
    lse = torch.full_like(ref_lse, 5.0)
    pkv.paged_attn_decode_noalloc(out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, w.max_context_len, lse=lse,
                                  **kw)
    torch.cuda.synchronize()
    return ref_out.cpu().numpy(), ref_lse.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def test_noalloc_matches_workspace_call_twice(pkv):
    big = wl.make_decode(lens=[3000, 100, 1777, 64, 2500, 1], num_heads=32, num_kv_heads=8, head_dim=128,
                         block_size=16, dtype="bf16", seed=71, k_scale=3.0)
    small = wl.make_decode(lens=[50, 7], num_heads=8, num_kv_heads=2, head_dim=64, block_size=32, dtype="bf16",
                           seed=72, window=20, sinks=4)
    for w in (big, small):
        print(f"noalloc decode S={w.num_seqs} H={w.num_heads} D={w.head_dim}", flush=True)
        d = _device(w)
        ro, rl, o, l = _both(pkv, d, w)
        assert np.array_equal(o, ro), "output differs from paged_attn_decode"
        assert np.array_equal(l, rl), "lse differs from paged_attn_decode"
        kp, vp = ref.build_pools(w)
        want, _ = ref.decode(w.q, kp, vp, w.block_tables, w.context_lens, block_size=w.block_size,
                             num_kv_heads=w.num_kv_heads, window=w.window, scale=w.scale, dtype=w.dtype,
                             sinks=w.sinks)
        assert np.abs(o - want).max() <= 2e-3


def test_noalloc_refuses_beyond_scratch(pkv):
    """A batch whose workspace exceeds the 32 MiB scratch: PKV_ESCRATCH, and
    the output keeps its bytes."""
    from paged_kv_cache_30_amd import session
    S, H, Hkv, D = 9000, 32, 8, 128
    k_pool = torch.zeros((4, 16, Hkv, D), dtype=torch.bfloat16, device="cuda")
    need = pkv.paged_attn_decode_workspace_bytes(k_pool, H, S, 64)
    assert need > 32 << 20
    q = torch.zeros((S, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.full((S, H, D), 7.0, dtype=torch.float32, device="cuda")
    tables = torch.zeros((S, 4), dtype=torch.int32, device="cuda")
    lens = torch.ones(S, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PagedAttnError) as e:
        pkv.paged_attn_decode_noalloc(out, q, k_pool, k_pool, tables, lens, 64, scale=0.1)
    assert e.value.status == pkv.PKV_ESCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
