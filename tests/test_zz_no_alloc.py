"""The allocation-free attention backward (mt_op_attn_bwd_rope_noalloc)
through the C-ABI against mt_op_attn_bwd_rope with a caller workspace: the
same kernels, so the same bits, on two calls in a row (the second smaller,
so it runs over what the first left in the shared scratch); sizes beyond
the scratch are refused before any launch, with an error stating the need."""
import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from host_memory_streamed_amd import mt  # noqa: E402

DEV = "cuda"


def _case(rng, dtype, B, T, H, Hkv, hd):
    tdt = torch.bfloat16 if dtype else torch.float32
    W = (H + 2 * Hkv) * hd
    qkv = rng.standard_normal((B * T, W)).astype(np.float32)
    if dtype:
        qkv = O.bf16(qkv).astype(np.float32)
    qd = torch.from_numpy(qkv).to(DEV).to(tdt)
    M = B * T
    o = torch.empty(M, H * hd, device=DEV)
    oc = torch.empty(M, H * hd, device=DEV, dtype=tdt) if dtype else None
    lse = torch.empty(B, H, T, device=DEV)
    mt.attn_fwd(dtype, qd, o, oc, lse, B, T, H, Hkv, hd)
    dout = torch.from_numpy(rng.standard_normal((M, H * hd)).astype(np.float32)).to(DEV)
    c, s = mt.rope_table(T, hd, 10000.0)
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    ws = torch.empty(mt.attn_bwd_ws_bytes(dtype, B, T, H, hd), device=DEV, dtype=torch.uint8)
    ref = torch.full((M, W), float("nan"), device=DEV, dtype=tdt)
    mt.attn_bwd_rope(dtype, qd, o, dout, lse, cd, sd, ref, ws, B, T, H, Hkv, hd)
    got = torch.full((M, W), float("nan"), device=DEV, dtype=tdt)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    mt.attn_bwd_rope_noalloc(dtype, qd, o, dout, lse, cd, sd, got, B, T, H, Hkv, hd)
    torch.cuda.synchronize()
    return ref.float().cpu().numpy(), got.float().cpu().numpy(), free0 - torch.cuda.mem_get_info()[0]


@pytest.mark.parametrize("dtype", [mt.MT_FP32, mt.MT_BF16])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    rng = np.random.default_rng(7)
    # first a 14B-shaped layer's heads over 1024 tokens, then a smaller,
    # ragged case on top of what the first left in the scratch. The first
    # call on a device may load the array itself (the library's set-up, once
    # per device); no call after it takes any device memory.
    for i, (B, T, H, Hkv, hd) in enumerate(((1, 1024, 40, 8, 128), (2, 77, 4, 2, 64))):
        ref, got, taken = _case(rng, dtype, B, T, H, Hkv, hd)
        assert np.all(np.isfinite(got))
        np.testing.assert_array_equal(got, ref)
        if i == 1:
            assert taken == 0, taken


def test_noalloc_refuses_sizes_beyond_its_scratch():
    # 1 x 65536 tokens x 32 heads x 128 needs 512 MiB + D: refused on the
    # host before anything is launched (NULL buffers are never touched)
    need = mt.attn_bwd_ws_bytes(mt.MT_BF16, 1, 65536, 32, 128)
    assert need > (64 << 20)
    with pytest.raises(mt.MTError) as e:
        mt.attn_bwd_rope_noalloc(mt.MT_BF16, 0, 0, 0, 0, 0, 0, 0, 1, 65536, 32, 32, 128)
    assert e.value.code == mt.MT_EINVAL
    msg = mt.lib().mt_last_error(None).decode()
    assert str(need) in msg and str(64 << 20) in msg
