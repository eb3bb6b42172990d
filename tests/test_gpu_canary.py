"""Canary-padded outputs: kv_compact, kv_compact_decode and kv_decode_attn
write nothing past the rows the offsets give (offsets[last], or the capacity
when it truncates), past offsets[B*Hkv], past out / lse, or past the
workspace size the library asked for."""
import numpy as np
import pytest
import torch

from kv_cache_compression_score_amd import api
from kv_cache_compression_score_amd import workloads as wl

from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu

PAD = 64          # guard rows / elements after every output
CANARY16 = 0x7FA5  # a bf16 NaN payload no kernel writes
CANARY32 = -123456789


def guarded(shape_rows, d, dtype):
    t = torch.empty(shape_rows + PAD, d, device="cuda", dtype=dtype)
    t.view(torch.int16).fill_(CANARY16)
    return t


def kept(seed, B, Hkv, N, ctx):
    rng = np.random.default_rng(seed)
    idx = np.zeros((B, Hkv, N), np.int32)
    cnt = np.zeros(B * Hkv, np.int32)
    for b in range(B):
        for h in range(Hkv):
            c = int(rng.integers(1, ctx[b] + 1))
            idx[b, h, :c] = np.sort(rng.choice(ctx[b], c, replace=False))
            cnt[b * Hkv + h] = c
    return dev(torch.from_numpy(idx)), dev(torch.from_numpy(cnt))


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("trunc", [False, True])
def test_no_write_past_the_packed_rows(fused, trunc):
    B, Hq, Hkv, N, d = 2, 8, 2, 1500, 128
    log(f"canary fused={fused} truncated={trunc}")
    lay = wl.random_case(31, B=B, Hq=Hq, Hkv=Hkv, d=d, N_max=N, W=1, ctx=[1500, 900])
    k, v, q = dev(lay.k), dev(lay.v), dev(lay.q_dec[0])
    idx, cnt = kept(5, B, Hkv, N, [1500, 900])
    total = int(cnt.sum())
    cap = total - 700 if trunc else total + 300
    k_c, v_c = guarded(cap, d, torch.bfloat16), guarded(cap, d, torch.bfloat16)
    pos = torch.full((cap + PAD,), CANARY32, device="cuda", dtype=torch.int32)
    off = torch.full((B * Hkv + 1 + PAD,), CANARY32, device="cuda", dtype=torch.int64)
    out = torch.full((B * Hq * d + PAD,), float("nan"), device="cuda")
    lse = torch.full((B * Hq + PAD,), float("nan"), device="cuda")
    need = api.kv_decode_workspace_size(B, Hq, Hkv, d, cap)
    ws = torch.full((need + 4096,), 0xA5, device="cuda", dtype=torch.uint8)
    outs = (k_c[:cap], v_c[:cap], pos[:cap], off[:B * Hkv + 1])
    if fused:
        api.kv_compact_decode(k, v, idx, cnt, cap, q, out=outs,
                              attn_out=out[:B * Hq * d].view(B, Hq, d), lse=lse[:B * Hq].view(B, Hq),
                              workspace=ws[:need])
    else:
        api.kv_compact(k, v, idx, cnt, cap, out=outs)
        api.kv_decode_attn(q, k_c[:cap], v_c[:cap], off[:B * Hkv + 1], Hkv,
                           out=out[:B * Hq * d].view(B, Hq, d), lse=lse[:B * Hq].view(B, Hq),
                           workspace=ws[:need])
    torch.cuda.synchronize()
    assert int(off[B * Hkv]) == total
    n = min(total, cap)
    assert torch.all(k_c[n:].view(torch.int16) == CANARY16).item()
    assert torch.all(v_c[n:].view(torch.int16) == CANARY16).item()
    assert torch.all(pos[n:] == CANARY32).item()
    assert torch.all(off[B * Hkv + 1:] == CANARY32).item()
    assert torch.all(torch.isnan(out[B * Hq * d:])).item()
    assert torch.all(torch.isnan(lse[B * Hq:])).item()
    assert torch.all(ws[need:] == 0xA5).item()
    # and everything inside was written
    assert not torch.any(k_c[:n].view(torch.int16) == CANARY16).item()
    assert not torch.any(pos[:n] == CANARY32).item()
    assert torch.all(torch.isfinite(out[:B * Hq * d])).item()
