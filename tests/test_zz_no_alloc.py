"""The allocation-free speculative + sparse decode (bsa_speculative_sparse_noalloc) against
bsa_speculative_sparse, the entry point whose kernels it shares: two calls in a row, the
second on a smaller problem (the library's scratch area then still holds the first call's
partials), each compared bit for bit, plus the float64 oracle within the parity tolerances.
Also the host-side refusal of a problem whose partials exceed the scratch area."""
import numpy as np
import pytest
import torch

import long_context_attention_sparse_amd as bsa
import oracle
from synth.workloads import spec_sparse_decode
from tests.gpu_util import check_lse, check_o, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, Sk, spec_tokens):
    w = spec_sparse_decode(seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=128, Sk=Sk, bs=64, spec_tokens=spec_tokens)
    q, k, v = dev_bf16(w["q"]), dev_bf16(w["k"]), dev_bf16(w["v"])
    s0 = w["spec_start"]
    n = w["missed"].shape[-1]
    cnt = np.full((B, Hkv, 1), n, np.int32)
    idx = np.ascontiguousarray(w["missed"][:, :, None, :])
    pat = bsa.BlockPattern(torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda(), 128, 64)
    return w, q, k, v, s0, cnt, idx, pat


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry_point(out_dtype):
    # the first call fills most of the scratch area; the second is smaller, so stale partials
    # of the first call sit past the ones it writes
    for seed, B, Hq, Hkv, Sk, spec in [(71, 16, 32, 8, 16384, 1024), (72, 3, 8, 2, 4096, 512)]:
        say("noalloc speculative+sparse", B, Hq, Hkv, Sk, spec, out_dtype)
        w, q, k, v, s0, cnt, idx, pat = _case(seed, B, Hq, Hkv, Sk, spec)
        ks, vs = k[:, s0:], v[:, s0:]
        o_ref, lse_ref = bsa.speculative_sparse(q, ks, vs, k, v, pat, out_dtype=out_dtype)
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device)
        bsa.speculative_sparse_noalloc(q, ks, vs, k, v, pat, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), "O differs from bsa_speculative_sparse"
        assert torch.equal(lse, lse_ref), "LSE differs from bsa_speculative_sparse"
        o64, l64 = oracle.speculative_sparse(w["q"], w["k"][:, s0:], w["v"][:, s0:], w["k"], w["v"], cnt, idx, 64)
        check_o(host(out), o64, f"noalloc B={B}", bf16_out=out_dtype == torch.bfloat16)
        check_lse(host(lse), l64, f"noalloc lse B={B}")


def test_noalloc_rejects_partials_past_the_scratch_area():
    # B=64, Hq=128 at 32768 keys needs about 34 MB of partials, twice the scratch area: refused
    # on the host before any launch (K/V broadcast over the batch with stride 0)
    B, Hq, Hkv, D, Sk = 64, 128, 8, 128, 32768
    q = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, Sk, Hkv, D), dtype=torch.bfloat16, device="cuda").expand(B, Sk, Hkv, D)
    cnt = torch.full((B, Hkv, 1), 120, dtype=torch.int32, device="cuda")
    idx = torch.arange(120, dtype=torch.int32, device="cuda").repeat(B, Hkv, 1, 1).contiguous()
    pat = bsa.BlockPattern(cnt, idx, 128, 64)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(bsa.BSAError) as e:
        bsa.speculative_sparse_noalloc(q, k[:, -2048:], k[:, -2048:], k, k, pat, out=out)
    assert e.value.status == 3  # BSA_ERR_WORKSPACE
