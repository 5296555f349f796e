"""mala_decode_noalloc, the decode step that allocates nothing (its partial
states and decision bits live in the library's fixed device scratch),
against mala_decode with a caller-owned workspace, through the C ABI: two
calls in a row on the same scratch, the 128K decode batch and then a smaller
problem, give the same outputs, decisions and counters bit for bit."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU only to be deselected
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"


def test_noalloc_decode_matches_workspace_decode():
    import contribution_gated_sparse_amd as m
    big = W.make_decode(W.CONFIGS[5], device=DEV)
    n = big["cache"] + 1
    small = W.make_decode(W.CONFIGS[5], cache=2100, steps=1, batch=3, planted=8, device=DEV)
    cases = [("128K decode batch, step 0", big, [n] * 8, 1e-4),
             ("3 ragged sequences", small, [2101, 1500, 65], 1.0)]
    for name, x, lens, tau in cases:
        print(f"[noalloc] {name}: lens={lens} tau={tau}", flush=True)
        q = x["q_steps"][0].contiguous()
        seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
        a = m.mala_decode(q, x["k_cache"], x["v_cache"], seq, tau, max_n_k=max(lens),
                          softmax_scale=x["scale"], want_mask=True)
        b = m.mala_decode(q, x["k_cache"], x["v_cache"], seq, tau, max_n_k=max(lens),
                          softmax_scale=x["scale"], want_mask=True, noalloc=True)
        torch.cuda.synchronize()
        assert b["ws"] is None
        for k in ("o", "lse", "mask", "kept"):
            assert torch.equal(a[k], b[k]), (name, k)
        assert (a["mask"] == 1).any() and int(a["kept"].sum()) > 0
