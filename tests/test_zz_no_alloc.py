"""The allocation-free decode entry point against dsa_layer_decode.

dsa_layer_decode_noalloc runs the same kernels with the library's fixed
per-GPU scratch array as workspace.  Two calls in a row, the second on a
smaller input (fewer sequences, shorter contexts), must each give exactly
the bits of dsa_layer_decode with a caller workspace: the same selected
positions and the same bf16 outputs.  A call whose workspace would exceed
the array is refused before any launch.
"""
import sys

import pytest
import torch

from long_context_sparse_dsa_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _pair(dsa, wl, d):
    L = max(wl.ctx_lens)
    ws = torch.empty(dsa.dsa_layer_decode_workspace_size(wl.B, L, wl.K, wl.Hq, wl.D),
                     dtype=torch.uint8, device=DEV)
    idx_a = torch.empty(wl.B, wl.K, dtype=torch.int32, device=DEV)
    out_a = dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"],
                                 d["k_cache"], d["v_cache"], d["gate"], wl.K, d["ctx_len"],
                                 d["cu_ctx"], max_ctx=L, idx_out=idx_a, ws=ws)
    idx_b = torch.empty_like(idx_a)
    out_b = torch.empty_like(out_a)
    dsa.dsa_layer_decode_noalloc(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"],
                                 d["k_cache"], d["v_cache"], d["gate"], wl.K, d["ctx_len"],
                                 d["cu_ctx"], L, out_b, idx_out=idx_b)
    torch.cuda.synchronize()
    return out_a, idx_a, out_b, idx_b


def test_noalloc_decode_matches_decode_twice(dsa):
    cases = [
        W.Workload("t", [40000, 23000, 131072], [1, 1, 1], 32, 128, 64, 128, 2048,
                   plant_frac=0.05, seed=61),
        W.Workload("t", [5000], [1], 16, 128, 64, 128, 2048, seed=62),
    ]
    for i, wl in enumerate(cases):
        print(f"noalloc decode call {i}: lens={wl.ctx_lens}", flush=True)
        sys.stdout.flush()
        d = W.make_inputs(wl, device=DEV)
        out_a, idx_a, out_b, idx_b = _pair(dsa, wl, d)
        assert torch.equal(idx_a, idx_b), f"call {i}: selected positions differ"
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), \
            f"call {i}: outputs differ"


def test_noalloc_decode_refuses_oversize(dsa):
    cap = dsa.load().dsa_layer_decode_noalloc_max_bytes()
    assert cap == 64 << 20
    # 64 sequences of 1M positions need 256 MiB of fp32 scores
    need = dsa.dsa_layer_decode_workspace_size(64, 1 << 20, 2048, 64, 128)
    assert need > cap
    f = dsa.load().dsa_layer_decode_noalloc
    fake = 0x10000
    st = f(fake, fake, 32, fake, 0, None, 32, 128, fake, fake, fake, fake, 1, 0.0, 64, 128,
           2048, fake, fake, 64, 1 << 20, fake, None, None)
    assert st == 3 and "fixed" in dsa.dsa_last_error()
