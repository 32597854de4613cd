"""The no-allocation entry point (moe_route_and_scatter_noalloc) against the
call it varies (moe_route_and_scatter with a caller workspace), through the C
ABI: two calls in a row on one GPU, the second with a smaller input, each
bit-identical in every output to the workspace call on the same input.  The
first call takes the multi-kernel path (MFMA router, counting-sort launches),
the second the one-workgroup decode path, so the scratch the second call finds
holds the first call's data."""

import pytest
import torch

from mixture_experts_ffn_05_amd import binding as B
from mixture_experts_ffn_05_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CALLS = [("v3", 4096), ("v2l", 512), ("v2l", 16), ("v3", 64)]   # the first: the largest benchmark layer


def _outputs(T, H, E, k, dtype):
    i32, f32 = torch.int32, torch.float32
    return {"topk_ids": torch.full((T, k), -7, dtype=i32, device=DEV),
            "topk_weights": torch.full((T, k), float("nan"), dtype=f32, device=DEV),
            "logits": torch.full((T, E), float("nan"), dtype=f32, device=DEV),
            "scatter_index": torch.full((T, k), -7, dtype=i32, device=DEV),
            "row_token": torch.full((T * k,), -7, dtype=i32, device=DEV),
            "expert_offsets": torch.full((E + 1,), -7, dtype=i32, device=DEV),
            "status_words": torch.full((2,), -7, dtype=i32, device=DEV),
            "x_scattered": torch.zeros((T * k, H), dtype=dtype, device=DEV)}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (t.view(torch.int32) if t.is_floating_point() else t)


def test_noalloc_matches_workspace_call_twice_with_a_smaller_second_input():
    assert torch.cuda.is_available()
    B.load()
    for name, T in CALLS:
        base = wl.WORKLOADS[name]
        cfg = base.at_tokens(T, f"t{T}")
        print(f"[noalloc] {name} T={T} H={cfg.H} E={cfg.E} k={cfg.top_k}", flush=True)
        x = wl.make_x(base, DEV)[:T].contiguous()
        wr = wl.make_router(cfg, DEV)
        bias = wl.load_route_bias(cfg)
        bias_t = torch.from_numpy(bias).to(DEV) if bias is not None else None
        need = B.moe_route_and_scatter_workspace_bytes(x.dtype, T, cfg.H, cfg.E, cfg.top_k)
        assert need <= B.moe_route_and_scatter_noalloc_max_bytes()
        ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
        ref = _outputs(T, cfg.H, cfg.E, cfg.top_k, x.dtype)
        B.moe_route_and_scatter(x, wr, bias_t, cfg.top_k, ref["topk_ids"], ref["topk_weights"], ref["logits"],
                                ref["scatter_index"], ref["row_token"], ref["expert_offsets"], ref["status_words"],
                                ref["x_scattered"], ws)
        got = _outputs(T, cfg.H, cfg.E, cfg.top_k, x.dtype)
        B.moe_route_and_scatter_noalloc(x, wr, bias_t, cfg.top_k, got["topk_ids"], got["topk_weights"],
                                        got["logits"], got["scatter_index"], got["row_token"],
                                        got["expert_offsets"], got["status_words"], got["x_scattered"])
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(_bits(got[key]), _bits(ref[key])), f"{name} T={T}: {key} differs"
        assert got["status_words"][1].item() == 0
        assert int(got["expert_offsets"][-1].item()) == T * cfg.top_k
