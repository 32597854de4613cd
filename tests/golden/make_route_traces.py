"""Writes the route-trace fixtures used by the tests (inputs only: seeded
routes from the package's sample generator, no expected values).

    python tests/golden/make_route_traces.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from mixture_experts_ffn_05_amd import route_trace as RT  # noqa: E402

small = dict(name="small-gated", hidden_size=512, num_experts=16, top_k=4, moe_intermediate_size=136,
             shared_experts=2, shared_intermediate_size=192, shared_gate=True)
docs = {
    "route_trace_tiny_v1.json": RT.sample_trace(RT.MODEL_PRESETS["tiny"], tokens=128, seed=11, version=1,
                                                dtype="f32"),
    "route_trace_small_v2_gated.json": RT.sample_trace(small, tokens=257, seed=12, routing="zipf:1.1"),
}
for name, doc in docs.items():
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(doc, f)
    print("wrote", name)
