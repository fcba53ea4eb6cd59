"""The bytes model reproduces the totals printed on the pages."""
from quantized_moe_router_amd import accounting as acc


def test_expert_bytes_match_pages():
    # model card "What is quantized": group A (routed experts, 512 per layer,
    # 48 layers, INT4 gs128) is 58.0 GiB
    assert acc.expert_bytes() == 2_534_400
    assert round(512 * 48 * acc.expert_bytes() / 2**30, 1) == 58.0
    # "vLLM Edition" section 2: routed experts are 120.8B parameters
    assert round(512 * 48 * acc.expert_params() / 1e9, 1) == 120.8
    # "vLLM Optimization Edition" 3.3 decode-05: about 25 MB of expert weights
    # per token and layer (top-10)
    assert round(10 * acc.expert_bytes() / 1e6) == 25
    # section 4.2 of the same page: about 2.46 MB of packed INT4 per expert
    assert round(acc.expert_params() * 4 / 8 / 1e6, 2) == 2.46
    # "vLLM Edition" 5.6: 1.22 GB of expert reads per decode token (48 layers)
    assert round(48 * 10 * acc.expert_bytes() / 1e9, 2) == 1.22


def test_layer_totals():
    assert acc.router_bytes() == 2_621_440
    assert acc.layer_bytes(1, 10) == 2_621_440 + 25_344_000 + 10_240
    assert acc.layer_flops(1) == 2 * 512 * 2560 + 2 * 10 * 4_915_200
