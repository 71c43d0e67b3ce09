"""Layer shapes printed on the pages (tests/golden/ultra_layer_shapes.json)."""
import json
import os

from selective_state_space_conv1d_amd.synth import WORKLOADS

GOLD = os.path.join(os.path.dirname(__file__), "golden", "ultra_layer_shapes.json")


def test_ultra_layer_shapes():
    g = json.load(open(GOLD))
    d = WORKLOADS["prefill_ultra_8k"]
    assert (d.nheads, d.head_dim, d.d_state, d.ngroups, d.conv_width) == (
        g["mamba_num_heads"], g["head_dim"], g["ssm_state_size"], g["n_groups"], g["conv_kernel"])
    assert [d.conv_dim, d.conv_width] == g["conv_states_shape_per_batch_row"]
    assert [d.nheads, d.head_dim, d.d_state] == g["ssm_states_shape_per_batch_row"]
    elems = d.nheads * d.head_dim * d.d_state
    # "about 2M elements, about 8 MB in fp32"
    assert abs(elems - g["ssm_state_elements_approx"]) / g["ssm_state_elements_approx"] < 0.05
    assert abs(4 * elems - g["ssm_state_fp32_bytes_approx"]) / g["ssm_state_fp32_bytes_approx"] < 0.05
    for name in ("decode_ultra_b64", "long_ultra_256k"):
        w = WORKLOADS[name]
        assert (w.nheads, w.head_dim, w.d_state, w.ngroups, w.conv_dim) == (256, 64, 128, 8, 18432)
