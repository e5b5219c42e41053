"""Whole-model parameter lists for the bucket-planner workloads.

The planner is evaluated on DeepSeek-V3-671B and GPT-OSS-120B at 1x and 16x
row granularity over a range of FSDP sizes (veScale-FSDP talk notes,
"2. Structure-aware planning algorithm", Fig. 11).  Each model is a list of
buckets, one per decoder layer plus one for the input embedding and one for
the output head with the final norm, as an FSDP wrapper per layer would
group them.  Shapes are the public architecture configurations of the two
models (hidden sizes, head counts, expert counts and widths); values are
never needed.  A tensor is ``rows x cols`` with ``cols`` the contiguous
dimension; a 1-D tensor is ``numel x 1``, so its row granularity is in
elements.  Row granularity g gives every tensor ``block_rows = g``.
"""

from __future__ import annotations

from typing import List

from .configs import TensorDef


def _t(name, rows, cols, g):
    return TensorDef(name, rows, cols, g, cols)


def _v(name, n, g):
    return TensorDef(name, n, 1, g, 1)


def deepseek_v3_671b(g: int = 1) -> List[List[TensorDef]]:
    """61 decoder layers (3 dense, 58 MoE with 256 routed experts and one
    shared expert), multi-head latent attention, vocabulary 129,280."""
    H, V = 7168, 129280
    heads, q_lora, kv_lora, nope, rope, vdim = 128, 1536, 512, 128, 64, 128
    dense_inter, expert_inter, experts = 18432, 2048, 256
    buckets = [[_t("embed", V, H, g)]]
    for layer in range(61):
        p = f"l{layer}."
        b = [_v(p + "input_norm", H, g),
             _t(p + "q_a", q_lora, H, g), _v(p + "q_a_norm", q_lora, g),
             _t(p + "q_b", heads * (nope + rope), q_lora, g),
             _t(p + "kv_a", kv_lora + rope, H, g), _v(p + "kv_a_norm", kv_lora, g),
             _t(p + "kv_b", heads * (nope + vdim), kv_lora, g),
             _t(p + "o", H, heads * vdim, g),
             _v(p + "post_norm", H, g)]
        if layer < 3:
            b += [_t(p + "gate", dense_inter, H, g), _t(p + "up", dense_inter, H, g),
                  _t(p + "down", H, dense_inter, g)]
        else:
            b += [_t(p + "router", experts, H, g), _v(p + "router_bias", experts, g)]
            for e in list(range(experts)) + ["shared"]:
                b += [_t(p + f"e{e}.gate", expert_inter, H, g), _t(p + f"e{e}.up", expert_inter, H, g),
                      _t(p + f"e{e}.down", H, expert_inter, g)]
        buckets.append(b)
    buckets.append([_v("final_norm", H, g), _t("lm_head", V, H, g)])
    return buckets


def gpt_oss_120b(g: int = 1) -> List[List[TensorDef]]:
    """36 decoder layers with 128 experts each (fused gate/up projection of
    2 x 2880 rows, down projection of 2880 rows, with biases), grouped-query
    attention of 64 query and 8 key/value heads of 64, attention sinks,
    vocabulary 201,088."""
    H, V = 2880, 201088
    heads, kv_heads, hd, experts, inter = 64, 8, 64, 128, 2880
    buckets = [[_t("embed", V, H, g)]]
    for layer in range(36):
        p = f"l{layer}."
        b = [_v(p + "input_norm", H, g),
             _t(p + "q", heads * hd, H, g), _v(p + "q_bias", heads * hd, g),
             _t(p + "k", kv_heads * hd, H, g), _v(p + "k_bias", kv_heads * hd, g),
             _t(p + "v", kv_heads * hd, H, g), _v(p + "v_bias", kv_heads * hd, g),
             _t(p + "o", H, heads * hd, g), _v(p + "o_bias", H, g),
             _v(p + "sinks", heads, g),
             _v(p + "post_norm", H, g),
             _t(p + "router", experts, H, g), _v(p + "router_bias", experts, g)]
        for e in range(experts):
            b += [_t(p + f"e{e}.gate_up", 2 * inter, H, g), _v(p + f"e{e}.gate_up_bias", 2 * inter, g),
                  _t(p + f"e{e}.down", H, inter, g), _v(p + f"e{e}.down_bias", H, g)]
        buckets.append(b)
    buckets.append([_v("final_norm", H, g), _t("unembed", V, H, g)])
    return buckets


MODELS = {"deepseek_v3_671b": deepseek_v3_671b, "gpt_oss_120b": gpt_oss_120b}
# FSDP sizes the planner is evaluated over
PLANNER_FSDP_SIZES = (8, 16, 32, 64, 128, 256, 512, 1024)
PLANNER_GRANULARITIES = (1, 16)
