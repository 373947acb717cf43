"""The storage formulas against the worked numbers printed on the pages."""

import json
import os

import pytest

from oracle import memory

UNITS = {"B": 1, "KiB": 1024, "MB": 1e6, "GB": 1e9, "bit": 1, "params": 1, "fraction": 1}


def _compute(q, a):
    if q == "dense_bytes":
        return memory.dense_bytes(a["n_params"], a["bytes_per_param"])
    if q == "lora_bytes_fp16":
        return 2 * memory.lora_params([tuple(s) for s in a["shapes"]], a["r"])
    if q == "dq_saving_bits":
        return memory.dq_saving_bits(a["blocksize"], a["group"])
    if q == "constant_bytes_no_dq":
        return memory.constant_bytes(a["n_params"], a["blocksize"], double_quant=False)
    if q == "dq_saving_bytes":
        return (memory.constant_bytes(a["n_params"], a["blocksize"], a["group"], False)
                - memory.constant_bytes(a["n_params"], a["blocksize"], a["group"], True))
    if q == "weight_saving_fraction":
        return 1 - a["to_bits"] / a["from_bits"]
    if q == "dq_constant_bytes_single_global":
        return memory.dq_constant_bytes_single_global(a["nblocks"])
    if q == "lora_params_llama7b":
        return memory.lora_params(memory.llama7b_target_shapes(), a["r"])
    if q == "code_bytes":
        return a["n_params"] // 2
    if q == "quantized_weight_bytes":
        return memory.quantized_weight_bytes(a["n_params"])
    raise KeyError(q)


def _examples():
    path = os.path.join(os.path.dirname(__file__), "golden", "page_worked_examples.json")
    with open(path, encoding="utf-8") as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["name"][:40])
def test_page_worked_example(ex):
    got = _compute(ex["quantity"], ex["args"]) / UNITS[ex["unit"]]
    want = ex["page_value"]
    if "abs_tol" in ex:
        assert abs(got - want) <= ex["abs_tol"], (got, want)
    else:
        assert abs(got - want) <= ex["rel_tol"] * abs(want), (got, want)


def test_llama7b_lora_count_closed_form():
    # r * sum(N + K) over 7 projections x 32 layers at r = 16.
    assert memory.lora_params(memory.llama7b_target_shapes(), 16) == 39976960
