"""Golden values of the algorithmic byte / flop model used for roofline reporting."""
import json
import os

from adapter_lora_serving_amd.roofline import lora_call_cost

GOLD = os.path.join(os.path.dirname(__file__), "golden", "byte_model.json")


def test_byte_model_golden():
    g = json.load(open(GOLD))
    for key, emb in (("linear", False), ("embedding", True)):
        c = g[key]
        total, flops, terms = lora_call_cost(c["T"], c["in_features"], c["out_slices"], c["R"],
                                             c["slots"], c["ranks"], c["token_slot"],
                                             c["elem_bytes"], embedding=emb, ids=c.get("ids"))
        assert terms == c["expect_terms"], key
        assert total == c["expect_bytes"], key
        assert flops == c["expect_flops"], key
