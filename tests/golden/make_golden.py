"""Writes the stored fixtures in this folder.  Each value is a constant the
pages print or the pages' own formula evaluated (no oracle output is stored
here).  Run from this folder: python make_golden.py"""
import json

PS = [0.05, 0.1, 0.2, 0.3, 0.5]

fallback = {
    "source": "aitujian.cn article on Clover-35B-A3B-Preview, section 三 (decoding loop), toy model of the fallback branch: "
              "with 32 independent positions that each pass in one round with probability p, the chance that no position passes "
              "is (1-p)^32; the page's table of values did not survive extraction, so the values below are that formula evaluated. "
              "The page's reading of the table: for p >= 0.2 the forced fill is a rare path.",
    "block_size": 32,
    "p": PS,
    "p_no_pass": [(1 - p) ** 32 for p in PS],
}

constants = {
    "block_size": {"value": 32, "source": "aitujian.cn article, opening list and section 三 pseudocode default; goremy.ai page, decoding-loop section defaults"},
    "threshold": {"value": 0.95, "source": "aitujian.cn article, opening list and section 三 (conf >= threshold); goremy.ai page, decoding-loop section defaults"},
    "max_steps": {"value": 32, "source": "aitujian.cn article, section 三 pseudocode default"},
    "routed_experts": {"value": 256, "source": "aitujian.cn article, section 四; goremy.ai page, architecture section; 10100.com article part 01"},
    "top_k": {"value": 8, "source": "aitujian.cn article, section 四; goremy.ai page, architecture and coreset sections"},
    "shared_experts": {"value": 1, "source": "aitujian.cn article, section 四; goremy.ai page, architecture section"},
    "layers": {"value": 40, "source": "aitujian.cn article, section 四; 10100.com article part 01"},
    "coreset_top_p_example": {"value": 0.9, "source": "goremy.ai page, coreset section: 0.9 keeps 90% of aggregated routing mass, not 90% of experts"},
    "max_request_tokens": {"value": 131072, "source": "goremy.ai page, generation-controls section; 10100.com article opening"},
}

if __name__ == "__main__":
    json.dump(fallback, open("fallback_toy_model.json", "w"), indent=1)
    json.dump(constants, open("page_constants.json", "w"), indent=1)
