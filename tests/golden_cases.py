"""Loader for tests/golden/hand_examples.json and a runner that evaluates one case
through either the oracle or the HIP binding (both expose the same call shapes)."""
from __future__ import annotations

import json
import os

import numpy as np

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def load():
    with open(_PATH) as f:
        return json.load(f)["cases"]


def arrays(case):
    out = {}
    for k, v in case["inputs"].items():
        out[k] = np.asarray(v, dtype=np.int64 if k == "actions" else np.float32)
    return out


def run_oracle(case):
    import oracle

    a, p = arrays(case), case["params"]
    est = case["estimator"]
    if est == "gae":
        adv, ret = oracle.gae(a["rewards"], a["values"], a["terminateds"], a.get("truncateds"),
                              p["gamma"], p["lambda"], a.get("bootstrap_values"), a.get("last_value"))
        return {"advantages": adv, "returns": ret}
    if est == "vtrace":
        vs, pg = oracle.vtrace(a["log_rhos"], None, a["values"], a["rewards"], a["terminateds"],
                               a.get("truncateds"), p["gamma"], p["rho_bar"], p["c_bar"],
                               a.get("bootstrap_values"), a.get("last_value"))
        return {"vs": vs, "pg_advantages": pg}
    if est == "retrace":
        q, adv = oracle.retrace(a["pi_target"], a["mu_taken"], a["q_taken"], a["next_q_all"],
                                a["actions"], a["rewards"], a["terminateds"], a.get("truncateds"),
                                p["gamma"], p["lambda"], p["c_bar"], p["rho_bar"])
        return {"q_ret": q, "advantages": adv}
    if est == "discounted":
        return {"returns": oracle.discounted_returns(a["rewards"], a["terminateds"], a.get("truncateds"),
                                                     p["gamma"], a.get("bootstrap_values"))}
    if est == "lambda_returns":
        return {"returns": oracle.lambda_returns(a["rewards"], a["next_values"], a["terminateds"],
                                                 a.get("truncateds"), p["gamma"], p["lambda"],
                                                 a.get("bootstrap_values"))}
    if est == "prefix":
        return {b: oracle.forward_scan(a["inputs"], a["dones"], a.get("seed_values"), p["decay"], b)
                for b in ("ends_at", "starts_at")}
    if est == "traces":
        return {"traces": oracle.forward_scan(a["inputs"], a["dones"], a.get("seed_values"),
                                              p["decay"], "ends_at")}
    raise KeyError(est)
