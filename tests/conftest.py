import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


# ---------------------------------------------------------------------------
# GPU fixtures (instantiated only by tests marked `gpu`)
# ---------------------------------------------------------------------------
_CACHE = {}


def gpu_inputs(name: str, T: int | None = None, **overrides):
    """Host inputs of a named workload (fields replaced by `overrides`) plus their device
    copies (cached per session; the Beam-shaped workloads share one weight draw per
    weight dtype, the dense MLP has its own)."""
    from dataclasses import replace

    import numpy as np
    import torch
    from beam_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[name] if T is None else WORKLOADS[name].with_T(T)
    if overrides:
        w = replace(w, **overrides)
    key_w = (w.H, w.I, w.E, w.weight_dtype, w.seed, w.dense, w.fp8_scales if w.weight_dtype == 2 else None)
    if key_w not in _CACHE:
        print(f"[inputs] generating weights for {name} ...", flush=True)
        full = make_inputs(w)
        dev = {}
        if w.weight_dtype == 0:
            dev["w13"] = torch.from_numpy(full.w13).cuda()
            dev["w2"] = torch.from_numpy(full.w2).cuda()
        elif w.weight_dtype == 1:
            dev["w13"] = torch.from_numpy(full.w13.view(np.int16)).cuda().view(torch.bfloat16)
            dev["w2"] = torch.from_numpy(full.w2.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            dev["w13"] = torch.from_numpy(full.w13).cuda()
            dev["w2"] = torch.from_numpy(full.w2).cuda()
            dev["w13_scale"] = torch.from_numpy(full.w13_scale).cuda()
            dev["w2_scale"] = torch.from_numpy(full.w2_scale).cuda()
        dev["w_router"] = None if full.w_router is None else torch.from_numpy(full.w_router).cuda()
        _CACHE[key_w] = (full, dev)
        print(f"[inputs] weights for {name} resident on the GPU", flush=True)
    full, dev = _CACHE[key_w]
    from beam_inputs import token_inputs, to_bf16_bits, zipf_logit_offsets
    x = token_inputs(w)
    if w.act_dtype == 1:
        x = to_bf16_bits(x)
    bias = zipf_logit_offsets(w.E, w.zipf_s, w.seed) if w.zipf_s is not None else None
    return w, full, dev, x, bias
