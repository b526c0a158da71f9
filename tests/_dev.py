"""numpy <-> device tensor helpers for the GPU tests (bf16 travels as its bit pattern)."""
import numpy as np
import torch

from gated_delta_rule_63_amd import inputs


def to_dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy; bf16 comes back as its uint16 bit pattern."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    return inputs.widen(to_host(t))


def problem_to_dev(p):
    d = {
        "q": to_dev(p.q), "k": to_dev(p.k), "v": to_dev(p.v), "g": to_dev(p.g), "beta": to_dev(p.beta),
        "cu": to_dev(p.cu_seqlens.astype(np.int32)),
    }
    if p.initial_state is not None:
        d["h0"] = to_dev(p.initial_state)
    return d


def oracle_inputs(p):
    return [inputs.widen(x) for x in (p.q, p.k, p.v, p.g, p.beta)]
