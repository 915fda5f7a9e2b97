"""Test helpers: storage-form conversions between torch tensors and NumPy."""
import numpy as np
import torch


def np_store(t):
    """Torch tensor -> NumPy array in storage form (bf16/fp16 codes as uint16)."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def np_f64(t):
    """Torch tensor -> float64 NumPy values."""
    return t.detach().cpu().to(torch.float64).numpy()


def layer_np(L, prefix=""):
    """Weights of one layer (generator dict) as a dict of NumPy storage arrays."""
    out = {}
    for n in ("gate", "up", "down"):
        w = L.get(prefix + n) if prefix else L.get("w_" + n)
        s = L.get(prefix + "s_" + n) if prefix else L.get("s_" + n)
        out["w_" + n] = np_store(w)
        out["s_" + n] = np_store(s)
    return out


def shared_np(L):
    if L.get("sh_gate") is None:
        return None
    return {"w_gate": np_store(L["sh_gate"]), "w_up": np_store(L["sh_up"]),
            "w_down": np_store(L["sh_down"]), "s_gate": np_store(L["sh_s_gate"]),
            "s_up": np_store(L["sh_s_up"]), "s_down": np_store(L["sh_s_down"])}


def rel_err_tokenwise(y, r):
    """max_t ||y_t - r_t||_inf / ||r_t||_inf (per-token infinity norm)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    num = np.abs(y - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((num / den).max())
