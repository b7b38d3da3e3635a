"""Deployment form of a calibrated block and the saved calibration state.

* ``export_block``: for a weight-only block (abits 16), the packed codes of every
  linear with their (h, z), the biases produced by folding the LET sites, the
  attention-output pair folded into the value projection, and the gains 1/s that
  take the input sites' place in the norms in front (the FFN input's scale for the
  FFN alone).  Paper reading, section "LET": after calibration the transformation
  is folded away and the deployed block keeps its original operators; section
  "LWC": the deployed weight is the integer code with its step and zero point.
  Every arithmetic step runs in the library's kernels (fake quantizer, packing,
  fold); this module only selects the parameter slices and collects the outputs.
* ``save`` / ``load``: tensors to a safetensors file (e.g. the exported block).
* ``save_state`` / ``load_state``: the packed parameter vector, the AdamW moments
  and the step count, so a calibration can resume where it stopped.
"""
from __future__ import annotations

import json
from typing import Dict, List

import torch

from . import (BlockDesc, block_theta_layout, fold_linear, lwc_fakequant, pack_codes)

_ALL = ("q", "k", "v", "o", "gate", "up", "down")


def theta_names(desc: BlockDesc) -> List[str]:
    """Names of the packed parameter vector's entries, in the library's order."""
    lin = ("gate", "up", "down") if desc.ffn_only else _ALL
    names = []
    for n in lin:
        names += ["a_gamma_" + n, "a_beta_" + n]
    for site in (("ffn",) if desc.ffn_only else ("qkv", "o", "ffn")):
        names += ["s_" + site, "delta_" + site]
    if not desc.ffn_only and desc.abits < 16:
        names.append("s_a")
    return names


def theta_dict(desc: BlockDesc, theta: torch.Tensor) -> Dict[str, torch.Tensor]:
    offs, _, total = block_theta_layout(desc)
    ends = list(offs[1:]) + [total]
    return {n: theta[a:b] for n, a, b in zip(theta_names(desc), offs, ends)}


def export_block(desc: BlockDesc, weights, theta: torch.Tensor) -> Dict[str, torch.Tensor]:
    """weights: the 7 bf16 [C_out x C_in] device tensors (q, k, v, o, gate, up, down;
    None for the attention ones of an FFN-only block); theta: the calibrated packed
    parameters.  Returns {name: device tensor}: <lin>.words (int32 view of the packed
    codes), <lin>.h, <lin>.z, <lin>.bias, attn_norm.gain, ffn_in.gain."""
    if desc.abits < 16:
        raise ValueError("the weight-only fold needs abits 16 (an activation quantizer "
                         "sits between the LET site and its layer)")
    th = theta_dict(desc, theta)
    W = dict(zip(_ALL, weights))
    g, nb = int(desc.group), int(desc.wbits)
    out: Dict[str, torch.Tensor] = {}

    def lin(name, s=None, delta=None, s_o=None, delta_o=None, want_gain=False):
        Wn = W[name]
        N, K = Wn.shape
        r = lwc_fakequant(Wn, th["a_gamma_" + name], th["a_beta_" + name], nb, s, delta,
                          out_dtype=torch.bfloat16, want_bias=delta is not None,
                          want_codes=True, group=g)
        words = pack_codes(r["codes"], nb)
        out[name + ".words"], out[name + ".z"] = words, r["z"]
        res = fold_linear(words, nb, N, K, r["h"], r["z"], g, r["B_tilde"], s, delta, s_o,
                          delta_o, want_gain=want_gain)
        out[name + ".bias"] = res[0]
        out[name + ".h"] = res[1] if s_o is not None else r["h"]
        return res[2] if want_gain else None

    if not desc.ffn_only:
        s, d = th["s_qkv"], th["delta_qkv"]
        out["attn_norm.gain"] = lin("q", s, d, want_gain=True)
        lin("k", s, d)
        lin("v", s, d, th["s_o"], th["delta_o"])
        grp = int(desc.n_q // desc.n_kv)
        hd = int(desc.head_dim)
        s_o = th["s_o"].view(-1, 1, hd).expand(-1, grp, hd).reshape(-1).contiguous()
        d_o = th["delta_o"].view(-1, 1, hd).expand(-1, grp, hd).reshape(-1).contiguous()
        # o keeps its own quantizer on s_o W_o and the bias fold B~ = delta_o W_o: its input
        # is exactly the folded site's output
        Wo = W["o"]
        r = lwc_fakequant(Wo, th["a_gamma_o"], th["a_beta_o"], nb, s_o, d_o,
                          out_dtype=torch.bfloat16, want_bias=True, want_codes=True, group=g)
        out["o.words"], out["o.h"], out["o.z"] = pack_codes(r["codes"], nb), r["h"], r["z"]
        out["o.bias"] = r["B_tilde"]
    s, d = th["s_ffn"], th["delta_ffn"]
    out["ffn_in.gain"] = lin("gate", s, d, want_gain=True)
    lin("up", s, d)
    lin("down")
    return out


def save(path: str, tensors: Dict[str, torch.Tensor], meta: Dict[str, str] = None) -> None:
    from safetensors.torch import save_file
    save_file({k: v.detach().contiguous().cpu() for k, v in tensors.items()}, path,
              metadata=meta or {})


def load(path: str, device: str = "cpu") -> Dict[str, torch.Tensor]:
    from safetensors.torch import load_file
    return load_file(path, device=device)


def _desc_meta(desc: BlockDesc) -> Dict[str, str]:
    keys = ("T", "d", "n_q", "n_kv", "head_dim", "F", "wbits", "abits", "ffn_only", "group",
            "optimizer", "lr_lwc", "lr_let", "beta1", "beta2", "adam_eps", "weight_decay")
    return {"block_desc": json.dumps({k: getattr(desc, k) for k in keys})}


def save_state(path: str, desc: BlockDesc, theta, m, v, step: int) -> None:
    """The calibration state (packed parameters, AdamW moments, step count)."""
    meta = _desc_meta(desc)
    meta["step"] = str(int(step))
    save(path, {"theta": theta, "adam_m": m, "adam_v": v}, meta)


def load_state(path: str, device: str = "cpu"):
    """Returns (theta, m, v, step, desc fields dict)."""
    from safetensors import safe_open
    with safe_open(path, framework="pt", device=device) as f:
        meta = f.metadata()
        t = {k: f.get_tensor(k) for k in f.keys()}
    return (t["theta"], t["adam_m"], t["adam_v"], int(meta["step"]),
            json.loads(meta["block_desc"]))
