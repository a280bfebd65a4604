"""A ``Linear8bitLt``-style PyTorch module over the lli8 C-ABI.

Follows the interface the pages document for bitsandbytes' ``Linear8bitLt``
("Class Linear8bitLt", its ``__init__`` arguments and the conversion example;
the issue page's ``state.idx``; "Hugging Face integrates LLM.int8() ...",
section "Integration into transformers", for ``weight.CB`` / ``weight.SCB``
and the recovery ``(CB * SCB) / 127``):

* ``Linear8bitLt(input_features, output_features, bias=True,
  has_fp16_weights=True, threshold=0.0, index=None, device=None)``;
* ``has_fp16_weights=False``: the 16-bit weight is quantised once, when the
  module lands on the GPU (``.to("cuda")``, ``.cuda()``, or built there), and
  the parameter then holds the int8 codes, with ``weight.CB`` (the same int8
  tensor) and ``weight.SCB`` (fp32 row absmax);
* ``has_fp16_weights=True``: the weight stays 16-bit and is quantised on every
  forward;
* ``threshold``: activation columns with some |x| > threshold are the outlier
  columns of that forward; ``threshold <= 0`` turns the split off;
* ``state.idx``: the ascending outlier columns of the last forward.

Every step of the forward runs in the library's HIP kernels; this module only
keeps tensors and calls the binding.  It has no CPU path: a forward on CPU
tensors raises.

Persistence (the pages list INT8 checkpoints without CB/SCB as a gap): a
quantised module's ``state_dict()`` carries ``weight`` (int8 CB) and ``SCB``,
and ``load_state_dict`` accepts either that form or a 16-bit ``weight`` (as
from ``torch.nn.Linear``).  ``save_int8`` / ``load_int8`` write and read such a
state dict as safetensors.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from ._lib import Workspace, lli8_int8_linear, lli8_quant_weight_rowwise, lli8_recover_weight

__all__ = ["Linear8bitLt", "Int8State", "save_int8", "load_int8"]

class Int8State:
    """What the last forward left: its workspace (CA, SCA, the outlier set)."""

    def __init__(self):
        self.ws: Optional[Workspace] = None
        self.CB: Optional[torch.Tensor] = None   # the codes the last forward used
        self.SCB: Optional[torch.Tensor] = None

    @property
    def idx(self) -> Optional[torch.Tensor]:
        """Ascending outlier columns of the last forward (device int32; reading
        the count synchronises with the stream)."""
        if self.ws is None:
            return None
        n = int(self.ws.n_idx.item())
        return self.ws.idx[:n]


def _is_int8(t: Optional[torch.Tensor]) -> bool:
    return t is not None and t.dtype == torch.int8


class Linear8bitLt(torch.nn.Module):
    """out = LLM.int8() linear of x [..., input_features] -> [..., output_features]."""

    def __init__(self, input_features: int, output_features: int, bias: bool = True,
                 has_fp16_weights: bool = True, threshold: float = 0.0, index=None, device=None,
                 dtype: torch.dtype = torch.float16):
        super().__init__()
        if dtype not in (torch.float16, torch.bfloat16):
            raise TypeError("the 16-bit weight dtype must be float16 or bfloat16")
        self.in_features = int(input_features)
        self.out_features = int(output_features)
        self.has_fp16_weights = bool(has_fp16_weights)
        self.threshold = float(threshold)
        self.index = index  # accepted for the documented signature; not used
        w = torch.empty((self.out_features, self.in_features), dtype=dtype, device=device)
        b = torch.empty((self.out_features,), dtype=dtype, device=device) if bias else None
        if w.device.type != "meta":
            # torch.nn.Linear's default initialisation, drawn in fp32
            bound = 1.0 / math.sqrt(self.in_features) if self.in_features > 0 else 0.0
            with torch.no_grad():
                w.copy_(torch.empty(w.shape, dtype=torch.float32, device=w.device).uniform_(-bound, bound))
                if b is not None:
                    b.copy_(torch.empty(b.shape, dtype=torch.float32, device=b.device).uniform_(-bound, bound))
        self.weight = torch.nn.Parameter(w, requires_grad=False)
        if b is not None:
            self.bias = torch.nn.Parameter(b, requires_grad=False)
        else:
            self.register_parameter("bias", None)
        self._scb: Optional[torch.Tensor] = None  # fp32 row scales once quantised (kept fp32 under .half())
        self.state = Int8State()
        self._bias_cast: Optional[torch.Tensor] = None
        if self.weight.is_cuda and not self.has_fp16_weights:
            self._quantize()

    # ----------------------------------------------------------- weights ----

    @property
    def SCB(self) -> Optional[torch.Tensor]:
        return self._scb

    @property
    def is_quantized(self) -> bool:
        return _is_int8(self.weight) and self._scb is not None

    def _set_int8(self, CB: torch.Tensor, SCB: torch.Tensor):
        self.weight = torch.nn.Parameter(CB, requires_grad=False)
        self._scb = SCB
        self.weight.CB = CB
        self.weight.SCB = SCB

    def _quantize(self):
        """16-bit weight on the GPU -> int8 codes and row scales (lli8 kernel)."""
        W = self.weight.data
        if not W.is_contiguous():
            W = W.contiguous()
        CB, SCB = lli8_quant_weight_rowwise(W)
        self._set_int8(CB, SCB)

    def _apply(self, fn, *args, **kwargs):
        int8 = self.is_quantized
        out = super()._apply(fn, *args, **kwargs)
        if int8 and self.weight.dtype != torch.int8:
            raise RuntimeError("a quantised Linear8bitLt keeps its int8 weight; cast the input instead")
        if self.is_quantized:  # the scales and attributes follow the moved weight
            self._scb = self._scb.to(self.weight.device)
            self.weight.CB = self.weight.data
            self.weight.SCB = self._scb
        elif self.weight.is_cuda and not self.has_fp16_weights:
            self._quantize()  # "quantization happens here"
        self._bias_cast = None
        self.state = Int8State()
        return out

    def _save_to_state_dict(self, destination, prefix, keep_vars):
        super()._save_to_state_dict(destination, prefix, keep_vars)
        if self._scb is not None:
            destination[prefix + "SCB"] = self._scb if keep_vars else self._scb.detach()

    def _load_from_state_dict(self, state_dict, prefix, local_metadata, strict, missing_keys,
                              unexpected_keys, error_msgs):
        wkey, skey = prefix + "weight", prefix + "SCB"
        w = state_dict.get(wkey)
        if _is_int8(w):
            scb = state_dict.get(skey)
            if scb is None:
                error_msgs.append(f"{skey} is missing: an int8 weight needs its row scales")
                return
            if tuple(w.shape) != (self.out_features, self.in_features) or tuple(scb.shape) != (self.out_features,):
                error_msgs.append(f"int8 weight {tuple(w.shape)} / SCB {tuple(scb.shape)} do not fit "
                                  f"({self.out_features}, {self.in_features})")
                return
            dev = self.weight.device
            self._set_int8(w.detach().to(dev).contiguous().clone(), scb.detach().to(dev, torch.float32).contiguous().clone())
            rest = {k: v for k, v in state_dict.items() if k not in (wkey, skey)}
            super()._load_from_state_dict(rest, prefix, local_metadata, False, [], [], error_msgs)
            if self.bias is not None and (prefix + "bias") not in state_dict:
                missing_keys.append(prefix + "bias")
            return
        if w is not None and self.is_quantized:
            # a 16-bit weight into a quantised module: quantise it here
            W = w.detach().to(self.weight.device)
            if W.dtype not in (torch.float16, torch.bfloat16):
                W = W.to(torch.float16)
            if tuple(W.shape) != (self.out_features, self.in_features):
                error_msgs.append(f"weight {tuple(W.shape)} does not fit ({self.out_features}, {self.in_features})")
                return
            if not W.is_cuda:
                error_msgs.append("a quantised Linear8bitLt lives on the GPU; its 16-bit weight is quantised there")
                return
            CB, SCB = lli8_quant_weight_rowwise(W.contiguous())
            self._set_int8(CB, SCB)
            rest = {k: v for k, v in state_dict.items() if k not in (wkey, skey)}
            super()._load_from_state_dict(rest, prefix, local_metadata, False, [], [], error_msgs)
            return
        # 16-bit weight into a 16-bit module: the ordinary path (SCB not expected)
        rest = {k: v for k, v in state_dict.items() if k != skey}
        super()._load_from_state_dict(rest, prefix, local_metadata, strict, missing_keys,
                                      unexpected_keys, error_msgs)
        self._bias_cast = None

    def recovered_weight(self) -> torch.Tensor:
        """(CB * SCB) / 127 in the bias' 16-bit dtype (float16 without a bias):
        the recovery form of "Integration into transformers", computed by the
        library (lli8_recover_weight).  A convenience outside the forward path."""
        if not self.is_quantized:
            raise RuntimeError("the module is not quantised (has_fp16_weights=True or not on the GPU)")
        dt = self.bias.dtype if self.bias is not None else torch.float16
        return lli8_recover_weight(self.weight.data, self._scb, dtype=dt)

    # ----------------------------------------------------------- forward ----

    def _workspace(self, T: int, device) -> Workspace:
        ws = self.state.ws
        if ws is not None and ws.fits(T, self.in_features, self.out_features, False) and ws.CA.device == device:
            return ws
        # one buffer, with room for the recovered weights of 8 outlier chunks
        # (256 columns); the GEMM gathers any further ones from CB itself
        return Workspace(T, self.in_features, self.out_features, None, device, want_acc=False)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not x.is_cuda:
            raise RuntimeError("Linear8bitLt runs on the GPU only (no CPU path): move the module "
                               "and the input to the GPU")
        if x.dtype is not torch.float16 and x.dtype is not torch.bfloat16:
            raise TypeError(f"input dtype {x.dtype}: LLM.int8() takes float16 or bfloat16 activations")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"input has {x.shape[-1]} features, the layer {self.in_features}")
        if not self.has_fp16_weights and self._scb is not None and self.weight.dtype is torch.int8:
            CB, SCB = self.weight.data, self._scb  # the common case, checked cheaply
        elif self.has_fp16_weights:
            if _is_int8(self.weight):
                raise RuntimeError("has_fp16_weights=True needs a 16-bit weight")
            W = self.weight.data
            if not W.is_cuda:
                raise RuntimeError("move the module to the GPU first")
            W = W if W.is_contiguous() else W.contiguous()
            st = self.state
            reuse = st.CB is not None and st.CB.shape == W.shape and st.CB.device == W.device
            CB, SCB = lli8_quant_weight_rowwise(W, st.CB if reuse else None, st.SCB if reuse else None)
        else:
            if not self.is_quantized:
                if not self.weight.is_cuda:
                    raise RuntimeError("move the module to the GPU first: the weight is quantised there")
                self._quantize()
            CB, SCB = self.weight.data, self._scb
        if CB.device != x.device:
            raise RuntimeError(f"input on {x.device}, weight on {CB.device}")
        bias = None
        if self.bias is not None:
            bc = self._bias_cast
            if bc is None or bc.dtype is not x.dtype or bc.device != x.device:
                bc = self._bias_cast = self.bias.data.to(device=x.device, dtype=x.dtype).contiguous()
            bias = bc
        xc = x if x.is_contiguous() else x.contiguous()
        T = xc.numel() // self.in_features if self.in_features else 0
        st = self.state
        ws = st.ws
        if ws is None or ws.T != T or ws.CA.device != x.device:
            ws = self._workspace(T, x.device)
        out, ws = lli8_int8_linear(xc, CB, SCB, bias, self.threshold, ws=ws)
        st.ws, st.CB, st.SCB = ws, CB, SCB
        return out

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, has_fp16_weights={self.has_fp16_weights}, "
                f"threshold={self.threshold}, quantized={self.is_quantized}")


def save_int8(module_or_state: "torch.nn.Module | dict", path: str) -> None:
    """Write a state dict (int8 weights with their SCB, or 16-bit ones) as
    safetensors; tensors are copied to the host."""
    from safetensors.torch import save_file
    sd = module_or_state.state_dict() if isinstance(module_or_state, torch.nn.Module) else module_or_state
    save_file({k: v.detach().contiguous().cpu() for k, v in sd.items() if v is not None}, path)


def load_int8(path: str, device="cpu") -> dict:
    """Read a state dict written by save_int8 (safetensors: no code is run)."""
    from safetensors.torch import load_file
    return load_file(path, device=str(device))
