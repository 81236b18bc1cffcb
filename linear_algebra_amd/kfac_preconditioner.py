"""K-FAC preconditioning of real layers on one GPU.

The method of "Accelerating Distributed K-FAC with Smart Parallelism of
Computing and Communication Tasks" attaches to every layer a forward
pre-hook, which takes the layer input for the factor A, and a backward hook,
which takes the gradient of the layer output for the factor G (pipelining
paragraph; the optimizer paragraph traverses the model's layers to find the
factor sizes).  This class does the same for ``torch.nn.Linear`` and
``torch.nn.Conv2d`` and runs one step of the hot path per call of
:meth:`step`, each stage one grouped call of the C library:

    kfac_im2col / kfac_grad_rows    factor inputs of every layer
    kfac_factors                    A and G with their running average
    kfac_damped_inverse             every ``inv_update_freq`` steps
    kfac_grad_matrix                [dW | db] of every layer
    kfac_precondition               (G + gamma I)^-1 [dW | db] (A + gamma I)^-1
    kfac_grad_matrix                the result back into .grad

The caller's optimizer then applies the preconditioned gradients.  Readings:
the rows of a convolution's factor inputs are its patches (batch * H_out *
W_out rows); the loss is taken as averaged over the batch, so the output
gradients are multiplied by the batch size to give per-sample gradients
(``batch_averaged=False`` leaves them as they are).
"""
from __future__ import annotations

from typing import List

from . import (KFAC_PACK, KFAC_UNPACK, conv_out_hw, kfac_damped_inverse, kfac_factors, kfac_grad_matrix,
               kfac_grad_rows, kfac_im2col, kfac_precondition)


class KFACPreconditioner:
    def __init__(self, model, damping: float = 1e-3, factor_decay: float = 0.95, inv_update_freq: int = 10,
                 batch_averaged: bool = True):
        import torch
        self.damping = float(damping)
        self.eps = float(factor_decay)
        self.inv_update_freq = int(inv_update_freq)
        self.batch_averaged = bool(batch_averaged)
        self.layers: List[torch.nn.Module] = []
        for m in model.modules():
            if isinstance(m, torch.nn.Conv2d):
                if m.groups != 1 or isinstance(m.padding, str) or m.padding_mode != "zeros":
                    raise ValueError("KFACPreconditioner: Conv2d needs groups=1, numeric zero padding")
                self.layers.append(m)
            elif isinstance(m, torch.nn.Linear):
                self.layers.append(m)
        if not self.layers:
            raise ValueError("KFACPreconditioner: the model has no Linear or Conv2d layer")
        self._inputs = {}
        self._grads = {}
        self._handles = []
        for m in self.layers:
            self._handles.append(m.register_forward_pre_hook(self._save_input))
            self._handles.append(m.register_full_backward_hook(self._save_grad))
        self.steps = 0
        self.A = self.G = self.Ainv = self.Ginv = None
        self.info = None
        self.failed: List[int] = []

    def _save_input(self, module, inputs):
        if module.training:
            self._inputs[module] = inputs[0].detach()

    def _save_grad(self, module, grad_input, grad_output):
        if module.training:
            self._grads[module] = grad_output[0].detach()

    def remove(self) -> None:
        for h in self._handles:
            h.remove()
        self._handles = []

    @staticmethod
    def _shape(m):
        import torch
        if isinstance(m, torch.nn.Conv2d):
            return dict(kernel=tuple(m.kernel_size), stride=tuple(m.stride), padding=tuple(m.padding),
                        dilation=tuple(m.dilation), ones=m.bias is not None)
        return dict(kernel=(1, 1), stride=(1, 1), padding=(0, 0), dilation=(1, 1), ones=m.bias is not None)

    def factor_inputs(self):
        """The factor inputs of every layer: (a, g) lists, rows as in the
        library's kfac_im2col and kfac_grad_rows."""
        import torch
        xs, shapes, outs, gys, gouts = [], [], [], [], []
        for m in self.layers:
            x, gy = self._inputs[m], self._grads[m]
            if isinstance(m, torch.nn.Linear):
                x = x.reshape(-1, x.shape[-1], 1, 1)
                gy = gy.reshape(-1, gy.shape[-1])
            x = x.contiguous()
            gy = gy.contiguous()
            s = self._shape(m)
            oh, ow = conv_out_hw(x.shape[2], x.shape[3], *s["kernel"], s["stride"], s["padding"], s["dilation"])
            xs.append(x)
            shapes.append(s)
            outs.append(torch.empty(x.shape[0] * oh * ow, x.shape[1] * s["kernel"][0] * s["kernel"][1] + int(s["ones"]),
                                    dtype=x.dtype, device=x.device))
            hw = 1
            for v in gy.shape[2:]:
                hw *= v
            gys.append(gy)
            gouts.append(torch.empty(gy.shape[0] * hw, gy.shape[1], dtype=gy.dtype, device=gy.device))
        kfac_im2col(xs, shapes, outs)
        # one scale for all layers: they share the batch
        batch = self._inputs[self.layers[0]].shape[0]
        scale = float(batch) if self.batch_averaged else 1.0
        kfac_grad_rows(gys, scale, gouts)
        return outs, gouts

    def _update_inverses(self, first: bool) -> None:
        """Damped inverses of every factor.  A factor whose Cholesky
        factorisation fails (info != 0: a non-finite input, or gamma = 0 on a
        singular factor) keeps its previous inverse and is listed in
        ``self.failed``; with no previous inverse the step raises."""
        import warnings

        import torch
        facs = self.A + self.G
        new = [torch.empty_like(f) for f in facs]
        kfac_damped_inverse(facs, self.damping, new, self.info)
        info = self.info.cpu().tolist()
        self.failed = [k for k, v in enumerate(info) if v != 0]
        if self.failed and first:
            raise RuntimeError(f"KFACPreconditioner: damped inverse failed (info {info}) with no previous inverse")
        nl = len(self.layers)
        for k, z in enumerate(new):
            if info[k] == 0:
                if k < nl:
                    self.Ainv[k] = z
                else:
                    self.Ginv[k - nl] = z
        if self.failed:
            warnings.warn(f"KFACPreconditioner: damped inverse failed for factors {self.failed} "
                          f"(info {[info[k] for k in self.failed]}); their previous inverses are kept")

    def step(self) -> None:
        """Precondition the gradients of every layer in place."""
        import torch
        missing = [m for m in self.layers if m not in self._inputs or m not in self._grads]
        if missing:
            raise RuntimeError("KFACPreconditioner.step: run a forward and backward pass first")
        a, g = self.factor_inputs()
        dev = a[0].device
        first = self.A is None
        if first:
            self.A = [torch.zeros(t.shape[1], t.shape[1], device=dev) for t in a]
            self.G = [torch.zeros(t.shape[1], t.shape[1], device=dev) for t in g]
            self.Ainv = [torch.empty_like(f) for f in self.A]
            self.Ginv = [torch.empty_like(f) for f in self.G]
            self.info = torch.zeros(2 * len(self.layers), dtype=torch.int32, device=dev)
        # the factor stage takes one input dtype per call
        for group in (a, g):
            if len({t.dtype for t in group}) != 1:
                raise ValueError("KFACPreconditioner: all layers must share one dtype")
        kfac_factors(a, self.A, self.eps, first)
        kfac_factors(g, self.G, self.eps, first)
        if self.steps % self.inv_update_freq == 0:
            self._update_inverses(first)
        wg = [m.weight.grad for m in self.layers]
        bg = [m.bias.grad if m.bias is not None else None for m in self.layers]
        mats = [torch.empty(w.shape[0], w[0].numel() + (b is not None), device=dev) for w, b in zip(wg, bg)]
        kfac_grad_matrix(wg, bg, mats, KFAC_PACK)
        outs = [torch.empty_like(t) for t in mats]
        kfac_precondition(self.Ginv, mats, self.Ainv, outs)
        kfac_grad_matrix(wg, bg, outs, KFAC_UNPACK)
        self.steps += 1
