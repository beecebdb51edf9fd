"""Torch plumbing around the C ABI: device buffers for one layer call and the
calls themselves.  PyTorch only allocates memory and provides the stream; the
layer's arithmetic runs in libmok's kernels."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import mok


@dataclass
class MoeShape:
    T: int
    d: int
    E: int
    k: int
    F: int
    precision: str = "bf16"
    expert_begin: int = 0
    expert_end: int = -1
    minibatch_rows: int = 0
    ring_bytes: int = 0
    save_for_backward: bool = False
    gating: str = "softmax"       # router affinities: "softmax" or "sigmoid"
    renorm: bool = False          # gates renormalised over the k chosen experts
    separate_route_sort: bool = False  # never the one-launch router + sort of small calls
    gemm_path: str = "auto"            # forward expert products: "auto", "tiled" or "stream" (small calls)
    mxfp8_wgrad: bool = False          # MXFP8 training: weight gradients on the scaled MFMA too
    mover_cus: int = 0                 # ring pipeline: workgroups that only copy (0: one shared queue)

    @property
    def e_end(self):
        return self.E if self.expert_end < 0 else self.expert_end

    @property
    def E_loc(self):
        return self.e_end - self.expert_begin

    def config(self) -> mok.mok_moe_config:
        if self.gating not in ("softmax", "sigmoid"):
            raise ValueError(f"gating must be 'softmax' or 'sigmoid', not {self.gating!r}")
        if self.gemm_path not in ("auto", "tiled", "stream"):
            raise ValueError(f"gemm_path must be 'auto', 'tiled' or 'stream', not {self.gemm_path!r}")
        flags = ((mok.MOK_FLAG_SAVE_FOR_BACKWARD if self.save_for_backward else 0)
                 | (mok.MOK_FLAG_SIGMOID_GATES if self.gating == "sigmoid" else 0)
                 | (mok.MOK_FLAG_RENORM_GATES if self.renorm else 0)
                 | (mok.MOK_FLAG_SEPARATE_ROUTE_SORT if self.separate_route_sort else 0)
                 | (mok.MOK_FLAG_TILED_GEMMS if self.gemm_path == "tiled" else 0)
                 | (mok.MOK_FLAG_STREAM_GEMMS if self.gemm_path == "stream" else 0)
                 | (mok.MOK_FLAG_MXFP8_WGRAD if self.mxfp8_wgrad else 0))
        return mok.make_config(self.T, self.d, self.E, self.F, self.expert_begin, self.e_end, self.precision,
                               self.minibatch_rows, self.ring_bytes, flags, self.mover_cus)

    @property
    def act_dtype(self):
        return torch.float32 if self.precision == "f32" else torch.bfloat16


def _stream():
    return torch.cuda.current_stream().cuda_stream


class MoeBuffers:
    """Outputs, saved state and workspace of one layer configuration on a device."""

    def __init__(self, shape: MoeShape, device="cuda"):
        self.shape = s = shape
        self.cfg = s.config()
        ws, sv = mok.mok_moe_workspace_query(self.cfg, s.k)
        self.layout = mok.mok_moe_saved_layout(self.cfg, s.k)
        self.ws_layout = mok.mok_moe_workspace_layout(self.cfg, s.k)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
        self.saved = torch.empty(max(sv, 256), dtype=torch.uint8, device=device)
        self.out = torch.empty((s.T, s.d), dtype=s.act_dtype, device=device)
        self.topk_idx = torch.empty((s.T, s.k), dtype=torch.int32, device=device)
        self.topk_gate = torch.empty((s.T, s.k), dtype=torch.float32, device=device)
        self.counts = torch.empty(s.E, dtype=torch.int32, device=device)
        self.offsets = torch.empty(s.E + 1, dtype=torch.int32, device=device)
        self.grads = None

    def alloc_grads(self):
        s = self.shape
        dev = self.out.device
        self.grads = dict(
            dx=torch.empty((s.T, s.d), dtype=s.act_dtype, device=dev),
            dW1=torch.empty((s.E_loc, s.F, s.d), dtype=torch.float32, device=dev),
            dW3=torch.empty((s.E_loc, s.F, s.d), dtype=torch.float32, device=dev),
            dW2=torch.empty((s.E_loc, s.d, s.F), dtype=torch.float32, device=dev),
            dgate=torch.empty((s.T, s.k), dtype=torch.float32, device=dev),
            dlogits=torch.empty((s.T, s.E), dtype=torch.float32, device=dev))
        return self.grads

    def device_status(self):
        """(status, failed-check bits) of the last call on this workspace: the
        two int32 words the library's device-side checks write (synchronises
        with the device, which the library itself never does)."""
        off = self.ws_layout["status"]
        w = self.workspace[off:off + 8].view(torch.int32).cpu()
        return int(w[0]), int(w[1])

    def workspace_view(self, name: str, dtype, shape):
        """A view of one array inside the workspace (see mok_workspace_layout)."""
        off = self.ws_layout[name]
        n = 1
        for v in shape:
            n *= v
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype).view(*shape)

    def saved_view(self, name: str, dtype, shape):
        """A view of one array inside the saved buffer (see mok_saved_layout)."""
        off = self.layout[name]
        n = 1
        for v in shape:
            n *= v
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.saved[off:off + nbytes].view(dtype).view(*shape)

    def forward(self, x, logits, W1, W3, W2, w_scales=None, stream=None):
        mok.mok_moe_forward(x, logits, W1, W3, W2, self.shape.k, self.cfg, w_scales, self.out, self.topk_idx,
                            self.topk_gate, self.counts, self.offsets, self.saved, self.workspace,
                            _stream() if stream is None else stream)
        return self.out

    def forward_router(self, x, Wr, W1, W3, W2, w_scales=None, logits=None, stream=None):
        """The forward with the router GEMM in front: logits = x . Wr^T are
        computed (into `logits`, or a buffer of this object) and routed in
        the same call; returns out.  The logits are kept in self.logits for
        the backward."""
        s = self.shape
        if logits is None:
            logits = getattr(self, "logits", None)
            if logits is None or tuple(logits.shape) != (s.T, s.E):
                logits = torch.empty((s.T, s.E), dtype=torch.float32, device=self.out.device)
        self.logits = logits
        mok.mok_moe_forward_router(x, Wr, W1, W3, W2, s.k, self.cfg, w_scales, logits, self.out, self.topk_idx,
                                   self.topk_gate, self.counts, self.offsets, self.saved, self.workspace,
                                   _stream() if stream is None else stream)
        return self.out

    def backward(self, dout, x, logits, W1, W3, W2, stream=None):
        g = self.grads or self.alloc_grads()
        mok.mok_moe_backward(dout, x, logits, W1, W3, W2, self.shape.k, self.cfg, self.saved, g["dx"], g["dW1"],
                             g["dW3"], g["dW2"], g["dgate"], g["dlogits"], self.workspace,
                             _stream() if stream is None else stream)
        return g


    def backward_mxfp8(self, dout, x, logits, wt, stream=None):
        """MXFP8 backward; wt = quantize_mxfp8_backward_weights(W1, W3, W2)."""
        g = self.grads or self.alloc_grads()
        mok.mok_moe_backward_mxfp8(dout, x, logits, self.shape.k, self.cfg, wt[0], wt[1], self.saved, g["dx"],
                                   g["dW1"], g["dW3"], g["dW2"], g["dgate"], g["dlogits"], self.workspace,
                                   _stream() if stream is None else stream)
        return g


def quantize_mxfp8_backward_weights(W1: torch.Tensor, W3: torch.Tensor, W2: torch.Tensor):
    """Transposed MXFP8 weights of the backward pass: (codes, scales) with
    codes = [W2^T as [E, F, d] | [W1^T | W3^T] as [E, d, 2F]] flattened and
    scales in pair planes (see include/mok.h)."""
    E, F, d = W1.shape
    n = E * F * d
    q = torch.empty(3 * n, dtype=torch.uint8, device=W1.device)
    sc = torch.empty(3 * n // 32, dtype=torch.uint8, device=W1.device)
    mok.mok_quantize_mxfp8_backward_weights(W1, W3, W2, E, d, F, q, sc, _stream())
    return q, sc


def quantize_mxfp8(w: torch.Tensor):
    """E4M3 codes and E8M0 scales of a bf16 tensor along its last axis.

    Scales come in the library's pair-plane layout, shape [K/64, rows, 2]
    with rows = numel / K (see scales_by_row for the [rows, K/32] view)."""
    K = w.shape[-1]
    rows = w.numel() // K
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    sc = torch.empty((K // 64, rows, 2), dtype=torch.uint8, device=w.device)
    mok.mok_quantize_mxfp8(w, rows, K, q, sc, _stream())
    return q, sc


def quantize_mxfp4(w: torch.Tensor):
    """E2M1 codes (two per byte, the lower element in the low nibble; shape
    [..., K/2]) and E8M0 scales [K/64, rows, 2] of a bf16 tensor along its
    last axis, for the weights of an MXFP4 forward."""
    K = w.shape[-1]
    rows = w.numel() // K
    q = torch.empty(w.shape[:-1] + (K // 2,), dtype=torch.uint8, device=w.device)
    sc = torch.empty((K // 64, rows, 2), dtype=torch.uint8, device=w.device)
    mok.mok_quantize_mxfp4(w, rows, K, q, sc, _stream())
    return q, sc


def scales_by_row(sc: torch.Tensor) -> torch.Tensor:
    """[rows, K/32] view (a copy) of pair-plane scales [K/64, rows, 2]."""
    planes, rows, _ = sc.shape
    return sc.permute(1, 0, 2).reshape(rows, planes * 2)


def router_logits(x: torch.Tensor, Wr: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 logits [T, E] = x [T, d] . Wr^T for bf16 x and Wr [E, d]."""
    T, d = x.shape
    E = Wr.shape[0]
    if x.dtype != torch.bfloat16 or Wr.dtype != torch.bfloat16 or Wr.shape[1] != d:
        raise ValueError("router_logits: bf16 x [T, d] and Wr [E, d] expected")
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    mok.mok_router_logits(x.contiguous(), Wr.contiguous(), T, d, E, out, _stream())
    return out


def router_logits_backward(x: torch.Tensor, Wr: torch.Tensor, dlogits: torch.Tensor):
    """(dx, dWr) = (dlogits . Wr, dlogits^T . x), both fp32."""
    T, d = x.shape
    E = Wr.shape[0]
    if dlogits.dtype != torch.float32 or tuple(dlogits.shape) != (T, E):
        raise ValueError("router_logits_backward: fp32 dlogits [T, E] expected")
    dx = torch.empty((T, d), dtype=torch.float32, device=x.device)
    dWr = torch.empty((E, d), dtype=torch.float32, device=x.device)
    mok.mok_router_logits_backward(x.contiguous(), Wr.contiguous(), dlogits.contiguous(), T, d, E, dx, dWr,
                                   _stream())
    return dx, dWr
