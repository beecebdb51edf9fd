"""Seeded synthetic workloads for the MoE layer (inputs only).

This module builds the input tensors of every workload: token activations,
router logits, expert weights and the incoming output gradient.  It holds none
of the layer's arithmetic (no softmax, no top-k, no sort, no FFN, no combine);
both the CPU oracle and the HIP path receive the arrays it produces.

Every value is a pure function of (workload seed, stream id, row id, column id)
through a counter-based integer hash, so a single token's activations can be
regenerated from its token id alone, on any device.  The hash works on int64
torch tensors holding 32-bit values (every product stays below 2**63), so the
integer part is bit-identical on CPU and GPU; the final Box-Muller transform
runs in float64.  Tests that compare devices always copy one device's arrays to
the other rather than relying on cross-device equality of that last step.

Stream ids: 0 = x, 1 = logit noise, 2 = W1, 3 = W3, 4 = W2, 5 = Wr (router
weight of the tiny workload), 6 = per-expert logit bias, 7 = incoming output
gradient, 8 = expert popularity permutation, 9 = incoming router-logit
gradient (router GEMM inputs).

Workloads (sizes from the pages' layer benchmark: expert parallelism of 64 with
2,048 tokens per GPU before routing, and the Kimi-2.5 shape with hidden 7168 and
expert width 2048; kucoin.com «Cursor's MoK réalise une amélioration des
performances de 2,37x sur NVIDIA GB300 NVL72», sections 02 and 03):

  tiny_fp32   T=256  d=128  E=8   k=2 F=256   fp32, logits = x·Wr
  bf16_fwd    T=4096 d=2048 E=64  k=6 F=1408  logits N(0,1) + per-expert N(0,1) bias
  ep_share    U tokens of 64*2048 routed top-8 over 256 experts with Zipf(1.1)
              popularity; the tokens with a pair on local experts 0..3; d=7168 F=2048
  ep_mxfp8    ep_share in MXFP8
  bf16_train  T=8192 d=4096 E=128 k=8 F=1536, Zipf(1.2) popularity (expert 0 hottest)
  mxfp8_train bf16_train in MXFP8
  mxfp8_infer, mxfp4_infer  bf16_train's forward alone in MXFP8 / MXFP4
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_M32 = 0xFFFFFFFF
# Odd multipliers below 2**31, so that a 32-bit value times one fits in int64.
_C1 = 0x7FEB352D
_C2 = 0x5BD1E995
_GOLD = 0x9E3779B9

S_X, S_LOGIT, S_W1, S_W3, S_W2, S_WR, S_BIAS, S_DOUT, S_PERM, S_DLOGIT = range(10)


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """Avalanche a tensor of 32-bit values held in int64 (two xorshift-multiply rounds)."""
    x = x ^ (x >> 16)
    x = (x * _C1) & _M32
    x = x ^ (x >> 15)
    x = (x * _C2) & _M32
    x = x ^ (x >> 16)
    x = (x * _C1) & _M32
    x = x ^ (x >> 15)
    return x


def _mix32_int(v: int) -> int:
    return int(_mix32(torch.tensor([v & _M32], dtype=torch.int64))[0])


def _stream_key(seed: int, stream: int) -> int:
    return _mix32_int(_mix32_int(seed * 0x3C6EF372 + 0x1234567) ^ (stream * 0x1B873593 & _M32))


def uniform_bits(seed: int, stream: int, rows: torch.Tensor, ncols: int, salt: int = 0) -> torch.Tensor:
    """32-bit hash for every (row, col); rows is an int64 tensor of global row ids."""
    key = _stream_key(seed, stream) ^ (salt * 0x2545F491 & _M32)
    hr = _mix32((rows.to(torch.int64) ^ key) & _M32)
    cols = torch.arange(ncols, dtype=torch.int64, device=rows.device)
    return _mix32((hr[:, None] + cols[None, :] * _GOLD) & _M32)


def uniform01(seed: int, stream: int, rows: torch.Tensor, ncols: int, salt: int = 0) -> torch.Tensor:
    """Uniform in the open interval (0, 1), float64, 24-bit resolution."""
    h = uniform_bits(seed, stream, rows, ncols, salt)
    return ((h >> 8).to(torch.float64) + 0.5) * (1.0 / 16777216.0)


def normal(seed: int, stream: int, rows: torch.Tensor, ncols: int, std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) via Box-Muller on two independent hashed uniforms; float32 (RNE from float64)."""
    u1 = uniform01(seed, stream, rows, ncols, salt=1)
    u2 = uniform01(seed, stream, rows, ncols, salt=2)
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
    return (z * std).to(torch.float32)


def gumbel(seed: int, stream: int, rows: torch.Tensor, ncols: int) -> torch.Tensor:
    """Standard Gumbel(0, 1) samples, float64."""
    u = uniform01(seed, stream, rows, ncols, salt=3)
    return -torch.log(-torch.log(u))


def _rows(n: int, device, offset: int = 0) -> torch.Tensor:
    return torch.arange(offset, offset + n, dtype=torch.int64, device=device)


@dataclass
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    precision: str                    # "f32" | "bf16" | "mxfp8" | "mxfp4" (forward only)
    seed: int
    expert_begin: int = 0
    expert_end: int = -1              # -1 means E
    backward: bool = False
    minibatch_rows: tuple = (0,)
    ring_bytes: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def e_end(self) -> int:
        return self.E if self.expert_end < 0 else self.expert_end

    @property
    def E_loc(self) -> int:
        return self.e_end - self.expert_begin

    @property
    def act_dtype(self):
        return torch.float32 if self.precision == "f32" else torch.bfloat16


# Popularity-permutation seed of ep_share: the first seed (0, 1, 2, ...) whose
# local pair count lands within 10 % of 64*2048*8*4/256 = 16,384, found by
# find_perm_seed() below and checked by the workload tests.
EP_PERM_SEED = 34

WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=256, d=128, E=8, k=2, F=256, precision="f32", seed=1, backward=True),
    "bf16_fwd": Workload("bf16_fwd", T=4096, d=2048, E=64, k=6, F=1408, precision="bf16", seed=2),
    "ep_share": Workload("ep_share", T=-1, d=7168, E=256, k=8, F=2048, precision="bf16", seed=3,
                         expert_begin=0, expert_end=4,
                         notes={"source_tokens": 64 * 2048, "zipf": 1.1, "perm_seed": EP_PERM_SEED}),
    "ep_mxfp8": Workload("ep_mxfp8", T=-1, d=7168, E=256, k=8, F=2048, precision="mxfp8", seed=3,
                         expert_begin=0, expert_end=4,
                         notes={"source_tokens": 64 * 2048, "zipf": 1.1, "perm_seed": EP_PERM_SEED}),
    "bf16_train": Workload("bf16_train", T=8192, d=4096, E=128, k=8, F=1536, precision="bf16", seed=5,
                           backward=True, minibatch_rows=(512, 1024, 2048, 4096), ring_bytes=268435456,
                           notes={"zipf": 1.2}),
    # the same layer, inputs and routing in MXFP8 (forward and backward)
    "mxfp8_train": Workload("mxfp8_train", T=8192, d=4096, E=128, k=8, F=1536, precision="mxfp8", seed=5,
                            backward=True, notes={"zipf": 1.2}),
    # the same layer's forward alone (inference: nothing saved) in MXFP8 and MXFP4
    "mxfp8_infer": Workload("mxfp8_infer", T=8192, d=4096, E=128, k=8, F=1536, precision="mxfp8", seed=5,
                            notes={"zipf": 1.2}),
    "mxfp4_infer": Workload("mxfp4_infer", T=8192, d=4096, E=128, k=8, F=1536, precision="mxfp4", seed=5,
                            notes={"zipf": 1.2}),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(name: str, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    import dataclasses
    return dataclasses.replace(WORKLOADS[name], **over)


# ---------------------------------------------------------------- logits

def zipf_log_popularity(E: int, s: float, perm_seed: int | None, device="cpu") -> torch.Tensor:
    """log pi_e with pi_r proportional to r^-s; rank r = 1 is the most popular.

    With perm_seed None expert e has rank e+1; otherwise ranks follow a seeded
    permutation (expert e gets rank perm[e]+1)."""
    r = torch.arange(1, E + 1, dtype=torch.float64, device=device)
    logpi = -s * torch.log(r)
    logpi = logpi - torch.logsumexp(logpi, 0)
    if perm_seed is None:
        return logpi
    keys = uniform_bits(perm_seed, S_PERM, _rows(1, device), E)[0]
    rank_of_e = torch.empty(E, dtype=torch.int64, device=device)
    rank_of_e[torch.argsort(keys, stable=True)] = torch.arange(E, device=device)
    return logpi[rank_of_e]


def zipf_gumbel_logits(seed: int, token_ids: torch.Tensor, E: int, s: float, perm_seed) -> torch.Tensor:
    """logits[t, e] = log pi_e + G[t, e], G ~ Gumbel(0, 1): taking the k largest
    samples k experts without replacement with probability proportional to pi."""
    logpi = zipf_log_popularity(E, s, perm_seed, device=token_ids.device)
    return (logpi[None, :] + gumbel(seed, S_LOGIT, token_ids, E)).to(torch.float32)


def ep_share_tokens(w: Workload, device="cpu", chunk: int = 16384) -> torch.Tensor:
    """Token ids (ascending) among the source tokens whose top-k choice includes
    a local expert: this is how the one-GPU share of the expert-parallel layer
    is defined.  A token qualifies when fewer than k experts outrank its best
    local expert (higher logit, or equal logit and lower index)."""
    n_src = w.notes["source_tokens"]
    keep = []
    eidx = torch.arange(w.E, device=device)
    for c0 in range(0, n_src, chunk):
        ids = _rows(min(chunk, n_src - c0), device, c0)
        lg = zipf_gumbel_logits(w.seed, ids, w.E, w.notes["zipf"], w.notes["perm_seed"])
        loc = lg[:, w.expert_begin:w.e_end]
        best_val, best_i = loc.max(dim=1)
        best_e = best_i + w.expert_begin
        above = (lg > best_val[:, None]) | ((lg == best_val[:, None]) & (eidx[None, :] < best_e[:, None]))
        keep.append(ids[above.sum(dim=1) < w.k])
    return torch.cat(keep)


def find_perm_seed(w: Workload, target: int = 16384, tol: float = 0.10, max_seed: int = 200, device="cpu") -> int:
    """First permutation seed whose local pair count is within tol of target."""
    import dataclasses
    for s in range(max_seed):
        ws = dataclasses.replace(w, notes=dict(w.notes, perm_seed=s))
        if abs(local_pair_count(ws, device) - target) <= tol * target:
            return s
    raise RuntimeError("no permutation seed found")


def local_pair_count(w: Workload, device="cpu", chunk: int = 16384) -> int:
    """Number of (token, expert) pairs among all source tokens that land on the
    local experts (workload sizing only): a local expert counts for a token when
    fewer than k experts outrank it."""
    n_src = w.notes["source_tokens"]
    total = 0
    eidx = torch.arange(w.E, device=device)
    for c0 in range(0, n_src, chunk):
        ids = _rows(min(chunk, n_src - c0), device, c0)
        lg = zipf_gumbel_logits(w.seed, ids, w.E, w.notes["zipf"], w.notes["perm_seed"])
        for e in range(w.expert_begin, w.e_end):
            v = lg[:, e:e + 1]
            above = (lg > v) | ((lg == v) & (eidx[None, :] < e))
            total += int((above.sum(dim=1) < w.k).sum())
    return total


# ---------------------------------------------------------------- tensors

def make_inputs(w: Workload, device="cpu", weights: bool = True) -> dict:
    """All inputs of one layer call, on `device`.

    Returns x [T,d], logits [T,E] fp32, W1/W3 [E_loc,F,d], W2 [E_loc,d,F]
    (bf16 for bf16/mxfp8/mxfp4 workloads, fp32 for f32), dout [T,d] when the workload
    has a backward pass, token_ids [T], and Wr [d,E] for tiny_fp32."""
    dt = w.act_dtype
    out = {}
    if w.name.startswith("ep_"):
        ids = ep_share_tokens(w, device)
        logits = zipf_gumbel_logits(w.seed, ids, w.E, w.notes["zipf"], w.notes["perm_seed"])
    else:
        ids = _rows(w.T, device)
        if w.name.startswith("tiny"):
            x32 = normal(w.seed, S_X, ids, w.d)
            Wr = normal(w.seed, S_WR, _rows(w.d, device), w.E, std=0.02)
            out["Wr"] = Wr
            logits = (x32.to(torch.float64) @ Wr.to(torch.float64)).to(torch.float32)
        elif "zipf" in w.notes:
            logits = zipf_gumbel_logits(w.seed, ids, w.E, w.notes["zipf"], None)
        else:
            bias = normal(w.seed, S_BIAS, _rows(1, device), w.E)[0]
            logits = normal(w.seed, S_LOGIT, ids, w.E) + bias[None, :]
    T = ids.numel()
    out["token_ids"] = ids
    out["x"] = normal(w.seed, S_X, ids, w.d).to(dt)
    out["logits"] = logits.contiguous()
    if weights:
        out.update(make_weights(w, device))
    if w.backward:
        out["dout"] = normal(w.seed, S_DOUT, _rows(T, device), w.d).to(dt)
    return out


def make_weights(w: Workload, device="cpu") -> dict:
    """W1, W3 [E_loc, F, d] and W2 [E_loc, d, F], N(0, 0.02^2), generated one
    expert at a time (rows of expert e start at global row e*F or e*d)."""
    dt = w.act_dtype
    W1 = torch.empty((w.E_loc, w.F, w.d), dtype=dt, device=device)
    W3 = torch.empty_like(W1)
    W2 = torch.empty((w.E_loc, w.d, w.F), dtype=dt, device=device)
    for i in range(w.E_loc):
        e = w.expert_begin + i
        W1[i] = normal(w.seed, S_W1, _rows(w.F, device, e * w.F), w.d, std=0.02).to(dt)
        W3[i] = normal(w.seed, S_W3, _rows(w.F, device, e * w.F), w.d, std=0.02).to(dt)
        W2[i] = normal(w.seed, S_W2, _rows(w.d, device, e * w.d), w.F, std=0.02).to(dt)
    return {"W1": W1, "W3": W3, "W2": W2}


def regenerate_x_rows(w: Workload, token_ids: torch.Tensor) -> torch.Tensor:
    """Activations of the given tokens, regenerated from their ids alone."""
    return normal(w.seed, S_X, token_ids, w.d).to(w.act_dtype)


def make_router_inputs(seed: int, T: int, d: int, E: int, device="cpu") -> dict:
    """Inputs of the router GEMM: x [T, d] bf16 ~ N(0, 1) (the layer's token
    stream), Wr [E, d] bf16 ~ N(0, 0.02^2), one row per expert, and an
    incoming gradient dlogits [T, E] fp32 ~ N(0, 1)."""
    ids = _rows(T, device)
    return {"x": normal(seed, S_X, ids, d).to(torch.bfloat16),
            "Wr": normal(seed, S_WR, _rows(E, device), d, std=0.02).to(torch.bfloat16),
            "dlogits": normal(seed, S_DLOGIT, ids, E)}
