"""Seeded synthetic inputs for the selective-batched iteration.

This module only draws numbers: batch shapes, parameters, hidden rows and
pre-filled K/V caches.  It holds none of the method's arithmetic, so both the
HIP path and the CPU oracle can take their inputs from it.

Workloads (all parameters random-init, no trained weights exist here):

  tiny-fp32      1 layer, H=64, 4 heads, FFN 256, fp32.  The four requests of
                 the selective-batching figure on garden.houmin.site/infra/orca
                 (section 3.1.2): x1 increment with 3 cached tokens, x2
                 increment with 4, x3 initiation of 2 prompt tokens, x4
                 initiation of 3.  Flattened rows: x1 | x2 | x3 | x4, sum L = 7.
  h1024-2l       2 layers, H=1024, 16 heads, FFN 4096, bf16.  4 initiations
                 with prompts U[64,512] and 28 increments with K/V lengths
                 U[128,2048].
  gpt13b-40l     GPT-3-13B shape: 40 layers, H=5120, 40 heads, FFN 20480, bf16.
                 2 initiations of 1024 tokens and 128 increments with K/V
                 lengths U[256,2048]; sum L = 2176.
  gpt175b-8l     GPT-3-175B layer shape: 8 layers, H=12288, 96 heads,
                 FFN 49152, bf16.  8 initiations with prompts U[128,1024] and
                 248 increments with K/V lengths U[512,2048].
  gpt13b-40l-decode64
                 the 13B shape with the steady-state batch of a serving trace
                 at a full 64-request batch: 64 increments, no initiation,
                 K/V lengths U[32,1024] (prompt U[32,512] plus up to 512
                 generated tokens).

Draw order for one seed (numpy PCG64, ``default_rng(seed)``): prompt lengths,
then K/V lengths; then for every layer ln1_g, ln1_b, W_qkv, b_qkv, W_o, b_o,
ln2_g, ln2_b, W_1, b_1, W_2, b_2; then the hidden rows x; then, layer by
layer and request by request in batch order, the cached K then V rows.
Integer draws are inclusive at both ends.  Linear weights and biases are
N(0, 0.02^2); LayerNorm gains are 1 + N(0, 0.02^2) and shifts N(0, 0.02^2);
hidden rows and cached K/V are N(0, 1).  For bf16 workloads every value is
drawn in fp32 and rounded to the nearest bf16 (ties to even) before either
side sees it.  Weights are stored [out, in].

The batch lists increment requests first, then initiation requests, the order
of the figure (x1, x2 | x3, x4).

The two largest workloads are too big to draw on the host; ``device_*``
helpers draw them on the GPU with a seeded ``torch.Generator`` in the same
order.  Their values differ from the host draw of the same seed; they are
seeded and reproducible, and checks copy back only what they compare.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

LAYER_KEYS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
              "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2")

MODELS: Dict[str, dict] = {
    "tiny-fp32": dict(layers=1, hidden=64, heads=4, ffn=256, dtype="f32"),
    "h1024-2l": dict(layers=2, hidden=1024, heads=16, ffn=4096, dtype="bf16"),
    "gpt13b-40l": dict(layers=40, hidden=5120, heads=40, ffn=20480, dtype="bf16"),
    "gpt175b-8l": dict(layers=8, hidden=12288, heads=96, ffn=49152, dtype="bf16"),
    "gpt13b-40l-decode64": dict(layers=40, hidden=5120, heads=40, ffn=20480, dtype="bf16"),
}

LN_EPS = 1e-5


@dataclass
class Workload:
    name: str
    layers: int
    hidden: int
    heads: int
    ffn: int
    dtype: str                       # "f32" | "bf16"
    q_len: List[int]                 # per request, batch order
    kv_len: List[int]                # cached entries before the iteration
    eps: float = LN_EPS

    @property
    def n_reqs(self) -> int:
        return len(self.q_len)

    @property
    def rows(self) -> int:
        return int(sum(self.q_len))

    @property
    def q_offset(self) -> List[int]:
        out, off = [], 0
        for q in self.q_len:
            out.append(off)
            off += q
        return out

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    def with_layers(self, layers: int) -> "Workload":
        w = Workload(**{**self.__dict__})
        w.layers = layers
        return w


def _lengths(name: str, rng: np.random.Generator) -> Tuple[List[int], List[int]]:
    """Returns (q_len, kv_len) in batch order: increments, then initiations."""
    if name == "tiny-fp32":
        return [1, 1, 2, 3], [3, 4, 0, 0]
    if name == "h1024-2l":
        prompts = rng.integers(64, 512, size=4, endpoint=True)
        kvs = rng.integers(128, 2048, size=28, endpoint=True)
    elif name == "gpt13b-40l":
        prompts = np.array([1024, 1024])
        kvs = rng.integers(256, 2048, size=128, endpoint=True)
    elif name == "gpt175b-8l":
        prompts = rng.integers(128, 1024, size=8, endpoint=True)
        kvs = rng.integers(512, 2048, size=248, endpoint=True)
    elif name == "gpt13b-40l-decode64":
        prompts = np.zeros(0, dtype=np.int64)
        kvs = rng.integers(32, 1024, size=64, endpoint=True)
    else:
        raise KeyError(name)
    q = [1] * len(kvs) + [int(p) for p in prompts]
    kv = [int(k) for k in kvs] + [0] * len(prompts)
    return q, kv


def workload(name: str, seed: int = 0) -> Workload:
    m = MODELS[name]
    q, kv = _lengths(name, np.random.default_rng(seed))
    return Workload(name=name, q_len=q, kv_len=kv, **m)


def custom_workload(layers: int, hidden: int, heads: int, ffn: int, dtype: str,
                    q_len: Sequence[int], kv_len: Sequence[int],
                    name: str = "custom") -> Workload:
    return Workload(name=name, layers=layers, hidden=hidden, heads=heads, ffn=ffn,
                    dtype=dtype, q_len=list(q_len), kv_len=list(kv_len))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even), returned as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _param_shapes(w: Workload) -> List[Tuple[str, Tuple[int, ...], str]]:
    h, f = w.hidden, w.ffn
    return [("ln1_g", (h,), "gain"), ("ln1_b", (h,), "small"),
            ("w_qkv", (3 * h, h), "small"), ("b_qkv", (3 * h,), "small"),
            ("w_o", (h, h), "small"), ("b_o", (h,), "small"),
            ("ln2_g", (h,), "gain"), ("ln2_b", (h,), "small"),
            ("w_1", (f, h), "small"), ("b_1", (f,), "small"),
            ("w_2", (h, f), "small"), ("b_2", (h,), "small")]


@dataclass
class HostInputs:
    work: Workload
    params: List[Dict[str, np.ndarray]]
    x: np.ndarray                                   # [rows, H] float32
    caches: List[List[Tuple[np.ndarray, np.ndarray]]]   # [layer][req] (K, V) [kv_len, H]


def host_inputs(w: Workload, seed: int = 0, rng: Optional[np.random.Generator] = None
                ) -> HostInputs:
    """Draw everything for a workload on the host, in the documented order.

    When `w` came from ``workload(name, seed)`` the generator continues after
    the length draws of that call; for custom workloads a fresh generator is
    used.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
        if w.name in MODELS:
            _lengths(w.name, rng)                       # replay the length draws
    rnd = round_to_bf16 if w.dtype == "bf16" else (lambda a: a)

    def normal(shape, kind):
        z = rng.standard_normal(shape, dtype=np.float32)
        if kind == "gain":
            return rnd(1.0 + 0.02 * z)
        if kind == "small":
            return rnd(0.02 * z)
        return rnd(z)

    params = []
    for _ in range(w.layers):
        params.append({k: normal(s, kind) for k, s, kind in _param_shapes(w)})
    x = normal((w.rows, w.hidden), "unit")
    caches = []
    for _ in range(w.layers):
        per = []
        for kv in w.kv_len:
            per.append((normal((kv, w.hidden), "unit"), normal((kv, w.hidden), "unit")))
        caches.append(per)
    return HostInputs(w, params, x, caches)


# ----------------------------------------------------------- device-side draws

def device_param_tensors(w: Workload, layer_seed: int, device, torch_dtype):
    """One layer's parameters drawn on the device (seeded torch.Generator),
    in the documented order, returned as a dict of tensors of `torch_dtype`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(layer_seed)
    out = {}
    for k, shape, kind in _param_shapes(w):
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if kind == "gain":
            z = 1.0 + 0.02 * z
        elif kind == "small":
            z = 0.02 * z
        out[k] = z.to(torch_dtype)
    return out


def device_normal_(t, seed: int):
    """Fill a device tensor with N(0,1) values from a seeded torch.Generator,
    in chunks so that no fp32 temporary larger than 256 MiB is needed."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    flat = t.view(-1)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=g, device=t.device,
                                dtype=torch.float32).to(t.dtype)
    return t


# ---------------------------------------------------------------- trace (c5)

@dataclass
class TraceRequest:
    id: int
    arrival: float
    prompt_len: int
    max_tokens: int
    out_len: int


def poisson_trace(n: int, rate: float, seed: int = 0, prompt=(32, 512),
                  out=(1, 512), max_tokens: int = 512) -> List[TraceRequest]:
    """Requests arriving as a Poisson stream of `rate` per second (rate=inf:
    all at t=0); prompt and output lengths uniform, inclusive.  Draw order:
    inter-arrival gaps, prompt lengths, output lengths."""
    rng = np.random.default_rng(seed)
    if np.isinf(rate):
        gaps = np.zeros(n)
    else:
        gaps = rng.exponential(1.0 / rate, size=n)
    arrivals = np.cumsum(gaps)
    prompts = rng.integers(prompt[0], prompt[1], size=n, endpoint=True)
    outs = rng.integers(out[0], out[1], size=n, endpoint=True)
    return [TraceRequest(i, float(arrivals[i]), int(prompts[i]), max_tokens, int(outs[i]))
            for i in range(n)]
