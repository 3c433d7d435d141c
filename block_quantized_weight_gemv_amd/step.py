"""One decode step (one token's forward pass) built from the library's calls.

The sequence of "picoLM, in Python" §4 (model_forward): dequantise the
token's embedding row; per layer RMSNorm, q/k/v (one batched launch), RoPE
with the fp16 cache store, attention over the cache, the output projection,
the residual add fused with the next RMSNorm, gate/up (one batched launch),
SwiGLU, down; after the last layer the residual add with the final RMSNorm
and the output matrix. Every operation is a call into libqk.so (qk.h,
qk_step.h); this module owns the buffers and issues the calls in order.

The position lives in a device int32, so the layer sequence can be captured
once in a HIP graph (``capture``) and replayed for every position: the host
writes the new position and the new embedding row before each replay.

Where the library has a transformed-input GEMV for every matrix's format
and shape (qk_gemv_input_supported), the residual add and the RMSNorm that
feed q/k/v, gate/up and the output matrix, and the SwiGLU that feeds down,
run inside those GEMVs (qk_gemv_batch_input), and RoPE with the cache store
inside the attention launch (qk_attention_rope): 6 launches per layer
instead of 10. The residual stream then alternates between two buffers (a GEMV
reads one and its workgroup 0 writes the sum to the other).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import qk, synth


@dataclass
class StepConfig:
    """Shapes of a Llama-style decoder (defaults: TinyLlama-1.1B, the model
    the picoLM page runs: 22 layers, 2048 wide, 32 query heads sharing 4 KV
    heads of 64, FFN 5632, 32000 tokens). Weight types default to a Q4_K_M
    file's: Q4_K, with V, down and the output matrix in Q6_K."""
    dim: int = 2048
    n_layers: int = 22
    n_heads: int = 32
    n_kv_heads: int = 4
    ffn: int = 5632
    vocab: int = 32000
    max_pos: int = 2048
    eps: float = 1e-5
    rope_base: float = 10000.0
    types: dict = field(default_factory=lambda: {
        "token_embd": qk.Q4_K, "q": qk.Q4_K, "k": qk.Q4_K, "v": qk.Q6_K, "o": qk.Q4_K, "gate": qk.Q4_K,
        "up": qk.Q4_K, "down": qk.Q6_K, "output": qk.Q6_K})

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def shapes(self) -> dict:
        """(rows, cols) of every weight matrix (rows = outputs)."""
        return {"token_embd": (self.vocab, self.dim), "q": (self.dim, self.dim), "k": (self.kv_dim, self.dim),
                "v": (self.kv_dim, self.dim), "o": (self.dim, self.dim), "gate": (self.ffn, self.dim),
                "up": (self.ffn, self.dim), "down": (self.dim, self.ffn), "output": (self.vocab, self.dim)}


WEIGHT_SCALE = 0.02  # block scales x 0.02: weights ~0.02, activations of order one


def synthetic_weights(cfg: StepConfig, seed: int) -> dict:
    """Seeded random weights on the host: packed blocks per matrix (the
    generator's field distributions with the block scales multiplied by
    WEIGHT_SCALE) and norm weights uniform in [0.5, 1.5].
    Keys: "token_embd", "output", "output_norm", and per layer l
    "l.attn_norm", "l.q", "l.k", "l.v", "l.o", "l.ffn_norm", "l.gate", "l.up",
    "l.down"."""
    shp = cfg.shapes()
    w = {}
    sid = 0

    def mat(name, key):
        nonlocal sid
        sid += 1
        r, c = shp[name]
        return synth.matrix(cfg.types[name], r, c, seed, stream=sid, scale=WEIGHT_SCALE)

    def norm(n):
        nonlocal sid
        sid += 1
        return synth.rng(seed, 50000 + sid).uniform(0.5, 1.5, n).astype(np.float32)

    w["token_embd"] = mat("token_embd", "token_embd")
    for l in range(cfg.n_layers):
        w[f"{l}.attn_norm"] = norm(cfg.dim)
        for name in ("q", "k", "v", "o"):
            w[f"{l}.{name}"] = mat(name, f"{l}.{name}")
        w[f"{l}.ffn_norm"] = norm(cfg.dim)
        for name in ("gate", "up", "down"):
            w[f"{l}.{name}"] = mat(name, f"{l}.{name}")
    w["output_norm"] = norm(cfg.dim)
    w["output"] = mat("output", "output")
    return w


class DecodeStep:
    """Device buffers and the call sequence of one step. ``weights`` maps the
    keys of synthetic_weights to host numpy arrays or device tensors. With
    ``fuse`` (the default) the norms and SwiGLU run inside the GEMVs wherever
    every matrix has such a kernel; fuse=False keeps them separate launches."""

    def __init__(self, cfg: StepConfig, weights: dict, device: str = "cuda", fuse: bool = True):
        if cfg.head_dim not in (64, 128) or cfg.n_heads % cfg.n_kv_heads:
            raise ValueError("head_dim must be 64 or 128 and n_heads a multiple of n_kv_heads")
        self.cfg = cfg
        dev = torch.device(device)

        def put(a):
            return a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.w = {k: put(v) for k, v in weights.items()}
        f32 = dict(dtype=torch.float32, device=dev)
        d, kv, ffn = cfg.dim, cfg.kv_dim, cfg.ffn
        self.x = torch.zeros(d, **f32)
        self.x2 = torch.zeros(d, **f32)  # the other residual buffer (fused path)
        self.xb = torch.zeros(d, **f32)
        self.q = torch.zeros(d, **f32)
        self.k = torch.zeros(kv, **f32)
        self.v = torch.zeros(kv, **f32)
        self.att = torch.zeros(d, **f32)
        self.o = torch.zeros(d, **f32)
        self.gate = torch.zeros(ffn, **f32)
        self.up = torch.zeros(ffn, **f32)
        self.hb = torch.zeros(ffn, **f32)
        self.down = torch.zeros(d, **f32)
        self.logits = torch.zeros(cfg.vocab, **f32)
        self.kv_stride = (kv + 7) // 8 * 8
        self.k_cache = torch.zeros(cfg.n_layers, cfg.max_pos, self.kv_stride, dtype=torch.int16, device=dev)
        self.v_cache = torch.zeros_like(self.k_cache)
        half = cfg.head_dim // 2
        self.cos = torch.empty(cfg.max_pos * half, **f32)
        self.sin = torch.empty(cfg.max_pos * half, **f32)
        qk.qk_rope_tables(cfg.max_pos, cfg.head_dim, cfg.rope_base, self.cos, self.sin)
        self.pos = torch.zeros(1, dtype=torch.int32, device=dev)
        self.att_ws = torch.empty((qk.qk_attention_workspace_bytes(cfg.n_heads, cfg.head_dim, cfg.max_pos) + 3) // 4,
                                  **f32)
        T = cfg.types
        self.qkv = []
        self.gateup = []
        for l in range(cfg.n_layers):
            self.qkv.append(qk.make_gemv_batch([
                (T["q"], self.w[f"{l}.q"], d, d, self.xb, self.q),
                (T["k"], self.w[f"{l}.k"], kv, d, self.xb, self.k),
                (T["v"], self.w[f"{l}.v"], kv, d, self.xb, self.v)]))
            self.gateup.append(qk.make_gemv_batch([
                (T["gate"], self.w[f"{l}.gate"], ffn, d, self.xb, self.gate),
                (T["up"], self.w[f"{l}.up"], ffn, d, self.xb, self.up)]))
        self.embd_row_bytes = qk.qk_row_bytes(T["token_embd"], d)
        shp = cfg.shapes()
        self.fused = fuse and all(qk.qk_gemv_input_supported(T[m], *shp[m])
                                  for m in ("q", "k", "v", "gate", "up", "down", "output"))
        if self.fused:
            # The residual stream alternates between R0 (= x, the embedding)
            # and R1: q/k/v of layer l > 0 read RMSNorm(R1 + down) and write
            # R1 + down to R0; gate/up of every layer read RMSNorm(R0 + o) and
            # write R0 + o to R1; the output matrix reads RMSNorm(R1 + down).
            # (Layer 0's q/k/v read RMSNorm(R0) from a plain norm launch.)
            R0, R1 = self.x, self.x2
            self.f_qkv, self.f_gateup, self.f_down = [], [], []
            for l in range(cfg.n_layers):
                self.f_qkv.append((qk.make_gemv_batch([
                    (T["q"], self.w[f"{l}.q"], d, d, R1, self.q), (T["k"], self.w[f"{l}.k"], kv, d, R1, self.k),
                    (T["v"], self.w[f"{l}.v"], kv, d, R1, self.v)]),
                    qk.make_gemv_input(qk.QK_INPUT_ADD_RMSNORM, self.down, self.w[f"{l}.attn_norm"], cfg.eps, R0)))
                self.f_gateup.append((qk.make_gemv_batch([
                    (T["gate"], self.w[f"{l}.gate"], ffn, d, R0, self.gate),
                    (T["up"], self.w[f"{l}.up"], ffn, d, R0, self.up)]),
                    qk.make_gemv_input(qk.QK_INPUT_ADD_RMSNORM, self.o, self.w[f"{l}.ffn_norm"], cfg.eps, R1)))
                self.f_down.append((qk.make_gemv_batch([(T["down"], self.w[f"{l}.down"], d, ffn, self.gate,
                                                         self.down)]),
                                    qk.make_gemv_input(qk.QK_INPUT_SWIGLU, self.up)))
            self.f_out = (qk.make_gemv_batch([(T["output"], self.w["output"], cfg.vocab, d, R1, self.logits)]),
                          qk.make_gemv_input(qk.QK_INPUT_ADD_RMSNORM, self.down, self.w["output_norm"], cfg.eps, R0))
        self.graph = None

    # -- the sequence --------------------------------------------------------
    def embed(self, token: int, stream=None) -> None:
        """x = the token's dequantised embedding row."""
        c = self.cfg
        if not 0 <= token < c.vocab:
            raise ValueError("token out of range")
        row = self.w["token_embd"].data_ptr() + token * self.embd_row_bytes
        qk.qk_dequantize_row(c.types["token_embd"], row, c.dim, self.x, stream=stream)

    def layers(self, stream=None) -> None:
        """Every layer and the output matrix for the position in self.pos,
        starting from x (the embedding); logits in self.logits."""
        if self.fused:
            return self._layers_fused(stream)
        c, T = self.cfg, self.cfg.types
        d, kv, ffn, hd = c.dim, c.kv_dim, c.ffn, c.head_dim
        for l in range(c.n_layers):
            if l == 0:
                qk.qk_rmsnorm(self.x, self.w["0.attn_norm"], d, c.eps, self.xb, stream)
            else:
                qk.qk_add_rmsnorm(self.x, self.down, self.w[f"{l}.attn_norm"], d, c.eps, self.xb, stream)
            qk.qk_gemv_batch(self.qkv[l], stream=stream)
            qk.qk_rope_kv(self.q, self.k, self.v, self.pos, c.max_pos, self.cos, self.sin, c.n_heads, c.n_kv_heads,
                          hd, self.k_cache[l], self.v_cache[l], self.kv_stride, stream)
            qk.qk_attention(self.q, self.k_cache[l], self.v_cache[l], self.pos, c.max_pos, c.n_heads, c.n_kv_heads,
                            hd, self.kv_stride, self.att_ws, self.att, stream)
            qk.qk_gemv(T["o"], self.w[f"{l}.o"], d, d, self.att, self.o, stream)
            qk.qk_add_rmsnorm(self.x, self.o, self.w[f"{l}.ffn_norm"], d, c.eps, self.xb, stream)
            qk.qk_gemv_batch(self.gateup[l], stream=stream)
            qk.qk_swiglu(self.gate, self.up, ffn, self.hb, stream)
            qk.qk_gemv(T["down"], self.w[f"{l}.down"], d, ffn, self.hb, self.down, stream)
        qk.qk_add_rmsnorm(self.x, self.down, self.w["output_norm"], d, c.eps, self.xb, stream)
        qk.qk_gemv(T["output"], self.w["output"], c.vocab, d, self.xb, self.logits, stream)

    def _layers_fused(self, stream=None) -> None:
        c = self.cfg
        d, hd = c.dim, c.head_dim
        for l in range(c.n_layers):
            descs, xin = self.f_qkv[l]
            if l == 0:
                qk.qk_rmsnorm(self.x, self.w["0.attn_norm"], d, c.eps, self.xb, stream)
                qk.qk_gemv_batch(self.qkv[0], stream=stream)
            else:
                qk.qk_gemv_batch_input(descs, xin, stream=stream)
            qk.qk_attention_rope(self.q, self.k, self.v, self.pos, c.max_pos, self.cos, self.sin, c.n_heads,
                                 c.n_kv_heads, hd, self.k_cache[l], self.v_cache[l], self.kv_stride, self.att_ws,
                                 self.att, stream)
            qk.qk_gemv(c.types["o"], self.w[f"{l}.o"], d, d, self.att, self.o, stream)
            qk.qk_gemv_batch_input(*self.f_gateup[l], stream=stream)
            qk.qk_gemv_batch_input(*self.f_down[l], stream=stream)
        qk.qk_gemv_batch_input(*self.f_out, stream=stream)

    def forward(self, token: int, pos: int) -> torch.Tensor:
        """Eager: one step at `pos`; returns the logits tensor (overwritten by
        the next step)."""
        if not 0 <= pos < self.cfg.max_pos:
            raise ValueError("pos out of range")
        self.pos.fill_(pos)
        self.embed(token)
        if self.graph is not None:
            self.graph.replay()
        else:
            self.layers()
        return self.logits

    def capture(self) -> None:
        """Capture layers() in a HIP graph; later forward() calls replay it.
        The capture runs at whatever position self.pos holds and writes that
        row of the caches, which forward() rewrites before it is read."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.layers()  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.layers()
        torch.cuda.synchronize()
        self.graph = g
