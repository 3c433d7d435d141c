"""CPU oracle of one decode step (one token's forward pass), composed from the
oracle's pinned operations.

TEST INFRASTRUCTURE: only the test suite, the package smoke check and the
benchmark's CPU baseline use it. The order is the forward pass of "picoLM,
in Python" §4 (model_forward): the token's embedding row; per layer RMSNorm,
q/k/v, RoPE on q and k with the position's table (the interleaved pairs of
§3), k and v rounded to fp16 into the cache row of the position (k after
RoPE), attention of every query head over positions 0..pos of its KV head,
the output projection and the residual add, RMSNorm, gate/up, SwiGLU, down
and the residual add; the final RMSNorm and the output matrix.

Activations are fp32 between operations, as on the path: each operation's
result (an fp64 sum or an fp64-evaluated formula inside the oracle) is
rounded once to fp32 before the next one uses it; the residual adds are fp32
additions. The logits are returned in fp64 with their tolerance scale
(sum |w * x| of the output matrix).

Pins (tests/test_oracle_step.py): the per-operation pins of tests/pins.py,
and on the composition: grouped-query attention equals multi-head attention
with the K/V projections copied (bit-identical logits); the cached K row is
the projection turned by RoPE (unchanged at position 0, pair norms kept and
values changed at later positions) and the cached V row the projection
itself; a step never changes cache rows other than its own position, and
replaying a prefix reproduces the logits bit for bit; attention is not
degenerate at these weight scales (several positions carry weight).
"""
from __future__ import annotations

import numpy as np


class OracleStep:
    """Host state of one sequence: the fp16 KV caches (as uint16 patterns).
    `cfg` is a StepConfig (dim, n_layers, n_heads, n_kv_heads, head_dim, ffn,
    vocab, max_pos, eps, rope_base, types); `w` maps the keys of
    synthetic_weights to host numpy arrays."""

    def __init__(self, o, cfg, w):
        self.o, self.cfg, self.w = o, cfg, w
        kv = cfg.n_kv_heads * (cfg.dim // cfg.n_heads)
        self.kv = kv
        self.k_cache = np.zeros((cfg.n_layers, cfg.max_pos, kv), dtype=np.uint16)
        self.v_cache = np.zeros_like(self.k_cache)
        self.trace = {}  # the last step's per-layer intermediates (fp32)

    def _mv(self, name, key, x, rows, cols):
        y, a = self.o.gemv(self.cfg.types[name], self.w[key], rows, cols, x)
        return y.astype(np.float32), y, a

    def forward(self, token: int, pos: int):
        """Returns (logits fp64, tolerance scale fp64, final normed x fp32)."""
        o, c, w = self.o, self.cfg, self.w
        d, hd, kv, ffn = c.dim, c.dim // c.n_heads, self.kv, c.ffn
        rb = o.row_bytes(c.types["token_embd"], d)
        x = o.dequantize_row(c.types["token_embd"], w["token_embd"][token * rb:(token + 1) * rb], d)
        cs, sn = o.rope_table(pos, hd, c.rope_base)
        for l in range(c.n_layers):
            xb = o.rmsnorm(x, w[f"{l}.attn_norm"], c.eps)
            q = self._mv("q", f"{l}.q", xb, d, d)[0]
            k = self._mv("k", f"{l}.k", xb, kv, d)[0]
            v = self._mv("v", f"{l}.v", xb, kv, d)[0]
            self.trace[f"{l}.xb"], self.trace[f"{l}.k_raw"], self.trace[f"{l}.v"] = xb, k, v
            q = o.rope(q, c.n_heads, hd, cs, sn)
            k = o.rope(k, c.n_kv_heads, hd, cs, sn)
            self.k_cache[l, pos] = o.halves(k)
            self.v_cache[l, pos] = o.halves(v)
            att, _ = o.attention(q, self.k_cache[l], self.v_cache[l], c.n_heads, c.n_kv_heads, hd, pos + 1, kv)
            out = self._mv("o", f"{l}.o", att.astype(np.float32), d, d)[0]
            x = x + out  # fp32 addition
            xb = o.rmsnorm(x, w[f"{l}.ffn_norm"], c.eps)
            g = self._mv("gate", f"{l}.gate", xb, ffn, d)[0]
            u = self._mv("up", f"{l}.up", xb, ffn, d)[0]
            hb = o.swiglu(g, u).astype(np.float32)
            dn = self._mv("down", f"{l}.down", hb, d, ffn)[0]
            x = x + dn
        xb = o.rmsnorm(x, w["output_norm"], c.eps)
        _, logits, absacc = self._mv("output", "output", xb, c.vocab, d)
        return logits, absacc, xb
