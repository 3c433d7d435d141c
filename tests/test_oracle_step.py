"""Pins of the oracle's composed decode step (oracle/step.py), on the CPU:
properties of the forward pass that a wiring mistake would break.

* Grouped-query attention equals multi-head attention whose K/V heads are
  copies of the grouped ones (weights copied across, logits compared), the
  check the batching page's README describes for its GQA model.
* K enters the cache after its rotation ("picoLM, in Python" §4: K is stored
  after RoPE because a cached position never changes): at position 0 the
  cached row is the projection itself (the rotation is the identity), at a
  later position its pairs keep their norms but not their values; V is
  cached as projected. A mutant that caches K before the rotation fails.
* A step writes only its own cache row, and replaying a prefix reproduces
  the logits bit for bit (the picoLM page's runnable file checks cache
  immutability and a bit-identical prefix replay).
"""
import numpy as np
import pytest

from block_quantized_weight_gemv_amd import synth
from oracle.step import OracleStep

Q4_K, Q6_K = 3, 4


class Cfg:
    def __init__(self, **kw):
        self.dim, self.n_layers, self.n_heads, self.n_kv_heads = 256, 2, 4, 2
        self.ffn, self.vocab, self.max_pos, self.eps, self.rope_base = 512, 300, 16, 1e-5, 10000.0
        self.types = {"token_embd": Q4_K, "q": Q4_K, "k": Q4_K, "v": Q6_K, "o": Q4_K, "gate": Q4_K, "up": Q4_K,
                      "down": Q6_K, "output": Q6_K}
        self.__dict__.update(kw)


def weights(cfg, seed=1):
    hd = cfg.dim // cfg.n_heads
    kv = cfg.n_kv_heads * hd
    shp = {"token_embd": (cfg.vocab, cfg.dim), "q": (cfg.dim, cfg.dim), "k": (kv, cfg.dim), "v": (kv, cfg.dim),
           "o": (cfg.dim, cfg.dim), "gate": (cfg.ffn, cfg.dim), "up": (cfg.ffn, cfg.dim), "down": (cfg.dim, cfg.ffn),
           "output": (cfg.vocab, cfg.dim)}
    w, sid = {}, 0

    def mat(name):
        nonlocal sid
        sid += 1
        return synth.matrix(cfg.types[name], *shp[name], seed, stream=sid, scale=0.02)

    w["token_embd"] = mat("token_embd")
    for l in range(cfg.n_layers):
        sid += 1
        w[f"{l}.attn_norm"] = synth.rng(seed, 900 + sid).uniform(0.5, 1.5, cfg.dim).astype(np.float32)
        for n in ("q", "k", "v", "o"):
            w[f"{l}.{n}"] = mat(n)
        sid += 1
        w[f"{l}.ffn_norm"] = synth.rng(seed, 900 + sid).uniform(0.5, 1.5, cfg.dim).astype(np.float32)
        for n in ("gate", "up", "down"):
            w[f"{l}.{n}"] = mat(n)
    w["output_norm"] = synth.rng(seed, 999).uniform(0.5, 1.5, cfg.dim).astype(np.float32)
    w["output"] = mat("output")
    return w


def test_gqa_equals_mha_with_copied_kv(orc):
    cfg = Cfg()
    w = weights(cfg)
    hd = cfg.dim // cfg.n_heads
    grp = cfg.n_heads // cfg.n_kv_heads
    mha = Cfg(n_kv_heads=cfg.n_heads)
    wm = dict(w)
    rb = orc.row_bytes(Q4_K, cfg.dim)
    rbv = orc.row_bytes(Q6_K, cfg.dim)
    for l in range(cfg.n_layers):
        for name, rbx in (("k", rb), ("v", rbv)):
            rows = w[f"{l}.{name}"].reshape(cfg.n_kv_heads, hd, rbx)
            wm[f"{l}.{name}"] = np.repeat(rows, grp, axis=0).reshape(-1)
    a, b = OracleStep(orc, cfg, w), OracleStep(orc, mha, wm)
    for pos, tok in enumerate([5, 17, 250]):
        la = a.forward(tok, pos)[0]
        lb = b.forward(tok, pos)[0]
        assert np.array_equal(la, lb)


def test_step_touches_only_its_cache_row_and_replays(orc):
    cfg = Cfg()
    w = weights(cfg, seed=3)
    a = OracleStep(orc, cfg, w)
    outs = []
    for i, t in enumerate([7, 8, 9]):
        before_k, before_v = a.k_cache.copy(), a.v_cache.copy()
        outs.append(a.forward(t, i)[0])
        others = [p for p in range(cfg.max_pos) if p != i]
        assert np.array_equal(a.k_cache[:, others], before_k[:, others])
        assert np.array_equal(a.v_cache[:, others], before_v[:, others])
    b = OracleStep(orc, cfg, w)
    for i, t in enumerate([7, 8, 9]):
        assert np.array_equal(b.forward(t, i)[0], outs[i])


def check_cache_rows(st, pos):
    """The cache rows of `pos` against the step's own projections."""
    cfg = st.cfg
    for l in range(cfg.n_layers):
        k_raw, v = st.trace[f"{l}.k_raw"], st.trace[f"{l}.v"]
        kc = st.k_cache[l, pos].view(np.float16).astype(np.float64)
        assert np.array_equal(st.v_cache[l, pos], v.astype(np.float16).view(np.uint16))
        if pos == 0:
            assert np.array_equal(st.k_cache[l, 0], k_raw.astype(np.float16).view(np.uint16))
        else:
            n_raw = np.hypot(*k_raw.astype(np.float64).reshape(-1, 2).T)
            n_c = np.hypot(*kc.reshape(-1, 2).T)
            assert np.allclose(n_c, n_raw, rtol=2e-3, atol=1e-4)
            assert np.max(np.abs(kc - k_raw)) > 1e-2 * np.max(np.abs(k_raw))


def test_cache_holds_rotated_k_and_plain_v(orc):
    cfg = Cfg()
    st = OracleStep(orc, cfg, weights(cfg, seed=2))
    for pos, tok in enumerate([3, 141, 59, 26]):
        st.forward(tok, pos)
        check_cache_rows(st, pos)


def test_cache_pin_catches_k_cached_before_rope(orc):
    """A mutant that stores the unrotated K fails the cache pin."""
    cfg = Cfg()

    class Mutant(OracleStep):
        def forward(self, token, pos):
            out = super().forward(token, pos)
            for l in range(self.cfg.n_layers):
                self.k_cache[l, pos] = self.trace[f"{l}.k_raw"].astype(np.float16).view(np.uint16)
            return out

    st = Mutant(orc, cfg, weights(cfg, seed=2))
    st.forward(3, 0)
    check_cache_rows(st, 0)
    st.forward(141, 1)
    with pytest.raises(AssertionError):
        check_cache_rows(st, 1)
