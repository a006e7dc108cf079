"""Pins of the fp64 prefill oracle against things other than itself (CPU only).

- HuggingFace transformers' Phi-3 model, the oracle the Phi-3-mini page
  compares against (section 2, Methods table), run in fp64 on the same
  weights and ids: pins the whole forward (fused row order, RoPE pairing and
  sign, causal mask, norms, residuals, SiLU(gate) * up, untied lm_head).
- torch's fp64 scaled-dot-product attention with a causal mask.
- closed forms and invariants (S = 1, zero queries, RoPE as complex
  multiplication, norm preservation, relative-position property, RMSNorm of a
  constant row, causal prefix invariance, int8 dequantization).
- planted mistakes: each variant of the oracle with one plausible slip must
  fail the transformers pin.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import parity, prefill


def _hf_logits(cfg, ws, ids):
    from transformers import Phi3Config, Phi3ForCausalLM

    hc = Phi3Config(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                    num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                    num_key_value_heads=cfg.n_kv_heads, max_position_embeddings=4096,
                    original_max_position_embeddings=4096, rms_norm_eps=cfg.rms_eps,
                    rope_theta=cfg.rope_theta, tie_word_embeddings=False,
                    pad_token_id=0, bos_token_id=1, eos_token_id=2)
    hc._attn_implementation = "eager"
    torch.manual_seed(0)
    m = Phi3ForCausalLM(hc).to(torch.float64).eval()
    t = lambda a: torch.from_numpy(prefill.widen(a))
    sd = {"model.embed_tokens.weight": t(ws.embed), "model.norm.weight": t(ws.final_norm),
          "lm_head.weight": t(ws.lm_head)}
    for l in range(cfg.n_layers):
        w, p = ws.layer(l), f"model.layers.{l}."
        sd.update({p + "self_attn.qkv_proj.weight": t(w["qkv"]), p + "self_attn.o_proj.weight": t(w["o"]),
                   p + "mlp.gate_up_proj.weight": t(w["gate_up"]), p + "mlp.down_proj.weight": t(w["down"]),
                   p + "input_layernorm.weight": t(w["ln1"]),
                   p + "post_attention_layernorm.weight": t(w["ln2"])})
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not missing and not unexpected
    with torch.no_grad():
        return m(torch.from_numpy(np.asarray(ids, dtype=np.int64))).logits.numpy()


class ScaledWeights:
    """Wraps a WeightSet, multiplying every linear weight by a factor so that
    activations and attention scores are O(1) (a harder regime than N(0, 0.02))."""

    def __init__(self, ws, factor):
        self.ws, self.f = ws, factor
        self.embed, self.final_norm = ws.embed, ws.final_norm
        self.lm_head = ws.lm_head

    def layer(self, l):
        w = dict(self.ws.layer(l))
        for k in ("qkv", "o", "gate_up", "down"):
            w[k] = w[k].astype(np.float64) * self.f
        return w


def _hf_pin(cfg, ws, ids, tol):
    ours = prefill.prefill_logits(cfg, ws, ids)
    ref = _hf_logits(cfg, ws, ids)
    scale = np.sqrt(np.mean(ref ** 2))
    err = np.abs(ours - ref).max() / scale
    assert err < tol, err
    return ours, ref


def test_matches_transformers_phi3_tiny():
    cfg = synth.TINY
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 16)
    ours, ref = _hf_pin(cfg, ws, ids, 1e-5)
    s = parity.summary(ours[0], ref[0])
    assert s["min_cos"] > 1 - 1e-10 and not s["failures"]


def test_matches_transformers_gqa_gain_one_peaked():
    # GQA grouping (4 query heads over 2 KV heads), unit norm gains and weights
    # scaled so that softmax rows are far from uniform.
    cfg = replace(synth.TINY, n_kv_heads=2, norm_gain="ones")
    ws = ScaledWeights(synth.WeightSet(cfg), 2.5)
    ids = synth.token_ids(cfg, 2, 24)
    _hf_pin(cfg, ws, ids, 1e-4)


def test_matches_transformers_head_dim_128_gqa_peaked():
    # the Phi-4 head geometry: head_dim 128, four query heads per KV head,
    # RoPE base 250000, unit gains and peaked attention
    cfg = replace(synth.TINY_GQA128, norm_gain="ones")
    ws = ScaledWeights(synth.WeightSet(cfg), 2.5)
    ids = synth.token_ids(cfg, 2, 24)
    ours, ref = _hf_pin(cfg, ws, ids, 1e-4)
    assert np.abs(ref).max() > 1.0   # the regime is not dominated by the embedding


def _mutants():
    good_rope, good_attn = prefill.apply_rope, prefill.causal_attention

    def rope_sign(x, ang):
        return good_rope(x, -ang)

    def rope_interleaved(x, ang):
        y = x.copy()
        c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
        y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
        return y

    def attn_no_mask(q, k, v, scale):
        out = np.empty_like(q)
        for h in range(q.shape[1]):
            g = h // (q.shape[1] // k.shape[1])
            sc = q[:, h] @ k[:, g].T * scale
            e = np.exp(sc - sc.max(axis=1, keepdims=True))
            out[:, h] = (e / e.sum(axis=1, keepdims=True)) @ v[:, g]
        return out

    def attn_no_scale(q, k, v, scale):
        return good_attn(q, k, v, 1.0)

    def silu_plain_sigmoid(x):
        return 1.0 / (1.0 + np.exp(-x))

    def norm_no_eps_mean(x, g, eps):
        return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * prefill.widen(g)

    return {"apply_rope": [rope_sign, rope_interleaved], "causal_attention": [attn_no_mask, attn_no_scale],
            "silu": [silu_plain_sigmoid], "rms_norm": [norm_no_eps_mean]}


def test_planted_mistakes_fail_the_transformers_pin(monkeypatch):
    cfg = replace(synth.TINY, norm_gain="ones")
    ws = ScaledWeights(synth.WeightSet(cfg), 2.5)
    ids = synth.token_ids(cfg, 1, 12)
    ref = _hf_logits(cfg, ws, ids)
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.abs(prefill.prefill_logits(cfg, ws, ids) - ref).max() / scale < 1e-4
    for name, variants in _mutants().items():
        for bad in variants:
            with monkeypatch.context() as mp:
                mp.setattr(prefill, name, bad)
                err = np.abs(prefill.prefill_logits(cfg, ws, ids) - ref).max() / scale
            assert err > 1e-2, (name, bad.__name__, err)
    # swapped fused row blocks (K and V sections; gate and up halves)

    class Swapped(ScaledWeights):
        def __init__(self, base, which):
            self.__dict__.update(base.__dict__)
            self.which = which

        def layer(self, l):
            w = ScaledWeights.layer(self, l)
            H, I = cfg.hidden, cfg.intermediate
            kv = cfg.n_kv_heads * cfg.head_dim
            if self.which == "qkv":
                q = w["qkv"]
                w["qkv"] = np.concatenate([q[:H], q[H + kv:], q[H:H + kv]])
            else:
                gu = w["gate_up"]
                w["gate_up"] = np.concatenate([gu[I:], gu[:I]])
            return w

    for which in ("qkv", "gate_up"):
        err = np.abs(prefill.prefill_logits(cfg, Swapped(ws, which), ids) - ref).max() / scale
        assert err > 1e-2, (which, err)


def test_attention_matches_torch_sdpa_peaked():
    rng = np.random.default_rng(3)
    S, nh, nkv, d = 37, 6, 3, 96
    q = rng.standard_normal((S, nh, d)) * 1.5
    k = rng.standard_normal((S, nkv, d)) * 1.5
    v = rng.standard_normal((S, nkv, d))
    ours = prefill.causal_attention(q, k, v, 1 / np.sqrt(d))
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(nh // nkv, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(nh // nkv, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2)
    assert np.abs(ours - ref.numpy()).max() < 1e-12


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((9, 2, 96))
    k = rng.standard_normal((9, 2, 96))
    # single position: the softmax has one term, the output is v[0]
    q1 = rng.standard_normal((1, 2, 96))
    assert np.array_equal(prefill.causal_attention(q1, k[:1], v[:1], 0.1), v[:1])
    # zero queries: uniform weights over the causal prefix
    out = prefill.causal_attention(np.zeros((9, 2, 96)), k, v, 0.1)
    want = np.cumsum(v, axis=0) / np.arange(1, 10)[:, None, None]
    assert np.abs(out - want).max() < 1e-14
    # V = 1 everywhere: every row of softmax weights sums to one
    out = prefill.causal_attention(rng.standard_normal((9, 2, 96)) * 3, k, np.ones_like(v), 0.3)
    assert np.abs(out - 1).max() < 1e-14


def test_rope_properties():
    rng = np.random.default_rng(5)
    d = 96
    pos = np.array([0, 1, 7, 100, 4095])
    ang = prefill.rope_angles(pos, d, 10000.0)
    x = rng.standard_normal((len(pos), 3, d))
    y = prefill.apply_rope(x, ang)
    # position 0 is the identity; norms are preserved
    assert np.array_equal(y[0], x[0])
    assert np.abs(np.linalg.norm(y, axis=-1) - np.linalg.norm(x, axis=-1)).max() < 1e-12
    # as complex multiplication of (x_i + j x_{i+48}) by exp(j p theta^(-2i/d))
    rot = np.exp(1j * np.outer(pos, 10000.0 ** (-2 * np.arange(48) / d)))
    z = (x[..., :48] + 1j * x[..., 48:]) * rot[:, None, :]
    assert np.abs(np.concatenate([z.real, z.imag], axis=-1) - y).max() < 1e-12
    # <R_m q, R_n k> = <R_{m-n} q, k>
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    for m, n in [(5, 2), (300, 17), (4000, 3999)]:
        lhs = np.sum(prefill.apply_rope(q, prefill.rope_angles([m], d, 1e4)) *
                     prefill.apply_rope(k, prefill.rope_angles([n], d, 1e4)))
        rhs = np.sum(prefill.apply_rope(q, prefill.rope_angles([m - n], d, 1e4)) * k)
        assert abs(lhs - rhs) < 1e-10


def test_rmsnorm_and_silu_closed_forms():
    g = np.linspace(-1, 2, 384)
    for c in (0.0, 1e-3, 3.0, -7.5):
        y = prefill.rms_norm(np.full((1, 384), c), g, 1e-5)
        assert np.abs(y - c / np.sqrt(c * c + 1e-5) * g).max() < 1e-14
    import scipy.special
    x = np.linspace(-30, 30, 1001)
    assert np.abs(prefill.silu(x) - x * scipy.special.expit(x)).max() < 1e-13
    assert prefill.silu(np.array([0.0]))[0] == 0.0


def test_causal_prefix_invariance():
    cfg = synth.TINY
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 16)
    full = prefill.prefill_logits(cfg, ws, ids)
    for k in (1, 5, 11):
        part = prefill.prefill_logits(cfg, ws, ids[:, :k])
        assert np.abs(part - full[:, :k]).max() < 1e-15 * 1e3


def test_int8_weights_mean_code_times_scale():
    # weights that are exactly code * scale give the same logits through the
    # int8 path as through the float path
    cfg = replace(synth.TINY, wtype="f16")
    ws = synth.WeightSet(cfg)

    class Exact:
        def __init__(self):
            self.embed, self.final_norm = ws.embed, ws.final_norm
            self.lm_head = synth.quantize_rows_i8(ws.lm_head)

        def layer(self, l):
            w = dict(ws.layer(l))
            for k in ("qkv", "o", "gate_up", "down"):
                w[k] = synth.quantize_rows_i8(w[k])
            return w

    class AsFloat(Exact):
        def __init__(self):
            super().__init__()
            self.lm_head = self.lm_head[0].astype(np.float64) * self.lm_head[1].astype(np.float64)[:, None]

        def layer(self, l):
            w = Exact.layer(self, l)
            for k in ("qkv", "o", "gate_up", "down"):
                q, s = w[k]
                w[k] = q.astype(np.float64) * s.astype(np.float64)[:, None]
            return w

    ids = synth.token_ids(cfg, 1, 8)
    a = prefill.prefill_logits(cfg, Exact(), ids)
    b = prefill.prefill_logits(cfg, AsFloat(), ids)
    assert np.array_equal(a, b)
    # and the int8 model is close to, but not the same as, the float16 one
    c = prefill.prefill_logits(cfg, ws, ids)
    cos = parity.row_cosines(a[0], c[0])
    assert 0.999 < cos.min() < 1.0
