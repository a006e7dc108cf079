"""End-to-end prefill parity: ids -> logits through the C ABI vs the oracle (GPU).

Gates: per-position logit cosine >= 0.99999 against the fp64 oracle and
argmax agreement wherever the oracle's top-2 gap exceeds 1e-3 (absolute
logits).  The int8 path is gated against the oracle run on the int8 weights
(code * scale); its cosine against the float16 oracle is reported.

Small cases run the oracle live.  Full Phi-3-mini shapes compare with oracle
results stored under tests/golden/ (written by make_goldens.py, which calls
only the oracle): the oracle's final normalised hidden state at every
position, from which each reference logit row is formed here by the oracle's
own lm_head step, so the cosine is gated at every position; argmax and top-2
gap at every position; and full rows at sampled positions.  The input digests
stored with them must match.
"""
import hashlib
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import parity, prefill

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
COS_GATE = 0.99999


def _say(*a):
    print(*a, flush=True)


def _run(phi, cfg, dev_weights, ids):
    m = phi.phi_load_fused(cfg, dev_weights)
    out = m.prefill_logits(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _gate(got, ref):
    s = parity.summary(got.reshape(-1, got.shape[-1]), ref.reshape(-1, ref.shape[-1]))
    _say(f"  min_cos={s['min_cos']:.9f} gated={s['gated']} agree={s['gated_agree']}")
    assert np.all(np.isfinite(got))
    assert s["min_cos"] >= COS_GATE, s
    assert not s["failures"], s
    return s


@pytest.mark.parametrize("batch,seq", [(1, 16), (2, 13), (3, 1)])
def test_tiny_f32_vs_oracle(phi, batch, seq):
    from logits_parity_amd.weights import to_device
    cfg = synth.TINY
    _say(f"tiny f32 {batch}x{seq}")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, batch, seq)
    got = _run(phi, cfg, to_device(ws, cfg.n_layers), ids)
    ref = prefill.prefill_logits(cfg, ws, ids)
    s = _gate(got, ref)
    assert s["min_cos"] > 1 - 1e-9


@pytest.mark.parametrize("wtype", ["f16", "i8"])
def test_tiny_low_precision_vs_oracle(phi, wtype):
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.TINY, wtype=wtype)
    _say(f"tiny {wtype}")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 2, 40)
    got = _run(phi, cfg, to_device(ws, cfg.n_layers), ids)
    _gate(got, prefill.prefill_logits(cfg, ws, ids))


def test_tiny_f16_prompt_of_max_pos_tokens(phi):
    # the longest prompt a model takes: positions up to max_pos - 1, the last
    # row of the RoPE tables (ragged against every tile and key block)
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.TINY, wtype="f16", max_pos=300)
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, cfg.max_pos)
    got = _run(phi, cfg, to_device(ws, cfg.n_layers), ids)
    _gate(got, prefill.prefill_logits(cfg, ws, ids))


def test_empty_prefill_is_refused_before_any_launch(phi):
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.TINY, wtype="f16")
    m = phi.phi_load_fused(cfg, to_device(synth.WeightSet(cfg), cfg.n_layers))
    L = phi.lib()
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    assert L.phi_prefill_logits(m.handle, p, 0, 8, p, p, 1 << 20, None) == 2  # PHI_E_SHAPE
    assert L.phi_prefill_logits(m.handle, p, 1, 0, p, p, 1 << 20, None) == 2
    assert L.phi_workspace_bytes(m.handle, 0, 8) == 0
    assert L.phi_workspace_bytes(m.handle, 1, 0) == 0
    torch.cuda.synchronize()
    assert int(buf.sum()) == 0  # nothing was written


def test_tiny_f32_gqa_unit_gains(phi):
    # harder regime: unit norm gains, GQA grouping
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.TINY, n_kv_heads=2, norm_gain="ones")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 33)
    got = _run(phi, cfg, to_device(ws, cfg.n_layers), ids)
    _gate(got, prefill.prefill_logits(cfg, ws, ids))


def test_tiny_bad_id_gives_nan_rows_only_in_its_sequence(phi):
    from logits_parity_amd.weights import to_device
    cfg = synth.TINY
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 2, 8).copy()
    ids[1, 3] = cfg.vocab + 5
    got = _run(phi, cfg, to_device(ws, cfg.n_layers), ids)
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1, :3]))
    assert np.all(np.isnan(got[1, 3:]))


def test_tiny_errors_are_reported(phi):
    from logits_parity_amd.weights import to_device
    cfg = synth.TINY
    dev = to_device(synth.WeightSet(cfg), cfg.n_layers)
    m = phi.phi_load_fused(cfg, dev)
    ids = torch.zeros((1, cfg.max_pos + 1), dtype=torch.int32, device="cuda")
    with pytest.raises(phi.PhiError) as e:
        m.prefill_logits(ids)
    assert e.value.status == 4  # PHI_E_RANGE
    ids = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(phi.PhiError) as e:
        m.prefill_logits(ids, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 5  # PHI_E_WORKSPACE


@pytest.mark.parametrize("wtype", ["f32", "f16"])
def test_tiny_host_ids_entry_point(phi, wtype):
    """phi_prefill_logits_host_ids: the same logits, bit for bit, as the
    device-ids entry point; an id outside [0, V) is refused on the host with
    PHI_E_RANGE and nothing is enqueued (the logits buffer keeps its
    sentinel)."""
    from logits_parity_amd.weights import to_device
    cfg = synth.TINY if wtype == "f32" else replace(synth.TINY, wtype=wtype)
    ws = synth.WeightSet(cfg)
    m = phi.phi_load_fused(cfg, to_device(ws, cfg.n_layers))
    ids = np.ascontiguousarray(synth.token_ids(cfg, 2, 11), dtype=np.int32)
    want = m.prefill_logits(torch.from_numpy(ids).cuda())
    got = torch.empty_like(want)
    phi.phi_prefill_logits_host_ids(m, ids, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    got_t = torch.full_like(want, 7.0)
    phi.phi_prefill_logits_host_ids(m, torch.from_numpy(ids), got_t)
    torch.cuda.synchronize()
    assert torch.equal(got_t, want)
    for bad in (-1, cfg.vocab):
        ids_bad = ids.copy()
        ids_bad[1, 4] = bad
        sentinel = torch.full_like(want, 7.0)
        with pytest.raises(phi.PhiError) as e:
            phi.phi_prefill_logits_host_ids(m, ids_bad, sentinel)
        assert e.value.status == 4  # PHI_E_RANGE
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all())


def test_mini_one_layer_ragged_1100_vs_oracle(phi):
    """Full Phi-3-mini width, one layer, 1100 tokens: the 1024-token-and-up
    GEMM tiles (QKV 256 x 192, gate/up and lm_head 256 x 256) with a ragged
    last M-tile of 76 rows, against the live oracle."""
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.MINI, n_layers=1)
    _say("mini 1 layer 1x1100")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 1100)
    got = _run(phi, cfg, to_device(ws, 1, "cuda"), ids)
    ref = prefill.prefill_logits(cfg, ws, ids)
    _gate(got, ref)


@pytest.mark.parametrize("batch,seq", [(1, 300), (3, 101)])
def test_mini_one_layer_head_and_a_half_qkv_vs_oracle(phi, batch, seq):
    """Full Phi-3-mini width, one layer, under 1024 tokens: QKV on 128 x 144
    tiles (one Q or K head plus half a V head each, nh + nkv = 64 tiles per
    128 tokens), with a ragged last M-tile; at S = 101 the V^T rows leave
    through the unaligned store path (8-token chunks straddle sequences)."""
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.MINI, n_layers=1)
    _say(f"mini 1 layer {batch}x{seq}")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, batch, seq)
    got = _run(phi, cfg, to_device(ws, 1, "cuda"), ids)
    ref = prefill.prefill_logits(cfg, ws, ids)
    _gate(got, ref)


def test_mini_w8_one_layer_ragged_1100_vs_oracle(phi):
    """The same shape with int8 weights against the oracle on those weights:
    the 8-wave 256 x 192 QKV tile (44 register-staged copies per stage padded
    to 6 per wave) and the int8 256 x 256 gate/up and lm_head tiles, with a
    ragged last M-tile."""
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.MINI_W8, n_layers=1)
    _say("mini int8 1 layer 1x1100")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 1100)
    got = _run(phi, cfg, to_device(ws, 1, "cuda"), ids)
    ref = prefill.prefill_logits(cfg, ws, ids)
    _gate(got, ref)


@pytest.mark.parametrize("batch,seq", [(1, 300), (3, 101)])
def test_mini_w8_one_layer_under_1024_vs_oracle(phi, batch, seq):
    """Full Phi-3-mini width, one layer, int8 weights, under 1024 tokens,
    against the oracle on those weights: the int8 128 x 192 QKV tile, the
    5-split residual GEMMs on 256 x 128 tiles (binary16 partials summed by the
    RMSNorm), the int8 256 x 128 gate/up tile and the 256 x 256 lm_head, with
    a ragged last M-tile (and, at S = 101, sequences that straddle tiles)."""
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.MINI_W8, n_layers=1)
    _say(f"mini int8 1 layer {batch}x{seq}")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, batch, seq)
    got = _run(phi, cfg, to_device(ws, 1, "cuda"), ids)
    ref = prefill.prefill_logits(cfg, ws, ids)
    _gate(got, ref)


@pytest.mark.parametrize("wtype", ["f16", "i8"])
def test_mini_one_layer_ragged_4000_vs_oracle(phi, wtype):
    """One layer, 4000 tokens: the residual GEMMs take the 8-wave 256 x 192
    tile (16 x 16 = 256 tiles; int8 with its register-staged copies padded)
    with a last M-tile of 160 rows, and attention the 8-wave
    shared-key-block kernel at a ragged S (the oracle takes about 40 s)."""
    from logits_parity_amd.weights import to_device
    cfg = replace(synth.MINI if wtype == "f16" else synth.MINI_W8, n_layers=1)
    _say(f"mini {wtype} 1 layer 1x4000")
    ws = synth.WeightSet(cfg)
    ids = synth.token_ids(cfg, 1, 4000)
    got = _run(phi, cfg, to_device(ws, 1, "cuda"), ids)
    _say("  oracle")
    ref = prefill.prefill_logits(cfg, ws, ids)
    _gate(got, ref)


# ---------------------------------------------------------------- full shapes
def _golden(name):
    path = os.path.join(GOLDEN, name + ".npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    return np.load(path)


def _all_position_cosines(g, got_flat, lm_head):
    """Cosine at every position: each reference row is the oracle's lm_head
    step on its stored final hidden state (float32-stored, moving a cosine by
    about 1e-14)."""
    hidden = g["hidden"]
    assert hidden.shape[0] == got_flat.shape[0]
    cos = np.empty(len(got_flat))
    for r0 in range(0, len(got_flat), 512):
        ref = prefill.logits_from_hidden(hidden[r0:r0 + 512], lm_head)
        cos[r0:r0 + 512] = parity.row_cosines(got_flat[r0:r0 + 512], ref)
    return cos


def _check_golden(g, got_flat, ids, digest, prefix="", lm_head=None):
    """Oracle-trust first: the stored results must belong to these exact
    inputs.  Returns the cosines (at every position when the stored hidden
    state and the lm_head are given, else at the sampled rows) and the
    positions whose gated argmax disagrees."""
    assert str(g["ids_sha256"]) == hashlib.sha256(np.ascontiguousarray(ids, np.int32).tobytes()).hexdigest()
    assert str(g[prefix + "weights_sha256"]) == digest
    pos = g["pos"]
    rows = g[prefix + "rows"].astype(np.float64)
    cos = parity.row_cosines(got_flat[pos], rows)
    gap = g[prefix + "gap"]
    agree = np.argmax(got_flat, axis=1) == g[prefix + "argmax"]
    gated = gap > 1e-3
    fails = np.nonzero(gated & ~agree)[0]
    _say(f"  sampled min_cos={cos.min():.9f} mean={cos.mean():.9f}; argmax gated={gated.sum()} "
         f"agree={(agree & gated).sum()} all-agree={agree.sum()}/{len(agree)}")
    if lm_head is not None and not prefix:
        full = _all_position_cosines(g, got_flat, lm_head)
        # the sampled rows agree with the rows formed from the stored hidden state
        assert np.abs(full[pos] - cos).max() < 1e-9
        _say(f"  every position ({len(full)}): min_cos={full.min():.9f} mean={full.mean():.9f} "
             f"worst at {int(np.argmin(full))}")
        cos = full
    return cos, fails


@pytest.fixture(scope="module")
def mini_digest(mini_f16):
    return mini_f16[0].digest()


@pytest.mark.parametrize("name", ["mini_f16_1x512", "mini_f16_1x4096"])
def test_mini_f16_vs_stored_oracle(phi, mini_f16, mini_digest, name):
    wl = synth.PREFILL_WORKLOADS[name]
    _say(f"{name}")
    g = _golden(name)
    ids = synth.token_ids(wl.cfg, wl.batch, wl.seq)
    got = _run(phi, wl.cfg, mini_f16[1], ids).reshape(-1, wl.cfg.vocab).astype(np.float64)
    assert np.all(np.isfinite(got))
    cos, fails = _check_golden(g, got, ids, mini_digest, lm_head=mini_f16[0].lm_head)
    assert len(cos) == wl.tokens
    assert cos.min() >= COS_GATE
    assert len(fails) == 0, fails[:20]


def test_mini_w8_vs_stored_oracle(phi, mini_w8, mini_digest):
    name = "mini_w8_4x1024"
    wl = synth.PREFILL_WORKLOADS[name]
    _say(name)
    g = _golden(name)
    ids = synth.token_ids(wl.cfg, wl.batch, wl.seq)
    got = _run(phi, wl.cfg, mini_w8[1], ids).reshape(-1, wl.cfg.vocab).astype(np.float64)
    assert np.all(np.isfinite(got))
    cos, fails = _check_golden(g, got, ids, mini_w8[0].digest(), lm_head=mini_w8[0].lm_head)
    assert len(cos) == wl.tokens
    assert cos.min() >= COS_GATE
    assert len(fails) == 0, fails[:20]
    # reported: distance to the float16 oracle is the quantisation's, not the kernel's
    cos16, _ = _check_golden(g, got, ids, mini_digest, prefix="f16_")
    ref_i8 = g["rows"].astype(np.float64)
    floor = parity.row_cosines(ref_i8, g["f16_rows"].astype(np.float64))
    _say(f"  vs f16 oracle: min_cos={cos16.min():.7f}; oracle(int8) vs oracle(f16) floor={floor.min():.7f}")
    assert abs(cos16.min() - floor.min()) < 1e-5


def test_mini_prefix_invariance_and_determinism(phi, mini_f16):
    wl = synth.PREFILL_WORKLOADS["mini_f16_1x512"]
    ids = synth.token_ids(wl.cfg, 1, 512)
    a = _run(phi, wl.cfg, mini_f16[1], ids)
    b = _run(phi, wl.cfg, mini_f16[1], ids)
    assert np.array_equal(a, b)
    # a shorter prefix may take other GEMM tile shapes and K splits (the plan
    # depends on the token count), so it sums in another order: equal to
    # within fp32 rounding, same argmax wherever the top-2 gap exceeds 1e-3
    c = _run(phi, wl.cfg, mini_f16[1], ids[:, :200])
    s = parity.summary(c[0], a[0, :200])
    _say(f"  200-token prefix vs the 512-token run: 1 - min_cos = {1 - s['min_cos']:.3e}, "
         f"bitwise equal rows {int(np.all(c[0] == a[0, :200], axis=1).sum())}/200")
    assert s["min_cos"] > 1 - 1e-6 and not s["failures"], s
