"""The C ABI library: exports and host-side argument checks (CPU only; no
entry point here reaches a HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import logits_parity_amd as phi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "phi.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declarations_are_all_exported():
    names = declared_functions()
    assert len(names) >= 12, names
    out = subprocess.run(["nm", "-D", "--defined-only", phi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(phi.EXPORTS)
    L = phi.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_status_strings():
    assert phi.strerror(0) == "ok"
    assert "workspace" in phi.strerror(5)
    assert phi.strerror(99) == "unknown status"


def test_pool_slots_reproduce_the_page():
    # Phi-4 page, pool paragraph: 223,696 (K16/V8) and 167,760 (FP16) slots per layer
    assert phi.phi_kv_pool_slots(32 << 30, 40, 10, 128, 2, 1, 16) == 223696
    assert phi.phi_kv_pool_slots(32 << 30, 40, 10, 128, 2, 2, 16) == 167760
    assert phi.phi_kv_pool_slots(0, 40, 10, 128, 2, 1, 16) == -1


def _cfg(**kw):
    import synth
    from dataclasses import replace
    return phi.make_config(replace(synth.TINY, **kw))


def _load(cfg, layers=None, state=0x1000, state_bytes=1 << 24, w=None):
    L = phi.lib()
    n = cfg.n_layers
    if layers is None:
        layers = (phi.phi_layer_weights * n)()
        for i in range(n):
            layers[i] = phi.phi_layer_weights(0x100, phi.phi_linear(0x200, None), phi.phi_linear(0x300, None),
                                              0x400, phi.phi_linear(0x500, None), phi.phi_linear(0x600, None))
    if w is None:
        w = phi.phi_weights(0x700, layers, 0x800, phi.phi_linear(0x900, None))
    h = ctypes.c_void_p()
    return L.phi_load_fused(ctypes.byref(cfg), ctypes.byref(w), state, state_bytes, None, ctypes.byref(h))


def test_load_rejects_bad_arguments_before_any_hip_call():
    assert _load(_cfg(), state=None) == 1                           # PHI_E_NULL
    assert _load(_cfg(head_dim=64)) == 2                            # PHI_E_SHAPE
    assert _load(_cfg(hidden=100)) == 2
    assert _load(_cfg(n_kv_heads=3)) == 2
    assert _load(_cfg(max_pos=8192)) == 2
    c = _cfg()
    c.wtype = 7
    assert _load(c) == 3                                            # PHI_E_DTYPE
    c = _cfg()
    c.rms_eps = 0.0
    assert _load(c) == 4                                            # PHI_E_RANGE
    assert _load(_cfg(), state_bytes=16) == 5                       # PHI_E_WORKSPACE
    assert _load(_cfg(), state=0x1008) == 6                         # PHI_E_ALIGN
    c = _cfg(wtype="i8")
    assert _load(c) == 1  # int8 weights need scales


def test_other_entry_points_reject_bad_arguments():
    L = phi.lib()
    assert L.phi_prefill_logits(None, None, 1, 1, None, None, 0, None) == 1
    assert L.phi_linear_f32out(1, 0x100, 0x200, None, 0x300, 4, 4, 60, None) == 2
    assert L.phi_linear_f32out(2, 0x100, 0x200, None, 0x300, 4, 4, 64, None) == 1
    assert L.phi_linear_f32out(1, 0x108, 0x200, None, 0x300, 4, 4, 64, None) == 6
    assert L.phi_attention_prefill(0, 0x100, 0x200, 0x300, 0x400, 1, 5000, 4, 4, 96, None) == 4
    assert L.phi_attention_prefill(0, 0x100, 0x200, 0x300, 0x400, 1, 16, 4, 3, 96, None) == 2
    args = [0x100, 0x200, 0x300, 0x400, 0x500, 0x600]
    ok = dict(batch=2, hq=8, hkv=2, d=128, page=16, n_pages=8, max_pages=4, max_ctx=64)

    def dec(ws_bytes=1 << 20, **kw):
        p = dict(ok, **kw)
        return L.attn_decode_k16v8(*args, p["batch"], p["hq"], p["hkv"], p["d"], p["page"], p["n_pages"],
                                   p["max_pages"], p["max_ctx"], 0.1, 0x700, 0x800, ws_bytes, None)
    assert dec(d=96) == 2
    assert dec(page=32) == 2
    assert dec(hq=6, hkv=4) == 2
    assert dec(hq=48, hkv=2) == 2          # GQA group of 24 unsupported
    assert dec(max_ctx=65) == 4            # beyond max_pages * 16
    assert dec(ws_bytes=8) == 5
    assert L.attn_decode_k16v8_workspace_bytes(32, 40, 10, 128, 1024) > 0
    assert L.attn_decode_k16v8_workspace_bytes(32, 40, 10, 96, 1024) == 0

    def app(**kw):
        p = dict(batch=2, hkv=2, d=128, page=16, n_pages=8, max_pages=4, k_new=0x100, k_pool=0x600)
        p.update(kw)
        return L.kv_append_k16v8(p["k_new"], 0x200, 0x300, 0x400, 0x500, p["batch"], p["hkv"], p["d"], p["page"],
                                 p["n_pages"], p["max_pages"], p["k_pool"], 0x700, None)
    assert app(k_new=None) == 1
    assert app(d=96) == 2
    assert app(page=8) == 2
    assert app(batch=-1) == 2
    assert app(k_pool=0x604) == 6
    assert app(batch=0) == 0               # nothing to write, nothing enqueued
    assert L.phi_prefill_fill_k16v8(None, 0x100, 1, 1, 0x200, None, 0x300, 1 << 20, None) == 1
    assert L.phi_decode_step_k16v8(None, 0x100, 0x200, 1, 1, None, 0x300, 0x400, 1 << 20, None) == 1
    assert L.phi_decode_workspace_bytes(None, 1, 16) == 0


def test_int32_offset_guards_before_any_hip_call():
    """The GEMM kernels form operand offsets in int32: a weight or activation
    of 2^31 elements or more is refused on the host (PHI_E_SHAPE)."""
    L = phi.lib()
    # lm_head [V][H] just below 2^31 elements passes the shape checks (and stops
    # at the misaligned state pointer, still before any HIP call)
    assert _load(_cfg(hidden=8192, vocab=262144 - 4), state=0x1008) == 6
    assert _load(_cfg(hidden=8192, vocab=262144)) == 2         # V * H = 2^31
    assert _load(_cfg(hidden=4096, intermediate=262144)) == 2  # gate_up [2I][H] = 2^31
    assert _load(_cfg(n_heads=1 << 20, n_kv_heads=1 << 20)) == 2   # head count bounded before any product
    assert _load(_cfg(n_heads=(1 << 16) - 32, n_kv_heads=1)) == 2  # fused QKV rows x H past 2^31
    assert L.phi_linear_f32out(1, 0x100, 0x200, None, 0x300, 1 << 25, 4, 64, None) == 2   # M * K = 2^31
    assert L.phi_linear_f32out(1, 0x100, 0x200, None, 0x300, 4, 1 << 25, 64, None) == 2   # N * K = 2^31
    assert L.phi_gate_up_silu(1, 0x100, 0x200, None, 0x300, 4, 1 << 24, 64, None) == 2    # 2 I * K = 2^31
    assert L.phi_gate_up_silu(1, 0x100, 0x200, None, 0x300, 1 << 25, 128, 64, None) == 2  # M * K = 2^31


def test_noalloc_decode_rejects_before_any_hip_call():
    """attn_decode_k16v8_noalloc takes the checks of attn_decode_k16v8, and a
    plan whose partials exceed the library's scratch array is refused with
    PHI_E_WORKSPACE before anything is enqueued."""
    L = phi.lib()
    args = [0x100, 0x200, 0x300, 0x400, 0x500, 0x600]

    def dec(batch=2, hq=8, hkv=2, d=128, page=16, n_pages=8, max_pages=4, max_ctx=64):
        return L.attn_decode_k16v8_noalloc(*args, batch, hq, hkv, d, page, n_pages, max_pages, max_ctx, 0.1,
                                           0x700, None)
    assert L.attn_decode_k16v8_noalloc(None, *args[1:], 2, 8, 2, 128, 16, 8, 4, 64, 0.1, 0x700, None) == 1
    assert dec(d=96) == 2
    assert dec(hq=6, hkv=4) == 2
    assert dec(max_ctx=65) == 4
    limit = 16 << 20
    need = L.attn_decode_k16v8_workspace_bytes(4096, 64, 8, 128, 100000)
    assert need > limit
    assert dec(batch=4096, hq=64, hkv=8, n_pages=1 << 20, max_pages=6250, max_ctx=100000) == 5
    assert L.attn_decode_k16v8_workspace_bytes(3, 40, 10, 128, 3000) <= limit


def test_host_ids_entry_point_rejects_null_arguments():
    """phi_prefill_logits_host_ids checks its pointers before anything else."""
    L = phi.lib()
    ids = (ctypes.c_int32 * 4)(0, 1, 2, 3)
    assert L.phi_prefill_logits_host_ids(None, ids, 1, 4, 0x1000, 0x2000, 1 << 20, None) == 1
    assert L.phi_prefill_logits_host_ids(0x100, None, 1, 4, 0x1000, 0x2000, 1 << 20, None) == 1
    assert L.phi_prefill_logits_host_ids(0x100, ids, 1, 4, None, 0x2000, 1 << 20, None) == 1


def test_binding_refuses_strided_tensors():
    """The binding passes raw addresses, and the library reads every operand as
    a dense row-major array: a strided view (a broadcast, a transpose, a
    stepped slice) is refused in Python before any library call."""
    import torch
    base = torch.zeros((4, 6), dtype=torch.float16)
    assert phi._ptr(None) is None
    assert phi._ptr(base) == base.data_ptr()
    assert phi._ptr(base[1:3]) == base[1:3].data_ptr()  # whole rows stay dense
    for view in (base.t(), base[:, :3], base[::2], torch.zeros(6, dtype=torch.float16).expand(4, 6)):
        with pytest.raises(ValueError, match="not contiguous"):
            phi._ptr(view)
    with pytest.raises(ValueError, match="not contiguous"):
        phi.phi_attention_prefill(torch.zeros((1, 2, 8, 96), dtype=torch.float16).transpose(1, 2),
                                  torch.zeros((1, 2, 8, 96), dtype=torch.float16),
                                  torch.zeros((1, 2, 96, 64), dtype=torch.float16), out=base)


def test_decode_plan_split_counts():
    # the decode workspace holds (o, max, sum) partials per (sequence, query
    # head, split), so its size shows the split plan: one split per sequence
    # (8-wave workgroups) where the context fits 512 pages and the (sequence,
    # KV head) pairs number at least 128; the 4-wave split plan below that
    L = phi.lib()
    r = lambda x: (x + 255) // 256 * 256

    def splits(B, ctx, hq=40, hkv=10):
        got = L.attn_decode_k16v8_workspace_bytes(B, hq, hkv, 128, ctx)
        found = [s for s in range(1, 65) if r(B * hq * s * 128 * 4) + r(B * hq * s * 2 * 4) == got]
        assert len(found) == 1, (B, ctx, got)
        return found[0]
    assert splits(32, 1024) == 1    # 320 pairs: one 64-page split each, 4 waves
    assert splits(16, 8192) == 1    # 160 pairs: one 512-page split each, 8 waves
    assert splits(16, 4096) == 1
    assert splits(24, 8192) == 1
    assert splits(12, 8192) == 4    # 120 pairs: four 128-page splits and the merge
    assert splits(8, 8192) == 4     # 80 pairs
    assert splits(16, 16384) == 4   # 1024 pages do not fit one split


def test_no_packed_fp32_instructions_in_device_code(tmp_path):
    """Device code is built with packed fp32 math disabled; check the ISA of
    this build for any v_pk_{add,mul,fma}_f32."""
    bundler = "/opt/rocm/llvm/bin/clang-offload-bundler"
    objdump = "/opt/rocm/llvm/bin/llvm-objdump"
    if not (os.path.exists(bundler) and os.path.exists(objdump)):
        pytest.skip("LLVM tools not found")
    fatbin = tmp_path / "fatbin"
    r = subprocess.run(["/opt/rocm/llvm/bin/llvm-objcopy", "--dump-section=.hip_fatbin=" + str(fatbin),
                        phi.LIB_PATH], capture_output=True)
    assert r.returncode == 0, r.stderr
    co = tmp_path / "gfx950.co"
    r = subprocess.run([bundler, "--type=o", "--unbundle", f"--input={fatbin}", f"--output={co}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950"], capture_output=True)
    assert r.returncode == 0, r.stderr
    dis = subprocess.run([objdump, "-d", str(co)], capture_output=True, text=True).stdout
    assert "v_mfma_f32_32x32x16_f16" in dis
    bad = [l for l in dis.splitlines() if re.search(r"v_pk_(add|mul|fma)_f32", l)]
    assert not bad, bad[:5]
