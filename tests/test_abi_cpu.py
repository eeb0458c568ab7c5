"""Host-side checks of the C ABI (no GPU calls): the library loads, exports every
declared symbol, and its configuration / sizing / validation logic is right."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from gpt_pretraining_step_train_amd import binding, configs, inputs
from oracle import polar_express

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.lib()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "gpt.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"\b((?:gpt|gptk|muon)_\w+)\s*\(", hdr))
    assert len(names) >= 30
    raw = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(raw, n)]
    assert not missing, missing


def test_cfg_from_depth(lib):
    want = {12: (768, 6, 3072), 24: (1536, 12, 6144), 26: (1664, 13, 6656)}
    for depth, (d, h, f) in want.items():
        c = binding.GptCfg()
        assert lib.gpt_cfg_from_depth(depth, ctypes.byref(c)) == 0
        assert (c.d_model, c.n_head, c.head_dim, c.d_ff) == (d, h, 128, f)
        assert (c.vocab, c.seq_len, c.batch) == (32768, 2048, 16)
        assert lib.gpt_cfg_validate(ctypes.byref(c)) == 0
        n = configs.n_params(dict(depth=depth, d_model=d, d_ff=f, vocab=32768))
        assert c.num_steps == round(8 * n / 2 ** 20)
    c = binding.GptCfg()
    assert lib.gpt_cfg_from_depth(0, ctypes.byref(c)) == 1
    c = binding.GptCfg()
    lib.gpt_cfg_from_depth(13, ctypes.byref(c))
    assert c.d_model % 128 == 0 and c.n_head * c.head_dim == c.d_model


def test_param_counts_of_the_five_configs():
    assert configs.n_params(configs.get("tiny")) == 1441792
    assert configs.n_params(configs.get("laptop")) == 2899968
    assert configs.n_params(configs.get("d12")) == 135266304
    assert configs.n_params(configs.get("d24")) == 780140544
    assert configs.n_params(configs.get("d26")) == 972947456


def test_default_ns_table(lib):
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "ns_printed_coeffs.json")))
    c = binding.GptCfg()
    c.attn_window, c.n_kv_head, c.extras = 7, 3, 5  # overwritten with the defaults
    lib.gpt_cfg_from_depth(24, ctypes.byref(c))
    tab = c.coeffs()
    assert c.ns_steps == gold["ns_steps"] and c.ns_split_steps == 0 and c.fp8_gemms == 7
    assert c.attn_window == 0 and c.n_kv_head == 0 and c.extras == 0
    assert c.normuon_beta2 == pytest.approx(0.95)
    assert ctypes.sizeof(binding.GptCfg) == lib.gpt_cfg_bytes() == 152
    np.testing.assert_allclose(tab[:2], gold["printed"], rtol=0, atol=1e-6)
    derived, _ = polar_express.coefficients()
    np.testing.assert_allclose(tab[2:], derived[2:], rtol=0, atol=2e-5)


def test_validation_errors(lib):
    base = binding.make_cfg(configs.get("laptop"))
    assert lib.gpt_cfg_validate(ctypes.byref(base)) == 0
    for field, val, code in [("head_dim", 48, 6), ("n_head", 5, 2), ("d_model", 2056, 2), ("precision", 7, 6),
                             ("ns_steps", 6, 1), ("batch", 0, 2), ("vocab", 4100, 2), ("fp8_gemms", 8, 1),
                             ("attn_window", -1, 1), ("n_kv_head", 2, 2), ("n_kv_head", 4, 2),
                             ("n_kv_head", -1, 2), ("extras", 32, 1), ("extras", -1, 1)]:
        c = binding.make_cfg(configs.get("laptop"))
        setattr(c, field, val)
        assert lib.gpt_cfg_validate(ctypes.byref(c)) == code, field
        assert lib.gpt_state_bytes(ctypes.byref(c)) == 0
    for b2, code in ((1.0, 1), (-0.1, 1), (float("nan"), 1), (0.0, 0)):  # NorMuon's decay, checked when on
        c = binding.make_cfg(configs.get("laptop", extras=16))
        c.normuon_beta2 = b2
        assert lib.gpt_cfg_validate(ctypes.byref(c)) == code, b2
    assert lib.gpt_cfg_validate(None) == 1
    assert lib.gpt_status_str(3).decode() == "token id out of range"


@pytest.mark.parametrize("name,over", [("tiny", {}), ("laptop", {}), ("d12", {}), ("d24", {}),
                                       ("tiny", {"n_kv_head": 2}), ("laptop", {"n_kv_head": 1}),
                                       ("d24", {"n_kv_head": 4}), ("tiny", {"extras": 7}),
                                       ("laptop", {"extras": 2}), ("d24", {"extras": 7, "n_kv_head": 4}),
                                       ("tiny", {"extras": 15}), ("laptop", {"extras": 8, "n_kv_head": 1}),
                                       ("d24", {"extras": 15, "n_kv_head": 4}), ("laptop", {"extras": 16}),
                                       ("tiny", {"extras": 31})])
def test_state_bytes_and_tensor_table(lib, name, over):
    for cfg in [configs.get(name, **over)]:
        c = binding.make_cfg(cfg)
        nb = lib.gpt_state_bytes(ctypes.byref(c))
        n = configs.n_params(cfg)
        assert nb > 3 * 4 * n                     # params + grads + momentum at least
        assert nb < 288 * 2 ** 30                # fits one MI355X
        ex = cfg.get("extras", 0)
        assert lib.gpt_tensor_count(ctypes.byref(c)) == (2 + 6 * cfg["depth"] + bool(ex & 15)
                                                         + (cfg["depth"] + 1) * bool(ex & 8))
        shapes = inputs.tensor_shapes(cfg)
        assert n == sum(r * k for _, (r, k) in shapes)
        for i, (nm, shp) in enumerate(shapes):
            r, k = ctypes.c_int32(), ctypes.c_int32()
            assert lib.gpt_tensor_shape(ctypes.byref(c), i, ctypes.byref(r), ctypes.byref(k)) == 0
            assert (r.value, k.value) == shp, nm
        r, k = ctypes.c_int32(), ctypes.c_int32()
        assert lib.gpt_tensor_shape(ctypes.byref(c), len(shapes), ctypes.byref(r), ctypes.byref(k)) == 1
    d24 = binding.make_cfg(configs.get("d24"))
    assert lib.gpt_state_bytes(ctypes.byref(d24)) < 100 * 2 ** 30


def test_kernel_names(lib):
    assert binding.gemm_kernel_name(1, 32768, 6144, 1536) == "gemm_bf16_dma_kernel<256,256,NT>"
    assert binding.gemm_kernel_name(1, 32768, 1536, 6144, b_kmaj=0) == "gemm_bf16_dma_kernel<256,256,NN>"
    assert binding.gemm_kernel_name(1, 512, 384, 128, a_kmaj=0, b_kmaj=0) == "gemm_bf16_kernel<128,128,TN>"
    assert binding.gemm_kernel_name(0, 512, 384, 128) == "gemm_f32_kernel<NT>"


def test_configs_flops_formula():
    f = configs.step_flops(configs.get("d24"))
    assert abs(f["total"] - 1.844e14) / 1.844e14 < 3e-3
    assert abs(f["muon"] - 300 * 24 * 1536 ** 3) < 1
    # attention: 12 L B d flops per visible (query, key) pair, counted by brute force
    for W in (1, 7, 100, 2047, 2048, 5000):
        c = configs.get("d24", attn_window=W)
        pairs = sum(min(i + 1, W) for i in range(c["seq_len"]))
        assert configs.step_flops(c)["attn"] == 12 * 24 * 16 * 1536 * pairs
    assert configs.step_flops(configs.get("d24", attn_window=2048))["attn"] == f["attn"]
    # grouped-query attention shrinks Wk, Wv (and their Newton-Schulz), not attention
    g = configs.step_flops(configs.get("d24", n_kv_head=4))
    assert g["attn"] == f["attn"] and g["linear"] < f["linear"] and g["muon"] < f["muon"]


def test_arena_too_small_is_rejected_before_any_device_call(lib):
    """gpt_init checks the arena against gpt_state_bytes (and its alignment) before it
    touches the device, so a short or misaligned arena is GPT_ERR_ARG on any host."""
    c = binding.make_cfg(configs.get("laptop"))
    need = lib.gpt_state_bytes(ctypes.byref(c))
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the checks come first
    out = ctypes.c_void_p()
    assert lib.gpt_init(ctypes.byref(c), 0, fake, need - 1, None, ctypes.byref(out)) == 1
    assert lib.gpt_init(ctypes.byref(c), 0, ctypes.c_void_p((1 << 20) + 16), need, None, ctypes.byref(out)) == 1
    assert lib.gpt_init(ctypes.byref(c), 0, None, need, None, ctypes.byref(out)) == 1
    assert not out.value
    bad = binding.make_cfg(configs.get("laptop", head_dim=48))
    assert lib.gpt_init(ctypes.byref(bad), 0, fake, need, None, ctypes.byref(out)) == 6


def test_gemm_argument_checks_run_before_any_launch(lib):
    """gptk_gemm rejects leading dimensions shorter than a stored row, negative or short
    batch strides and grids beyond 65535 rows before launching anything."""
    p = ctypes.c_void_p(1 << 20)  # never dereferenced

    def call(ak=1, bk=1, M=64, N=64, K=64, batch=1, lda=64, sA=0, ldb=64, sB=0, ldc=64, sC=0, splits=1):
        return lib.gptk_gemm(1, ak, bk, M, N, K, batch, p, lda, sA, p, ldb, sB, p, ldc, sC, 0, splits, p, 0, None)
    assert call(lda=63) == 1                       # k-major A needs lda >= K
    assert call(ak=0, M=128, lda=100) == 1         # transposed A needs lda >= M
    assert call(ldb=32) == 1
    assert call(bk=0, N=128, ldb=64) == 1
    assert call(ldc=63) == 1
    assert call(batch=2, sA=-1, sC=64 * 64) == 1
    assert call(batch=2, sA=100, sC=64 * 64) == 1  # neither shared (0) nor a whole matrix
    assert call(batch=2, sB=64, sC=64 * 64) == 1
    assert call(batch=2, sC=64 * 63) == 1          # outputs of two batch entries would overlap
    assert call(batch=40000, sC=64 * 64, splits=2) == 1   # grid rows
    assert call(M=-1) == 1
    assert lib.gptk_gemm(7, 1, 1, 64, 64, 64, 1, p, 64, 0, p, 64, 0, p, 64, 0, 0, 1, p, 0, None) == 6
    assert lib.gptk_gemm_fp8(64, 64, 64, p, 32, p, 64, p, p, p, 64, 1, p, 0, None) == 1
    assert lib.gptk_gemm_split(1, 1, 64, 64, 64, 1, p, p, 64, 0, p, p, 64, 0, p, 32, 0, None) == 1


def test_auto_split_factors_of_the_d24_weight_gradients(lib):
    """The factors gpt_step's d24 weight-gradient launches take over K = 32768 tokens
    (the GPU test checks those launches against fp64)."""
    f = {(m, n): binding.gemm_auto_splits(1, m, n, 32768, 1, 0, 0)
         for m, n in [(4608, 1536), (1536, 1536), (6144, 1536), (1536, 6144), (32768, 1536)]}
    assert f[(4608, 1536)] == 2 and f[(1536, 1536)] == 7 and f[(6144, 1536)] == 5 and f[(1536, 6144)] == 5
    assert f[(32768, 1536)] == 1


def test_capture_sizes(lib):
    """gpt_capture_bytes: 15 items of a block layer, 4 of the LM head, 256-byte aligned."""
    cfg = configs.get("d24", batch=1)
    c = binding.make_cfg(cfg)
    N, d, F, V = 2048, 1536, 6144, 32768
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    QD = 3 * d
    block = [N * d * 2, N * QD * 2, N * d * 4, N * d * 2, N * d * 4, N * d * 2, N * F * 2, N * d * 4,
             N * d * 2, N * F * 2, N * d * 4, N * d * 2, N * d * 2, N * QD * 2, N * d * 4]
    head = [N * d * 2, N * V * 4, N * V * 2, N * d * 4]
    assert lib.gpt_capture_bytes(ctypes.byref(c), 0) == sum(al(x) for x in block)
    assert lib.gpt_capture_bytes(ctypes.byref(c), 23) == sum(al(x) for x in block)
    assert lib.gpt_capture_bytes(ctypes.byref(c), 24) == sum(al(x) for x in head)
    assert lib.gpt_capture_bytes(ctypes.byref(c), 25) == 0
    assert lib.gpt_capture_bytes(ctypes.byref(c), -1) == 0
    assert lib.gpt_capture(None, 0, None, 0) == 1
    names = [n for n, _, _ in binding.Model.CAPTURE_BLOCK]
    assert len(names) == len(block) and len(binding.Model.CAPTURE_HEAD) == len(head)


ERR_ARG = 1  # GPT_ERR_ARG in include/gpt.h


def test_process_switches_validate_and_report(lib):
    """The process-wide switches set no device state: they validate their argument and
    return the previous setting (a negative argument only queries)."""
    prev = lib.gptk_side_stream(-1)
    assert prev == 1                                   # default: where CUs would idle
    assert lib.gptk_side_stream(0) == 1
    assert lib.gptk_side_stream(2) == 0
    assert lib.gptk_side_stream(-1) == 2
    assert lib.gptk_side_stream(prev) == 2
    assert lib.gptk_side_stream(-1) == prev
    assert lib.gptk_ce_variant(1) == 0 and lib.gptk_ce_variant(0) == 0
    for bad in (-1, 2, 7):
        assert lib.gptk_ce_variant(bad) == ERR_ARG
    for p, v in ((0, 2), (1, 3), (2, 0), (-1, 0), (0, -1)):
        assert lib.gptk_attn_variant(p, v) == ERR_ARG
    assert lib.gptk_attn_variant(0, 0) == 0 and lib.gptk_attn_variant(1, 0) == 0
