"""The C-ABI library loads, exports every entry point include/moe.h
declares, and rejects bad arguments on the host before any launch (CPU only:
no compute call is made)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_permute_amd as M
from mixture_experts_layer_permute_amd import _lib, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return M.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_gate_topk", "moe_permute", "moe_expert_ffn_fwd",
              "moe_expert_ffn_bwd", "moe_combine", "moe_unpermute_grad",
              "moe_combine_bwd", "moe_gate_topk_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, "binding lacks " + n


def test_binding_names_match_c_names():
    for n in ("moe_gate_topk", "moe_permute", "moe_expert_ffn_fwd",
              "moe_expert_ffn_bwd", "moe_combine", "moe_unpermute_grad",
              "moe_combine_bwd", "moe_gate_topk_bwd", "moe_init",
              "moe_expert_ffn_fwd_gather", "moe_expert_ffn_bwd_gather"):
        assert callable(getattr(M, n))


def test_status_strings_and_version(lib):
    assert lib.moe_abi_version() == 7
    for s in (0, -1, -2, -3, -4):
        assert lib.moe_status_string(s)


def test_workspace_queries(lib):
    assert lib.moe_permute_workspace_bytes(8192, 8, 2) > 0
    assert lib.moe_permute_workspace_bytes(-1, 8, 2) == 0
    # backward FFN workspace holds dH [R, f] (x2 for SwiGLU)
    R, E, d, f = 16384, 8, 1024, 4096
    bw = lib.moe_ffn_workspace_bytes(R, E, d, f, 0, 1, 1)
    assert bw >= 2 * R * f
    assert lib.moe_ffn_workspace_bytes(R, E, d, f, 1, 1, 1) >= 4 * R * f
    assert lib.moe_ffn_workspace_bytes(R, E, d, 100, 0, 1, 0) == 0   # f % 64
    assert lib.moe_gate_bwd_workspace_bytes(8192, 1024, 8) > 0


def test_invalid_arguments_rejected_before_launch(lib):
    N = None
    INV = _lib.MOE_ERR_INVALID_ARG
    # k > E
    assert lib.moe_gate_topk(N, N, N, 10, 64, 4, 5, 1, 0, N, N, N, N) == INV
    # E > 1024
    assert lib.moe_gate_topk(N, N, N, 10, 64, 2000, 2, 1, 0, N, N, N, N) == INV
    # bad dtype
    assert lib.moe_gate_topk(N, N, N, 10, 64, 4, 1, 1, 7, N, N, N, N) == INV
    # T = 0 is a no-op
    assert lib.moe_gate_topk(N, N, N, 0, 64, 4, 1, 1, 0, N, N, N, N) == 0
    # null pointers
    assert lib.moe_gate_topk(N, N, N, 10, 64, 4, 1, 1, 0, N, N, N, N) == INV
    # d not a multiple of 64 for the row kernels
    assert lib.moe_combine(N, N, N, 10, 2, 100, 1, N, N) == INV
    assert lib.moe_unpermute_grad(N, N, 10, 2, 100, 1, N, 0, N) == INV
    # f not a multiple of 64
    assert lib.moe_expert_ffn_fwd(N, N, 10, 2, 64, 100, 0, 1, N, N, N, N, N, N, N, 0,
                                  N) == INV
    # workspace too small
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    assert lib.moe_permute(p, p, 100, 64, 4, 2, 0, p, p, p, p, p, p, 0, N) == \
        _lib.MOE_ERR_WORKSPACE


def test_gather_entry_points_validate_on_host(lib):
    N = None
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    # the bf16 source must stay under 2^31 bytes (32-bit buffer offsets)
    assert lib.moe_expert_ffn_fwd_gather(p, p, p, 1 << 20, 16, 2, 1024, 64, 0, 1, p, N, p,
                                         p, p, p, p, 1 << 20, N) == _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_ffn_bwd_gather(p, p, p, p, p, p, 1 << 20, 16, 2, 1024, 64, 0, 1,
                                         p, N, p, p, p, N, p, p, 1 << 20, N) == \
        _lib.MOE_ERR_UNSUPPORTED
    # rows to gather but no source or no map
    assert lib.moe_expert_ffn_fwd_gather(N, p, p, 100, 16, 2, 64, 64, 0, 1, p, N, p, p, p,
                                         p, p, 1 << 20, N) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn_fwd_gather(p, N, p, 100, 16, 2, 64, 64, 0, 1, p, N, p, p, p,
                                         p, p, 1 << 20, N) == _lib.MOE_ERR_INVALID_ARG
    # rows but an empty source
    assert lib.moe_expert_ffn_fwd_gather(p, p, p, 0, 16, 2, 64, 64, 0, 1, p, N, p, p, p,
                                         p, p, 1 << 20, N) == _lib.MOE_ERR_INVALID_ARG
    # routing-only permute still needs dest and src
    assert lib.moe_permute(p, N, 10, 64, 4, 2, 1, p, p, N, p, N, p, 1 << 20, N) == \
        _lib.MOE_ERR_INVALID_ARG


def test_no_gpu_means_error_not_fallback(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    # valid arguments reach the device check, which fails without a GPU
    assert lib.moe_init(0) in (_lib.MOE_ERR_HIP, _lib.MOE_ERR_UNSUPPORTED)


def test_empty_gate_backward_needs_no_token_pointers(lib):
    """T = 0: the gate backward accepts NULL token pointers (empty tensors)
    and gets past its argument checks to the device check (which fails here,
    with no GPU); it still needs Wg and dWg, which it writes."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    N = None
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    wsb = lib.moe_gate_bwd_workspace_bytes(0, 64, 4)
    wbuf = ctypes.create_string_buffer(max(wsb, 16) + 16)
    wp = ctypes.addressof(wbuf) + (-ctypes.addressof(wbuf)) % 16
    args = lambda Wg, dWg: (N, Wg, N, N, N, N, 0, 64, 4, 2, 1, 1, N, 0, dWg, wp, wsb, N)
    assert lib.moe_gate_topk_bwd(*args(p, p)) in (_lib.MOE_ERR_HIP, _lib.MOE_ERR_UNSUPPORTED)
    assert lib.moe_gate_topk_bwd(*args(N, p)) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_gate_topk_bwd(*args(p, N)) == _lib.MOE_ERR_INVALID_ARG


def _ctype_of(decl):
    """ctypes kind of one C parameter or return type in include/moe.h."""
    decl = decl.strip()
    if "*" in decl or decl.startswith("hipStream_t"):
        return "char_p" if decl.startswith("const char") and decl.count("*") == 1 and \
            not re.search(r"\w\s*$", decl.replace("*", "")) else "ptr"
    t = decl.split()[0] if decl.split()[0] != "const" else decl.split()[1]
    return {"int": "int", "moe_status": "int", "moe_dtype": "int", "moe_act": "int",
            "int32_t": "int", "size_t": "size", "void": "void"}[t]


def header_signatures():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    out = {}
    for m in re.finditer(r"([A-Za-z_][\w\s\*]*?)\b(moe_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        ret, name, args = m.group(1), m.group(2), m.group(3).strip()
        params = [] if args in ("", "void") else [a for a in args.split(",")]
        # a parameter is "type name": drop the name
        kinds = [_ctype_of(re.sub(r"\b\w+\s*$", "", p)) for p in params]
        rk = "char_p" if re.search(r"const\s+char\s*\*", ret) else _ctype_of(ret.split()[-1])
        out[name] = (rk, kinds)
    return out


def test_binding_types_match_the_header():
    """Every argument list in the ctypes table has the header's length and
    kinds (pointer / int / size_t), so a changed C signature cannot be
    called with stale marshalling."""
    kind = {ctypes.c_void_p: "ptr", ctypes.c_int: "int", ctypes.c_size_t: "size",
            ctypes.c_char_p: "char_p", None: "void"}
    decl = header_signatures()
    assert len(decl) >= 20
    for name, (rk, kinds) in decl.items():
        assert name in _lib.SIGNATURES, name
        res, args = _lib.SIGNATURES[name]
        got = [kind.get(a, "ptr") for a in args]     # POINTER(...) is a pointer
        assert got == kinds, (name, got, kinds)
        assert kind.get(res) == rk, (name, res, rk)


def test_benchmark_probes_reject_bad_arguments(lib):
    INV = _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_mfma_loop(0, 10, None, 0, None) == INV          # no blocks, no buffer
    assert lib.moe_mfma_loop(4, 0, 16, 16, None) == INV            # no iterations
    assert lib.moe_mfma_loop(4, 10, 16, 15, None) == INV           # buffer under blocks * 4
    assert lib.moe_mfma_loop_random(0, 16, None, 0, None) == INV   # no blocks, no buffer
    assert lib.moe_mfma_loop_random(4, 12, 16, 16, None) == INV    # not a multiple of 8
    assert lib.moe_mfma_loop_random(4, 0, 16, 16, None) == INV     # no iterations
    assert lib.moe_lds_probe(0, 4, 10, None, 0, 16, 16, None) == INV       # no kind
    assert lib.moe_lds_probe(8, 4, 10, None, 0, 16, 16, None) == INV       # multiplier only
    assert lib.moe_lds_probe(16, 4, 10, None, 0, 16, 16, None) == INV      # unknown bit
    assert lib.moe_lds_probe(1, 4, 10, None, 0, 16, 15, None) == INV       # buffer short
    assert lib.moe_lds_probe(3, 0, 10, None, 0, 16, 16, None) == INV       # no blocks
    assert lib.moe_lds_probe(4, 4, 10, None, 1 << 20, 16, 16, None) == INV  # loads, no source
    assert lib.moe_lds_probe(4, 4, 10, 256, 3 << 20, 16, 16, None) == INV   # not a power of two
    assert lib.moe_lds_probe(5, 4, 10, 256, 4096, 16, 16, None) == INV      # under 8 KB
    assert lib.moe_lds_probe(6, 4, 10, 8, 1 << 20, 16, 16, None) == INV     # unaligned source
    assert lib.moe_mfma_loop_random(4, 16, 16, 15, None) == INV    # buffer under blocks * 4
