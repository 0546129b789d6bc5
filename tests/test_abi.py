"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host before any
device work (these calls return before touching the GPU)."""
import ctypes

import pytest

import sparse_mixture_experts_renorm_amd as m
from sparse_mixture_experts_renorm_amd import _lib

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def L():
    return m.lib()


def test_exports_every_declared_symbol(L):
    names = m.declared_symbols()
    assert set(names) == {"moe_status_string", "moe_workspace_size", "moe_route",
                          "moe_route_logits", "moe_permute", "moe_expert_ffn", "moe_forward",
                          "moe_forward_profiled", "moe_router_stats_workspace_size",
                          "moe_router_stats", "moe_forward_ext_workspace_size", "moe_forward_ext",
                          "moe_permute_workspace_size", "moe_forward_no_alloc"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, s in enumerate(["MOE_OK", "MOE_INVALID_ARG", "MOE_UNSUPPORTED",
                              "MOE_WORKSPACE_TOO_SMALL", "MOE_HIP_ERROR"]):
        assert m.status_string(code) == s
    assert m.status_string(99) == "MOE_UNKNOWN_STATUS"


def test_workspace_holds_reachable_splits(L):
    """The down pass cuts its reduction over ffn into at most one part per
    12 steps of 64 (one to four parts), and the workspace holds exactly that
    many partial sums of y (3 bytes per element in a bf16 layer), besides h
    (two bf16 terms below width 1024) and a few small arrays."""
    T, d, E, k = 8192, 2048, 64, 8
    for ffn, parts in [(1408, 1), (2816, 3), (14336, 4), (512, 1), (768, 1), (1536, 2)]:
        n = L.moe_workspace_size(T, d, ffn, E, k, BF16)
        y = T * k * d * 3
        h = T * k * ffn * 2 * (2 if ffn < 1024 else 1)
        assert parts * y + h <= n < parts * y + h + (8 << 20), (ffn, n)


def test_workspace_size(L):
    T, d, ffn, E, k = 4096, 4096, 14336, 8, 2
    n = m.moe_workspace_size(T, d, ffn, E, k, BF16)
    assert n >= T * k * (ffn + d) * 2 + 4 * T * k * 4
    assert n % 256 == 0
    assert m.moe_workspace_size(T, d, ffn, E, k, F32) > n
    assert m.moe_workspace_size(T, d, ffn, E, 0, BF16) == 0      # k < 1
    assert m.moe_workspace_size(T, d, ffn, E, 9, BF16) == 0      # k > E
    assert m.moe_workspace_size(T, 4095, ffn, E, k, BF16) == 0   # d % 16
    assert m.moe_workspace_size(T, d, ffn, 300, k, BF16) == 0    # E > 256
    assert m.moe_workspace_size(0, d, ffn, E, k, BF16) > 0       # T = 0 is valid


def _route_logits(L, T, E, k, ptr=16):
    p = ctypes.c_void_p(ptr)
    return L.moe_route_logits(p, T, E, k, None, p, p, None)


def test_route_logits_validation(L):
    # the page's rules: 1 <= k <= E (axonml MoERouter::new, KempnerForge ModelConfig)
    assert _route_logits(L, 10, 8, 0) == INVALID
    assert _route_logits(L, 10, 8, 9) == INVALID
    assert _route_logits(L, 10, 0, 1) == INVALID
    assert _route_logits(L, -1, 8, 2) == INVALID
    assert _route_logits(L, 10, 300, 2) == UNSUPPORTED
    assert _route_logits(L, 10, 32, 17) == UNSUPPORTED
    assert _route_logits(L, 0, 8, 2, ptr=0) == OK          # T = 0: no launch
    assert L.moe_route_logits(None, 10, 8, 2, None, None, None, None) == INVALID
    assert _route_logits(L, 10, 8, 2, ptr=8) == INVALID    # misaligned


def test_forward_validation(L):
    p = ctypes.c_void_p(256)
    base = dict(T=16, d=64, ffn=64, E=4, k=2, dt=BF16, odt=F32)

    def call(ws_bytes=1 << 30, **kw):
        a = {**base, **kw}
        return L.moe_forward(p, p, p, p, p, None, a["T"], a["d"], a["ffn"], a["E"], a["k"],
                             a["dt"], p, a["odt"], None, None, None, p, ws_bytes, None)

    assert call(T=1 << 20, d=4096) == UNSUPPORTED          # T*d*2 bytes reach 2^32
    assert call(k=0) == INVALID
    assert call(k=5) == INVALID
    assert call(d=0) == INVALID
    assert call(ffn=-16) == INVALID
    assert call(d=72) == UNSUPPORTED
    assert call(ffn=40) == UNSUPPORTED
    assert call(dt=7) == UNSUPPORTED
    assert call(odt=7) == UNSUPPORTED
    assert call(ws_bytes=100) == WS_SMALL
    assert call(T=0) == OK
    assert L.moe_forward(p, p, p, p, p, None, 16, 64, 64, 4, 2, BF16, None, F32, None, None,
                         None, p, 1 << 30, None) == INVALID
    # workspace must be 256-byte aligned
    assert L.moe_forward(p, p, p, p, p, None, 16, 64, 64, 4, 2, BF16, p, F32, None, None, None,
                         ctypes.c_void_p(272), 1 << 30, None) == INVALID


def test_forward_no_alloc_validation(L):
    """The fixed-scratch forward checks its arguments as moe_forward does and
    refuses, on the host, a shape whose workspace exceeds its array."""
    p = ctypes.c_void_p(256)

    def call(T=16, d=64, ffn=64, E=4, k=2, dt=BF16, out=p):
        return L.moe_forward_no_alloc(p, p, p, p, p, None, T, d, ffn, E, k, dt, out, F32, None,
                                      None, None, None)

    assert call(k=0) == INVALID
    assert call(k=5) == INVALID
    assert call(d=72) == UNSUPPORTED
    assert call(out=None) == INVALID
    assert call(T=0) == OK
    limit = 64 << 20
    T = 1
    while L.moe_workspace_size(T + 1, 4096, 14336, 8, 2, BF16) <= limit:
        T += 1
    assert T == 430     # the limit include/moe.h states for the Mixtral widths
    assert call(T=T + 1, d=4096, ffn=14336, E=8, k=2) == WS_SMALL


def test_expert_ffn_and_permute_validation(L):
    p = ctypes.c_void_p(256)
    bad = ctypes.c_void_p(260)  # not 16-byte aligned
    assert L.moe_expert_ffn(p, p, p, p, p, p, 8, 64, 64, 4, 5, BF16, p, F32, p, 1 << 30, None) == INVALID
    assert L.moe_expert_ffn(p, p, p, p, p, p, 8, 64, 64, 4, 2, BF16, p, F32, p, 10, None) == WS_SMALL
    assert L.moe_permute(p, None, 8, 4, 5, p, p, p, p, None, None, 0, None) == INVALID
    assert L.moe_permute(p, None, 8, 257, 2, p, p, p, p, None, None, 0, None) == UNSUPPORTED
    assert L.moe_permute(None, None, 8, 4, 2, p, p, p, p, None, None, 0, None) == INVALID
    # the weights and their permuted copy come together or not at all
    assert L.moe_permute(p, p, 8, 4, 2, p, p, p, p, None, None, 0, None) == INVALID
    assert L.moe_permute(p, None, 8, 4, 2, p, p, p, p, p, None, 0, None) == INVALID
    assert L.moe_permute(p, p, 8, 4, 2, p, p, p, p, bad, None, 0, None) == INVALID
    # one workgroup up to 4096 assignments (no scratch), then per-block histograms
    assert L.moe_permute_workspace_size(2048, 8, 2) == 0
    assert L.moe_permute_workspace_size(8192, 64, 8) == 64 * 64 * 4
    assert L.moe_permute_workspace_size(1 << 20, 8, 2) == 256 * 8 * 4
    assert L.moe_permute(p, None, 8192, 64, 8, p, p, p, p, None, None, 0, None) == INVALID
    assert L.moe_permute(p, None, 8192, 64, 8, p, p, p, p, None, p, 64 * 64 * 4 - 1, None) == WS_SMALL
    assert L.moe_route(p, p, None, 8, 40, 4, 2, BF16, None, None, p, p, None) == UNSUPPORTED
    ev = (ctypes.c_void_p * 6)(*([16] * 5 + [0]))
    assert L.moe_forward_profiled(p, p, p, p, p, None, 16, 64, 64, 4, 2, BF16, p, F32, None, None,
                                  None, p, 1 << 30, None, ev) == INVALID
    assert L.moe_forward_profiled(p, p, p, p, p, None, 16, 64, 64, 4, 2, BF16, p, F32, None, None,
                                  None, p, 1 << 30, None, None) == INVALID


def test_assignment_limit(L):
    """T*k stays below 2^31 - 2^20: the permutation's per-block assignment
    ranges run up to T*k + 2^18 in int32. At the limit every routing entry
    point rejects the call; just below it the checks pass (the permutation
    then stops at its workspace check, before any device work)."""
    p = ctypes.c_void_p(256)
    lim = (1 << 31) - (1 << 20)
    k = 2
    T_over, T_under = lim // k, lim // k - 1
    assert L.moe_permute(p, None, T_over, 8, k, p, p, p, p, None, p, 0, None) == UNSUPPORTED
    assert L.moe_permute(p, None, T_under, 8, k, p, p, p, p, None, p, 0, None) == WS_SMALL
    assert L.moe_permute_workspace_size(T_over, 8, k) == 0
    assert L.moe_permute_workspace_size(T_under, 8, k) == 256 * 8 * 4
    assert L.moe_route_logits(p, T_over, 8, k, None, p, p, None) == UNSUPPORTED
    assert L.moe_route(p, p, None, T_over, 64, 8, k, BF16, None, None, p, p, None) == UNSUPPORTED


def test_router_stats_validation(L):
    p = ctypes.c_void_p(256)
    n = L.moe_router_stats_workspace_size(1000, 8)
    assert n == 16 * 8 * 4          # 16 blocks of 64 rows, one float per expert each
    assert L.moe_router_stats_workspace_size(-1, 8) == 0
    assert L.moe_router_stats_workspace_size(10, 257) == 0
    assert L.moe_router_stats(p, p, -1, 8, p, None, p, p, n, None) == INVALID
    assert L.moe_router_stats(p, p, 10, 0, p, None, p, p, n, None) == INVALID
    assert L.moe_router_stats(p, p, 10, 257, p, None, p, p, n, None) == UNSUPPORTED
    assert L.moe_router_stats(None, p, 10, 8, p, None, p, p, n, None) == INVALID
    assert L.moe_router_stats(p, p, 10, 8, None, None, p, p, n, None) == INVALID
    assert L.moe_router_stats(p, p, 10, 8, p, ctypes.c_void_p(260), p, p, n, None) == INVALID
    assert L.moe_router_stats(p, p, 1000, 8, p, None, p, p, n - 4, None) == WS_SMALL


def test_options_struct_layout(tmp_path):
    """The ctypes mirror of moe_options has the C struct's size and offsets
    (compiled from include/moe.h with the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"moe.h\"\n"
        "int main(void) { printf(\"%zu\", sizeof(moe_options));\n"
        + "".join(f'  printf(" %zu", offsetof(moe_options, {f}));\n'
                  for f, _ in _lib.MoeOptions._fields_)
        + "  return 0; }\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I", _lib.os.path.dirname(_lib.HEADER),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                           text=True).stdout.split()]
    want = [ctypes.sizeof(_lib.MoeOptions)] + [getattr(_lib.MoeOptions, f).offset
                                               for f, _ in _lib.MoeOptions._fields_]
    assert got == want


def test_forward_ext_validation(L):
    p = ctypes.c_void_p(256)
    o = _lib.MoeOptions()
    def call(opt=ctypes.byref(o), T=16, ws_bytes=1 << 30):
        return L.moe_forward_ext(p, p, p, p, p, None, T, 64, 64, 4, 2, BF16, opt, p, F32, None,
                                 None, None, None, p, ws_bytes, None)
    assert L.moe_forward_ext_workspace_size(16, 64, 64, 4, 2, BF16, ctypes.byref(o)) == \
        L.moe_workspace_size(16, 64, 64, 4, 2, BF16)
    assert call(opt=None) == INVALID
    o.capacity_factor = -0.5
    assert call() == INVALID
    o.capacity_factor = float("nan")
    assert call() == INVALID
    o.capacity_factor = 1.25
    o.norm_weight = 256
    o.norm_eps = 0.0
    assert call() == INVALID
    o.norm_eps = 1e-5
    o.n_shared = 17
    o.shared_ffn = 64
    o.shared_gate = o.shared_up = o.shared_down = 256
    assert call() == UNSUPPORTED
    o.n_shared = 2
    o.shared_ffn = 40
    assert call() == UNSUPPORTED
    o.shared_ffn = 64
    o.shared_down = None
    assert call() == INVALID
    o.shared_down = 256
    # one shared expert's weights are addressed with 32-bit byte offsets, as
    # the routed experts' are: shared_ffn * d * 2 bytes must stay below 2^32
    o.n_shared = 1
    o.shared_ffn = (1 << 32) // (4096 * 2)
    def call_d(T=1, ws_bytes=0):
        return L.moe_forward_ext(p, p, p, p, p, None, T, 4096, 64, 4, 2, BF16, ctypes.byref(o), p,
                                 F32, None, None, None, None, p, ws_bytes, None)
    assert call_d() == UNSUPPORTED
    assert L.moe_forward_ext_workspace_size(1, 4096, 64, 4, 2, BF16, ctypes.byref(o)) == 0
    o.shared_ffn -= 16
    assert call_d() == WS_SMALL
    o.n_shared = 2
    o.shared_ffn = 64
    need = L.moe_forward_ext_workspace_size(16, 64, 64, 4, 2, BF16, ctypes.byref(o))
    assert need > L.moe_workspace_size(16, 64, 64, 4, 2, BF16)
    assert call(ws_bytes=need - 1) == WS_SMALL
    assert call(T=0) == OK   # nothing to do


def test_binding_requires_library(monkeypatch, tmp_path):
    """No fallback: without the built library every binding call raises."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()
