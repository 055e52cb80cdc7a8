"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/w4a4.h, reports blob sizes, and rejects bad arguments on
the host before anything is enqueued."""
import ctypes
import os
import re
import sys

import pytest

import w4a4_gemm_lora_amd as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(W.lib_path()),
                                reason="libw4a4.so not built (run __graft_entry__.build())")


def _declared(header="w4a4.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a4_[a-z0-9_]+)\s*\(", src)))


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["w4a4.h", "w4a4_peaks.h"]


def test_exports_every_declared_symbol():
    lib = W.load_library()
    names = _declared()
    assert set(names) == set(W.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n
    assert W.w4a4_status_string(0) == "W4A4_OK"
    assert "SHAPE" in W.w4a4_status_string(2)


def test_peaks_library_exports_every_declared_symbol():
    lib = W.load_peaks_library()
    names = _declared("w4a4_peaks.h")
    assert set(names) == set(W.PEAKS_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n
    # host-only queries and argument checks (nothing is launched)
    assert lib.w4a4_peak_i8_mfma_ops(10) == 512 * 4 * 8 * 10 * 2 * 16 * 16 * 64
    assert lib.w4a4_peak_i8_mfma_out_ints() == 512 * 256
    assert lib.w4a4_peak_hbm_read_out_ints() > 0
    assert lib.w4a4_peak_i8_mfma(0, ctypes.c_void_p(1 << 20), None) == 4
    assert lib.w4a4_peak_i8_mfma(1, None, None) == 4
    assert lib.w4a4_peak_hbm_read(ctypes.c_void_p(1 << 20), 24, ctypes.c_void_p(1 << 20), None) == 4
    assert lib.w4a4_peak_hbm_read(ctypes.c_void_p((1 << 20) + 8), 32, ctypes.c_void_p(1 << 20), None) == 4
    assert lib.w4a4_peak_roles_out_ints() == 256 * 512
    assert lib.w4a4_peak_roles_ops(1, 10) == 256 * 4 * 8 * 10 * 2 * 16 * 16 * 64
    assert lib.w4a4_peak_roles_ops(2, 10) == 256 * 4 * 32 * 10 * 64
    assert lib.w4a4_peak_roles(8, 0, 1, 1, ctypes.c_void_p(1 << 20), None) == 4   # roles are 0..7
    assert lib.w4a4_peak_roles(0, -1, 1, 1, ctypes.c_void_p(1 << 20), None) == 4
    assert lib.w4a4_peak_roles(1, 2, 1, 1, None, None) == 4


def test_no_unresolved_library_symbols():
    """Every kernel launch stub the library references is defined in it (a
    stub the compiler fails to emit only shows up as an unresolved symbol)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", W.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    bad = [l for l in out.splitlines() if "w4a4" in l]
    assert not bad, bad


def test_layout_sizes():
    N, K, R = 3072, 1024, 32
    tot, offs = W.w4a4_weight_layout(N, K, R)
    assert offs[0] == 0 and all(o % 256 == 0 for o in offs)
    assert offs[1] >= K * R * 2
    assert offs[2] - offs[1] >= N * K // 2
    assert offs[3] - offs[2] >= N * (K // 64) * 2
    assert offs[4] - offs[3] >= N * R * 2
    assert tot >= offs[5] + 4 * N
    tot, offs, ks = W.w4a4_act_layout(700, K, R, with_splits=True)
    Mp = 704
    assert offs[1] - offs[0] >= Mp * K // 2
    assert offs[2] - offs[1] >= Mp * (K // 64) * 2
    assert ks == 1   # 8 k-pairs: too short to split
    assert tot >= offs[2] + ks * Mp * R * 4


def test_lora_split_rule():
    """The header's rule: M <= 16: clamp((K/128)/4, 1, 8); M > 16: the
    smallest power of two S with ceil(M/16)*S >= 256, capped at 4 and KP/8."""
    def rule(M, K):
        kp = K // 128
        if M <= 16:
            return min(max(1, kp // 4), 8)
        mt = -(-M // 16)
        s = 1
        while s < 4 and mt * s < 256 and 16 * s <= kp:
            s *= 2
        return s
    assert rule(700, 1024) == 1 and rule(700, 3072) == 2 and rule(8192, 4096) == 1 and rule(17, 256) == 1
    assert rule(130, 2048) == 2 and rule(40, 4096) == 4 and rule(100, 8192) == 4
    for M in (1, 4, 16, 17, 100, 700, 2048, 4095, 4096, 8192):
        for K in (128, 256, 512, 1024, 2048, 3072, 4096, 8192):
            _, _, ks = W.w4a4_act_layout(M, K, 32, with_splits=True)
            assert ks == rule(M, K), (M, K, ks)


@pytest.mark.parametrize("N,K,R", [(16, 64, 16), (16, 192, 16), (8, 128, 16), (24, 128, 16),
                                   (16, 128, 8), (16, 128, 80), (16, 128, -16), (0, 128, 16)])
def test_bad_shapes_rejected(N, K, R):
    with pytest.raises(W.W4A4Error) as e:
        W.w4a4_weight_layout(N, K, R)
    assert e.value.status == 2
    assert W.load_library().w4a4_query_variant(1, N, K, R) == -2


def _lib():
    return W.load_library()


FAKE = 1 << 20  # a non-NULL, 256-byte aligned host address; never dereferenced


def test_validation_errors_before_any_launch():
    lib = _lib()
    # linear: NULL y, misaligned y, ldy < N, bad ldy, bad shape
    assert lib.w4a4_linear(4, 64, 128, 16, FAKE, FAKE, None, 64, None) == 1
    assert lib.w4a4_linear(4, 64, 128, 16, FAKE, FAKE, FAKE + 2, 64, None) == 3
    assert lib.w4a4_linear(4, 64, 128, 16, FAKE, FAKE, FAKE, 32, None) == 2
    assert lib.w4a4_linear(4, 64, 128, 16, FAKE, FAKE, FAKE, 68, None) == 3
    assert lib.w4a4_linear(4, 64, 100, 16, FAKE, FAKE, FAKE, 64, None) == 2
    assert lib.w4a4_linear(4, 64, 128, 16, None, FAKE, FAKE, 64, None) == 1
    assert lib.w4a4_linear(4, 64, 128, 16, FAKE + 16, FAKE, FAKE * 4, 64, None) == 3
    # y overlapping a blob
    assert lib.w4a4_linear(4, 64, 128, 16, FAKE, FAKE * 4, FAKE, 64, None) == 4
    # M == 0 is a no-op success; negative M is a shape error
    assert lib.w4a4_linear(0, 64, 128, 16, None, None, None, 64, None) == 0
    assert lib.w4a4_linear(-1, 64, 128, 16, FAKE, FAKE, FAKE, 64, None) == 2
    # gated linear: N not whole (gate, up) tile pairs, ldy below N/2, NULL y,
    # misaligned y, y overlapping a blob, M == 0 no-op, rank above the maximum,
    # gate rank outside [0, R]
    assert lib.w4a4_linear_glu(4, 48, 128, 16, 8, FAKE, FAKE, FAKE, 24, None) == 2
    assert lib.w4a4_linear_glu(4, 64, 128, 16, 8, FAKE, FAKE, FAKE, 16, None) == 2
    assert lib.w4a4_linear_glu(4, 64, 128, 16, 8, FAKE, FAKE, None, 32, None) == 1
    assert lib.w4a4_linear_glu(4, 64, 128, 16, 8, FAKE, FAKE, FAKE + 2, 32, None) == 3
    assert lib.w4a4_linear_glu(4, 64, 128, 16, 8, FAKE, FAKE, FAKE, 36, None) == 3
    assert lib.w4a4_linear_glu(4, 64, 128, 16, 8, FAKE, FAKE * 4, FAKE, 32, None) == 4
    assert lib.w4a4_linear_glu(0, 64, 128, 16, 8, None, None, None, 32, None) == 0
    assert lib.w4a4_linear_glu(4, 64, 128, 80, 16, FAKE, FAKE, FAKE, 32, None) == 2
    assert lib.w4a4_linear_glu(4, 64, 128, 16, 17, FAKE, FAKE, FAKE, 32, None) == 2
    assert lib.w4a4_linear_glu(4, 64, 128, 16, -1, FAKE, FAKE, FAKE, 32, None) == 2
    # quantize: ldx < K, misaligned x, NULL act, missing weight blob with R > 0
    assert lib.w4a4_quantize_act(4, 128, 16, FAKE, 64, FAKE, FAKE, None) == 2
    assert lib.w4a4_quantize_act(4, 128, 16, FAKE + 8, 128, FAKE, FAKE, None) == 3
    assert lib.w4a4_quantize_act(4, 128, 16, FAKE, 130, FAKE, FAKE, None) == 3
    assert lib.w4a4_quantize_act(4, 128, 16, FAKE, 128, FAKE, None, None) == 1
    assert lib.w4a4_quantize_act(4, 128, 16, FAKE, 128, None, FAKE, None) == 1
    assert lib.w4a4_quantize_act(0, 128, 16, None, 128, None, None, None) == 0
    # layer graphs: argument errors return before any HIP call
    import ctypes
    h = ctypes.c_void_p()
    gc = lib.w4a4_layer_graph_create
    assert gc(4, 64, 128, 16, FAKE, 128, None, 0.0, FAKE, FAKE, FAKE, 64, None) == 1
    assert gc(0, 64, 128, 16, FAKE, 128, None, 0.0, FAKE, FAKE, FAKE, 64, ctypes.byref(h)) == 2
    assert h.value is None
    assert gc(4, 60, 128, 16, FAKE, 128, None, 0.0, FAKE, FAKE, FAKE, 64, ctypes.byref(h)) == 2
    assert gc(4, 64, 100, 16, FAKE, 128, None, 0.0, FAKE, FAKE, FAKE, 64, ctypes.byref(h)) == 2
    assert lib.w4a4_graph_launch(None, None) == 1
    assert lib.w4a4_graph_destroy(None) == 0
    assert lib.w4a4_graph_begin(None) == 1
    assert lib.w4a4_graph_end(None, ctypes.byref(h)) == 1
    # fused RMSNorm quantizer: NULL gamma, eps <= 0 / NaN / inf, misaligned gamma,
    # then the plain quantizer's checks
    q = lib.w4a4_quantize_act_rmsnorm
    assert q(4, 128, 16, FAKE, 128, None, 1e-6, FAKE, FAKE, None) == 1
    assert q(4, 128, 16, FAKE, 128, FAKE, 0.0, FAKE, FAKE, None) == 4
    assert q(4, 128, 16, FAKE, 128, FAKE, -1e-6, FAKE, FAKE, None) == 4
    assert q(4, 128, 16, FAKE, 128, FAKE, float("nan"), FAKE, FAKE, None) == 4
    assert q(4, 128, 16, FAKE, 128, FAKE, float("inf"), FAKE, FAKE, None) == 4
    assert q(4, 128, 16, FAKE, 128, FAKE + 8, 1e-6, FAKE, FAKE, None) == 3
    assert q(4, 128, 16, FAKE, 64, FAKE, 1e-6, FAKE, FAKE, None) == 2
    assert q(4, 128, 16, FAKE, 128, FAKE, 1e-6, FAKE, None, None) == 1
    # pack: both or neither code source, half a checkpoint pair, missing LoRA
    assert lib.w4a4_pack_weights(16, 128, 16, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None) == 4
    assert lib.w4a4_pack_weights(16, 128, 16, None, None, None, FAKE, FAKE, None, None, FAKE, None) == 4
    assert lib.w4a4_pack_weights(16, 128, 16, None, FAKE, None, FAKE, FAKE, None, None, FAKE, None) == 1
    assert lib.w4a4_pack_weights(16, 128, 16, FAKE, None, None, None, FAKE, None, None, FAKE, None) == 1
    assert lib.w4a4_pack_weights(16, 128, 16, FAKE, None, None, FAKE, FAKE, None, None, FAKE + 16, None) == 3
    assert lib.w4a4_pack_weights(16, 128, 16, FAKE, None, None, FAKE, FAKE, None, None, None, None) == 1
    # debug psums: window not on 16 boundaries / outside
    assert lib.w4a4_debug_group_psums(20, 64, 128, 16, FAKE, FAKE, 8, 16, 0, 16, FAKE, None) == 2
    assert lib.w4a4_debug_group_psums(20, 64, 128, 16, FAKE, FAKE, 16, 32, 0, 16, FAKE, None) == 2
    assert lib.w4a4_debug_group_psums(20, 64, 128, 16, FAKE, FAKE, 0, 16, 64, 16, FAKE, None) == 2
    assert lib.w4a4_debug_group_psums(20, 64, 128, 16, FAKE, FAKE, 0, 16, 0, 16, None, None) == 1
    # the gated twin: also N % 32 (whole (gate, up) tile pairs)
    assert lib.w4a4_debug_group_psums_glu(20, 48, 128, 16, FAKE, FAKE, 0, 16, 0, 16, FAKE, None) == 2
    assert lib.w4a4_debug_group_psums_glu(20, 64, 128, 16, FAKE, FAKE, 8, 16, 0, 16, FAKE, None) == 2
    # the window must not overlap the blobs
    _, _ = W.w4a4_weight_layout(64, 128, 16)
    assert lib.w4a4_debug_group_psums(20, 64, 128, 16, FAKE, FAKE + 1024 * 1024, 0, 16, 0, 16, FAKE + 256,
                                      None) == 4


def test_glu_quant_workspace_and_validation():
    """The quantized gated output: workspace sizes, and every argument error
    returned on the host (nothing launched)."""
    lib = _lib()
    ws = W.w4a4_glu_quant_workspace
    # the larger of the per-group LoRA-down partials, 4 * (N/128) * Mp * R_down
    # bytes, and h, 2 * M * N/2 bytes (rounded up to 256)
    assert ws(700, 6144, 32) == 4 * 48 * 704 * 32
    assert ws(17, 256, 16) == 2 * 17 * 128   # h (4352 B, a multiple of 256) over 4096 B of shares
    assert ws(700, 6144, 0) == 2 * 700 * 3072
    assert ws(1, 6144, 32) == 4 * 48 * 16 * 32
    assert ws(5, 256, 0) == 2 * 5 * 128
    assert ws(0, 6144, 32) == 0
    n = ctypes.c_size_t()
    assert lib.w4a4_glu_quant_workspace(4, 6144, 32, None) == 1
    assert lib.w4a4_glu_quant_workspace(4, 6016, 32, ctypes.byref(n)) == 2   # N/2 not a multiple of 128
    assert lib.w4a4_glu_quant_workspace(4, 6144, 24, ctypes.byref(n)) == 2
    assert lib.w4a4_glu_quant_workspace(-1, 6144, 32, ctypes.byref(n)) == 2
    big = 1 << 30   # far from FAKE: no overlap between the fake buffers
    q = lib.w4a4_linear_glu_quant
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("M", 40), ("N", 256), ("K", 128), ("R", 32), ("rg", 16), ("act", FAKE), ("wb", 2 * big),
        ("Rd", 16), ("dwb", 3 * big), ("out", 4 * big), ("ws", 5 * big), ("s", None))]
    assert q(*args(N=192)) == 2            # N/2 not a multiple of 128
    assert q(*args(N=240)) == 2            # not whole (gate, up) pairs
    assert q(*args(rg=48)) == 2            # gate rank above R
    assert q(*args(Rd=8)) == 2             # down rank not a multiple of 16
    assert q(*args(Rd=80)) == 2
    assert q(*args(K=100)) == 2
    assert q(*args(M=-1)) == 2
    assert q(*args(M=0, act=None, wb=None, dwb=None, out=None, ws=None)) == 0
    assert q(*args(out=None)) == 1
    assert q(*args(dwb=None)) == 1         # needed for R_down > 0
    assert q(*args(ws=None)) == 1
    assert q(*args(act=None)) == 1
    assert q(*args(out=4 * big + 16)) == 3
    assert q(*args(ws=5 * big + 128)) == 3
    assert q(*args(dwb=3 * big + 8)) == 3
    # overlaps: the output blob with the input blob, the workspace with the output
    assert q(*args(out=FAKE + 256)) == 4
    assert q(*args(ws=4 * big + 256)) == 4
    assert q(*args(ws=3 * big)) == 4       # the workspace over the down layer's L_down


def test_glu_quant_noalloc_validation():
    """The allocation-free variant: the size limit of its array and every
    argument error are returned on the host before any device call."""
    lib = _lib()
    assert W.NOALLOC_SCRATCH_BYTES == 32 << 20
    big = 1 << 30
    q = lib.w4a4_linear_glu_quant_noalloc
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("M", 40), ("N", 256), ("K", 128), ("R", 32), ("rg", 16), ("act", FAKE), ("wb", 2 * big),
        ("Rd", 16), ("dwb", 3 * big), ("out", 4 * big), ("s", None))]
    assert q(*args(N=192)) == 2
    assert q(*args(Rd=8)) == 2
    assert q(*args(out=None)) == 1
    assert q(*args(dwb=None)) == 1
    assert q(*args(act=FAKE + 16)) == 3
    assert q(*args(out=FAKE + 256)) == 4
    assert q(*args(M=0, act=None, wb=None, dwb=None, out=None)) == 0
    # a workspace need above the array (M=8192, 3072 columns of h, rank 32:
    # 48 MiB of LoRA-down shares) is a shape error
    assert W.w4a4_glu_quant_workspace(8192, 6144, 32) > W.NOALLOC_SCRATCH_BYTES
    assert q(*args(M=8192, N=6144, K=1024, wb=2 * big, dwb=3 * big, out=4 * big)) == 2
    assert W.w4a4_glu_quant_workspace(4096, 6144, 32) <= W.NOALLOC_SCRATCH_BYTES


def test_query_variant_is_host_only():
    for M in (1, 4, 16, 700, 8192):
        assert W.w4a4_query_variant(M, 4096, 4096, 32) == (1 if M <= 16 else 2)


def test_library_shares_torch_hip_runtime():
    """Loading the library before any torch import still leaves one HIP
    runtime in the process (torch's): a second copy would find no device
    once torch's copy has opened the GPU."""
    import subprocess
    code = ("import w4a4_gemm_lora_amd as W; W.load_library(); "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr[-2000:]
    import ast
    libs = ast.literal_eval(out.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs
