"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/moe.h declares, sizes its buffers consistently, and rejects
bad arguments before touching the device.  Every call here returns before
any HIP runtime call."""
import ctypes
import subprocess

import pytest

from sparse_moe_layer_rmsnorm_amd import binding as B

REPLICA = dict(d=1024, l=256, E=256, k=6, f=512, f_s=2048)


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_function(L):
    names = B.header_functions()
    assert {"moe_init", "moe_route", "moe_forward", "qb_update"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(L, n)


def test_status_strings(L):
    for code, name in enumerate(["MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_SHAPE", "MOE_ERR_DTYPE",
                                 "MOE_ERR_WORKSPACE", "MOE_ERR_STATE", "MOE_ERR_HIP"]):
        assert L.moe_status_string(code).decode() == name
    assert L.moe_kernel_name(0).decode() == "rmsnorm"
    assert [L.moe_kernel_name(i).decode() for i in range(B.MOE_NUM_KERNELS)] == B.KERNELS


def test_sizes_and_layouts():
    cfg = B.make_config(**REPLICA, max_tokens=8192)
    st = B.moe_state_layout_of(cfg)
    assert B.moe_state_bytes(cfg) == st.total
    assert st.bias == 0 and st.count >= 4 * 256 and st.q > st.count and st.hist > st.q
    assert st.total >= st.hist + st.hist_slices * 256 * 256 * 4
    assert st.load >= st.hist + st.hist_slices * 256 * 256 * 4 and st.total >= st.load + 256 * 4
    for T in (0, 1, 1000, 8192):
        ws = B.moe_workspace_layout(cfg, T)
        assert B.moe_workspace_bytes(cfg, T) == ws.total
        offs = [getattr(ws, n) for n, _ in B.moe_ws_layout._fields_]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    ws = B.moe_workspace_layout(cfg, 8192)
    assert ws.H - ws.G >= 8192 * 2048 * 2 and ws.Y - ws.H >= 8192 * 6 * 512 * 2
    assert B.moe_workspace_bytes(cfg, 8193) == 0          # above max_tokens
    assert B.moe_workspace_bytes(cfg, -1) == 0


@pytest.mark.parametrize("field,value,status", [
    ("d", 1000, B.MOE_ERR_SHAPE), ("l", 0, B.MOE_ERR_SHAPE), ("f", 96, B.MOE_ERR_SHAPE),
    ("f_s", 100, B.MOE_ERR_SHAPE), ("E", 0, B.MOE_ERR_SHAPE), ("E", 1025, B.MOE_ERR_SHAPE),
    ("k", 0, B.MOE_ERR_SHAPE), ("k", 33, B.MOE_ERR_SHAPE), ("k", 300, B.MOE_ERR_SHAPE),
    ("qb_bins", 1, B.MOE_ERR_SHAPE), ("qb_bins", 257, B.MOE_ERR_SHAPE), ("dtype", 7, B.MOE_ERR_DTYPE),
    ("qb_mode", 5, B.MOE_ERR_INVALID_ARG), ("rms_eps", 0.0, B.MOE_ERR_INVALID_ARG),
    ("max_tokens", 0, B.MOE_ERR_SHAPE), ("max_tokens", 2 ** 30, B.MOE_ERR_SHAPE),
    ("balancer", 2, B.MOE_ERR_INVALID_ARG), ("balancer", -1, B.MOE_ERR_INVALID_ARG),
    ("n_shared", -1, B.MOE_ERR_SHAPE), ("n_shared", 1024, B.MOE_ERR_SHAPE),
    ("qb_lo", 1.0, B.MOE_ERR_INVALID_ARG), ("qb_lo", 2.0, B.MOE_ERR_INVALID_ARG),
    ("qb_hi", float("inf"), B.MOE_ERR_INVALID_ARG), ("qb_lo", float("nan"), B.MOE_ERR_INVALID_ARG),
    ("qb_hi", 1e-42, B.MOE_ERR_INVALID_ARG),
])
def test_bad_config_rejected_before_any_device_call(L, field, value, status):
    cfg = B.make_config(**REPLICA, max_tokens=64)
    setattr(cfg, field, value)
    assert B.moe_state_bytes(cfg) == 0
    ctx = ctypes.c_void_p()
    w = B.moe_weights(*([1] * 11))                       # never dereferenced: the config fails first
    assert L.moe_init(ctypes.byref(cfg), ctypes.byref(w), 256, None, ctypes.byref(ctx)) == status
    assert ctx.value is None
    assert L.moe_last_error()


@pytest.mark.parametrize("gamma,ok", [(1e-2, True), (1e-3, True), (0.0, False), (-1e-2, False),
                                      (float("inf"), False), (float("nan"), False)])
def test_sign_gamma_checked_only_for_the_sign_balancer(gamma, ok):
    sign = B.make_config(**REPLICA, max_tokens=64, balancer="sign", sign_gamma=gamma)
    assert (B.moe_state_bytes(sign) > 0) == ok
    qb = B.make_config(**REPLICA, max_tokens=64, balancer="qb", sign_gamma=gamma)
    assert B.moe_state_bytes(qb) > 0                      # ignored by the QB rule


@pytest.mark.parametrize("over,status", [
    (dict(), None), (dict(dtype="f32"), B.MOE_ERR_DTYPE), (dict(l=64), B.MOE_ERR_SHAPE),
    (dict(f=192), B.MOE_ERR_SHAPE), (dict(f=640), B.MOE_ERR_SHAPE), (dict(l=1024), B.MOE_ERR_SHAPE),
])
@pytest.mark.parametrize("fmt,bpe", [("mxfp8", 1.0), ("mxfp4", 0.5)])
def test_mxfp8_experts_config(L, over, status, fmt, bpe):
    """Block-scaled experts (MXFP8; MXFP4 weights): bf16 mode only, l and f
    multiples of 128 up to 512; the state then holds the quantised expert
    weights (1 or 1/2 byte per element) and their scales."""
    args = dict(REPLICA)
    over = dict(over)
    dtype = over.pop("dtype", "bf16")
    args.update(over)
    cfg = B.make_config(**args, dtype=dtype, max_tokens=64, experts=fmt)
    if status is None:
        st = B.moe_state_layout_of(cfg)
        w = args["E"] * args["f"] * args["l"]
        need = int(3 * w * bpe) + 3 * w // 32
        assert need <= st.total - st.mx <= need + 256
        ref = B.make_config(**args, dtype=dtype, max_tokens=64)
        assert B.moe_state_bytes(cfg) >= B.moe_state_bytes(ref) + int(3 * w * bpe)
    else:
        assert B.moe_state_bytes(cfg) == 0
        ctx = ctypes.c_void_p()
        w_ = B.moe_weights(*([1] * 11))
        assert L.moe_init(ctypes.byref(cfg), ctypes.byref(w_), 256, None, ctypes.byref(ctx)) == status


def test_keep_preact_config_and_workspaces(L):
    """keep_preact is 0 or 1 and needs bf16 experts; it adds exactly the four
    pre-activation buffers to the forward workspace and takes the backward's
    own copies of them away."""
    T = 1000
    es = 2
    base = B.make_config(**REPLICA, max_tokens=T)
    keep = B.make_config(**REPLICA, max_tokens=T, keep_preact=True)
    Lb, Lk = B.moe_workspace_layout(base, T), B.moe_workspace_layout(keep, T)
    fs, f, k = REPLICA["f_s"], REPLICA["f"], REPLICA["k"]
    assert Lb.P == Lb.Q == Lb.A == Lb.U == Lb.total
    assert Lk.Q - Lk.P >= T * fs * es and Lk.U - Lk.A >= T * k * f * es and Lk.total - Lk.U >= T * k * f * es
    grow = B.moe_workspace_bytes(keep, T) - B.moe_workspace_bytes(base, T)
    need = 2 * (T * fs + T * k * f) * es
    assert need <= grow <= need + 4 * 256
    shrink = B.moe_backward_workspace_bytes(base, T) - B.moe_backward_workspace_bytes(keep, T)
    assert need <= shrink <= need + 4 * 256
    for bad in (dict(keep_preact=2), dict(keep_preact=-1)):
        cfg = B.make_config(**REPLICA, max_tokens=T)
        cfg.keep_preact = bad["keep_preact"]
        assert B.moe_state_bytes(cfg) == 0
    assert B.moe_state_bytes(B.make_config(**REPLICA, max_tokens=T, keep_preact=True, experts="mxfp8")) == 0


def test_shared_experts_and_histogram_range_fields():
    """n_shared shared experts of hidden f_s are one GLU of hidden
    n_shared*f_s (the workspace's shared hidden grows with it; n_shared = 0 or
    f_s = 0 means no shared path); the QB score range is any finite
    qb_lo < qb_hi whose bins per unit of score fit fp32."""
    T = 1000
    ws1 = B.moe_workspace_layout(B.make_config(**REPLICA, max_tokens=T), T)
    ws3 = B.moe_workspace_layout(B.make_config(**REPLICA, max_tokens=T, n_shared=3), T)
    ws0 = B.moe_workspace_layout(B.make_config(**REPLICA, max_tokens=T, n_shared=0), T)
    assert ws1.z - ws1.G >= T * 2048 * 2 and ws3.z - ws3.G >= T * 3 * 2048 * 2 and ws0.z - ws0.G == 0
    args = dict(REPLICA, f_s=0)
    assert B.moe_workspace_layout(B.make_config(**args, max_tokens=T, n_shared=4), T).z == \
        B.moe_workspace_layout(B.make_config(**args, max_tokens=T, n_shared=0), T).z
    for lo, hi in ((0.0, 1.0), (0.25, 0.75), (-3.0, 3.0), (0.5, 0.5000001)):
        assert B.moe_state_bytes(B.make_config(**REPLICA, max_tokens=T, qb_lo=lo, qb_hi=hi)) > 0
    assert B.moe_state_bytes(B.make_config(**REPLICA, max_tokens=T, qb_lo=0.5, qb_hi=0.5)) == 0


def test_null_arguments_rejected(L):
    cfg = B.make_config(**REPLICA, max_tokens=64)
    ctx = ctypes.c_void_p()
    w = B.moe_weights(*([1] * 11))
    assert L.moe_init(None, ctypes.byref(w), 256, None, ctypes.byref(ctx)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_init(ctypes.byref(cfg), None, 256, None, ctypes.byref(ctx)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_init(ctypes.byref(cfg), ctypes.byref(w), None, None, ctypes.byref(ctx)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_init(ctypes.byref(cfg), ctypes.byref(w), 128, None, ctypes.byref(ctx)) == B.MOE_ERR_INVALID_ARG
    w2 = B.moe_weights(*([1] * 11))
    w2.W_g = None
    assert L.moe_init(ctypes.byref(cfg), ctypes.byref(w2), 256, None, ctypes.byref(ctx)) == B.MOE_ERR_INVALID_ARG
    w3 = B.moe_weights(*([1] * 11))
    w3.W_sd = None                                       # shared weights are needed when f_s > 0
    assert L.moe_init(ctypes.byref(cfg), ctypes.byref(w3), 256, None, ctypes.byref(ctx)) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward(None, 1, 8, 1, None, 256, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, 1, None, 8, None, 256, 1 << 30, None) == B.MOE_ERR_INVALID_ARG
    assert L.qb_update(None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_get_bias(None, 1, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_set_bias(None, 1, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_set_qb_mode(None, 0) == B.MOE_ERR_INVALID_ARG
    assert L.moe_profile_begin(None, 4, 0) == B.MOE_ERR_INVALID_ARG
    L.moe_destroy(None)


def test_python_wrappers_raise_with_message():
    cfg = B.make_config(**REPLICA, max_tokens=64)
    cfg.k = 0
    with pytest.raises(B.MoeError, match="MOE_ERR_SHAPE"):
        B.moe_state_layout_of(cfg)


def test_counter_hash_follows_code_not_comments(tmp_path):
    """The HBM-traffic figures are keyed by a hash of the kernel sources: a
    comment or blank-line edit keeps it, any code edit changes it."""
    import shutil
    from sparse_moe_layer_rmsnorm_amd import profsum
    src = tmp_path / "csrc"
    shutil.copytree(profsum.CSRC, src)
    h0 = profsum.source_hash(str(src))
    assert h0 == profsum.source_hash()
    f = src / "gemm_kernels.hip"
    text = f.read_text()
    f.write_text("// a new header line\n\n" + text.replace("\n", "  /* x */\n", 1))
    assert profsum.source_hash(str(src)) == h0
    f.write_text(text.replace("BM = BM_", "BM = BM_ + 0", 1))
    assert profsum.source_hash(str(src)) != h0
    assert profsum.strip_comments('s = "a//b"; c = \'/\'; // note\n/* x\n y */ t;') == 's = "a//b"; c = \'/\';\n t;'


def test_noalloc_scratch_size_matches_header():
    """The binding's copy of MOE_NOALLOC_SCRATCH_BYTES is the header's, and
    the array holds one replica-shaped forward of 8192 tokens."""
    import re
    text = open(B.HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.MOE_NOALLOC_SCRATCH_BYTES
    cfg = B.make_config(**REPLICA, max_tokens=16384)
    assert B.moe_workspace_bytes(cfg, 8192) <= B.MOE_NOALLOC_SCRATCH_BYTES < B.moe_workspace_bytes(cfg, 16384)


def test_fast_score_bound_constant():
    """The binding's copy of MOE_FAST_SCORE_ERR is the header's."""
    import re
    text = open(B.HEADER).read()
    m = re.search(r"#define MOE_FAST_SCORE_ERR 0x1p-(\d+)f", text)
    assert m and 2.0 ** -int(m.group(1)) == B.MOE_FAST_SCORE_ERR

