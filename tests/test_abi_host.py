"""Host-only checks of the C ABI: the library loads, exports every function
include/muonclip.h declares, and rejects bad arguments before any launch
(no GPU needed: validation runs before the first HIP call)."""
import ctypes
import os
import re

import pytest

import muonclip_step_amd as mc

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "muonclip.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    # every function declaration: a return type at the start of a line, then the name
    names = re.findall(r"^(?:const\s+)?(?:mc_status|void|size_t|int32_t|char)\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = mc.load()
    decl = declared_functions()
    assert set(decl) >= {"muonclip_step", "max_logits_per_head", "qk_clip_apply", "mc_last_error"}
    for name in decl:
        assert hasattr(lib, name), name
    assert set(mc.EXPORTS) == set(decl)


def test_default_hparams():
    hp = mc.hparams()
    assert abs(hp.lr - 2e-4) < 1e-10 and abs(hp.mu - 0.95) < 1e-7 and abs(hp.weight_decay - 0.1) < 1e-7
    assert abs(hp.rms_scale - 0.2) < 1e-7 and hp.tau == 100.0 and hp.ns_steps == 5
    assert (round(hp.ns_a, 4), round(hp.ns_b, 4), round(hp.ns_c, 4)) == (3.4445, -4.775, 2.0315)
    assert abs(hp.ns_eps - 1e-7) < 1e-12
    assert hp.nesterov == 0 and hp.clip_global == 0


def test_hparams_struct_size_matches_the_library():
    # mc_default_hparams writes the whole C struct: on a buffer one struct
    # long plus a sentinel tail, the tail must stay untouched and the last
    # fields must be written (so the binding's layout is the library's)
    size = ctypes.sizeof(mc.HParams)
    buf = (ctypes.c_uint8 * (size + 64))(*([0xAB] * (size + 64)))
    mc.load().mc_default_hparams(ctypes.cast(buf, ctypes.POINTER(mc.HParams)))
    assert bytes(buf[size:]) == b"\xab" * 64
    hp = mc.HParams.from_buffer_copy(bytes(buf[:size]))
    assert hp.ns_steps == 5 and hp.nesterov == 0 and hp.clip_global == 0


def fake_matrix(rows, cols, ld=None, w_dtype=mc.MC_BF16, g_dtype=mc.MC_F32, clip_slot=-1, period=0, segs=()):
    m = mc.Matrix()
    m.w, m.g, m.m = 0x100000, 0x200000, 0x300000   # never dereferenced: only validated
    m.rows, m.cols, m.ld = rows, cols, cols if ld is None else ld
    m.w_dtype, m.g_dtype = w_dtype, g_dtype
    m.clip_slot, m.period, m.nseg = clip_slot, period, len(segs)
    for i, s in enumerate(segs):
        m.seg[i] = mc.Segment(*s)
    return m


def step_status(mats, hp=None, s_max=None, slots=0, heads=0, gamma=None, ws=0x400000, ws_bytes=1 << 40):
    lib = mc.load()
    hp = hp or mc.hparams()
    arr = (mc.Matrix * max(1, len(mats)))(*mats)
    return lib.muonclip_step(arr, len(mats), ctypes.byref(hp), s_max, slots, heads, gamma, ws, ws_bytes, None)


def test_overlapped_step_validates_like_the_step():
    """muonclip_step_overlapped runs the step's argument checks before any
    launch or event wait: the same status for the same bad arguments."""
    lib = mc.load()

    def both(mats, hp=None, ws=0x400000, ws_bytes=1 << 40):
        hp = hp or mc.hparams()
        arr = (mc.Matrix * max(1, len(mats)))(*mats)
        a = lib.muonclip_step(arr, len(mats), ctypes.byref(hp), None, 0, 0, None, ws, ws_bytes, None)
        b = lib.muonclip_step_overlapped(arr, len(mats), ctypes.byref(hp), None, 0, 0, None, ws, ws_bytes, None,
                                         0x600000)
        return a, b

    for args, want in [(([fake_matrix(64, 0)],), mc.MC_ERR_SHAPE),
                       (([fake_matrix(64, 64)], mc.hparams(ns_steps=0)), mc.MC_ERR_HPARAM),
                       (([fake_matrix(64, 64)], None, None), mc.MC_ERR_WORKSPACE),
                       (([fake_matrix(64, 64)], None, 0x400000, 1024), mc.MC_ERR_WORKSPACE)]:
        assert both(*args) == (want, want)


def test_step_rejects_bad_arguments():
    assert step_status([fake_matrix(64, 0)]) == mc.MC_ERR_SHAPE
    assert step_status([fake_matrix(64, 64, ld=32)]) == mc.MC_ERR_SHAPE
    assert step_status([fake_matrix(64, 64, w_dtype=7)]) == mc.MC_ERR_DTYPE
    m = fake_matrix(64, 64); m.g = None
    assert step_status([m]) == mc.MC_ERR_NULL
    m = fake_matrix(64, 64); m.w = 0x100001
    assert step_status([m]) == mc.MC_ERR_ALIGN
    hp = mc.hparams(ns_steps=0)
    assert step_status([fake_matrix(64, 64)], hp=hp) == mc.MC_ERR_HPARAM
    hp = mc.hparams(tau=-1.0)
    assert step_status([fake_matrix(64, 64)], hp=hp) == mc.MC_ERR_HPARAM
    hp = mc.hparams(lr=float("nan"))
    assert step_status([fake_matrix(64, 64)], hp=hp) == mc.MC_ERR_HPARAM
    assert step_status([fake_matrix(64, 64)], hp=mc.hparams(nesterov=2)) == mc.MC_ERR_HPARAM
    assert step_status([fake_matrix(64, 64)], hp=mc.hparams(clip_global=-1)) == mc.MC_ERR_HPARAM
    # workspace: NULL, misaligned, too small
    assert step_status([fake_matrix(64, 64)], ws=None) == mc.MC_ERR_WORKSPACE
    assert step_status([fake_matrix(64, 64)], ws=0x400010) == mc.MC_ERR_WORKSPACE
    assert step_status([fake_matrix(64, 64)], ws_bytes=1024) == mc.MC_ERR_WORKSPACE
    assert "workspace" in mc.load().mc_last_error().decode()
    # clip layout: slot out of range, period not dividing rows, segment outside period, overlap
    seg = ((0, 16, 0.5),)
    assert step_status([fake_matrix(64, 64, clip_slot=1, period=16, segs=seg)], s_max=0x500000, slots=1,
                       heads=4) == mc.MC_ERR_SHAPE
    assert step_status([fake_matrix(64, 64, clip_slot=0, period=24, segs=seg)], s_max=0x500000, slots=1,
                       heads=4) == mc.MC_ERR_SHAPE
    assert step_status([fake_matrix(64, 64, clip_slot=0, period=16, segs=((8, 16, 0.5),))], s_max=0x500000,
                       slots=1, heads=4) == mc.MC_ERR_SHAPE
    assert step_status([fake_matrix(64, 64, clip_slot=0, period=16, segs=((0, 10, 0.5), (8, 4, 1.0)))],
                       s_max=0x500000, slots=1, heads=4) == mc.MC_ERR_SHAPE
    assert step_status([fake_matrix(64, 64, clip_slot=0, period=16, segs=seg)], s_max=0x500000, slots=1,
                       heads=2) == mc.MC_ERR_SHAPE
    # gamma_out without s_max
    assert step_status([fake_matrix(64, 64)], gamma=0x600000) == mc.MC_ERR_NULL
    # empty list is a no-op
    assert step_status([]) == mc.MC_OK


def test_workspace_sizes_are_monotone_and_grouped():
    one = [fake_matrix(2048, 2048)]
    four = one * 4
    s1 = mc.workspace_size(one)
    s4 = mc.workspace_size(four)
    assert s4 > s1 > 0
    assert mc.workspace_size(four, minimal=True) == s1
    # a tall and a wide matrix of the same shape share one group
    mixed = [fake_matrix(7168, 2048), fake_matrix(2048, 7168)]
    assert mc.workspace_size(mixed) == mc.workspace_size([fake_matrix(2048, 7168)] * 2)
    # 64 matrices per wave at most; more than one shape group asks for room
    # for two waves in flight
    w64 = mc.workspace_size([fake_matrix(256, 512)] * 64)
    assert mc.workspace_size([fake_matrix(256, 512)] * 200) == w64
    assert mc.workspace_size([fake_matrix(256, 512)] * 200, minimal=True) == \
        mc.workspace_size([fake_matrix(256, 512)], minimal=True)
    two_groups = [fake_matrix(256, 512), fake_matrix(512, 1024)]
    assert mc.workspace_size(two_groups) == 2 * mc.workspace_size([fake_matrix(512, 1024)])


def test_max_logits_rejects_bad_arguments():
    lib = mc.load()
    st = (ctypes.c_int64 * 3)(0, 0, 0)
    ks = (ctypes.c_int64 * 2)(0, 0)
    f = lib.max_logits_per_head
    out = 0x700000
    assert f(0x1000, 0x2000, None, 1, 1, 8, 2, 192, 128, 0, st, st, None, 1, 0.1, out, None) == mc.MC_ERR_SHAPE
    assert f(0x1000, 0x2000, None, 1, 1, 8, 2, 192, 128, 64, st, st, None, 1, 0.1, out, None) == mc.MC_ERR_NULL
    assert f(0x1000, 0x2000, None, 5, 1, 8, 2, 128, 128, 0, st, st, None, 1, 0.1, out, None) == mc.MC_ERR_DTYPE
    assert f(0x1000, 0x2000, None, 1, 1, 8, 2, 128, 128, 0, st, st, None, 1, -1.0, out, None) == mc.MC_ERR_HPARAM
    assert f(0x1000, 0x2000, None, 1, 1, 8, 2, 128, 128, 0, st, st, None, 1, 0.1, None, None) == mc.MC_ERR_NULL
    assert f(0x1001, 0x2000, None, 1, 1, 8, 2, 128, 128, 0, st, st, None, 1, 0.1, out, None) == mc.MC_ERR_ALIGN
    _ = ks


def test_qk_clip_apply_rejects_bad_arguments():
    lib = mc.load()
    seg = ((0, 16, 0.5),)
    arr = (mc.Matrix * 1)(fake_matrix(64, 64, clip_slot=0, period=16, segs=seg))
    assert lib.qk_clip_apply(arr, 1, None, 1, 4, 100.0, None, None) == mc.MC_ERR_NULL
    assert lib.qk_clip_apply(arr, 1, 0x500000, 1, 4, 0.0, None, None) == mc.MC_ERR_HPARAM
    assert lib.qk_clip_apply(arr, 1, 0x500000, 1, 2, 100.0, None, None) == mc.MC_ERR_SHAPE


def test_oracle_and_product_are_independent():
    # the product package never imports the oracle, and the oracle never
    # imports the product package or the HIP library
    root = os.path.dirname(os.path.dirname(__file__))
    for dirpath, _, files in os.walk(os.path.join(root, "muonclip_step_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
    for f in os.listdir(os.path.join(root, "oracle")):
        if f.endswith(".py"):
            txt = open(os.path.join(root, "oracle", f)).read()
            assert "muonclip_step_amd" not in txt and "libmuonclip" not in txt
    ws = open(os.path.join(root, "workloads", "__init__.py")).read()
    assert "import oracle" not in ws and "muonclip_step_amd" not in ws


def test_adamw_defaults_and_rejections():
    hp = mc.adamw_hparams()
    assert abs(hp.lr - 2e-4) < 1e-10 and abs(hp.beta1 - 0.9) < 1e-7 and abs(hp.beta2 - 0.95) < 1e-7
    assert abs(hp.eps - 1e-8) < 1e-14 and abs(hp.weight_decay - 0.1) < 1e-7 and hp.step == 1
    lib = mc.load()

    def status(vecs, **kw):
        arr = (mc.Vector * max(1, len(vecs)))(*vecs)
        return lib.adamw_step(arr, len(vecs), ctypes.byref(mc.adamw_hparams(**kw)), None)

    def vec(n=16, p=0x100000, g=0x200000, m=0x300000, v=0x400000, pd=mc.MC_BF16, gd=mc.MC_F32):
        d = mc.Vector()
        d.p, d.g, d.m, d.v, d.n, d.p_dtype, d.g_dtype = p, g, m, v, n, pd, gd
        return d

    assert status([]) == mc.MC_OK
    assert status([vec(n=0, p=None)]) == mc.MC_OK            # empty vectors are never touched
    assert status([vec(p=None)]) == mc.MC_ERR_NULL
    assert status([vec(n=-1)]) == mc.MC_ERR_SHAPE
    assert status([vec(pd=5)]) == mc.MC_ERR_DTYPE
    assert status([vec(m=0x300002)]) == mc.MC_ERR_ALIGN
    assert status([vec(p=0x100001)]) == mc.MC_ERR_ALIGN
    assert status([vec()], step=0) == mc.MC_ERR_HPARAM
    assert status([vec()], beta1=1.0) == mc.MC_ERR_HPARAM
    assert status([vec()], beta2=-0.1) == mc.MC_ERR_HPARAM
    assert status([vec()], eps=-1e-8) == mc.MC_ERR_HPARAM
    assert status([vec()], lr=float("inf")) == mc.MC_ERR_HPARAM


def test_matrix_beyond_32bit_offsets_is_rejected():
    """rows x cols (padded to 64) of 2^31 elements or more is refused before
    any launch (host-side validation; no device memory is touched)."""
    import ctypes
    import muonclip_step_amd as mc
    lib = mc.load()
    m = mc.Matrix()
    m.w = m.g = m.m = 256   # never dereferenced: validation fails first
    m.rows, m.cols, m.ld = 65536, 32768, 32768
    m.w_dtype = m.g_dtype = 1
    m.clip_slot = -1
    hp = mc.hparams()
    arr = (mc.Matrix * 1)(m)
    assert lib.mc_workspace_size(arr, 1, ctypes.byref(hp)) == 0
    assert b"2^31" in lib.mc_last_error()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with status 2 and a
    message before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_noalloc_step_rejects_matrices_beyond_its_scratch():
    # the dense 7168 x 18432 FFN matrix needs about 1.3 GB of workspace, more
    # than the static scratch: rejected before anything touches a device
    lib = mc.load()
    hp = mc.hparams()
    arr = (mc.Matrix * 1)(fake_matrix(7168, 18432))
    st = lib.muonclip_step_noalloc(arr, 1, ctypes.byref(hp), None, 0, 0, None, None)
    assert st == mc.MC_ERR_WORKSPACE
    assert b"static scratch" in lib.mc_last_error()
    assert lib.mc_workspace_min_size(arr, 1, ctypes.byref(hp)) > mc.NOALLOC_SCRATCH_BYTES
    # bad arguments are reported as by muonclip_step
    bad = (mc.Matrix * 1)(fake_matrix(64, 64, ld=32))
    assert lib.muonclip_step_noalloc(bad, 1, ctypes.byref(hp), None, 0, 0, None, None) == mc.MC_ERR_SHAPE
    hp.ns_steps = 0
    assert lib.muonclip_step_noalloc(arr, 1, ctypes.byref(hp), None, 0, 0, None, None) == mc.MC_ERR_HPARAM


def test_dispatcher_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The dispatcher (argument validation and workspace planning, host code
    of mc_api.hip) built with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host side, linked with the regular kernel objects and driven by
    tests/sanitize/dispatch_checks.cpp: every documented rejection returns its
    status and the planning of every configuration's shape set runs clean."""
    import subprocess

    from muonclip_step_amd import build as b
    root = os.path.dirname(os.path.dirname(__file__))
    objs = [os.path.join(b.BUILD, f + ".hip.o") for f in ("ns_gemm", "elementwise", "max_logits", "attn_fwd", "adamw")]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    hipcc = b._hipcc()
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    api = str(tmp_path / "mc_api_san.o")
    drv = str(tmp_path / "dispatch_checks.o")
    exe = str(tmp_path / "dispatch_checks")
    inc = ["-I", os.path.join(root, "include"), "-I", b.CSRC]
    steps = [
        [hipcc, f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", *inc, *san,
         "-c", os.path.join(b.CSRC, "mc_api.hip"), "-o", api],
        [clang, "-std=c++17", "-O1", "-g", "-I", os.path.join(root, "include"), "-fsanitize=address,undefined",
         "-fno-omit-frame-pointer", "-c", os.path.join(root, "tests", "sanitize", "dispatch_checks.cpp"), "-o", drv],
        [hipcc, f"--offload-arch={b.ARCH}", *san, drv, api, *objs, "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "dispatch checks ok" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
