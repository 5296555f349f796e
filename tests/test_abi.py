"""C ABI of libmala, on the CPU: the library loads, exports every function
include/mala.h declares, reports its tiling, sizes workspaces, and rejects bad
arguments with a status code and a message before touching any device (no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from contribution_gated_sparse_amd import mala as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        from contribution_gated_sparse_amd import build
        build.build()
    return M.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mala.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mala_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 14, names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(names) == set(M.EXPORTS)


def test_tiling(lib):
    assert M.mala_get_tiling(M.OP_FWD) == (32, 64, 0)
    assert M.mala_get_tiling(M.OP_BWD) == (32, 16, 0)
    assert M.mala_get_tiling(M.OP_DECODE) == (1, 64, 256)
    fb = M.mala_get_tiling(M.OP_FWD)
    bb = M.mala_get_tiling(M.OP_BWD)
    assert fb[0] % bb[0] == 0 and fb[1] % bb[1] == 0     # backward refines forward
    with pytest.raises(M.MalaError):
        M.mala_get_tiling(7)


def prob(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, n_q=100, n_k=100, head_dim=128,
                dtype=M.MALA_BF16, causal=1, tau=1e-4, softmax_scale=0.088, flags=0)
    base.update(kw)
    return M.Problem(*[base[f] for f, _ in M.Problem._fields_])


BAD = [
    (dict(n_kv_heads=3), M.MALA_ERR_INVALID_ARG, "multiple"),
    (dict(head_dim=96), M.MALA_ERR_UNSUPPORTED, "head_dim"),
    (dict(tau=-1.0), M.MALA_ERR_INVALID_ARG, "tau"),
    (dict(tau=float("nan")), M.MALA_ERR_INVALID_ARG, "tau"),
    (dict(tau=float("inf")), M.MALA_ERR_INVALID_ARG, "tau"),
    (dict(softmax_scale=0.0), M.MALA_ERR_INVALID_ARG, "softmax_scale"),
    (dict(n_q=101), M.MALA_ERR_INVALID_ARG, "causal"),
    (dict(n_k=0, n_q=0, causal=0), None, None),
    (dict(n_k=0, causal=0), M.MALA_ERR_INVALID_ARG, "n_k"),
    (dict(batch=0), M.MALA_ERR_INVALID_ARG, "batch"),
    (dict(dtype=5), M.MALA_ERR_INVALID_ARG, "dtype"),
    (dict(flags=8), M.MALA_ERR_INVALID_ARG, "flags"),
    (dict(n_k=20_000_000, n_q=1), M.MALA_ERR_UNSUPPORTED, "2 GiB"),
]


@pytest.mark.parametrize("kw,status,word", BAD)
def test_forward_rejects_bad_problems(lib, kw, status, word):
    p = prob(**kw)
    buf = (ctypes.c_char * 64)()
    addr = ctypes.addressof(buf)
    addr += (-addr) % 16
    ptr = ctypes.c_void_p(addr)
    if status is None:      # n_q = 0: nothing to do, returns OK without a launch
        assert lib.mala_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None) == 0
        return
    st = lib.mala_fwd(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, None, None, None)
    assert st == status
    assert word in lib.mala_last_error().decode()


def test_null_and_misaligned_pointers(lib):
    p = prob()
    buf = (ctypes.c_char * 64)()
    addr = ctypes.addressof(buf)
    addr += (-addr) % 16
    good, bad = ctypes.c_void_p(addr), ctypes.c_void_p(addr + 2)
    assert lib.mala_fwd(ctypes.byref(p), None, good, good, good, good, None, None,
                        None) == M.MALA_ERR_INVALID_ARG
    assert "q is NULL" in lib.mala_last_error().decode()
    assert lib.mala_fwd(ctypes.byref(p), good, bad, good, good, good, None, None,
                        None) == M.MALA_ERR_INVALID_ARG
    assert "aligned" in lib.mala_last_error().decode()
    assert lib.mala_fwd(None, good, good, good, good, good, None, None, None) == \
        M.MALA_ERR_INVALID_ARG


def test_backward_workspace(lib):
    p = prob()
    need = lib.mala_bwd_workspace_size(ctypes.byref(p))
    # D (B*Hq*Nq fp32) + decision bits, each rounded up to 256 bytes
    tr, tc = -(-100 // 32), -(-100 // 16)
    expect = -(-(4 * 100 * 4) // 256) * 256 + -(-(4 * tr * -(-tc // 32) * 4) // 256) * 256
    assert need == expect
    assert lib.mala_bwd_workspace_size(ctypes.byref(prob(head_dim=80))) == 0
    # MALA_FLAG_GATE_PASS adds the fp32 dK, dV partials of the per-head walks
    # (2 x B x Hq x Nk x D floats) and the walks' plan (one int per batch, KV
    # head and 128-key block) for bf16; fp32 problems ignore the flag
    part = -(-(2 * 4 * 100 * 128 * 4) // 256) * 256
    plan = -(-(1 * 2 * 1 * 4) // 256) * 256
    assert lib.mala_bwd_workspace_size(ctypes.byref(prob(flags=M.MALA_FLAG_GATE_PASS))) == \
        need + part + plan
    assert lib.mala_bwd_workspace_size(ctypes.byref(prob(flags=3))) == need + part + plan
    f32 = lib.mala_bwd_workspace_size(ctypes.byref(prob(dtype=M.MALA_F32)))
    assert lib.mala_bwd_workspace_size(ctypes.byref(prob(dtype=M.MALA_F32, flags=2))) == f32
    buf = (ctypes.c_char * 1024)()
    addr = ctypes.addressof(buf)
    addr += (-addr) % 256
    g = ctypes.c_void_p(addr)
    st = lib.mala_bwd(ctypes.byref(p), g, g, g, g, g, g, g, g, g, g, need - 1, None, None, None)
    assert st == M.MALA_ERR_WORKSPACE
    st = lib.mala_bwd(ctypes.byref(p), g, g, g, g, g, g, g, g, g, ctypes.c_void_p(addr + 16),
                      need, None, None, None)
    assert st == M.MALA_ERR_INVALID_ARG and "256-byte" in lib.mala_last_error().decode()


def test_nested_backward_arguments(lib):
    """mala_bwd_nested runs in the gate-pass mode and needs the forward's
    mask; both are checked before anything is enqueued, and its workspace is
    the gate-pass one."""
    buf = (ctypes.c_char * 1024)()
    addr = ctypes.addressof(buf)
    addr += (-addr) % 256
    g = ctypes.c_void_p(addr)
    fm = ctypes.c_void_p(addr + 1)          # a byte mask needs no alignment
    p = prob()
    need = lib.mala_bwd_workspace_size(ctypes.byref(p))
    st = lib.mala_bwd_nested(ctypes.byref(p), g, g, g, g, g, g, fm, g, g, g, g, need, None, None,
                             None)
    assert st == M.MALA_ERR_INVALID_ARG and "MALA_FLAG_GATE_PASS" in lib.mala_last_error().decode()
    p = prob(flags=M.MALA_FLAG_GATE_PASS)
    need_gp = lib.mala_bwd_workspace_size(ctypes.byref(p))
    st = lib.mala_bwd_nested(ctypes.byref(p), g, g, g, g, g, g, None, g, g, g, g, need_gp, None,
                             None, None)
    assert st == M.MALA_ERR_INVALID_ARG and "fwd_tile_mask" in lib.mala_last_error().decode()
    st = lib.mala_bwd_nested(ctypes.byref(p), g, g, g, g, g, g, fm, g, g, g, g, need_gp - 1, None,
                             None, None)
    assert st == M.MALA_ERR_WORKSPACE
    assert lib.mala_bwd_nested(None, g, g, g, g, g, g, fm, g, g, g, g, need_gp, None, None,
                               None) == M.MALA_ERR_INVALID_ARG


def test_auto_backward_arguments(lib):
    """mala_bwd_auto needs the forward's kept-tile counters, chooses the walk
    itself (MALA_FLAG_GATE_PASS set by the caller is an error) and takes the
    gate-pass workspace; all checked before anything is enqueued."""
    buf = (ctypes.c_char * 1024)()
    addr = ctypes.addressof(buf)
    addr += (-addr) % 256
    g = ctypes.c_void_p(addr)
    fk = ctypes.c_void_p(addr + 4)
    p = prob()
    need = lib.mala_bwd_workspace_size(ctypes.byref(p))
    need_gp = lib.mala_bwd_workspace_size(ctypes.byref(prob(flags=M.MALA_FLAG_GATE_PASS)))
    assert need_gp > need
    st = lib.mala_bwd_auto(ctypes.byref(p), g, g, g, g, g, g, None, g, g, g, g, need_gp, None,
                           None, None)
    assert st == M.MALA_ERR_INVALID_ARG and "fwd_kept_tiles" in lib.mala_last_error().decode()
    gp = prob(flags=M.MALA_FLAG_GATE_PASS)
    st = lib.mala_bwd_auto(ctypes.byref(gp), g, g, g, g, g, g, fk, g, g, g, g, need_gp, None,
                           None, None)
    assert st == M.MALA_ERR_INVALID_ARG and "MALA_FLAG_GATE_PASS" in lib.mala_last_error().decode()
    # the default backward's workspace is too small: the gate pass's is needed
    st = lib.mala_bwd_auto(ctypes.byref(p), g, g, g, g, g, g, fk, g, g, g, g, need, None, None,
                           None)
    assert st == M.MALA_ERR_WORKSPACE
    assert lib.mala_bwd_auto(None, g, g, g, g, g, g, fk, g, g, g, g, need_gp, None, None,
                             None) == M.MALA_ERR_INVALID_ARG


def dprob(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=1, head_dim=128, cache_capacity=1000,
                max_n_k=900, dtype=M.MALA_BF16, tau=1e-4, softmax_scale=0.088, split_keys=0)
    base.update(kw)
    return M.DecodeProblem(*[base[f] for f, _ in M.DecodeProblem._fields_])


def test_decode_validation_and_workspace(lib):
    p = dprob()
    n = lib.mala_decode_workspace_size(ctypes.byref(p))
    # 4 splits of 256 keys: (m, S) pairs padded to 64 words, then (O, kept
    # bits) per (sequence, query head, split) and V-read bits per (sequence,
    # KV head, split), 4 bytes each
    ms = -(-(2 * 8 * 4 * 2) // 64) * 64
    assert n == -(-((ms + 2 * 8 * 4 * 129 + 2 * 1 * 4) * 4) // 256) * 256
    for kw, word in [(dict(n_q_heads=34, n_kv_heads=2), "16"), (dict(max_n_k=2000), "max_n_k"),
                     (dict(batch=40000, n_q_heads=2, n_kv_heads=2), "65535"),
                     (dict(head_dim=64), "head_dim"), (dict(tau=-2.0), "tau"),
                     (dict(n_q_heads=7, n_kv_heads=2), "multiple")]:
        q = dprob(**kw)
        assert lib.mala_decode_workspace_size(ctypes.byref(q)) == 0
        buf = (ctypes.c_char * 64)()
        addr = ctypes.addressof(buf)
        addr += (-addr) % 256
        g = ctypes.c_void_p(addr)
        st = lib.mala_decode(ctypes.byref(q), g, g, g, g, g, g, g, 1 << 20, None, None, None)
        assert st != 0 and word in lib.mala_last_error().decode()
    # fp32 decode supports head_dim 64
    assert lib.mala_decode_workspace_size(ctypes.byref(dprob(head_dim=64, dtype=M.MALA_F32))) > 0


def test_decode_noalloc_rejects_problems_past_its_scratch(lib):
    """mala_decode_noalloc refuses a problem whose workspace exceeds the fixed
    scratch, before touching a device; the 128K decode batch fits."""
    big = dprob(batch=64, n_q_heads=16, n_kv_heads=1, cache_capacity=131136, max_n_k=131136)
    assert lib.mala_decode_workspace_size(ctypes.byref(big)) > (32 << 20)
    g = ctypes.c_void_p(1 << 20)
    st = lib.mala_decode_noalloc(ctypes.byref(big), g, g, g, g, g, g, None, None, None)
    assert st == M.MALA_ERR_UNSUPPORTED and "scratch" in lib.mala_last_error().decode()
    c5 = dprob(batch=8, n_q_heads=8, n_kv_heads=1, cache_capacity=131136, max_n_k=131136)
    assert lib.mala_decode_workspace_size(ctypes.byref(c5)) <= (32 << 20)
    bad = dprob(tau=-1.0)
    st = lib.mala_decode_noalloc(ctypes.byref(bad), g, g, g, g, g, g, None, None, None)
    assert st == M.MALA_ERR_INVALID_ARG


def test_decode_split_keys_rule(lib):
    """The split length each split_keys setting selects (the rule the header
    states), its validation, and the workspace of multi-word decision bits."""
    def split(**kw):
        return lib.mala_decode_split_keys(ctypes.byref(dprob(**kw)))
    assert split() == 256
    assert split(split_keys=64) == 64
    assert split(split_keys=512) == 512
    # longer than the sequence: one split, max_n_k rounded up to 64
    assert split(split_keys=4096) == 960
    for bad in (100, -2, 63):
        assert split(split_keys=bad) == 0
        assert "split_keys" in lib.mala_last_error().decode()
    # AUTO: 256 * ceil(max_n_k / (256 * max(1, 1024 // (batch * n_kv_heads))))
    assert split(split_keys=M.DECODE_SPLIT_AUTO) == 256                    # 2 x 1 heads, 900 keys
    big = dict(batch=8, max_n_k=131073, cache_capacity=131073, split_keys=M.DECODE_SPLIT_AUTO)
    assert split(**big) == 1280                  # 128 splits per sequence: 256 * ceil(131073 / 32768)
    assert split(**dict(big, n_kv_heads=2, n_q_heads=16)) == 2304        # 64: 256 * ceil(131073 / 16384)
    assert split(batch=1024, split_keys=M.DECODE_SPLIT_AUTO) == 960       # one split, capped
    # fp32, 2 splits of 40 tiles: two bit words per (head, split)
    p = dprob(max_n_k=5000, cache_capacity=5000, split_keys=2560, dtype=M.MALA_F32)
    ms = -(-(2 * 8 * 2 * 2) // 64) * 64
    words = ms + 2 * 8 * 2 * (128 + 2) + 2 * 1 * 2 * 2
    assert lib.mala_decode_workspace_size(ctypes.byref(p)) == -(-(words * 4) // 256) * 256
    # bf16 splits longer than 1024 keys run as three passes: the partial states
    # are per part of 4 tiles (10 parts per 40-tile split), and the
    # per-(head, tile) statistics follow the bits
    p = dprob(max_n_k=5000, cache_capacity=5000, split_keys=2560)
    parts = 2 * 10
    ms = -(-(2 * 8 * parts * 2) // 64) * 64
    bits_end = ms + 2 * 8 * parts * 128 + 2 * 8 * 2 * 2 + 2 * 1 * 2 * 2
    words = bits_end + bits_end % 2 + 2 * 8 * 2 * 40 * 2
    assert lib.mala_decode_workspace_size(ctypes.byref(p)) == -(-(words * 4) // 256) * 256


def test_header_and_abi_from_c(lib, tmp_path):
    """include/mala.h compiles as pedantic C99, and a C program linked
    against libmala gets the documented tiling, workspace, split-length and
    error behaviour (no GPU needed)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(M.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    src = os.path.join(ROOT, "tests", "c_abi_check.c")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), src, "-L", libdir, "-lmala",
                        f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr


def test_version(lib):
    assert "gfx950" in M.version()
