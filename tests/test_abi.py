"""CPU checks of the C ABI: the library loads, exports every function include/spectree.h
declares, and rejects bad host arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spectree.h")


@pytest.fixture(scope="module")
def lib():
    from tree_attention_verification_spec_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from tree_attention_verification_spec_amd import build
        build.build()
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(spec_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("spec_tree_build", "spec_tree_assemble", "spec_tree_attn", "spec_tree_attn_workspace",
              "spec_verify", "spec_verify_workspace", "spec_medusa_heads", "spec_medusa_heads_workspace",
              "spec_kv_compact", "spec_tree_select", "spec_lm_head_stats", "spec_lm_head_stats_workspace",
              "spec_verify_greedy_stats", "spec_verify_lm_head", "spec_verify_lm_head_workspace",
              "spec_strerror"):
        assert n in names, n
    for n in ("spec_prof_enable", "spec_prof_reset", "spec_prof_read", "spec_internal_tune"):
        assert n not in names, f"{n} is internal and must not be in the public header"


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} is declared but not exported"
    for n in internal_functions():
        assert hasattr(lib, n), f"{n} is declared in internal.h but not exported"


def internal_functions():
    text = open(os.path.join(ROOT, "tree_attention_verification_spec_amd", "csrc", "internal.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(spec_\w+)\s*\(", text, flags=re.M)))


def test_tuning_overrides(lib):
    """Launch-shape overrides are explicit calls (never environment variables); unknown names
    are refused, and a workspace query without an override depends on its arguments alone."""
    from tree_attention_verification_spec_amd import binding
    assert set(internal_functions()) == {"spec_prof_enable", "spec_prof_reset", "spec_prof_read",
                                         "spec_internal_tune"}
    assert lib.spec_internal_tune(b"no_such_knob", 1) == -1
    base = lib.spec_verify_workspace(4, 63, 128256)
    with binding.tuned(verify_chunk=16384, verify_store_w=0, verify_rows_list=1):
        assert lib.spec_verify_workspace(4, 63, 128256) == base
    a0 = lib.spec_tree_attn_workspace(1, 63, 32, 8, 128, 2111, 1)
    with binding.tuned(attn_splits=2):
        a2 = lib.spec_tree_attn_workspace(1, 63, 32, 8, 128, 2111, 1)
    assert lib.spec_tree_attn_workspace(1, 63, 32, 8, 128, 2111, 1) == a0 and a2 > 0
    src = os.path.join(ROOT, "tree_attention_verification_spec_amd", "csrc")
    for f in os.listdir(src):
        assert "getenv" not in open(os.path.join(src, f)).read(), f"{f} reads the environment"


def test_status_strings(lib):
    for code, text in ((0, "ok"), (1, "invalid argument"), (2, "unsupported configuration"),
                       (3, "workspace missing or too small"), (4, "HIP runtime error")):
        assert lib.spec_strerror(code).decode() == text


def test_host_argument_checks(lib):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below returns before a launch
    # tree build: B < 1, N > 256, NULL outputs
    assert lib.spec_tree_build(fake, None, None, None, 0, 10, fake, fake, fake, fake, None) == 1
    assert lib.spec_tree_build(fake, None, None, None, 1, 257, fake, fake, fake, fake, None) == 1
    assert lib.spec_tree_build(fake, None, None, None, 1, 10, None, fake, fake, fake, None) == 1
    # tree attention: unsupported head_dim / group, missing workspace
    args = [fake, fake, fake, fake, fake, None]
    assert lib.spec_tree_attn(*args, 1, 10, 8, 2, 96, 100, 0.1, 1, fake, None, None, fake, 1 << 30, None) == 2
    assert lib.spec_tree_attn(*args, 1, 10, 6, 4, 128, 100, 0.1, 1, fake, None, None, fake, 1 << 30, None) == 2
    assert lib.spec_tree_attn(*args, 1, 10, 8, 2, 128, 100, 0.1, 7, fake, None, None, fake, 1 << 30, None) == 2
    for bad in (0.0, -0.1, float("inf"), float("nan")):   # the scale must be positive and finite
        assert lib.spec_tree_attn(*args, 1, 10, 8, 2, 128, 100, bad, 1, fake, None, None, fake, 1 << 30, None) == 1
    need = lib.spec_tree_attn_workspace(1, 63, 32, 8, 128, 2111, 1)
    assert need > 0
    assert lib.spec_tree_attn(*args, 1, 63, 32, 8, 128, 2111, 0.1, 1, fake, None, None, None, 0, None) == 3
    assert lib.spec_tree_attn(*args, 1, 63, 32, 8, 128, 2111, 0.1, 1, fake, None, None, fake, need - 1, None) == 3
    # verify: reject without draft rows, t2d missing with Vd != V, bad mode, small workspace
    vargs = [fake, None, None, None, fake, fake, None, fake, 2, 10, 100]
    outs = [fake, fake, fake, None, fake]
    wsz = lib.spec_verify_workspace(2, 10, 100)
    assert lib.spec_verify(*vargs, 0, 0, 9, 2, 0.1, 0.3, *outs, fake, wsz, None) == 1
    vargs2 = [fake, fake, fake, None, fake, fake, None, fake, 2, 10, 100]
    assert lib.spec_verify(*vargs2, 3, 50, 9, 2, 0.1, 0.3, *outs, fake, wsz, None) == 1
    assert lib.spec_verify(*vargs2, 3, 100, 9, 5, 0.1, 0.3, *outs, fake, wsz, None) == 1
    assert lib.spec_verify(*vargs2, 3, 100, 9, 2, 0.1, 0.3, *outs, fake, wsz - 1, None) == 3
    # heads: unsupported shapes
    hw = lib.spec_medusa_heads_workspace(4, 2, 256, 1000, 8)
    assert lib.spec_medusa_heads(fake, fake, fake, 17, 2, 256, 1000, 8, fake, fake, None, fake, hw, None) == 2
    assert lib.spec_medusa_heads(fake, fake, fake, 4, 2, 200, 1000, 8, fake, fake, None, fake, hw, None) == 2
    assert lib.spec_medusa_heads(fake, fake, fake, 4, 2, 256, 1000, 65, fake, fake, None, fake, hw, None) == 2
    assert lib.spec_medusa_heads(fake, fake, fake, 4, 2, 256, 1000, 8, fake, fake, None, fake, hw - 1, None) == 3


def test_kv_compact_host_checks(lib):
    fake = ctypes.c_void_p(0x1000)     # 16-byte aligned; never dereferenced (no call launches)
    other = ctypes.c_void_p(0x2000)
    odd = ctypes.c_void_p(0x1008)      # 8-byte aligned only
    one = 1 * 8 * 100 * 128            # elements of one layer at B 1, Hkv 8, S_max 100, d 128

    def call(k=fake, v=fake, stride=one, L=1, pl=fake, plo=other, path=fake, acc=fake, err=None,
             B=1, H=8, S=100, d=128, md=8, dt=1):
        return lib.spec_kv_compact(k, v, stride, L, pl, plo, path, acc, err, B, H, S, d, md, dt, None)

    assert call(k=None) == 1 and call(path=None) == 1 and call(acc=None) == 1
    assert call(L=0) == 1 and call(B=0) == 1 and call(md=-1) == 1
    assert call(plo=fake) == 1                           # prefix_len_out aliases prefix_len
    assert call(L=2, stride=one - 1) == 1                # layers overlap
    assert call(dt=7) == 2                               # dtype
    assert call(d=100) == 2                              # 200-byte rows: not a multiple of 16
    assert call(d=512, dt=0) == 2                        # 2 KB rows: longer than a wave's pass
    assert call(k=odd) == 2                              # alignment
    assert call(L=2, stride=one + 4) == 2                # 8-byte layer stride in bf16


def test_workspace_sizes_are_monotone(lib):
    small = lib.spec_verify_workspace(1, 63, 128256)
    big = lib.spec_verify_workspace(16, 127, 128256)
    assert 0 < small < big
    assert lib.spec_medusa_heads_workspace(8, 4, 4096, 32000, 8) > 8 * 4 * 32000 * 4
    assert lib.spec_tree_attn_workspace(1, 10, 4, 1, 64, 266, 0) == 0   # fp32 path needs none
    # the bf16 kernel addresses one (sequence, KV head) cache with 32-bit offsets: below 2 GiB
    assert lib.spec_tree_attn_workspace(1, 63, 32, 8, 128, (1 << 23) - 1, 1) > 0
    assert lib.spec_tree_attn_workspace(1, 63, 32, 8, 128, 1 << 23, 1) == 0
    assert lib.spec_tree_attn_workspace(1, 63, 32, 8, 64, (1 << 24) - 1, 1) > 0
    assert lib.spec_tree_attn_workspace(1, 63, 32, 8, 64, 1 << 24, 1) == 0


def test_tree_select_argument_checks(lib):
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: every call below returns before a launch

    def call(par=fake, prob=fake, tok_in=None, row_in=None, B=2, C=100, N=63, sel=fake, parents=fake,
             tok=None, row=None, nn=fake, err=fake):
        return lib.spec_tree_select(par, prob, None, tok_in, row_in, B, C, N, sel, parents, tok, row, nn, err,
                                    None)

    assert call(par=None) == 1 and call(prob=None) == 1 and call(sel=None) == 1
    assert call(parents=None) == 1 and call(nn=None) == 1 and call(err=None) == 1
    assert call(B=0) == 1 and call(C=0) == 1 and call(C=4097) == 1
    assert call(N=0) == 1 and call(N=257) == 1
    assert call(tok_in=fake) == 1 and call(tok=fake) == 1          # tokens in without out, and back
    assert call(row_in=fake) == 1 and call(row=fake) == 1


def test_lm_head_stats_argument_checks(lib):
    fake = ctypes.c_void_p(0x1000)     # 16-byte aligned; never dereferenced (no call launches)
    odd = ctypes.c_void_p(0x1008)
    ws = lib.spec_lm_head_stats_workspace(1, 63, 4096, 128256)
    assert ws >= 63 * 2004 * 24 + 63 * 4096 * 2

    def call(h=fake, W=fake, B=1, N=63, Dm=4096, V=128256, out=fake, wsz=ws, wsp=fake):
        return lib.spec_lm_head_stats(h, W, fake, fake, None, B, N, Dm, V, out, fake, fake, fake, fake, fake,
                                      wsp, wsz, None)

    assert call(h=None) == 1 and call(W=None) == 1 and call(out=None) == 1
    assert call(B=0) == 1 and call(V=0) == 1
    assert call(B=17, N=256) == 2                        # more than 4096 rows
    assert call(B=1, N=257) == 2                         # more than 256 nodes
    assert call(Dm=4000) == 2                            # not a multiple of 128
    assert call(h=odd) == 2 and call(W=odd) == 2         # alignment
    assert call(wsz=ws - 1) == 3 and call(wsp=None) == 3


def test_verify_greedy_stats_argument_checks(lib):
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: every call below returns before a launch

    def call(am=fake, B=1, N=63, V=100, md=62, acc=fake, err=fake):
        return lib.spec_verify_greedy_stats(am, fake, fake, None, B, N, V, md, acc, fake, fake, None, err, None)

    assert call(am=None) == 1 and call(acc=None) == 1 and call(err=None) == 1
    assert call(B=0) == 1 and call(N=257) == 1 and call(V=0) == 1 and call(md=-1) == 1


def test_verify_lm_head_argument_checks(lib):
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: every call below returns before a launch
    ws = lib.spec_verify_lm_head_workspace(1, 63, 4096, 128256, 1)
    assert ws > lib.spec_lm_head_stats_workspace(1, 63, 4096, 128256)
    ws_rej = lib.spec_verify_lm_head_workspace(1, 63, 4096, 128256, 2)
    assert ws_rej >= ws + 63 * 128256 * 4                # REJECT keeps every row's logits

    def call(mode=0, eps=0.09, delta=0.3, uni=fake, wsz=ws, B=1, N=63, Dm=4096, draft=None, drow=None, R=0, Vd=0):
        return lib.spec_verify_lm_head(fake, fake, fake, fake, None, uni, draft, drow, None, B, N, Dm, 128256, R, Vd,
                                       N - 1, mode, eps, delta, fake, fake, fake, None, fake, fake, wsz, None)

    assert call(uni=None) == 1 and call(B=0) == 1
    assert call(mode=3) == 1                             # WALK without draft arrays
    assert call(mode=2) == 1                             # REJECT without draft arrays
    assert call(mode=2, draft=fake, drow=fake, R=4, Vd=1000) == 1   # no t2d: Vd must be V
    assert call(mode=1, eps=float("nan")) == 1
    assert call(Dm=4000) == 2 and call(wsz=ws - 1) == 3
    assert call(mode=2, draft=fake, drow=fake, R=63, Vd=128256, wsz=ws) == 3   # REJECT needs its rows
    ws_walk = lib.spec_verify_lm_head_workspace(1, 63, 4096, 128256, 3)
    assert ws_walk >= ws + 63 * 128256 * 4 + lib.spec_verify_workspace(1, 63, 128256)   # rows + spec_verify's
    assert call(mode=3, draft=fake, drow=fake, R=63, Vd=128256, wsz=ws_rej) == 3


def test_status_strings_cover_every_code(lib):
    assert lib.spec_strerror(5).decode() == "request exceeds the fixed scratch array"
    for code in (-1, 6, 99, 1 << 30):
        assert lib.spec_strerror(code).decode() == "unknown status"


def test_verify_static_host_checks(lib):
    """spec_verify_static refuses, before any device call, arguments spec_verify refuses and a
    request larger than its fixed scratch array."""
    fake = ctypes.c_void_p(0x1000)
    limit = 16 << 20
    assert lib.spec_verify_static_bytes(1, 63, 128256) <= lib.spec_verify_workspace(1, 63, 128256)
    assert lib.spec_verify_static_bytes(16, 127, 128256) <= lib.spec_verify_workspace(16, 127, 128256)
    # above 64 bonus chunks the workspace reserves stored draw weights that batch 16 does not use
    assert lib.spec_verify_static_bytes(16, 127, 300_000) < lib.spec_verify_workspace(16, 127, 300_000)
    for B, N, V in ((1, 63, 128256), (16, 127, 128256), (4, 255, 128256), (8, 127, 32000)):
        assert lib.spec_verify_static_bytes(B, N, V) <= limit, (B, N, V)
    assert lib.spec_verify_static_bytes(8, 256, 1_000_000) > limit
    assert lib.spec_verify_static_bytes(0, 10, 10) == 0

    def call(B=2, N=10, V=100, mode=0, R=0, Vd=0, draft=None, drow=None, logits=fake, acc=fake):
        return lib.spec_verify_static(logits, draft, drow, None, fake, fake, None, fake, B, N, V, R, Vd, N - 1, mode,
                                      0.09, 0.3, acc, fake, fake, None, fake, None)

    assert call(logits=None) == 1 and call(acc=None) == 1 and call(B=0) == 1 and call(N=257) == 1
    assert call(mode=2) == 1 and call(mode=9) == 1                 # REJECT without drafts; bad mode
    assert call(mode=2, R=3, Vd=50, draft=fake, drow=fake) == 1     # Vd != V without t2d
    assert call(B=8, N=256, V=1_000_000) == 5


def test_tree_assemble_rows_argument_checks(lib):
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: every call below returns before a launch
    ws = lib.spec_tree_assemble_rows_workspace(4, 255, 32000)
    assert ws >= 4 * 4 * 255 * 12                        # per chunk and slot: a key and a NaN flag
    assert lib.spec_tree_assemble_rows_workspace(1, 10, 262145) == 0

    def call(d=fake, par=fake, row=fake, d2t=None, B=4, N=255, R=60, Vd=32000, V=32000, tok=fake, wsz=ws):
        return lib.spec_tree_assemble_rows(d, par, row, d2t, None, None, B, N, R, Vd, V, tok, fake, fake, fake,
                                           wsz, None)

    assert call(d=None) == 1 and call(par=None) == 1 and call(row=None) == 1 and call(tok=None) == 1
    assert call(B=0) == 1 and call(N=257) == 1 and call(R=0) == 1 and call(Vd=0) == 1
    assert call(V=128256) == 1                           # a larger target vocabulary needs d2t
    assert call(Vd=262145, V=262145) == 2
    assert call(wsz=ws - 1) == 3


# Checks that need no torch: run again against the host-sanitised build below.
HOST_CHECKS = ["test_every_declared_symbol_is_exported", "test_status_strings", "test_host_argument_checks",
               "test_kv_compact_host_checks", "test_workspace_sizes_are_monotone", "test_tree_select_argument_checks",
               "test_lm_head_stats_argument_checks", "test_verify_greedy_stats_argument_checks",
               "test_verify_lm_head_argument_checks", "test_status_strings_cover_every_code",
               "test_verify_static_host_checks", "test_tree_assemble_rows_argument_checks"]


def _host_check_script(path):
    return (
        "import sys\n"
        f"sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]\n"
        "from tree_attention_verification_spec_amd import abi\n"
        "import test_abi\n"
        f"L = abi.load({path!r})\n"
        f"for name in {HOST_CHECKS!r}:\n"
        "    getattr(test_abi, name)(L)\n"
        "for B in (1, 7, 16, 4096, 1 << 20, 2**31 - 1):\n"
        "    for N in (1, 63, 255, 256, 257, 2**31 - 1):\n"
        "        for V in (1, 4096, 128256, 2**31 - 1):\n"
        "            L.spec_verify_workspace(B, N, V); L.spec_verify_static_bytes(B, N, V)\n"
        "            L.spec_tree_attn_workspace(B, N, 32, 8, 128, V, 1); L.spec_tree_assemble_rows_workspace(B, N, V)\n"
        "            L.spec_lm_head_stats_workspace(B, N, 4096, V)\n"
        "            L.spec_medusa_heads_workspace(B, 4, 4096, V, 8)\n"
        "            for m in range(4): L.spec_verify_lm_head_workspace(B, N, 4096, V, m)\n"
        "assert L.spec_internal_tune(None, 1) == -1 and L.spec_internal_tune(b'attn_cb', -1) == 0\n"
        "print('HOST_CHECKS_OK')\n")


@pytest.mark.slow
@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="host-only check: on a machine with a GPU the HIP runtime maps more address "
                           "space at start-up than AddressSanitizer allows")
def test_host_checks_under_address_and_ub_sanitizers():
    """The host side of the C ABI (argument checks, workspace sizing including extreme sizes,
    status strings, the tuning setter) under AddressSanitizer + UndefinedBehaviorSanitizer: a
    build whose host pass is instrumented (device code unchanged), loaded in a child process
    with clang's ASan runtime preloaded.  Any report aborts the child."""
    import subprocess
    import sys
    from tree_attention_verification_spec_amd import asan_build
    path = asan_build.build()
    env = dict(os.environ, LD_PRELOAD=asan_build.runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", _host_check_script(path)], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "HOST_CHECKS_OK" in r.stdout, (r.returncode, r.stdout[-3000:], r.stderr[-6000:])
