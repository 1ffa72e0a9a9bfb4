"""Host-code exercises of libmoe_ep's C ABI, run by tests/test_host_asan.py in a
child process under AddressSanitizer (a host-instrumented build of the
library, the ASan runtime preloaded).

Only calls that return before any device work are made -- configuration and
argument checks, handle creation and destruction (the workspace pointer is
never dereferenced on the host), the CU-mask computation, the no-allocation
layout's size checks, status strings -- so the script is safe on a machine
with or without a GPU. It imports ctypes and the binding's declarations
only (not torch). Exits 0 after printing "asan host checks ok".
"""
import ctypes
import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
spec = importlib.util.spec_from_file_location(
    "moe_lib_decls", os.path.join(ROOT, "combine_moe_dispatch_02_amd", "_lib.py"))
decl = importlib.util.module_from_spec(spec)
spec.loader.exec_module(decl)

# The ASan runtime must be in the process (preloaded) for the checks to mean anything.
if not hasattr(ctypes.CDLL(None), "__asan_init"):
    raise SystemExit("the AddressSanitizer runtime is not loaded")
lib = decl.declare(ctypes.CDLL(sys.argv[1]))
Cfg = decl.MoeConfig
OK, INVALID, UNSUP, STATE = decl.MOE_OK, decl.MOE_ERR_INVALID_ARG, decl.MOE_ERR_UNSUPPORTED, decl.MOE_ERR_STATE
FAKE_WS = ctypes.c_void_p(1 << 40)   # a 256-byte-aligned address the host never dereferences


def expect(got, want, what):
    if got != want:
        raise SystemExit(f"{what}: status {got}, expected {want}: {lib.moe_last_error().decode()}")


# configurations: every check, and the long messages that name the fix
for cfg, want in [((4096, 7168, 8, 256, 8), OK), ((0, 8, 1, 1, 1), OK), ((16, 16392, 32, 1024, 8), OK),
                  ((-1, 256, 2, 8, 2), INVALID), ((8, 0, 2, 8, 2), INVALID), ((8, 12, 2, 8, 2), UNSUP),
                  ((8, 256, 2, 2000, 2), UNSUP), ((8, 256, 2, 10, 4), UNSUP), ((8, 256, 9, 8, 2), UNSUP),
                  ((8, 256, 33, 64, 8), UNSUP), ((8, 256, 0, 8, 2), INVALID), ((8, 256, 2, 8, 0), INVALID),
                  ((1 << 28, 8192, 8, 256, 8), UNSUP)]:
    c = Cfg(*cfg)
    n = lib.moe_workspace_bytes(ctypes.byref(c))
    if (n > 0) != (want == OK):
        raise SystemExit(f"workspace bytes {n} for {cfg}")
    for _ in range(50):   # create and destroy repeatedly: no leaks, no double frees
        h = ctypes.c_void_p()
        st = lib.moe_handle_create(ctypes.byref(c), FAKE_WS, max(n, 1 << 20) if n else 1 << 20,
                                   ctypes.byref(h))
        expect(st, want, f"create {cfg}")
        if st == OK:
            v = decl.MoeLayoutView()
            expect(lib.moe_layout_view(h, ctypes.byref(v)), STATE, "view before layout")
            expect(lib.moe_set_max_workgroups(h, -3), INVALID, "negative cap")
            expect(lib.moe_set_max_workgroups(h, 64), OK, "cap")
            expect(lib.moe_dispatch(h, FAKE_WS, 0, FAKE_WS, None, 1, None), STATE, "dispatch before layout")
            expect(lib.moe_combine(h, FAKE_WS, 1, FAKE_WS, FAKE_WS, None), STATE, "combine before layout")
            expect(lib.moe_dispatch_layout(h, FAKE_WS, cfg[0] + 1, None), INVALID, "too many tokens")
            lib.moe_handle_destroy(h)
lib.moe_handle_destroy(None)
small = Cfg(128, 256, 2, 8, 2)
expect(lib.moe_handle_create(ctypes.byref(small), FAKE_WS, 16, ctypes.byref(ctypes.c_void_p())),
       INVALID, "short workspace")
expect(lib.moe_handle_create(ctypes.byref(small), ctypes.c_void_p((1 << 40) + 8), 1 << 20,
                             ctypes.byref(ctypes.c_void_p())), INVALID, "misaligned workspace")
expect(lib.moe_handle_create(None, FAKE_WS, 1 << 20, ctypes.byref(ctypes.c_void_p())), INVALID, "NULL config")

# CU masks over every valid count, and the errors
for total in (256, 128, 512):
    words = (total + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for n in range(8, total + 1, 8):
        expect(lib.moe_cu_mask(total, n, mask, words), OK, f"cu mask {n}/{total}")
        if sum(bin(w).count("1") for w in mask) != n:
            raise SystemExit(f"cu mask {n}/{total} has the wrong bit count")
    expect(lib.moe_cu_mask(total, 12, mask, words), INVALID, "cu mask 12")
    expect(lib.moe_cu_mask(total, 64, mask, words - 1), INVALID, "cu mask short")
expect(lib.moe_cu_mask(256, 64, None, 8), INVALID, "cu mask NULL")
expect(lib.moe_stream_create_cu_limited(64, None), INVALID, "stream out NULL")

# the no-allocation layout: every check that comes before device work
p = FAKE_WS
args = [p] * 7
expect(lib.moe_dispatch_layout_noalloc(p, 300000, 8, 256, 8, *args, None), UNSUP, "noalloc oversized")
expect(lib.moe_dispatch_layout_noalloc(p, 100, 8, 250, 8, *args, None), UNSUP, "noalloc E % R")
expect(lib.moe_dispatch_layout_noalloc(p, -1, 8, 256, 8, *args, None), INVALID, "noalloc T < 0")
expect(lib.moe_dispatch_layout_noalloc(p, 100, 8, 256, 8, p, p, None, p, p, p, p, None), INVALID,
       "noalloc NULL counts")
expect(lib.moe_dispatch_layout_noalloc(None, 100, 8, 256, 8, *args, None), INVALID, "noalloc NULL ids")
expect(lib.moe_dispatch_layout_noalloc(ctypes.c_void_p((1 << 40) + 2), 100, 8, 256, 8, *args, None),
       INVALID, "noalloc misaligned")

for s in range(-1, 7):
    lib.moe_status_string(s)
print("asan host checks ok", flush=True)
