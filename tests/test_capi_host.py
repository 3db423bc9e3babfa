"""Host-only checks of the C ABI (no GPU, no kernel launch): the library loads,
exports every function that include/bte.h declares, and rejects invalid
host-side arguments with the documented status codes before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bte.h")

bte = pytest.importorskip("block_token_eviction_amd")
lib = bte.lib
OK, NULL, DIM, UNSUP, ALIGN = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced on these paths
MIS = ctypes.c_void_p((1 << 20) + 2)     # misaligned


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bte_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) == 21
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    for s in (OK, NULL, DIM, UNSUP, ALIGN, -5, 7):
        assert bte.status_string(s)
    assert lib.bte_version() >= 100


def _focus(**kw):
    a = dict(q0=FAKE, k0=FAKE, q1=FAKE, k1=FAKE, dec=FAKE, out=FAKE, batch=2, block=32, hq=8,
             hkv=2, d=128, pool=7, dtype=1)
    a.update(kw)
    return lib.bte_focus_importance_delta(a["q0"], a["k0"], a["q1"], a["k1"], a["dec"], a["out"],
                                          a["batch"], a["block"], a["hq"], a["hkv"], a["d"],
                                          a["pool"], a["dtype"], None)


def test_focus_errors():
    assert _focus(q0=None) == NULL
    assert _focus(dec=None) == NULL
    assert _focus(batch=0) == DIM
    assert _focus(hq=6, hkv=4) == DIM
    assert _focus(block=0) == DIM
    assert _focus(block=65) == DIM             # blocks of 1..64 positions
    assert _focus(d=96) == UNSUP
    assert _focus(pool=4) == UNSUP
    assert _focus(pool=0) == UNSUP
    assert _focus(dtype=5) == UNSUP
    assert _focus(k1=MIS) == ALIGN


def test_esdllm_errors():
    f = lib.bte_esdllm_score
    assert f(None, FAKE, FAKE, FAKE, 0.5, FAKE, 1, 1, 1, 4096, 1, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, 0.5, FAKE, 0, 1, 1, 4096, 1, None) == DIM
    assert f(FAKE, FAKE, FAKE, FAKE, 0.5, FAKE, 1, 1, 1, 4100, 1, None) == UNSUP
    assert f(FAKE, FAKE, FAKE, FAKE, 0.5, FAKE, 1, 1, 1, 4096, 9, None) == UNSUP
    assert f(MIS, FAKE, FAKE, FAKE, 0.5, FAKE, 1, 1, 1, 4096, 1, None) == ALIGN


def test_topk_errors():
    f = lib.bte_topk_select
    assert f(None, FAKE, FAKE, FAKE, FAKE, 1, 32, 8, None) == NULL
    assert f(FAKE, FAKE, None, FAKE, FAKE, 1, 32, 8, None) == NULL      # idx needed when k_max > 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, 8, None) == DIM
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 8, None) == DIM
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1025, 8, None) == DIM
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 32, -1, None) == DIM


def test_rows_errors():
    g = lib.bte_gather_rows
    assert g(None, FAKE, FAKE, FAKE, FAKE, 1, 32, 8, 8192, None) == NULL
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, 8, 8192, None) == DIM
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 32, 8, 8190, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, MIS, 1, 32, 8, 8192, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 32, 0, 8192, None) == OK   # nothing to do
    s = lib.bte_kv_scatter
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None, 1, 8, 2048, None) == NULL
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, FAKE, 1, 8, 2048, None) == NULL
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1, 8, 2048, None) == DIM
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, FAKE, 1, 8, 2040, None) == ALIGN
    assert s(FAKE, None, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None, 1, 0, 2048, None) == OK


def test_attention_errors():
    f = lib.bte_reduced_attention
    # q, count, cu, cache_k, cache_v, seq_start, kv_len, order, out, batch, k_max, hq, hkv,
    # head_dim, scale, dtype, stream
    args = [FAKE] * 9 + [4, 8, 32, 8, 128, 0.088, 1, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == NULL
    assert call(a8=None) == NULL
    assert call(a9=0) == DIM
    assert call(a10=-1) == DIM
    assert call(a11=30) == DIM
    assert call(a14=0.0) == DIM
    assert call(a14=-0.1) == DIM
    assert call(a14=float("inf")) == DIM
    assert call(a14=float("nan")) == DIM
    assert call(a13=96) == UNSUP
    assert call(a15=3) == UNSUP
    assert call(a3=MIS) == ALIGN
    assert call(a10=0) == OK                  # nothing kept: no launch
    assert call(a7=None, a10=0) == OK         # the order is optional
    assert call(a10=1 << 18) == DIM           # 2^18 * 32 heads * 256 B = 2^31 output bytes


def test_scatter_attention_errors():
    f = lib.bte_kv_scatter_attention
    # q, count, cu, idx, n, pos_base, new_k, new_v, cache_k, cache_v, seq_start, kv_len, order,
    # out, batch, k_max, hq, hkv, head_dim, scale, dtype, stream
    args = [FAKE] * 4 + [32] + [FAKE] * 9 + [4, 8, 32, 8, 128, 0.088, 1, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a3=None) == NULL             # idx
    assert call(a5=None) == NULL             # pos_base
    assert call(a6=None) == NULL             # new_k
    assert call(a10=None) == NULL            # seq_start
    assert call(a4=0) == DIM
    assert call(a4=65) == UNSUP
    assert call(a11=None) == NULL            # kv_len
    assert call(a17=3) == DIM                # hq % hkv
    assert call(a18=96) == UNSUP
    assert call(a7=MIS) == ALIGN             # new_v
    assert call(a8=MIS) == ALIGN             # cache_k
    assert call(a15=0) == OK                 # nothing kept: no launch
    g = lib.bte_kv_scatter_attention_paged
    # q, count, cu, idx, n, pos_base, new_k, new_v, ck, cv, block_table, max_pages, page_size,
    # kv_len, order, out, batch, k_max, hq, hkv, head_dim, scale, dtype, stream
    pargs = [FAKE] * 4 + [32] + [FAKE] * 6 + [4, 64] + [FAKE] * 3 + [4, 8, 32, 8, 128, 0.088, 1,
                                                                       None]

    def pcall(**kw):
        a = list(pargs)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return g(*a)
    assert pcall(a10=None) == NULL           # block_table
    assert pcall(a3=None) == NULL
    assert pcall(a4=65) == UNSUP
    assert pcall(a11=0) == DIM
    assert pcall(a12=48) == UNSUP
    assert pcall(a6=MIS) == ALIGN
    assert pcall(a17=0) == OK


def test_attention_order_errors():
    f = lib.bte_attention_order
    # kv_len, count, group, batch, order_out, stream
    assert f(None, None, 1, 4, FAKE, None) == NULL
    assert f(FAKE, None, 1, 4, None, None) == NULL
    assert f(FAKE, None, 1, 0, FAKE, None) == DIM
    assert f(FAKE, None, 1, 16385, FAKE, None) == DIM
    assert f(FAKE, FAKE, 0, 4, FAKE, None) == DIM         # a count needs group >= 1


def test_budget_select_errors():
    f = lib.bte_focus_budget
    assert f(None, FAKE, FAKE, 1.5, 0, FAKE, 4, 32, None) == NULL
    assert f(FAKE, FAKE, FAKE, 1.5, 0, FAKE, 0, 32, None) == DIM
    assert f(FAKE, FAKE, FAKE, 1.5, 0, FAKE, 4, 0, None) == DIM
    assert f(FAKE, FAKE, FAKE, -1.0, 0, FAKE, 4, 32, None) == DIM
    assert f(FAKE, FAKE, FAKE, float("nan"), 0, FAKE, 4, 32, None) == DIM
    assert f(FAKE, FAKE, FAKE, 1.5, 2, FAKE, 4, 32, None) == DIM
    h = lib.bte_focus_history_update
    assert h(FAKE, None, FAKE, FAKE, 4, 32, None) == NULL
    assert h(FAKE, FAKE, FAKE, FAKE, 4, 0, None) == DIM
    s = lib.bte_focus_select
    assert s(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4, 32, None) == NULL
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, None) == DIM
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 65, None) == UNSUP


def test_paged_errors():
    f = lib.bte_reduced_attention_paged
    # q, count, cu, ck, cv, block_table, max_pages, page_size, kv_len, order, out, batch, k_max,
    # hq, hkv, head_dim, scale, dtype, stream
    args = [FAKE] * 6 + [4, 64] + [FAKE] * 3 + [4, 8, 32, 8, 128, 0.088, 1, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a5=None) == NULL
    assert call(a0=None) == NULL
    assert call(a6=0) == DIM
    assert call(a7=48) == UNSUP
    assert call(a7=4) == UNSUP
    assert call(a16=0.0) == DIM
    assert call(a12=0) == OK
    s = lib.bte_kv_scatter_paged
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, 4, 16, FAKE, FAKE, 2, 8, 2048, None) == NULL
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, 0, 16, FAKE, FAKE, 2, 8, 2048, None) == DIM
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, 4, 12, FAKE, FAKE, 2, 8, 2048, None) == UNSUP
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, 4, 16, FAKE, FAKE, 2, 0, 2048, None) == OK


def test_commit_and_multi_errors():
    f = lib.bte_focus_commit_mask
    assert f(None, FAKE, FAKE, None, 4, 32, None) == NULL
    assert f(FAKE, FAKE, FAKE, None, 0, 32, None) == DIM
    assert f(FAKE, FAKE, FAKE, None, 4, 2000, None) == DIM
    g = lib.bte_gather_rows_multi
    T = bte._RowsTensor
    ok = (T * 2)(T(1 << 20, 1 << 21, 8192), T(1 << 22, 1 << 23, 4))
    assert g(None, 2, FAKE, FAKE, FAKE, 4, 32, 8, None) == NULL
    assert g(ctypes.cast(ok, ctypes.c_void_p), 0, FAKE, FAKE, FAKE, 4, 32, 8, None) == DIM
    assert g(ctypes.cast(ok, ctypes.c_void_p), 9, FAKE, FAKE, FAKE, 4, 32, 8, None) == DIM
    bad = (T * 1)(T(1 << 20, 1 << 21, 6))
    assert g(ctypes.cast(bad, ctypes.c_void_p), 1, FAKE, FAKE, FAKE, 4, 32, 8, None) == ALIGN
    nul = (T * 1)(T(None, 1 << 21, 8))
    assert g(ctypes.cast(nul, ctypes.c_void_p), 1, FAKE, FAKE, FAKE, 4, 32, 8, None) == NULL
    assert g(ctypes.cast(ok, ctypes.c_void_p), 2, FAKE, FAKE, FAKE, 4, 32, 0, None) == OK


def test_esdllm_score_update_errors():
    f = lib.bte_esdllm_score_update
    a = [FAKE, FAKE, FAKE, None, None, FAKE, ctypes.c_float(0.5), FAKE, 1, 4, 8, 4096, 1, None]
    call = lambda **kw: f(*[kw.get(f"a{i}", v) for i, v in enumerate(a)])
    assert call(a0=None) == NULL
    assert call(a1=None) == NULL
    assert call(a3=FAKE) == NULL              # count without cu
    assert call(a4=FAKE) == NULL              # cu without count
    assert call(a8=0) == DIM
    assert call(a9=0) == DIM
    assert call(a11=4100) == UNSUP
    assert call(a12=7) == UNSUP
    assert call(a1=MIS) == ALIGN


def test_esdllm_schedule_errors():
    f = lib.bte_esdllm_schedule
    keep = (ctypes.c_int32 * 3)(128, 64, 80)
    kp = ctypes.cast(keep, ctypes.c_void_p)
    a = [FAKE, FAKE, 256, 3, kp, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None]
    call = lambda **kw: f(*[kw.get(f"a{i}", v) for i, v in enumerate(a)])
    assert call(a0=None) == NULL
    assert call(a4=None) == NULL              # keep counts needed with n_layers > 0
    assert call(a9=None) == NULL
    assert call(a11=0) == DIM
    assert call(a2=0) == DIM
    assert call(a3=-1) == DIM
    assert call(a5=9) == DIM                  # more than BTE_ES_MAX_SKIP_LAYERS
    assert call(a5=3) == DIM                  # keep[2] = 80 > keep[1] = 64
    big = (ctypes.c_int32 * 1)(300)
    assert call(a4=ctypes.cast(big, ctypes.c_void_p), a5=1) == DIM   # keep > block_len
    assert call(a2=1 << 20, a11=1 << 12) == DIM                      # batch * block >= 2^31


def test_gather_rows_multi_ragged_errors():
    f = lib.bte_gather_rows_multi_ragged
    ok = (bte._RowsTensor * 1)(bte._RowsTensor(1 << 20, 1 << 21, 8192))
    arr = ctypes.cast(ok, ctypes.c_void_p)
    assert f(arr, 1, None, FAKE, FAKE, FAKE, 4, 8, None) == NULL
    assert f(arr, 0, FAKE, FAKE, FAKE, FAKE, 4, 8, None) == DIM
    assert f(arr, 1, FAKE, FAKE, FAKE, FAKE, 0, 8, None) == DIM


def test_header_is_plain_c_and_links(tmp_path):
    """include/bte.h compiles as C99 on its own (gcc, no C++ and no torch), every declared
    entry point links against libbte.so, and a C caller gets the documented host-side
    status codes without a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not installed")
    names = declared()
    src = tmp_path / "caller.c"
    src.write_text(
        "#include <stdio.h>\n#include \"bte.h\"\n"
        "int main(void) {\n"
        "  void* const entry[] = {\n" + "".join(f"    (void*){n},\n" for n in names) + "  };\n"
        "  size_t i;\n"
        "  for (i = 0; i < sizeof(entry) / sizeof(entry[0]); ++i) if (!entry[i]) return 10;\n"
        "  if (bte_version() < 100) return 11;\n"
        "  if (bte_topk_select(NULL, NULL, NULL, NULL, NULL, 1, 1, 1, NULL) != BTE_ERR_NULL) return 12;\n"
        "  if (bte_esdllm_score((void*)16, (void*)16, (int32_t*)16, (float*)16, 0.5f, (float*)16,\n"
        "                       0, 1, 1, 8, BTE_BF16, NULL) != BTE_ERR_DIM) return 13;\n"
        "  printf(\"%s\\n\", bte_status_string(BTE_ERR_DIM));\n"
        "  return 0;\n}\n")
    libdir = os.path.join(ROOT, "block_token_eviction_amd")
    exe = tmp_path / "caller"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           str(src), "-L", libdir, "-lbte", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    assert r.stdout.strip() == bte.status_string(DIM)
