"""CPU-only checks of the C ABI (no kernel is launched; nothing here needs a GPU):

* libmp.so loads and exports every function include/mp.h declares;
* the ctypes mirror of mp_graph matches the C layout (sizeof / offsetof by gcc);
* host-side validation rejects bad arguments before any HIP call;
* the forward / input-gradient kernels contain no atomic instruction (scan of
  the disassembled gfx950 code of spmm.hip in the libmp.so built here);
* the product package never imports the oracle.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mp.h")
PKG = os.path.join(ROOT, "gnn_sparse_message_amd")
LIB = os.path.join(PKG, "libmp.so")


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mp_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("mp_graph_build", "mp_graph_build_workspace_size", "mp_spmm_fwd",
                     "mp_spmm_dx", "mp_edge_grad_dw", "mp_spmm_dx_edge_grad", "mp_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(mp):
    lib = ctypes.CDLL(mp.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mp.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(mp_\w+)", out))
    assert set(declared_functions()) <= exported


def test_graph_struct_layout_matches_ctypes(mp, tmp_path):
    fields = [f for f, _ in mp._MpGraph._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "mp.h"', "int main(void) {",
            'printf("%zu\\n", sizeof(mp_graph));']
    prog += [f'printf("%zu\\n", offsetof(mp_graph, {f}));' for f in fields]
    prog += ["return 0; }"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(mp._MpGraph)
    for f, off in zip(fields, vals[1:]):
        assert getattr(mp._MpGraph, f).offset == off, f


def _header_defines():
    text = open(HEADER).read()
    return {k: int(v.rstrip("ull"), 0) for k, v in
            re.findall(r"^#define\s+(MP_\w+)\s+\(?(-?(?:0x[0-9a-fA-F]+|\d+)(?:ull)?)\)?", text, re.M)}


def test_binding_constants_match_header(mp):
    d = _header_defines()
    assert d["MP_GRAPH_INFO_WORDS"] == mp.GRAPH_INFO_WORDS
    assert d["MP_GRAPH_BUILT"] == mp.GRAPH_BUILT
    assert d["MP_GRAPH_ON_DEVICE"] == mp.GRAPH_ON_DEVICE
    assert d["MP_NUM_CLASSES"] == mp.NUM_CLASSES
    for name in ("MP_ERR_NULL", "MP_ERR_SHAPE", "MP_ERR_INDEX", "MP_ERR_GRAPH", "MP_F32",
                 "MP_BF16", "MP_I32", "MP_I64", "MP_NORM_MEAN", "MP_NORM_SYM"):
        assert d[name] == getattr(mp, name), name


def test_finish_rejects_unbuilt_graph(mp):
    lib = mp._lib
    g = _fake_graph(mp, 10, 20)
    assert lib.mp_graph_finish(None, None) == mp.MP_ERR_NULL
    assert lib.mp_graph_finish(ctypes.byref(g), None) == mp.MP_ERR_GRAPH
    g.built = mp.GRAPH_BUILT               # an already finished graph is left as it is
    assert lib.mp_graph_finish(ctypes.byref(g), None) == mp.MP_OK


def test_status_strings(mp):
    for code in range(0, -11, -1):
        s = mp.mp_status_string(code)
        assert s.startswith("MP_OK" if code == 0 else "MP_ERR_"), (code, s)
    assert "unknown" in mp.mp_status_string(-99)


def test_workspace_size_validation(mp):
    lib = mp._lib
    out = ctypes.c_size_t(0)
    assert lib.mp_graph_build_workspace_size(0, 10, ctypes.byref(out)) == mp.MP_ERR_SHAPE
    assert lib.mp_graph_build_workspace_size(10, -1, ctypes.byref(out)) == mp.MP_ERR_SHAPE
    assert lib.mp_graph_build_workspace_size(1 << 31, 1, ctypes.byref(out)) == mp.MP_ERR_SHAPE
    assert lib.mp_graph_build_workspace_size(10, 10, None) == mp.MP_ERR_NULL
    assert lib.mp_graph_build_workspace_size(2_000_000, 100_000_000, ctypes.byref(out)) == 0
    assert out.value >= 16 * 100_000_000          # four [E] u32 sort buffers
    assert out.value < 17 * 100_000_000           # O(N + E): no [E, H] buffer


def _fake_graph(mp, n, e, base=0x10000):
    g = mp._MpGraph()
    g.num_nodes, g.num_edges = n, e
    for i, f in enumerate(mp.Graph._ARRAYS):
        setattr(g, f, base + i * 0x100000)
    g.info = base + len(mp.Graph._ARRAYS) * 0x100000
    return g


def test_build_rejects_before_any_device_call(mp):
    lib = mp._lib
    g = _fake_graph(mp, 10, 20)
    fake_src, fake_dst = 0x9000000, 0xA000000
    ws_need = mp.mp_graph_build_workspace_size(10, 20)
    assert lib.mp_graph_build(fake_src, fake_dst, mp.MP_I64, 10, 20, None, 0x100, ws_need, None) \
        == mp.MP_ERR_NULL
    assert lib.mp_graph_build(fake_src, fake_dst, 7, 10, 20, ctypes.byref(g), 0x100, ws_need,
                              None) == mp.MP_ERR_DTYPE
    assert lib.mp_graph_build(fake_src, fake_dst, mp.MP_I64, 0, 20, ctypes.byref(g), 0x100,
                              ws_need, None) == mp.MP_ERR_SHAPE
    assert lib.mp_graph_build(None, fake_dst, mp.MP_I64, 10, 20, ctypes.byref(g), 0x100, ws_need,
                              None) == mp.MP_ERR_NULL
    assert lib.mp_graph_build(fake_src, fake_dst, mp.MP_I64, 10, 20, ctypes.byref(g), None,
                              ws_need, None) == mp.MP_ERR_WORKSPACE
    assert lib.mp_graph_build(fake_src, fake_dst, mp.MP_I64, 10, 20, ctypes.byref(g), 0x100,
                              ws_need - 1, None) == mp.MP_ERR_WORKSPACE
    assert lib.mp_graph_build(fake_src, fake_dst, mp.MP_I64, 10, 20, ctypes.byref(g), 0x104,
                              ws_need, None) == mp.MP_ERR_ALIGN
    g.col = None
    assert lib.mp_graph_build(fake_src, fake_dst, mp.MP_I64, 10, 20, ctypes.byref(g), 0x100,
                              ws_need, None) == mp.MP_ERR_NULL
    g.col = 0x20002
    assert lib.mp_graph_build(fake_src, fake_dst, mp.MP_I64, 10, 20, ctypes.byref(g), 0x100,
                              ws_need, None) == mp.MP_ERR_ALIGN
    assert g.built == 0
    assert "aligned" in lib.mp_last_error_detail().decode()


def test_compute_calls_reject_unbuilt_graphs(mp):
    lib = mp._lib
    g = _fake_graph(mp, 10, 20)
    for fn in (lib.mp_spmm_fwd, lib.mp_spmm_dx):
        assert fn(None, 0x100, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_NULL
        assert fn(ctypes.byref(g), 0x100, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_GRAPH
    assert lib.mp_edge_grad_dw(None, 0x100, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_NULL
    assert lib.mp_edge_grad_dw(ctypes.byref(g), 0x100, 0x200, mp.MP_F32, 4, 0x300, None) \
        == mp.MP_ERR_GRAPH
    fused = lib.mp_spmm_dx_edge_grad
    assert fused(None, 0x100, 0x200, 0x300, mp.MP_F32, 4, 0x400, 0x500, None) == mp.MP_ERR_NULL
    assert fused(ctypes.byref(g), 0x100, 0x200, 0x300, mp.MP_F32, 4, 0x400, 0x500, None) \
        == mp.MP_ERR_GRAPH
    for fn in (lib.mp_spmm_fwd_heads, lib.mp_spmm_dx_heads):
        assert fn(None, 0x100, 2, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_NULL
        assert fn(ctypes.byref(g), 0x100, 2, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_GRAPH
    dwh = lib.mp_edge_grad_dw_heads
    assert dwh(None, 0x100, 0x200, mp.MP_F32, 4, 2, 0x300, None) == mp.MP_ERR_NULL
    assert dwh(ctypes.byref(g), 0x100, 0x200, mp.MP_F32, 4, 2, 0x300, None) == mp.MP_ERR_GRAPH
    fh = lib.mp_spmm_dx_edge_grad_heads
    assert fh(None, 0x100, 2, 0x200, 0x300, mp.MP_F32, 4, 0x400, 0x500, None) == mp.MP_ERR_NULL
    assert fh(ctypes.byref(g), 0x100, 2, 0x200, 0x300, mp.MP_F32, 4, 0x400, 0x500, None) \
        == mp.MP_ERR_GRAPH
    for fn in (lib.mp_spmm_fwd_norm, lib.mp_spmm_dx_norm):
        assert fn(None, 1, 0x100, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_NULL
        assert fn(ctypes.byref(g), 2, 0x100, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_GRAPH
        assert fn(ctypes.byref(g), 9, 0x100, 0x200, mp.MP_F32, 4, 0x300, None) == mp.MP_ERR_DTYPE
    fn = lib.mp_spmm_dx_edge_grad_norm
    assert fn(None, 1, 0x100, 0x200, 0x300, mp.MP_F32, 4, 0x400, 0x500, None) == mp.MP_ERR_NULL
    assert fn(ctypes.byref(g), 1, 0x100, 0x200, 0x300, mp.MP_F32, 4, 0x400, 0x500, None) \
        == mp.MP_ERR_GRAPH
    fs = lib.mp_spmm_fwd_softmax
    assert fs(None, 0x100, 0x200, mp.MP_F32, 4, 0x300, 0x400, None) == mp.MP_ERR_NULL
    assert fs(ctypes.byref(g), 0x100, 0x200, mp.MP_F32, 4, 0x300, 0x400, None) == mp.MP_ERR_GRAPH
    ab = lib.mp_attention_backward
    args = (0x100, 2, 0x200, 0x300, 0x380, mp.MP_F32, 4, 0x400, 0x500, 0x600, None)
    assert ab(None, *args) == mp.MP_ERR_NULL
    assert ab(ctypes.byref(g), *args) == mp.MP_ERR_GRAPH
    abs_ = lib.mp_attention_backward_scores
    args = (0x100, 0x180, 0x200, 0x300, 0x380, mp.MP_F32, 4, 0x400, 0x500, 0x600, None)
    assert abs_(None, *args) == mp.MP_ERR_NULL
    assert abs_(ctypes.byref(g), *args) == mp.MP_ERR_GRAPH
    assert abs_(ctypes.byref(g), 0x100, None, *args[2:]) == mp.MP_ERR_NULL


def _device_disassembly(tmp_path):
    """The gfx950 disassembly of every code object in the built libmp.so: its
    .hip_fatbin section holds one offload bundle per source file, each
    unbundled for the gfx950 target and disassembled with llvm-objdump.
    Returns a list of texts, one per source file."""
    llvm = "/opt/rocm/llvm/bin"
    fat = tmp_path / "fat.bin"
    subprocess.run([f"{llvm}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", LIB,
                    str(tmp_path / "lib.copy")], check=True, capture_output=True)
    data = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    assert starts and starts[0] == 0, "no offload bundle in the library"
    texts = []
    for k, s0 in enumerate(starts):
        end = starts[k + 1] if k + 1 < len(starts) else len(data)
        bundle, code = tmp_path / f"b{k}.bin", tmp_path / f"b{k}.co"
        bundle.write_bytes(data[s0:end])
        subprocess.run([f"{llvm}/clang-offload-bundler", "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={bundle}",
                        f"--output={code}"], check=True, capture_output=True)
        out = subprocess.run([f"{llvm}/llvm-objdump", "-d", "--mcpu=gfx950", str(code)],
                             check=True, capture_output=True, text=True).stdout
        texts.append(out)
    return texts


def test_forward_and_input_grad_kernels_have_no_atomics(tmp_path):
    """Scan the gfx950 code of spmm.hip, as built into libmp.so here, for atomic
    instructions (the aggregations own each output row: no atomics)."""
    texts = [t for t in _device_disassembly(tmp_path) if re.search(r"<_Z\w*spmm_kernel", t)]
    assert len(texts) == 1, "the aggregation kernels are in one source file"
    text = texts[0]
    kernels = re.findall(r"^[0-9a-f]+ <(_Z\w*spmm_kernel\w*)>:$", text, re.M)
    assert len(kernels) >= 84                       # 2 dtypes x 2 widths x 7 lane counts x 3 modes
    insts = [ln for ln in text.splitlines() if re.match(r"\s+[a-z_0-9]*atomic", ln)]
    assert not insts, insts[:5]
    assert "global_load_dwordx4" in text            # 16-byte feature-row loads are emitted


def test_product_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle.c" not in text and "liboracle" not in text, f


def test_build_script_loads_without_the_library():
    """build() must work on a fresh tree, where the package cannot be imported yet
    (it loads libmp.so at import): the build script is loaded by path."""
    code = ("import sys, __graft_entry__ as ge\n"
            "m = ge._build_module()\n"
            "assert callable(m.build) and m.ARCH == 'gfx950'\n"
            "assert 'gnn_sparse_message_amd' not in sys.modules\n")
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True)
