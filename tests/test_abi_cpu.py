"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/iqlher.h, and rejects bad arguments on the host before
any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iqlher.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|char|int64_t|int32_t|void)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


def test_every_declared_symbol_is_exported(m):
    names = declared_functions()
    assert len(names) >= 14, names
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_header_layout(m):
    assert ctypes.sizeof(m.IqlConfig) == 72
    assert ctypes.sizeof(m.HerConfig) == 32
    assert ctypes.sizeof(m.HerBuffer) == 72
    assert ctypes.sizeof(m.HerOut) == 80
    assert ctypes.sizeof(m.Adam) == 72
    assert ctypes.sizeof(m.HerStep) == 48
    assert ctypes.sizeof(m.BudgetStep) == 80


STRUCTS = {"iqlh_config": "IqlConfig", "her_config": "HerConfig", "her_buffer": "HerBuffer",
           "her_out": "HerOut", "iqlh_adam": "Adam", "iqlh_her_step": "HerStep",
           "iqlh_budget_step": "BudgetStep"}


def test_binding_structs_match_the_c_compiler(m, tmp_path):
    """Every field of every binding struct sits at the offset gcc gives it."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "iqlher.h"', "int main(void) {"]
    for c_name, py_name in STRUCTS.items():
        cls = getattr(m, py_name)
        lines.append(f'printf("{c_name} sizeof %zu\\n", sizeof({c_name}));')
        for f in cls._fields_:
            lines.append(f'printf("{c_name} {f[0]} %zu\\n", offsetof({c_name}, {f[0]}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for ln in out:
        if ln.strip():
            a, b, c = ln.split()
            got[(a, b)] = int(c)
    for c_name, py_name in STRUCTS.items():
        cls = getattr(m, py_name)
        assert got[(c_name, "sizeof")] == ctypes.sizeof(cls), c_name
        for f in cls._fields_:
            assert got[(c_name, f[0])] == getattr(cls, f[0]).offset, (c_name, f[0])


def test_num_params(m):
    assert m.iql_num_params(16, 32) == 1633
    assert m.iql_num_params(42, 128) == 22145
    assert m.iql_num_params(128, 128) == 33153
    assert m.iql_num_params(256, 512) == 394753
    with pytest.raises(m.IqlhError) as e:
        m.iql_num_params(0, 4)
    assert e.value.code == m.EINVAL


def test_workspace_bytes(m):
    b = m.grad_budget_workspace_bytes(132612, 4)
    assert b >= 5 * 4 and b % 4 == 0
    with pytest.raises(m.IqlhError):
        m.grad_budget_workspace_bytes(100, 9)
    with pytest.raises(m.IqlhError):
        m.grad_budget_workspace_bytes(0, 4)


@pytest.mark.parametrize("field,value,code", [
    ("num_groups", 3, -1), ("max_batch", 0, -1), ("states_ld", 5, -1), ("compute_dtype", 7, -1),
    ("hidden", 5000, -2), ("max_grad_norm", 0.0, -1), ("beta2", 1.0, -1), ("eps", 0.0, -1),
])
def test_create_rejects_bad_config_on_host(m, field, value, code):
    import numpy as np
    cfg = m.make_config(16, 32, 256, num_groups=1, compute_dtype=m.F32)
    setattr(cfg, field, value)
    with pytest.raises(m.IqlhError) as e:
        m.iql_create(cfg, np.zeros(m.iql_num_params(16, 32), np.float32))
    assert e.value.code == code
    assert m.last_error() != ""


def test_create_rejects_tau_outside_unit_interval(m):
    import numpy as np
    cfg = m.make_config(16, 32, 256, tau=(1.5,))
    with pytest.raises(m.IqlhError) as e:
        m.iql_create(cfg, np.zeros(1633, np.float32))
    assert "tau" in str(e.value)


def test_host_validation_of_kernel_entry_points(m):
    lib = ctypes.CDLL(m.LIB_PATH)
    # AW: bad action count / NULL pointers
    assert m._lib_iql_aw_policy(None, None, 1, 10, 9, 3.0, None, None) == m.EINVAL
    assert m._lib_iql_aw_policy(ctypes.c_void_p(16), ctypes.c_void_p(16), 1, 10, 65, 3.0,
                                ctypes.c_void_p(16), None) == m.EINVAL
    # HER: goal_dim > state_dim, unknown strategy, n < 0
    cfg = m.her_config(8, 9, m.HER_FUTURE)
    buf, out = m.HerBuffer(), m.HerOut()
    buf.capacity = buf.buffer_size = 10
    out.states_ld = 8
    rc = m._lib_her_relabel(ctypes.byref(cfg), ctypes.byref(buf), None, 4, 1, None, ctypes.byref(out), None)
    assert rc == m.EINVAL and "goal_dim" in m.last_error()
    cfg = m.her_config(8, 2, 5)
    rc = m._lib_her_relabel(ctypes.byref(cfg), ctypes.byref(buf), None, 4, 1, None, ctypes.byref(out), None)
    assert rc == m.EINVAL
    cfg = m.her_config(8, 2, m.HER_RANDOM)
    rc = m._lib_her_relabel(ctypes.byref(cfg), ctypes.byref(buf), None, -1, 1, None, ctypes.byref(out), None)
    assert rc == m.EINVAL
    # n == 0 is a no-op that touches nothing
    rc = m._lib_her_relabel(ctypes.byref(cfg), ctypes.byref(buf), None, 0, 1, None, ctypes.byref(out), None)
    assert rc == m.OK
    # final/future without episode ends
    cfg = m.her_config(8, 2, m.HER_FINAL)
    rc = m._lib_her_relabel(ctypes.byref(cfg), ctypes.byref(buf), None, 3, 1, None, ctypes.byref(out), None)
    assert rc == m.EINVAL
    # budget: too many sources, small workspace
    srcs = (ctypes.c_void_p * 9)(*([16] * 9))
    fr = (ctypes.c_float * 9)(*([0.1] * 9))
    rc = m._lib_budget(ctypes.c_void_p(16), srcs, fr, fr, 9, 100, 1.0, None, None, ctypes.c_void_p(16), 4096, None)
    assert rc == m.EINVAL
    rc = m._lib_budget(ctypes.c_void_p(16), srcs, fr, fr, 4, 100, 1.0, None, None, ctypes.c_void_p(16), 4, None)
    assert rc == m.EINVAL and "workspace" in m.last_error()
    # train step / whole step on a NULL handle
    assert m._lib_iql_train_step(None, None, None, 1, None, None, None, None) == m.EINVAL
    assert m._lib_iql_aux_step(None, None, None, None, 1, None, 0, 0.0, None, None, None, None, None,
                               None) == m.EINVAL
    assert m._lib_iql_aux_step_phase_stamps(None, None, None, None, 1, None, 0, 0.0, None, None, None, None, None,
                                            None, 0, None) == m.EINVAL
    assert m._lib_iql_step_counter(None) is None
    rows, floats = ctypes.c_int32(), ctypes.c_int64()
    assert m._lib_iql_partial_layout(None, 1, ctypes.byref(rows), ctypes.byref(floats)) == m.EINVAL
    # PER: outputs that overlap each other or the priorities (they hold the
    # draws' counter words between the launches)
    ws_bytes = m.per_workspace_bytes(100)
    for idx_at, w_at in ((1 << 20, (1 << 20) + 16), ((1 << 16) + 64, 1 << 24), (1 << 20, (1 << 16) + 128)):
        rc = m._lib_per_sample(ctypes.c_void_p(1 << 16), 100, 8, 1, None, 0.4, ctypes.c_void_p(idx_at),
                               ctypes.c_void_p(w_at), None, ctypes.c_void_p(1 << 28), ws_bytes, None)
        assert rc == m.EINVAL and "overlap" in m.last_error()


def test_binding_structs_keep_their_tensors(m):
    """The structs hold raw addresses; they must keep the tensors alive (a
    temporary freed after the call and released by the allocator would leave
    a captured launch reading unmapped memory)."""
    import gc
    import weakref
    import torch
    t = torch.zeros((8, 4))
    ref = weakref.ref(t)
    b = m.her_buffer(t, torch.zeros((8, 4)), None, None, torch.zeros(2, dtype=torch.int32))
    del t
    gc.collect()
    assert ref() is not None and b.states == ref().data_ptr()
    p = torch.zeros(16)
    ref = weakref.ref(p)
    a = m.make_adam(p, torch.zeros(16), torch.zeros(16), torch.zeros(1, dtype=torch.int32))
    del p
    gc.collect()
    assert ref() is not None and a.params == ref().data_ptr()
    g = torch.zeros(16)
    ref = weakref.ref(g)
    st = m.budget_step(g, [torch.zeros(16)], (1.0,), (1.0,), 16, 1.0, None, a, torch.zeros(64))
    del g
    gc.collect()
    assert ref() is not None and st.grad_buf == ref().data_ptr()
