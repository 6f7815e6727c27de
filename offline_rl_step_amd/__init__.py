"""Python binding of libiqlher.so, the MI355X IQL + HER step.

Argument marshalling only: every function forwards to the C entry point of
the same name in ``include/iqlher.h``; tensors are passed by ``data_ptr()``
and the work is enqueued on torch's current HIP stream.  There is no CPU or
PyTorch fallback: importing this module fails loudly when the library has not
been built (``python offline_rl_step_amd/build.py``).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libiqlher.so")

# torch owns device memory and streams; importing it first makes the library
# bind to the same HIP runtime instance.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python offline_rl_step_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, ESHAPE, ENOMEM, EHIP, ENONFINITE = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
HER_FINAL, HER_FUTURE, HER_RANDOM = 0, 1, 2
FLAG_NONFINITE_GRAD, FLAG_BAD_INDEX, FLAG_NONFINITE_LOSS, FLAG_NONFINITE_STATE = 0x1, 0x2, 0x4, 0x8
MAX_SOURCES = 8

_p = ctypes.c_void_p
_i32, _i64, _u64, _f = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float


class IqlConfig(ctypes.Structure):
    _fields_ = [("state_dim", _i32), ("hidden", _i32), ("max_batch", _i32), ("num_groups", _i32),
                ("compute_dtype", _i32), ("hidden2", _i32), ("states_ld", _i64),
                ("tau", _f * 2), ("lr", _f), ("beta1", _f), ("beta2", _f), ("eps", _f),
                ("weight_decay", _f), ("max_grad_norm", _f), ("weight_clamp_max_abs", _f)]


class HerConfig(ctypes.Structure):
    _fields_ = [("state_dim", _i32), ("goal_dim", _i32), ("strategy", _i32), ("reserved0", _i32),
                ("goal_threshold", _f), ("reward_hit", _f), ("reward_miss", _f), ("reserved1", _f)]


class HerBuffer(ctypes.Structure):
    _fields_ = [("states", _p), ("next_states", _p), ("actions", _p), ("rewards", _p), ("dones", _p),
                ("episode_ends", _p), ("capacity", _i64), ("buffer_size", _i64),
                ("num_episodes", _i32), ("reserved0", _i32)]


class HerOut(ctypes.Structure):
    _fields_ = [("donor_idx", _p), ("states", _p), ("states_dtype", _i32), ("reserved0", _i32),
                ("states_ld", _i64), ("next_states", _p), ("actions", _p), ("rewards", _p),
                ("dones", _p), ("d_flags", _p), ("is_weights", _p)]


class Adam(ctypes.Structure):
    _fields_ = [("params", _p), ("m", _p), ("v", _p), ("t", _p), ("d_flags", _p),
                ("lr", _f), ("beta1", _f), ("beta2", _f), ("eps", _f), ("weight_decay", _f),
                ("max_grad_norm", _f), ("weight_clamp_max_abs", _f), ("reserved0", _f)]


class HerStep(ctypes.Structure):
    _fields_ = [("cfg", ctypes.POINTER(HerConfig)), ("buf", ctypes.POINTER(HerBuffer)), ("source_idx", _p),
                ("out", ctypes.POINTER(HerOut)), ("seed", _u64), ("n", _i32), ("reserved0", _i32)]


class BudgetStep(ctypes.Structure):
    _fields_ = [("grad_buf", _p), ("sources", ctypes.POINTER(_p)), ("fractions", ctypes.POINTER(_f)),
                ("alphas", ctypes.POINTER(_f)), ("out_norms", _p), ("adam", ctypes.POINTER(Adam)),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t), ("n", _i64), ("num_sources", _i32),
                ("max_grad_norm", _f)]


def _sig(name, res, args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = args
    return fn


_lib_iql_num_params = _sig("iql_num_params", _i32, [_i32, _i32, ctypes.POINTER(_i64)])
_lib_iql_config_num_params = _sig("iql_config_num_params", _i32, [ctypes.POINTER(IqlConfig), ctypes.POINTER(_i64)])
_lib_iql_create = _sig("iql_create", _i32, [ctypes.POINTER(IqlConfig), _p, ctypes.POINTER(_p)])
_lib_iql_destroy = _sig("iql_destroy", _i32, [_p])
_lib_iql_train_step = _sig("iql_train_step", _i32, [_p, _p, _p, _i32, _p, _p, _p, _p])
_lib_iql_train_step_aw = _sig("iql_train_step_aw", _i32, [_p, _p, _p, _i32, _p, _i32, _f, _p, _p, _p, _p, _p])
_lib_iql_compute_gradients = _sig("iql_compute_gradients", _i32, [_p, _p, _p, _i32, _p, _p])
_lib_iql_apply_gradients = _sig("iql_apply_gradients", _i32, [_p, _i32, _p, _p, _p])
_lib_iql_time_cg = _sig("iql_time_compute_gradients", _i32, [_p, _p, _p, _i32, _i32, ctypes.POINTER(_f), _p])
_lib_iql_partial_layout = _sig("iql_partial_layout", _i32, [_p, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i64)])
_lib_iql_get_state = _sig("iql_get_state", _i32, [_p, _i32, _p, _p, _p, _p, _p])
_lib_iql_set_state = _sig("iql_set_state", _i32, [_p, _i32, _p, _p, _p, _p, _p])
_lib_iql_forward_values = _sig("iql_forward_values", _i32, [_p, _p, _i32, _i64, _i32, _p, _p, _p, _f, _p, _p])
_lib_iql_target_ema_update = _sig("iql_target_ema_update", _i32, [_p, _f, _p])
_lib_iql_set_target_ema = _sig("iql_set_target_ema", _i32, [_p, _f])
_lib_iql_get_target = _sig("iql_get_target", _i32, [_p, _i32, _p, _p])
_lib_iql_set_target = _sig("iql_set_target", _i32, [_p, _i32, _p, _p])
_lib_iql_step_counter = _sig("iql_step_counter", _p, [_p])
_lib_iql_flags = _sig("iql_flags", _p, [_p])
_lib_iql_status = _sig("iql_status", _i32, [_p, ctypes.POINTER(_i32)])
_lib_iql_aw_policy = _sig("iql_aw_policy", _i32, [_p, _p, _i32, _i32, _i32, _f, _p, _p])
_lib_her_relabel = _sig("her_relabel", _i32, [ctypes.POINTER(HerConfig), ctypes.POINTER(HerBuffer), _p, _i32,
                                              _u64, _p, ctypes.POINTER(HerOut), _p])
_lib_ws_bytes = _sig("grad_budget_workspace_bytes", _i32, [_i64, _i32, ctypes.POINTER(ctypes.c_size_t)])
_lib_budget = _sig("grad_budget_accumulate", _i32, [_p, ctypes.POINTER(_p), ctypes.POINTER(_f),
                                                    ctypes.POINTER(_f), _i32, _i64, _f, _p,
                                                    ctypes.POINTER(Adam), _p, ctypes.c_size_t, _p])
_lib_budget_noalloc = _sig("grad_budget_accumulate_noalloc", _i32, [_p, ctypes.POINTER(_p), ctypes.POINTER(_f),
                                                                    ctypes.POINTER(_f), _i32, _i64, _f, _p,
                                                                    ctypes.POINTER(Adam), _p])
_lib_iql_aux_step = _sig("iql_aux_step", _i32, [_p, ctypes.POINTER(HerStep), _p, _p, _i32, _p, _i32, _f, _p, _p,
                                                _p, _p, ctypes.POINTER(BudgetStep), _p])
_lib_iql_time_aux_step = _sig("iql_time_aux_step", _i32, [_p, ctypes.POINTER(HerStep), _p, _p, _i32, _p, _i32, _f,
                                                          _p, _p, _p, _p, ctypes.POINTER(BudgetStep), _i32,
                                                          ctypes.POINTER(_f), _p])
_lib_iql_aux_step_phase_stamps = _sig("iql_aux_step_phase_stamps", _i32,
                                      [_p, ctypes.POINTER(HerStep), _p, _p, _i32, _p, _i32, _f, _p, _p, _p, _p,
                                       ctypes.POINTER(BudgetStep), _p, _i32, _p])
_lib_per_ws = _sig("per_workspace_bytes", _i32, [_i64, ctypes.POINTER(ctypes.c_size_t)])
_lib_per_sample = _sig("per_sample_indices", _i32, [_p, _i64, _i32, _u64, _p, _f, _p, _p, _p, _p, ctypes.c_size_t, _p])
_lib_nonfinite_check = _sig("iqlh_nonfinite_check", _i32, [ctypes.POINTER(_p), ctypes.POINTER(_i64), _i32, _p, _p])
_lib_last_error = _sig("iqlh_last_error", ctypes.c_char_p, [])


class IqlhError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        msg = _lib_last_error().decode(errors="replace")
        super().__init__(f"{where} failed with status {code}: {msg}")


def _check(code, where):
    if code != OK:
        raise IqlhError(code, where)
    return code


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def last_error():
    return _lib_last_error().decode(errors="replace")


# ------------------------------------------------------------------- IQL
def iql_num_params(state_dim, hidden):
    out = _i64()
    _check(_lib_iql_num_params(state_dim, hidden, ctypes.byref(out)), "iql_num_params")
    return out.value


def iql_config_num_params(cfg):
    out = _i64()
    _check(_lib_iql_config_num_params(ctypes.byref(cfg), ctypes.byref(out)), "iql_config_num_params")
    return out.value


def make_config(state_dim, hidden, max_batch, num_groups=1, compute_dtype=F32, states_ld=None,
                tau=(0.7, 0.7), lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                max_grad_norm=1.0, weight_clamp_max_abs=0.0, hidden2=0):
    """hidden: first hidden width H1; hidden2: second (0 = hidden)."""
    c = IqlConfig()
    c.state_dim, c.hidden, c.max_batch, c.num_groups = state_dim, hidden, max_batch, num_groups
    c.hidden2 = hidden2
    c.compute_dtype = compute_dtype
    c.states_ld = state_dim if states_ld is None else states_ld
    taus = list(tau) + [tau[-1]] * (2 - len(tau))
    c.tau[0], c.tau[1] = taus[0], taus[1]
    c.lr, c.beta1, c.beta2, c.eps = lr, beta1, beta2, eps
    c.weight_decay, c.max_grad_norm, c.weight_clamp_max_abs = weight_decay, max_grad_norm, weight_clamp_max_abs
    return c


def iql_create(cfg, init_params_host):
    """init_params_host: contiguous float32 host array/tensor of num_groups * P."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(init_params_host, dtype=np.float32))
    h = _p()
    _check(_lib_iql_create(ctypes.byref(cfg), arr.ctypes.data_as(_p), ctypes.byref(h)), "iql_create")
    return h


def iql_destroy(h):
    _check(_lib_iql_destroy(h), "iql_destroy")


def iql_train_step(h, states, q_taken, batch, out_v=None, out_loss=None, out_grad_norm=None, stream=None):
    _check(_lib_iql_train_step(h, _ptr(states), _ptr(q_taken), batch, _ptr(out_v), _ptr(out_loss),
                               _ptr(out_grad_norm), _stream(stream)), "iql_train_step")


def iql_train_step_aw(h, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, out_loss=None,
                      out_grad_norm=None, stream=None):
    _check(_lib_iql_train_step_aw(h, _ptr(states), _ptr(q_taken), batch, _ptr(q_all), num_actions, beta,
                                  _ptr(out_pi), _ptr(out_v), _ptr(out_loss), _ptr(out_grad_norm),
                                  _stream(stream)), "iql_train_step_aw")


def iql_compute_gradients(h, states, q_taken, batch, out_v=None, stream=None):
    _check(_lib_iql_compute_gradients(h, _ptr(states), _ptr(q_taken), batch, _ptr(out_v), _stream(stream)),
           "iql_compute_gradients")


def iql_apply_gradients(h, batch, out_loss=None, out_grad_norm=None, stream=None):
    _check(_lib_iql_apply_gradients(h, batch, _ptr(out_loss), _ptr(out_grad_norm), _stream(stream)),
           "iql_apply_gradients")


def iql_time_compute_gradients(h, states, q_taken, batch, reps, stream=None):
    """Mean duration (us) of the fused forward/backward kernel over `reps` launches."""
    out = _f()
    _check(_lib_iql_time_cg(h, _ptr(states), _ptr(q_taken), batch, reps, ctypes.byref(out), _stream(stream)),
           "iql_time_compute_gradients")
    return out.value


def iql_partial_layout(h, batch):
    """(partial rows per group, floats per row) of the per-workgroup gradient
    partials written for `batch` rows."""
    rows, floats = _i32(), _i64()
    _check(_lib_iql_partial_layout(h, batch, ctypes.byref(rows), ctypes.byref(floats)), "iql_partial_layout")
    return rows.value, floats.value


def per_workspace_bytes(size):
    out = ctypes.c_size_t()
    _check(_lib_per_ws(size, ctypes.byref(out)), "per_workspace_bytes")
    return out.value


def per_sample_indices(priorities, n, seed, beta, out_idx, out_weights, workspace, d_step=None, d_flags=None,
                       stream=None):
    """n prioritized draws over the rows of `priorities` (f32 tensor)."""
    _check(_lib_per_sample(_ptr(priorities), priorities.numel(), n, seed, _ptr(d_step), beta, _ptr(out_idx),
                           _ptr(out_weights), _ptr(d_flags), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)), "per_sample_indices")


def nonfinite_check(buffers, slot_flags, stream=None):
    """Sets slot_flags[s] = 1 for every buffer (fp32 tensor or None) holding
    a NaN or an infinity; clean slots keep their value."""
    n = len(buffers)
    ptrs = (_p * n)(*[None if b is None else b.data_ptr() for b in buffers])
    lens = (_i64 * n)(*[0 if b is None else b.numel() for b in buffers])
    _check(_lib_nonfinite_check(ptrs, lens, n, _ptr(slot_flags), _stream(stream)), "iqlh_nonfinite_check")


def iql_forward_values(h, next_states, batch, out_v, rewards=None, dones=None, gamma=0.99, out_target=None,
                       states_ld=None, stream=None):
    """V(s') of every group (online parameters) and, with rewards, the
    bootstrap target r + gamma (1 - done) V(s')."""
    import torch
    dt = BF16 if next_states.dtype == torch.bfloat16 else F32
    ld = states_ld if states_ld is not None else next_states.stride(0)
    _check(_lib_iql_forward_values(h, _ptr(next_states), dt, ld, batch, _ptr(out_v), _ptr(rewards), _ptr(dones),
                                   gamma, _ptr(out_target), _stream(stream)), "iql_forward_values")


def iql_target_ema_update(h, tau, stream=None):
    _check(_lib_iql_target_ema_update(h, tau, _stream(stream)), "iql_target_ema_update")


def iql_set_target_ema(h, tau):
    _check(_lib_iql_set_target_ema(h, tau), "iql_set_target_ema")


def iql_get_target(h, group, params, stream=None):
    _check(_lib_iql_get_target(h, group, _ptr(params), _stream(stream)), "iql_get_target")


def iql_set_target(h, group, params, stream=None):
    _check(_lib_iql_set_target(h, group, _ptr(params), _stream(stream)), "iql_set_target")


def iql_get_state(h, group, params=None, m=None, v=None, t=None, stream=None):
    _check(_lib_iql_get_state(h, group, _ptr(params), _ptr(m), _ptr(v), _ptr(t), _stream(stream)),
           "iql_get_state")


def iql_set_state(h, group, params, m, v, t, stream=None):
    _check(_lib_iql_set_state(h, group, _ptr(params), _ptr(m), _ptr(v), _ptr(t), _stream(stream)),
           "iql_set_state")


def iql_step_counter(h):
    return _lib_iql_step_counter(h)


def iql_flags(h):
    return _lib_iql_flags(h)


def iql_status(h):
    """Returns (status, flags); synchronises the device."""
    f = _i32()
    rc = _lib_iql_status(h, ctypes.byref(f))
    return rc, f.value


def iql_aw_policy(q, v, num_groups, batch, num_actions, beta, out_pi, stream=None):
    _check(_lib_iql_aw_policy(_ptr(q), _ptr(v), num_groups, batch, num_actions, beta, _ptr(out_pi),
                              _stream(stream)), "iql_aw_policy")


# ------------------------------------------------------------------- HER
def her_relabel(cfg, buf, source_idx, n, seed, d_step, out, stream=None):
    """cfg: HerConfig, buf: HerBuffer, out: HerOut (device addresses filled in)."""
    step = None if d_step is None else (d_step if isinstance(d_step, int) else d_step.data_ptr())
    _check(_lib_her_relabel(ctypes.byref(cfg), ctypes.byref(buf), _ptr(source_idx), n, seed,
                            None if step is None else ctypes.c_void_p(step), ctypes.byref(out),
                            _stream(stream)), "her_relabel")


def her_config(state_dim, goal_dim, strategy, goal_threshold=0.01, reward_hit=1.0, reward_miss=-0.01):
    c = HerConfig()
    c.state_dim, c.goal_dim, c.strategy = state_dim, goal_dim, strategy
    c.goal_threshold, c.reward_hit, c.reward_miss = goal_threshold, reward_hit, reward_miss
    return c


def her_buffer(states, next_states, actions, dones, episode_ends, buffer_size=None, rewards=None):
    """HerBuffer over device tensors.  The struct holds raw addresses, so it
    keeps references to the tensors: they stay allocated while it lives (a
    captured graph that replays a launch built from it needs that too)."""
    b = HerBuffer()
    b._keep = (states, next_states, actions, dones, episode_ends, rewards)
    b.states, b.next_states = states.data_ptr(), next_states.data_ptr()
    b.actions = actions.data_ptr() if actions is not None else None
    b.rewards = rewards.data_ptr() if rewards is not None else None
    b.dones = dones.data_ptr() if dones is not None else None
    b.episode_ends = episode_ends.data_ptr() if episode_ends is not None else None
    b.capacity = states.shape[0]
    b.buffer_size = states.shape[0] if buffer_size is None else buffer_size
    b.num_episodes = 0 if episode_ends is None else episode_ends.shape[0]
    return b


def her_out(states, states_dtype, states_ld, rewards, next_states=None, actions=None, dones=None,
            donor_idx=None, d_flags=None, is_weights=None):
    """HerOut; keeps references to the tensors it was given (see her_buffer).
    `states` and `is_weights` may be a tensor or a raw device address (a view
    into the merged batch)."""
    o = HerOut()
    o._keep = (states, rewards, next_states, actions, dones, donor_idx, d_flags, is_weights)
    o.states = states if isinstance(states, int) else states.data_ptr()
    o.states_dtype, o.states_ld = states_dtype, states_ld
    o.rewards = rewards.data_ptr()
    o.next_states = next_states.data_ptr() if next_states is not None else None
    o.actions = actions.data_ptr() if actions is not None else None
    o.dones = dones.data_ptr() if dones is not None else None
    o.donor_idx = donor_idx.data_ptr() if donor_idx is not None else None
    o.d_flags = d_flags if (d_flags is None or isinstance(d_flags, int)) else d_flags.data_ptr()
    o.is_weights = is_weights if (is_weights is None or isinstance(is_weights, int)) else is_weights.data_ptr()
    return o


# --------------------------------------------------------------- budget
def grad_budget_workspace_bytes(n, num_sources):
    out = ctypes.c_size_t()
    _check(_lib_ws_bytes(n, num_sources, ctypes.byref(out)), "grad_budget_workspace_bytes")
    return out.value


def make_adam(params, m, v, t, lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
              max_grad_norm=1.0, weight_clamp_max_abs=0.0, d_flags=None):
    """Adam state struct; keeps references to the tensors (see her_buffer)."""
    a = Adam()
    a._keep = (params, m, v, t, d_flags)
    a.params, a.m, a.v, a.t = params.data_ptr(), m.data_ptr(), v.data_ptr(), t.data_ptr()
    a.d_flags = None if d_flags is None else (d_flags if isinstance(d_flags, int) else d_flags.data_ptr())
    a.lr, a.beta1, a.beta2, a.eps = lr, beta1, beta2, eps
    a.weight_decay, a.max_grad_norm, a.weight_clamp_max_abs = weight_decay, max_grad_norm, weight_clamp_max_abs
    return a


def grad_budget_accumulate(grad_buf, sources, fractions, alphas, n, max_grad_norm, out_norms, adam,
                           workspace, stream=None):
    k = len(sources)
    srcs = (_p * k)(*[s.data_ptr() for s in sources])
    fr = (_f * k)(*fractions)
    al = (_f * k)(*alphas)
    _check(_lib_budget(_ptr(grad_buf), srcs, fr, al, k, n, max_grad_norm, _ptr(out_norms),
                       None if adam is None else ctypes.byref(adam), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _stream(stream)),
           "grad_budget_accumulate")


def grad_budget_accumulate_noalloc(grad_buf, sources, fractions, alphas, n, max_grad_norm, out_norms, adam,
                                   stream=None):
    """grad_budget_accumulate on the library's static device scratch (no workspace)."""
    k = len(sources)
    srcs = (_p * k)(*[s.data_ptr() for s in sources])
    fr = (_f * k)(*fractions)
    al = (_f * k)(*alphas)
    _check(_lib_budget_noalloc(_ptr(grad_buf), srcs, fr, al, k, n, max_grad_norm, _ptr(out_norms),
                               None if adam is None else ctypes.byref(adam), _stream(stream)),
           "grad_budget_accumulate_noalloc")


# ------------------------------------------------------------ whole step
def her_step(cfg, buf, source_idx, n, seed, out):
    """HerStep for iql_aux_step (the HER arguments of her_relabel minus d_step)."""
    st = HerStep()
    st._keep = (cfg, buf, out, source_idx)
    st.cfg, st.buf, st.out = ctypes.pointer(cfg), ctypes.pointer(buf), ctypes.pointer(out)
    st.source_idx = None if source_idx is None else source_idx.data_ptr()
    st.seed, st.n = seed, n
    return st


def budget_step(grad_buf, sources, fractions, alphas, n, max_grad_norm, out_norms, adam, workspace):
    """BudgetStep for iql_aux_step (the arguments of grad_budget_accumulate)."""
    k = len(sources)
    st = BudgetStep()
    st._keep = (grad_buf, tuple(sources), out_norms, adam, workspace)
    st.grad_buf = grad_buf.data_ptr()
    st.sources = (_p * k)(*[x.data_ptr() for x in sources])
    st.fractions = (_f * k)(*fractions)
    st.alphas = (_f * k)(*alphas)
    st.out_norms = None if out_norms is None else out_norms.data_ptr()
    if adam is not None:
        st.adam = ctypes.pointer(adam)
    st.workspace = workspace.data_ptr()
    st.workspace_bytes = workspace.numel() * workspace.element_size()
    st.n, st.num_sources, st.max_grad_norm = n, k, max_grad_norm
    return st


def iql_aux_step(h, her, states, q_taken, batch, q_all=None, num_actions=0, beta=0.0, out_pi=None, out_v=None,
                 out_loss=None, out_grad_norm=None, budget=None, stream=None):
    """HER + IQL step (+ AW policy) + budgeted accumulation in four launches."""
    _check(_lib_iql_aux_step(h, None if her is None else ctypes.byref(her), _ptr(states), _ptr(q_taken), batch,
                             _ptr(q_all), num_actions, beta, _ptr(out_pi), _ptr(out_v), _ptr(out_loss),
                             _ptr(out_grad_norm), None if budget is None else ctypes.byref(budget),
                             _stream(stream)), "iql_aux_step")


def iql_time_aux_step(h, her, states, q_taken, batch, q_all=None, num_actions=0, beta=0.0, out_pi=None,
                      out_v=None, out_loss=None, out_grad_norm=None, budget=None, reps=100, stream=None):
    """Runs `reps` whole steps with per-launch dispatch events; returns the mean
    duration (us) of launches [relabel+norms, forward/backward, reduce+SAXPY, Adam]."""
    out = (_f * 4)()
    _check(_lib_iql_time_aux_step(h, None if her is None else ctypes.byref(her), _ptr(states), _ptr(q_taken), batch,
                                  _ptr(q_all), num_actions, beta, _ptr(out_pi), _ptr(out_v), _ptr(out_loss),
                                  _ptr(out_grad_norm), None if budget is None else ctypes.byref(budget), reps, out,
                                  _stream(stream)), "iql_time_aux_step")
    return list(out)


PHASE_STAMPS = 8  # clock values per workgroup recorded by iql_aux_step_phase_stamps


def iql_aux_step_phase_stamps(h, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, out_loss,
                              out_grad_norm, budget, stamps, stream=None):
    """iql_aux_step with the forward/backward kernel's phase ends recorded:
    `stamps` is a device int64 tensor of groups * ceil(batch / 128) *
    PHASE_STAMPS elements (100 MHz clock values, tile order)."""
    _check(_lib_iql_aux_step_phase_stamps(h, None if her is None else ctypes.byref(her), _ptr(states),
                                          _ptr(q_taken), batch, _ptr(q_all), num_actions, beta, _ptr(out_pi),
                                          _ptr(out_v), _ptr(out_loss), _ptr(out_grad_norm),
                                          None if budget is None else ctypes.byref(budget), _ptr(stamps),
                                          stamps.numel(), _stream(stream)), "iql_aux_step_phase_stamps")


class IqlTrainer:
    """Owns an iql_handle; methods forward to the C entry points."""

    def __init__(self, cfg, init_params_host):
        self.cfg = cfg
        self.h = iql_create(cfg, init_params_host)
        self.n_params = iql_config_num_params(cfg)

    def forward_values(self, next_states, batch, out_v, rewards=None, dones=None, gamma=0.99, out_target=None,
                       states_ld=None, stream=None):
        iql_forward_values(self.h, next_states, batch, out_v, rewards, dones, gamma, out_target, states_ld, stream)

    def target_ema_update(self, tau, stream=None):
        iql_target_ema_update(self.h, tau, stream)

    def set_target_ema(self, tau):
        iql_set_target_ema(self.h, tau)

    def get_target(self, group, params, stream=None):
        iql_get_target(self.h, group, params, stream)

    def set_target(self, group, params, stream=None):
        iql_set_target(self.h, group, params, stream)

    def partial_layout(self, batch):
        return iql_partial_layout(self.h, batch)

    def train_step(self, states, q_taken, batch, out_v=None, out_loss=None, out_grad_norm=None, stream=None):
        iql_train_step(self.h, states, q_taken, batch, out_v, out_loss, out_grad_norm, stream)

    def train_step_aw(self, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, out_loss=None,
                      out_grad_norm=None, stream=None):
        iql_train_step_aw(self.h, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, out_loss,
                          out_grad_norm, stream)

    def aux_step(self, her, states, q_taken, batch, q_all=None, num_actions=0, beta=0.0, out_pi=None, out_v=None,
                 out_loss=None, out_grad_norm=None, budget=None, stream=None):
        iql_aux_step(self.h, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, out_loss,
                     out_grad_norm, budget, stream)

    def time_aux_step(self, her, states, q_taken, batch, q_all=None, num_actions=0, beta=0.0, out_pi=None,
                      out_v=None, out_loss=None, out_grad_norm=None, budget=None, reps=100, stream=None):
        return iql_time_aux_step(self.h, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v,
                                 out_loss, out_grad_norm, budget, reps, stream)

    def aux_step_phase_stamps(self, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, out_loss,
                              out_grad_norm, budget, stamps, stream=None):
        iql_aux_step_phase_stamps(self.h, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v,
                                  out_loss, out_grad_norm, budget, stamps, stream)

    def compute_gradients(self, states, q_taken, batch, out_v=None, stream=None):
        iql_compute_gradients(self.h, states, q_taken, batch, out_v, stream)

    def apply_gradients(self, batch, out_loss=None, out_grad_norm=None, stream=None):
        iql_apply_gradients(self.h, batch, out_loss, out_grad_norm, stream)

    def get_state(self, group, params=None, m=None, v=None, t=None, stream=None):
        iql_get_state(self.h, group, params, m, v, t, stream)

    def set_state(self, group, params, m, v, t, stream=None):
        iql_set_state(self.h, group, params, m, v, t, stream)

    @property
    def step_counter(self):
        return iql_step_counter(self.h)

    @property
    def flags(self):
        return iql_flags(self.h)

    def status(self):
        return iql_status(self.h)

    def close(self):
        if self.h:
            iql_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
