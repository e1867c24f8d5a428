"""The pins of the distillation objective, its gradients and the backward have teeth:
each plausible mistake, planted in a copy of one oracle function (its source re-compiled in
the oracle's namespace, on the CPU), makes at least one pin in test_oracle_distill.py,
test_oracle_distill_grad.py or test_oracle_backward.py fail."""
import inspect
import itertools

import pytest

import oracle
import test_oracle_backward
import test_oracle_distill
import test_oracle_distill_grad

MUTANTS = {
    "teacher_scale_1_over_D": ("full_softmax", "s = q[b, h] @ k[b, h].T / np.sqrt(p.D)", "s = q[b, h] @ k[b, h].T / p.D"),
    "teacher_normalised_over_queries": ("full_softmax", "/ e.sum(axis=1, keepdims=True)", "/ e.sum(axis=0, keepdims=True)"),
    "loss_l1": ("distill_loss", "((hyb - soft) ** 2).sum(axis=(2, 3))", "np.abs(hyb - soft).sum(axis=(2, 3))"),
    "phi_grad_no_power_factor": ("_phi_backward", "power[f] * u[:, elem[f]] ** (power[f] - 1)", "u[:, elem[f]] ** (power[f] - 1)"),
    "softplus_grad_sign": ("_phi_backward", "dpre = du / (1.0 + np.exp(-pre))", "dpre = du / (1.0 + np.exp(pre))"),
    "kappa_grad_no_h_term": ("distill_phi_grads", "dkap = np.where(lin, a @ v[b, h].T - hv, 0.0)", "dkap = np.where(lin, a @ v[b, h].T, 0.0)"),
    "key_grad_untransposed": ("distill_phi_grads", "_phi_backward(p, prk, uk, k[b, h], dkap.T @ fq)", "_phi_backward(p, prk, uk, k[b, h], dkap @ fq)"),
    "chunked_key_frames_one_late": ("distill_phi_grads_chunked", "ks = slice(lprev * n, ls * n)", "ks = slice(lprev * n + n, ls * n + n)"),
    "backward_dk_unscaled": ("backward", 'res["dk"][b, h] += ds.T @ q[b, h] * rs', 'res["dk"][b, h] += ds.T @ q[b, h]'),
    "backward_dv_softmax_only": ("backward", 'res["dv"][b, h] += (ws_ + wl).T @ a', 'res["dv"][b, h] += ws_.T @ a'),
    "backward_ds_sign": ("backward", "ds = ws_ * dw", "ds = -ws_ * dw"),
    "input_grad_through_w_transposed": ("_phi_backward_x", "return dpre.T @ x, dpre.sum(axis=0), dpre @ w", "return dpre.T @ x, dpre.sum(axis=0), dpre @ w[:, ::-1]"),
    "chunked_window_unnormalised": ("backward_chunked", "- np.log(den[qs])[:, None])", ")"),
    "chunked_dv_linear_dropped": ("backward_chunked", 'res["dv"][b, h][ks] += fk[ks] @ R', 'pass'),
}

PIN_MODULES = (test_oracle_distill, test_oracle_distill_grad, test_oracle_backward)


def pin_calls():
    """Every (function, kwargs) of the pin modules, parametrizations expanded."""
    for mod in PIN_MODULES:
        for name, fn in vars(mod).items():
            if not name.startswith("test_") or not callable(fn):
                continue
            marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
            if not marks:
                yield f"{mod.__name__}.{name}", fn, {}
                continue
            grids = []
            for m in marks:
                names = [s.strip() for s in m.args[0].split(",")]
                vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
                grids.append([dict(zip(names, v)) for v in vals])
            for combo in itertools.product(*grids):
                kw = {}
                for d in combo:
                    kw.update(d)
                yield f"{mod.__name__}.{name}{kw}", fn, kw


def test_pins_pass_on_the_oracle():
    for label, fn, kw in pin_calls():
        fn(**kw)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, monkeypatch):
    fname, before, after = MUTANTS[name]
    src = inspect.getsource(getattr(oracle, fname))
    assert before in src, f"mutation site for {name} not found"
    ns = {}
    exec(compile(src.replace(before, after), f"<mutant {name}>", "exec"), oracle.__dict__, ns)
    monkeypatch.setattr(oracle, fname, ns[fname])
    for label, fn, kw in pin_calls():
        try:
            fn(**kw)
        except Exception:
            return
    pytest.fail(f"mutant {name} passed every pin")
