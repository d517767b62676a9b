"""dp_reduce_adam_step_noalloc, the single pass for callers that cannot
allocate, against dp_reduce_adam_step on a one-tensor plan with flat bindings:
the same inputs and the same starting state must give the same two state
banks, parameters and scalar state, bit for bit, at every step.  Two
configurations run one after the other in one process, the second on a
smaller flat space, so the second reuses the static scratch the first left
behind."""
import ctypes

import numpy as np
import pytest
import torch

import gradient_reduce_adam_amd as dp

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, eps=1e-8, weight_decay=0.01)
BETAS = (0.9, 0.999)
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}

# (P, n, grad dtype, param dtype, earlier micro-steps, scaler, initial scale,
#  steps, step whose gradient holds an inf)
CONFIGS = [
    (200003, 3, "bf16", "bf16", 1, "dynamic", 1024.0, 3, 2),
    (70001, 2, "f16", "f16", 0, "static", 8.0, 3, 3),
]


def _state_block(scale: float) -> torch.Tensor:
    """A device dp_step_state at the start of a run."""
    s = dp.StepState(0, 0, 0, 1.0, 1.0, scale, 0, 0, 0.0, 0.0, 1.0, 0.0)
    raw = np.frombuffer(ctypes.string_at(ctypes.addressof(s), ctypes.sizeof(s)), dtype=np.uint8).copy()
    return torch.from_numpy(raw).cuda()


def _read_block(t: torch.Tensor) -> dict:
    torch.cuda.synchronize()
    raw = t.cpu().numpy().tobytes()
    return dp.StepState.from_buffer_copy(raw).as_dict()


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32).cpu().numpy()


def _run_pair(P, n, gdt, pdt, earlier, scaler, scale0, steps, inf_step, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    dev = "cuda"
    stream = torch.cuda.current_stream()
    master0 = torch.randn(P, generator=gen, device=dev) * 0.02
    # the plan's arrays and the static path's arrays start equal
    sides = []
    for _ in range(2):
        banks = [[master0.clone(), torch.zeros(P, device=dev), torch.zeros(P, device=dev)] for _ in range(2)]
        param = master0.to(TORCH[pdt])
        accs = [torch.empty(P, device=dev) for _ in range(n)] if earlier else []
        sides.append((banks, param, accs))
    grads = [torch.empty(P, dtype=TORCH[gdt], device=dev) for _ in range(n)]
    plan = dp.Plan([P], n, gdt, pdt)
    try:
        (pb, pp, pa), (sb, sp, sa) = sides
        for b in range(2):
            for role, t in zip(("master", "exp_avg", "exp_avg_sq"), pb[b]):
                plan.bind(role, t, b)
        plan.bind("param", pp)
        for r in range(n):
            plan.bind("grad", grads[r], r)
            if earlier:
                plan.bind("acc", pa[r], r)
        plan.state_init(*BETAS, scaler=scaler, init_scale=scale0, stream=stream)
        block = _state_block(1.0 if scaler == "none" else scale0)
        for step in range(1, steps + 1):
            if earlier:  # the earlier micro-step: its gradients into the plan's accumulators
                for g in grads:
                    g.copy_((torch.randn(P, generator=gen, device=dev) * 1e-3 * scale0).to(TORCH[gdt]))
                plan.accumulate_all(first=True, stream=stream)
                for a_s, a_p in zip(sa, pa):
                    a_s.copy_(a_p)
            for g in grads:
                g.copy_((torch.randn(P, generator=gen, device=dev) * 1e-3 * scale0).to(TORCH[gdt]))
            if step == inf_step:
                grads[n - 1][P // 3] = float("inf")
            plan.reduce_adam_step(**HP, stream=stream)
            dp.dp_reduce_adam_step_noalloc(P, n, gdt, pdt, grads, sa if earlier else None, [b[0] for b in sb],
                                           [b[1] for b in sb], [b[2] for b in sb], sp, block, *HP.values(), *BETAS,
                                           scaler=scaler, init_scale=scale0, stream=stream)
            want = plan.read_state(stream=stream)
            got = _read_block(block)
            assert got == want, (P, step, got, want)
            assert got["found_inf"] == int(step == inf_step)
            for b in range(2):
                for k, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
                    assert np.array_equal(_bits(sb[b][k]), _bits(pb[b][k])), (P, step, name, b)
            assert np.array_equal(_bits(sp), _bits(pp)), (P, step, "param")
        return got
    finally:
        plan.close()


def test_noalloc_single_pass_equals_plan_single_pass_twice():
    t_prev = None
    for i, cfg in enumerate(CONFIGS):
        print(f"no-alloc single pass: P={cfg[0]} n={cfg[1]} {cfg[2]}/{cfg[3]} earlier={cfg[4]} scaler={cfg[5]} "
              f"steps={cfg[7]} inf at step {cfg[8]}", flush=True)
        st = _run_pair(*cfg, seed=11 + i)
        assert st["iter"] == cfg[7] and st["t"] == cfg[7] - 1
        if t_prev is not None:
            assert cfg[0] < t_prev  # the second call covers a smaller space
        t_prev = cfg[0]
