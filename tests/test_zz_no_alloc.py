"""moedc_route_noalloc -- the route on the library's static device array,
for callers that cannot allocate -- against moedc_route, both through the C
ABI.  Each case makes two calls in a row, the second on a smaller batch
(and, in the mixed case, with another plan), and compares every output of
each call bit for bit with moedc_route's on the same inputs: the large-batch
kernels (per-block counts in the array), the small-batch two-launch and
one-launch paths (tables only), replicas and a shared expert."""
import numpy as np
import pytest
import torch

from combine_moedc_route_amd import moedc as M
from combine_moedc_route_amd import workloads as W

from gpu_common import dev, gpu_route, log

pytestmark = pytest.mark.gpu


def _route_noalloc(plan, logits):
    T = logits.shape[0]
    K, P = plan.K, plan.num_phys
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(
        topk_ids=torch.full((T, K), -7, **i32),
        topk_w=torch.full((T, K), -7.0, dtype=torch.float32, device="cuda"),
        counts=torch.full((P,), -7, **i32),
        offsets=torch.full((P + 1,), -7, **i32),
        slots=torch.full((T, K), -7, **i32),
        dropped=torch.full((1,), -7, **i32),
    )
    lg = dev(logits) if T else torch.empty((0, plan.num_logical), dtype=torch.float32,
                                           device="cuda")
    plan.route_noalloc(lg, out["topk_ids"], out["topk_w"], out["counts"], out["offsets"],
                       out["slots"], out["dropped"], num_tokens=T)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["dropped"] = int(res["dropped"][0])
    return res


def _same(got, want, what):
    for k in want:
        assert np.array_equal(np.asarray(got[k]), np.asarray(want[k])), f"{what}: {k} differs"


@pytest.mark.parametrize("name,first,second", [
    ("global", 30720, 5000),         # large-batch kernels, then a smaller large batch
    ("skewed", 30720, 700),          # replicas (288 physical experts)
    ("prefill", 65536, 300),         # shared expert; largest per-block count array
    ("replica_shared", 517, 100),    # large, then the two-launch small-batch path
    ("decode", 96, 16),              # two-launch, then one-launch small batches
])
def test_route_noalloc_matches_route_on_two_calls(name, first, second):
    wl = W.get(name)
    plan = M.Plan.from_workload(wl)
    for T in (first, second):
        log(f"[case] route_noalloc {name} T={T}")
        _, logits = W.make_inputs(wl, T)
        want, _ = gpu_route(plan, wl, logits)
        got = _route_noalloc(plan, logits)
        _same(got, want, f"{name} T={T}")


def test_route_noalloc_two_plans_share_the_array():
    """A large batch of one plan, then a smaller batch of a plan with another
    table layout: the second call's tables replace the first's."""
    calls = [("skewed", 30720), ("ragged", 333), ("global", 4000)]
    for name, T in calls:
        wl = W.get(name)
        plan = M.Plan.from_workload(wl)
        log(f"[case] route_noalloc {name} T={T} after another plan")
        _, logits = W.make_inputs(wl, T)
        want, _ = gpu_route(plan, wl, logits)
        _same(_route_noalloc(plan, logits), want, f"{name} T={T}")
