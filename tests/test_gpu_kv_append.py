"""KV-cache append with attention sinks (decode-time streaming of the sink mode of
the ScaleSearch summary page, ScaleSearchAttention, アテンション・シンク対応混合精度
キャッシング): after every append the cache must hold exactly what the one-shot sink
mode gives for the whole sequence under the same given tensor scale — checked
bit for bit against the oracle."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def check_against_oracle(orc, cache, kv_all, sg, offsets, hadamard):
    nf, nl, T = cache["n_first"], cache["n_last"], cache["length"]
    if T < nf + nl:
        np.testing.assert_array_equal(to_host(cache["head"])[:, :, :min(T, nf)],
                                      kv_all[:, :, :min(T, nf)])
        return
    rc, rs, _, rsink = orc.quantize_kv_sink(np.ascontiguousarray(kv_all[:, :, :T]), nf, nl,
                                            *offsets, hadamard=hadamard, gscale=float(sg))
    tm = T - nf - nl
    np.testing.assert_array_equal(to_host(cache["codes"])[:, :, :tm], rc)
    np.testing.assert_array_equal(to_host(cache["scales"])[:, :, :tm], rs)
    np.testing.assert_array_equal(to_host(cache["head"]), rsink[:, :, :nf])
    if nl:
        ring = to_host(cache["tail"])
        order = [(T - nl + k) % nl for k in range(nl)]
        np.testing.assert_array_equal(ring[:, :, order], rsink[:, :, nf:])


@pytest.mark.parametrize("nf,nl,steps,dtype_bf16,hadamard,offsets", [
    (128, 128, [300, 1, 1, 1, 70, 1, 256, 3], True, False, (-2, 6)),
    (16, 32, [5, 60, 1, 33, 1, 100], True, False, (-8, 8)),
    (0, 0, [40, 1, 17], True, False, (-2, 6)),
    (32, 0, [50, 2, 1], True, False, (-2, 6)),
    (0, 24, [10, 30, 1, 5], False, False, (-2, 6)),
    (64, 64, [200, 1, 9], True, True, (-8, 8)),
])
def test_append_sequence_matches_one_shot(gpu, orc, nf, nl, steps, dtype_bf16, hadamard, offsets):
    B, H, D = 1, 3, 128
    total = sum(steps)
    kv_all = workloads.workload(3, (B, H, total, D))
    if not dtype_bf16:
        kv_all = workloads.bf16_bits_to_f32(kv_all)
    # the caller's tensor scale: fixed up front from the first 200 tokens' magnitudes
    sg = np.float32(np.abs(workloads.bf16_bits_to_f32(kv_all[:, :, :200]) if dtype_bf16
                           else kv_all[:, :, :200]).max() / np.float32(2688))
    g = torch.tensor([sg], dtype=torch.float32, device="cuda:0")
    tdt = torch.bfloat16 if dtype_bf16 else torch.float32
    cache = gpu.kv_cache_alloc(B, H, D, capacity=total + 8, n_first=nf, n_last=nl, dtype=tdt)
    t = 0
    for k in steps:
        print(f"[case] append {k} tokens at {t} (nf={nf}, nl={nl}, hadamard={hadamard})",
              flush=True)
        gpu.kv_append(cache, to_dev(np.ascontiguousarray(kv_all[:, :, t:t + k])), g, offsets,
                      hadamard=hadamard)
        torch.cuda.synchronize()
        t += k
        check_against_oracle(orc, cache, kv_all, sg, offsets, hadamard)


def test_append_capacity_check(gpu):
    cache = gpu.kv_cache_alloc(1, 1, 128, capacity=300, n_first=128, n_last=128)
    g = torch.ones(1, dtype=torch.float32, device="cuda:0")
    x = torch.zeros(1, 1, 301, 128, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        gpu.kv_append(cache, x, g)
