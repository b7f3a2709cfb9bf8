"""KV-cache append with attention sinks (decode-time streaming of the sink mode of
the ScaleSearch summary page, ScaleSearchAttention, アテンション・シンク対応混合精度
キャッシング): after every append the cache must hold exactly what the one-shot sink
mode gives for the whole sequence under the same given tensor scale — checked
bit for bit against the oracle. With the Hadamard transform the contract is that of
the transform: the oracle's quantizer on the GPU's own FP32 transform of the middle
tokens gives the cache's codes bit for bit, and against the oracle's exactly rounded
transform at most 1e-4 of the blocks differ."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def check_against_oracle(orc, cache, kv_all, sg, offsets, hadamard, nv=None):
    nf, nl, T = cache["n_first"], cache["n_last"], cache["length"]
    if T < nf + nl:
        np.testing.assert_array_equal(to_host(cache["head"])[:, :, :min(T, nf)],
                                      kv_all[:, :, :min(T, nf)])
        return
    rc, rs, _, rsink = orc.quantize_kv_sink(np.ascontiguousarray(kv_all[:, :, :T]), nf, nl,
                                            *offsets, hadamard=hadamard, gscale=float(sg))
    tm = T - nf - nl
    gc, gs = to_host(cache["codes"])[:, :, :tm], to_host(cache["scales"])[:, :, :tm]
    if hadamard:
        # split parity on the GPU's own transform of the middle tokens
        mid = to_dev(np.ascontiguousarray(kv_all[:, :, nf:T - nl]))
        y = to_host(nv.hadamard128(mid)).reshape(-1, mid.shape[-1])
        pc, ps, _ = orc.quantize(y, *offsets, gscale=float(sg))
        np.testing.assert_array_equal(gc.reshape(pc.shape), pc)
        np.testing.assert_array_equal(gs.reshape(ps.shape), ps)
        bad = (gs.reshape(-1) != rs.reshape(-1)) | np.any(
            gc.reshape(-1, 8) != rc.reshape(-1, 8), axis=1)
        assert bad.mean() <= 1e-4, f"{bad.sum()} of {bad.size} blocks differ end to end"
    else:
        np.testing.assert_array_equal(gc, rc)
        np.testing.assert_array_equal(gs, rs)
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
    # 3 heads x 8 blocks a token: 10 tokens (240 blocks) take the one-workgroup
    # append, 11 (264) the multi-kernel one
    (16, 16, [40, 10, 11, 10, 11, 1], True, False, (-2, 6)),
    (16, 16, [40, 10, 11, 10, 11, 1], False, False, (-8, 8)),
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
        check_against_oracle(orc, cache, kv_all, sg, offsets, hadamard, gpu)


def test_append_capacity_check(gpu):
    cache = gpu.kv_cache_alloc(1, 1, 128, capacity=300, n_first=128, n_last=128)
    g = torch.ones(1, dtype=torch.float32, device="cuda:0")
    x = torch.zeros(1, 1, 301, 128, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        gpu.kv_append(cache, x, g)


# --- the device-resident length (capturable decode steps) ---

def _same_cache(a, b, tm):
    for key in ("head", "tail"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["codes"][:, :, :tm], b["codes"][:, :, :tm])
    assert torch.equal(a["scales"][:, :, :tm], b["scales"][:, :, :tm])


@pytest.mark.parametrize("dtype,signs", [(torch.bfloat16, None), (torch.float32, None),
                                         (torch.bfloat16, (5, 6, 7, 8))])
def test_device_length_matches_host_length(gpu, dtype, signs):
    B, H, D, nf, nl = 1, 2, 128, 32, 48
    steps = [150, 1, 1, 40, 1, 7, 0, 3]
    kv_all = workloads.workload(3, (B, H, sum(steps), D))
    xall = to_dev(kv_all)
    if dtype == torch.float32:
        xall = xall.float()
    g = gpu.global_scale(xall[:, :, :150].contiguous())
    host = gpu.kv_cache_alloc(B, H, D, 300, nf, nl, dtype)
    devc = gpu.kv_cache_alloc(B, H, D, 300, nf, nl, dtype)
    had = signs is not None
    t = 0
    for k in steps:
        print(f"[case] device-length append {k} tokens at {t} ({dtype}, signs={signs})", flush=True)
        chunk = xall[:, :, t:t + k].contiguous()
        gpu.kv_append(host, chunk, g, (-2, 6), signs=signs)
        gpu.kv_append_dev(devc, chunk, g, (-2, 6), signs=signs)
        t += k
        torch.cuda.synchronize()
        assert gpu.kv_length(devc) == host["length"] == t
        _same_cache(host, devc, max(t - nf - nl, 0))


@pytest.mark.parametrize("dtype,k_signs", [(torch.bfloat16, None), (torch.float32, None),
                                           (torch.bfloat16, (5, 6, 7, 8))])
def test_paired_append_matches_two_appends(gpu, dtype, k_signs):
    """kv_append2_dev (the K and V appends of a step in one call: one launch of two
    workgroups when both are small) leaves both caches and both lengths exactly as two
    kv_append_dev calls do: prefill chunks (the multi-kernel path), single tokens, an
    empty append, an append that does not fit, and K with the randomized Hadamard
    transform (V without, so the call takes the two-call path)."""
    B, H, D, nf, nl, cap = 1, 2, 128, 32, 48, 220
    steps = [150, 1, 1, 40, 1, 7, 0, 3, 100]  # the last: 203 + 100 > 32 + 220 + 48
    kv_all = workloads.workload(3, (B, H, sum(steps), D))
    xk = to_dev(kv_all)
    xv = to_dev(np.ascontiguousarray(kv_all[..., ::-1]))
    if dtype == torch.float32:
        xk, xv = xk.float(), xv.float()
    gk = gpu.global_scale(xk[:, :, :150].contiguous())
    gv = gpu.global_scale(xv[:, :, :150].contiguous())
    one_k, one_v, pair_k, pair_v = (gpu.kv_cache_alloc(B, H, D, cap, nf, nl, dtype)
                                    for _ in range(4))
    t = 0
    for k in steps:
        print(f"[case] paired append {k} tokens at {t} ({dtype}, k_signs={k_signs})", flush=True)
        kc = xk[:, :, t:t + k].contiguous()
        vc = xv[:, :, t:t + k].contiguous()
        gpu.kv_append_dev(one_k, kc, gk, (-2, 6), signs=k_signs)
        gpu.kv_append_dev(one_v, vc, gv, (-2, 6))
        gpu.kv_append2_dev(pair_k, kc, gk, pair_v, vc, gv, (-2, 6), k_signs=k_signs)
        torch.cuda.synchronize()
        t += k
        n = gpu.kv_length(one_k)
        assert n == min(t, 203)
        assert gpu.kv_length(pair_k) == gpu.kv_length(pair_v) == gpu.kv_length(one_v) == n
        _same_cache(one_k, pair_k, max(n - nf - nl, 0))
        _same_cache(one_v, pair_v, max(n - nf - nl, 0))


def test_device_length_overflow_is_a_noop(gpu):
    B, H, D, nf, nl = 1, 1, 128, 16, 16
    kv = to_dev(workloads.workload(3, (B, H, 120, D)))
    g = gpu.global_scale(kv)
    c = gpu.kv_cache_alloc(B, H, D, 100, nf, nl)  # holds 100 tokens
    gpu.kv_append_dev(c, kv[:, :, :90].contiguous(), g)
    torch.cuda.synchronize()
    before = {k: v.clone() for k, v in c.items() if isinstance(v, torch.Tensor)}
    gpu.kv_append_dev(c, kv[:, :, 90:120].contiguous(), g)  # 90 + 30 > 100
    torch.cuda.synchronize()
    assert gpu.kv_length(c) == 90
    for k, v in before.items():
        assert torch.equal(c[k], v), k


@pytest.mark.parametrize("split,paired", [(0, False), (64, False), (64, True)])
def test_graph_replayed_decode_step(gpu, split, paired):
    """One decode step (append a K and a V token at the device length, attention of one
    query over the caches) captured once and replayed token after token; every replay is
    checked against the host-length calls made eagerly on a second pair of caches. With
    split keys the captured grid covers every unit of a full cache and the units past
    the tokens present add nothing, so the result equals the host-length call's bit for
    bit. paired: the two appends as one kv_append2_dev call (one launch)."""
    B, H, D, nf, nl = 1, 2, 128, 32, 32
    n_pre, n_dec = 120, 12  # the middle grows from 56 to 68 tokens: across a 64-token piece
    rng = np.random.default_rng(5)
    kall = to_dev(workloads.workload(3, (B, H, n_pre + n_dec, D)))
    vall = to_dev(workloads.to_bf16_bits(rng.standard_normal((B, H, n_pre + n_dec, D))
                                         .astype(np.float32)))
    qx = to_dev(workloads.to_bf16_bits(rng.standard_normal((B, 2 * H, 1, D)).astype(np.float32)))
    q = gpu.quantize(qx)
    kg = gpu.global_scale(kall[:, :, :n_pre].contiguous())
    vg = gpu.global_scale(vall[:, :, :n_pre].contiguous())
    kd, vd = (gpu.kv_cache_alloc(B, H, D, 256, nf, nl) for _ in range(2))
    kh, vh = (gpu.kv_cache_alloc(B, H, D, 256, nf, nl) for _ in range(2))
    for c, x, gs in ((kd, kall, kg), (vd, vall, vg)):
        gpu.kv_append_dev(c, x[:, :, :n_pre].contiguous(), gs)
    for c, x, gs in ((kh, kall, kg), (vh, vall, vg)):
        gpu.kv_append(c, x[:, :, :n_pre].contiguous(), gs)
    knew = torch.empty(B, H, 1, D, dtype=torch.bfloat16, device="cuda")
    vnew = torch.empty_like(knew)
    nws = gpu.attention_split_workspace_bytes(B, 2 * H, 1, 256, split) if split else 0
    ws_dev = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ws_host = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def step():
        if paired:
            gpu.kv_append2_dev(kd, knew, kg, vd, vnew, vg)
        else:
            gpu.kv_append_dev(kd, knew, kg)
            gpu.kv_append_dev(vd, vnew, vg)
        return gpu.attention_kv_cache(q, kd, kg, vd, vg, device_length=True, split=split,
                                      workspace=ws_dev if split else None)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        out = step()
    torch.cuda.synchronize()
    assert gpu.kv_length(kd) == n_pre  # capture launched nothing
    for i in range(n_dec):
        t = n_pre + i
        print(f"[case] graph replay {i}: token {t}", flush=True)
        knew.copy_(kall[:, :, t:t + 1])
        vnew.copy_(vall[:, :, t:t + 1])
        graph.replay()
        gpu.kv_append(kh, kall[:, :, t:t + 1].contiguous(), kg)
        gpu.kv_append(vh, vall[:, :, t:t + 1].contiguous(), vg)
        ref = gpu.attention_kv_cache(q, kh, kg, vh, vg, split=split,
                                     workspace=ws_host if split else None)
        torch.cuda.synchronize()
        assert gpu.kv_length(kd) == gpu.kv_length(vd) == t + 1
        assert torch.equal(out, ref), f"replay {i}"
        _same_cache(kh, kd, t + 1 - nf - nl)
        _same_cache(vh, vd, t + 1 - nf - nl)


@pytest.mark.parametrize("split,tokens", [(32, 137), (64, 150), (160, 389)])
def test_split_device_length_ignores_rows_past_the_tokens(gpu, split, tokens):
    """The split decode kernel with the token count in device memory loads a middle
    unit's first chunk from the cache's capacity before the count arrives, so rows past
    the tokens present are read and must drop out: here they hold 0xFF bytes (NaN block
    scales, largest codes), and the result must equal, bit for bit, the host-length
    call on caches whose unused rows were never written."""
    B, H, D, nf, nl, cap = 1, 2, 128, 32, 32, 512
    rng = np.random.default_rng(11)
    kall = to_dev(workloads.workload(3, (B, H, tokens, D)))
    vall = to_dev(workloads.to_bf16_bits(rng.standard_normal((B, H, tokens, D))
                                         .astype(np.float32)))
    q = gpu.quantize(to_dev(workloads.to_bf16_bits(
        rng.standard_normal((B, 2 * H, 1, D)).astype(np.float32))))
    kg = gpu.global_scale(kall)
    vg = gpu.global_scale(vall)
    kd, vd = (gpu.kv_cache_alloc(B, H, D, cap, nf, nl) for _ in range(2))
    kh, vh = (gpu.kv_cache_alloc(B, H, D, cap, nf, nl) for _ in range(2))
    for c in (kd, vd):
        c["codes"].fill_(0xFF)
        c["scales"].fill_(0xFF)
    for c in (kh, vh):
        c["codes"].zero_()
        c["scales"].zero_()
    gpu.kv_append_dev(kd, kall, kg)
    gpu.kv_append_dev(vd, vall, vg)
    gpu.kv_append(kh, kall, kg)
    gpu.kv_append(vh, vall, vg)
    nws = gpu.attention_split_workspace_bytes(B, 2 * H, 1, cap - nf - nl, split)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    print(f"[case] split {split}, {tokens} tokens in a cache of {cap}", flush=True)
    out = gpu.attention_kv_cache(q, kd, kg, vd, vg, device_length=True, split=split,
                                 workspace=ws).clone()
    ref = gpu.attention_kv_cache(q, kh, kg, vh, vg, split=split, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref)
