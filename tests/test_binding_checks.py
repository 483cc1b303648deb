"""Host-side checks of the Python binding and of the launch planning (CPU; no compute call).

The C layer receives bare pointers, so the binding must reject every tensor that the kernels would
misread: host tensors, strided views, wrong shapes or dtypes, and workspaces that are not contiguous
device byte tensors.  fa_plan exposes the launch heuristics (causal tile pairing, wave counts, the
fp32 key split, automatic split counts) as a function of the compute-unit count, so the threshold
arithmetic is checked here for the full part and for smaller and larger devices.
"""
import os

import pytest

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_tiled_attention_09_amd")


@pytest.fixture(scope="module", autouse=True)
def need_lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    fa.lib()


class FakeDeviceTensor:
    """Stands in for a device tensor on a machine without a GPU: only the attributes the checks read."""

    def __init__(self, shape, dtype, contiguous=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.is_cuda = True
        self._contig = contiguous

    def is_contiguous(self):
        return self._contig

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def data_ptr(self):  # pragma: no cover - never reached: every test call is rejected first
        raise AssertionError("a rejected call must not reach the library")


BF = torch.bfloat16


def dev(shape, dtype=BF, contiguous=True):
    return FakeDeviceTensor(shape, dtype, contiguous)


def test_fwd_rejects_host_and_strided_tensors():
    q = torch.zeros(1, 2, 8, 64, dtype=BF)
    with pytest.raises(ValueError, match="device tensor"):
        fa.fa_fwd(q, q, q, q, None, 0.125, True)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_fwd(dev((1, 2, 8, 64), contiguous=False), dev((1, 2, 8, 64)), dev((1, 2, 8, 64)),
                  dev((1, 2, 8, 64)), None, 0.125, True)


@pytest.mark.parametrize("bad", ["q", "k", "workspace"])
def test_decode_checks_every_argument(bad):
    B, H, N, d = 2, 2, 16, 64
    args = {"q": dev((B, H, d)), "k": dev((B, H, N, d)), "v": dev((B, H, N, d)), "o": dev((B, H, d)),
            "workspace": dev((4096,), torch.uint8)}
    args[bad] = torch.zeros(args[bad].shape, dtype=args[bad].dtype)  # a host tensor
    with pytest.raises(ValueError, match="device tensor"):
        fa.fa_decode(args["q"], args["k"], args["v"], args["o"], None, 0.1, 1, args["workspace"])
    with pytest.raises(ValueError, match="device tensor"):
        fa.fa_decode_split(args["q"], args["k"], args["v"], 0.1, 1, args["workspace"])


def test_workspace_must_be_contiguous_bytes():
    B, H, N, d = 2, 2, 16, 64
    q, k, o = dev((B, H, d)), dev((B, H, N, d)), dev((B, H, d))
    with pytest.raises(ValueError, match="uint8"):
        fa.fa_decode(q, k, k, o, None, 0.1, 1, dev((1024,), torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_decode(q, k, k, o, None, 0.1, 1, dev((4096,), torch.uint8, contiguous=False))
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_decode_combine(dev((4096,), torch.uint8), dev((B, H, d), contiguous=False), None, 1)


def test_split_gqa_paged_bwd_check_q_and_workspace():
    B, H, Nq, N, d = 1, 4, 8, 64, 64
    q, k = dev((B, H, Nq, d), contiguous=False), dev((B, H, N, d))
    o, ws = dev((B, H, Nq, d)), dev((1 << 16,), torch.uint8)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_fwd_split(q, k, k, o, None, 0.1, True, 2, ws)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_bwd(q, k, k, o, dev((B, H, Nq), torch.float32), o, o, k, k, 0.1, True, ws)
    qd, kv = dev((B, H, d)), dev((B, 2, N, d), contiguous=False)
    with pytest.raises(ValueError, match="contiguous"):
        fa.fa_decode_gqa(qd, kv, dev((B, 2, N, d)), qd, None, 0.1, 1, ws)
    pool = dev((8, 2, 16, d))
    with pytest.raises(ValueError, match="uint8"):
        fa.fa_decode_paged(qd, pool, pool, dev((B, 4), torch.int32), dev((B,), torch.int32), qd, None, 0.1, 1,
                           dev((1 << 16,), torch.float32))


# ----------------------------------------------------------------------------- launch planning

def P(op, B, H, Nq, Nkv, d, causal=True, dtype=fa.FA_DTYPE_BF16, num_splits=0, num_cu=256):
    return fa.plan(op, B, H, Nq, Nkv, d, causal, dtype, num_splits, num_cu)


def test_plan_headline_prefill_on_the_full_part():
    p = P(fa.FA_PLAN_FWD, 1, 32, 8192, 8192, 128)
    # 32 heads x 32 tiles of 256 rows = 1024 >= 256 CUs: 8 waves; >= 2 x 256: causal tiles paired
    assert p == {"kernel": "bf16_8wave", "waves_per_group": 8, "rows_per_group": 256, "paired": True,
                 "groups": 32 * 16, "num_splits": 0}


@pytest.mark.parametrize("num_cu,kernel,paired,groups", [
    (64, "bf16_8wave", True, 512),      # a partitioned device: same shape, fewer CUs
    (256, "bf16_8wave", True, 512),
    (512, "bf16_8wave", True, 512),     # 1024 groups >= 2 x 512: still paired
    (1024, "bf16_8wave", False, 1024),  # 1024 >= 1024 CUs: 8 waves, but fewer than 2 groups per CU
    (2048, "bf16_4wave", False, 2048),  # 1024 8-wave groups < 2048 CUs: 128-row tiles, 2048 < 4096
])
def test_plan_prefill_thresholds_follow_the_cu_count(num_cu, kernel, paired, groups):
    p = P(fa.FA_PLAN_FWD, 1, 32, 8192, 8192, 128, num_cu=num_cu)
    assert (p["kernel"], p["paired"], p["groups"]) == (kernel, paired, groups)


def test_plan_d64_and_noncausal():
    p = P(fa.FA_PLAN_FWD, 4, 16, 2048, 2048, 64)
    assert (p["kernel"], p["rows_per_group"], p["paired"], p["groups"]) == ("bf16_4wave", 128, True, 64 * 8)
    p = P(fa.FA_PLAN_FWD, 4, 16, 2048, 2048, 64, num_cu=1024)  # 1024 tiles < 2 x 1024: unpaired
    assert (p["paired"], p["groups"]) == (False, 1024)
    p = P(fa.FA_PLAN_FWD, 1, 32, 8192, 8192, 128, causal=False)
    assert (p["kernel"], p["paired"], p["groups"]) == ("bf16_8wave", False, 1024)


def test_plan_fp32_key_split_switch():
    f32 = fa.FA_DTYPE_F32
    p = P(fa.FA_PLAN_FWD, 1, 1, 256, 256, 64, causal=False, dtype=f32)  # 2 row groups < 256 CUs
    assert (p["kernel"], p["waves_per_group"], p["rows_per_group"], p["groups"]) == ("f32_keysplit", 8, 32, 8)
    p = P(fa.FA_PLAN_FWD, 1, 1, 256, 256, 64, causal=False, dtype=f32, num_cu=2)  # 2 >= 2: whole rows
    assert (p["kernel"], p["rows_per_group"], p["groups"]) == ("f32_rows", 128, 2)
    p = P(fa.FA_PLAN_FWD, 2, 128, 128, 128, 128, dtype=f32)  # 256 groups: whole rows
    assert p["kernel"] == "f32_rows"


def test_plan_split_counts_follow_the_cu_count():
    # chunked prefill: 1000 queries x 32 heads = 256 units of 128 rows
    assert P(fa.FA_PLAN_FWD_SPLIT, 1, 32, 1000, 8192, 128)["num_splits"] == 2
    assert P(fa.FA_PLAN_FWD_SPLIT, 1, 32, 1000, 8192, 128, num_cu=64)["num_splits"] == 1
    assert P(fa.FA_PLAN_FWD_SPLIT, 1, 32, 1000, 8192, 128, num_cu=4096)["num_splits"] == 16  # 8192 / 512 cap
    p = P(fa.FA_PLAN_FWD_SPLIT, 1, 32, 1000, 8192, 128, num_splits=5)
    assert (p["kernel"], p["num_splits"], p["groups"]) == ("bf16_split", 5, 32 * 8 * 5)
    # decode: eight (b, h, split) groups per CU, no split under 256 keys
    assert P(fa.FA_PLAN_DECODE, 64, 32, 1, 8192, 128)["num_splits"] == 1
    assert P(fa.FA_PLAN_DECODE, 64, 32, 1, 8192, 128, num_cu=1024)["num_splits"] == 4
    assert P(fa.FA_PLAN_DECODE, 1, 8, 1, 8192, 128)["num_splits"] == 32  # capped by 8192 / 256
    p = P(fa.FA_PLAN_DECODE, 64, 32, 1, 8192, 128, num_splits=16)
    assert (p["kernel"], p["groups"], p["num_splits"]) == ("decode_split", 64 * 32 * 16, 16)


def test_plan_backward_pairing():
    dq = P(fa.FA_PLAN_BWD_DQ, 1, 32, 8192, 8192, 128)
    dkdv = P(fa.FA_PLAN_BWD_DKDV, 1, 32, 8192, 8192, 128)
    assert (dq["rows_per_group"], dq["paired"], dq["groups"]) == (128, True, 32 * 32)
    assert (dkdv["waves_per_group"], dkdv["rows_per_group"], dkdv["paired"], dkdv["groups"]) == (8, 256, True, 32 * 16)
    dkdv = P(fa.FA_PLAN_BWD_DKDV, 1, 32, 8192, 8192, 128, num_cu=1024)
    assert (dkdv["paired"], dkdv["groups"]) == (False, 32 * 32)


def test_plan_rejects_what_the_entry_points_reject():
    with pytest.raises(fa.FaError):
        P(fa.FA_PLAN_FWD, 1, 1, 8, 8, 96)
    with pytest.raises(fa.FaError):
        P(fa.FA_PLAN_DECODE, 1, 1, 1, 8, 64, dtype=fa.FA_DTYPE_F32)
    with pytest.raises(fa.FaError):
        P(fa.FA_PLAN_FWD, 0, 1, 8, 8, 64)
