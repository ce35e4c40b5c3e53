"""GPU parity: the HIP path (through the C ABI binding) against the CPU oracle.

Bar: layout, slot indices and dispatched bytes bit-exact; fp8 codes and scales
exact (they are part of the dispatched bytes); combine within 1 bf16 ulp
(|err| <= 2^-7 |ref|), and expected bit-exact since both sides round the same
fp32 mul-then-add sequence once. Inputs are the seeded workloads at full size
with the bench's channel count, plus tiny adversarial tables. Windows and
outputs are poisoned before each call so unwritten bytes show up.
"""

import functools
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, draw_expert_out, f32_to_bf16_input, make_inputs, random_tiny_routing

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
POISON = 0xAB
LAYOUT_KEYS = [
    "is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert", "rank_prefix_matrix",
    "expert_prefix_matrix", "rank_slot_base", "expert_slot_base", "slot_idx",
]


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import combine_moe_layout_02_amd as m

    return m


@functools.lru_cache(maxsize=None)
def inputs(cfg):
    """x, topk_idx, topk_weights of a workload (kept for the whole module)."""
    return make_inputs(WORKLOADS[cfg], with_expert_out=False)


@functools.lru_cache(maxsize=1)
def expert_out(cfg):
    w = WORKLOADS[cfg]
    return draw_expert_out(w.seed + 1000, w.S * w.K, w.H)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_dev(bits):
    return to_dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def poisoned_layout(moe, S, K, E, P, C):
    out = moe.empty_layout(S, K, E, P, C, DEV)
    for t in out:
        t.view(torch.uint8).fill_(POISON)
    return out


def gpu_layout(moe, idx, E, P, C, path=None):
    S, K = idx.shape
    lay = moe.moe_layout(to_dev(idx), E, P, C, out=poisoned_layout(moe, S, K, E, P, C), path=path)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in lay._asdict().items()}


def assert_layout_equal(got, ref, what=""):
    for key in LAYOUT_KEYS:
        g = got[key].astype(np.uint8) if key == "is_token_in_rank" else got[key]
        if not np.array_equal(g, ref[key]):
            bad = np.argwhere(g != ref[key])[:5]
            raise AssertionError(f"{what} {key} differs at {bad.tolist()}")
    assert int(got["status"][0]) == ref["status"], what


def checked_layout(moe, idx, E, P, C, path=None):
    """The HIP layout of the host table idx (device tensors, for later HIP calls) and the oracle's
    layout of the same table, after asserting that the two agree on every output. Expected values
    downstream are computed from the oracle's layout only."""
    S, K = idx.shape
    lay = moe.moe_layout(to_dev(idx), E, P, C, out=poisoned_layout(moe, S, K, E, P, C), path=path)
    torch.cuda.synchronize()
    ref = oracle.layout(idx, E, P, C)
    assert_layout_equal({k: v.cpu().numpy() for k, v in lay._asdict().items()}, ref, "chained layout")
    return lay, ref


def gpu_dispatch(moe, x_bits, slot, quant, src_rank=0):
    S, H = x_bits.shape
    K = slot.shape[1]
    win = torch.full((moe.moe_window_bytes(S, K, H),), POISON, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(bf16_dev(x_bits), to_dev(slot), win, quant, src_rank)
    torch.cuda.synchronize()
    return win.cpu().numpy().reshape(S * K, -1)


def assert_window_equal(win, ref_regions, geom, what=""):
    n = ref_regions.shape[0]
    got = win[:n, : geom.tail_end]
    if not np.array_equal(got, ref_regions):
        s, b = np.argwhere(got != ref_regions)[0]
        raise AssertionError(f"{what} slot {s} byte {b}: gpu {got[s, b]:#x} oracle {ref_regions[s, b]:#x}")
    assert np.all(win[:n, geom.tail_end:] == POISON), f"{what} wrote past tail_end"
    assert np.all(win[n:] == POISON), f"{what} wrote an unused slot"


def gpu_combine(moe, rows_bits, slot, w):
    y = moe.moe_combine(bf16_dev(rows_bits), to_dev(slot), to_dev(w))
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bf16_within_ulp(got, ref, what=""):
    g = oracle.bf16_bits_to_f32(got).astype(np.float64)
    r = oracle.bf16_bits_to_f32(ref).astype(np.float64)
    err = np.abs(g - r)
    ok = err <= np.abs(r) * 2.0**-7
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what} at {i.tolist()}: gpu {g[tuple(i)]} oracle {r[tuple(i)]}")


# ---------------------------------------------------------------- layout


# Small tables go to the single-launch layout under MOE_LAYOUT_AUTO; MOE_LAYOUT_MULTI forces the
# three-launch form. The tests run both on the same inputs through moe_layout_ex /
# moe_layout_dispatch_ex.
LAYOUT_PATHS = {"auto": 0, "three_launch": 1}


@pytest.fixture(params=sorted(LAYOUT_PATHS))
def layout_path(request):
    return LAYOUT_PATHS[request.param]


@pytest.mark.parametrize("cfg", sorted(WORKLOADS))
def test_layout_workloads(moe, cfg, layout_path):
    w = WORKLOADS[cfg]
    idx = inputs(cfg)["topk_idx"]
    for C in sorted({w.C, 1, 3, min(w.S, 4096)}):
        note(f"layout cfg{cfg} {w.describe()} C={C} path={layout_path}")
        assert_layout_equal(gpu_layout(moe, idx, w.E, w.P, C, layout_path), oracle.layout(idx, w.E, w.P, C),
                            f"cfg{cfg} C={C}")


TINY_LAYOUTS = [
    # (S, K, E, P, C, p_mask, p_bad, seed)
    (1, 1, 1, 1, 1, 0.0, 0.0, 1),
    (5, 3, 6, 3, 2, 0.3, 0.0, 2),
    (37, 4, 12, 4, 3, 0.2, 0.1, 3),       # bad ids -> status bit 0
    (300, 16, 512, 1, 7, 0.1, 0.0, 4),    # K_MAX, E_MAX, one rank
    (257, 2, 384, 384, 257, 0.0, 0.0, 5),  # P_MAX, one expert per rank, C = S
    (1000, 8, 64, 8, 1, 0.05, 0.0, 6),    # one channel, many chunks
    (600, 6, 5, 5, 600, 0.5, 0.02, 7),    # heavy masking, duplicate-prone
    (512, 8, 256, 8, 128, 0.0, 0.0, 8),   # S*K = 4096: largest table of the single-launch path
    (513, 8, 256, 8, 128, 0.0, 0.0, 9),   # one token more: three launches
    (4096, 1, 16, 4, 1000, 0.1, 0.0, 14),  # S = 4096: 64 bitset words per rank row
    (64, 8, 512, 256, 64, 0.1, 0.05, 10),  # E at its maximum on the single-launch path
    (64, 4, 384, 384, 64, 0.1, 0.0, 12),  # P at its maximum on the single-launch path
    (2048, 2, 16, 4, 1024, 0.1, 0.0, 13),  # S*K = 4096 with C at its maximum (1024)
    (200, 3, 9, 3, 7, 0.0, 0.0, 11),      # S not a multiple of 64, ragged channels
]


@pytest.mark.parametrize("case", TINY_LAYOUTS)
def test_layout_tiny_adversarial(moe, case, layout_path):
    S, K, E, P, C, p_mask, p_bad, seed = case
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=p_mask, p_bad=p_bad)
    note(f"layout tiny {case} path={layout_path}")
    assert_layout_equal(gpu_layout(moe, idx, E, P, C, layout_path), oracle.layout(idx, E, P, C), str(case))


def test_layout_special_tables(moe, layout_path):
    S, K, E, P = 96, 4, 16, 4
    cases = {
        "all_masked": np.full((S, K), -1, np.int32),
        "one_expert": np.full((S, K), 5, np.int32),  # every entry to expert 5, duplicates in rows
        "empty_experts": np.tile(np.array([0, 1, 14, 15], np.int32), (S, 1)),
        "all_bad": np.full((S, K), E + 3, np.int32),
    }
    for name, idx in cases.items():
        for C in (1, 3, S):
            note(f"layout special {name} C={C} path={layout_path}")
            assert_layout_equal(gpu_layout(moe, idx, E, P, C, layout_path), oracle.layout(idx, E, P, C), name)


# ---------------------------------------------------------------- layout + dispatch in one call


def gpu_layout_dispatch(moe, idx, x_bits, E, P, C, quant, src_rank=0, path=None):
    S, K = idx.shape
    H = x_bits.shape[1]
    win = torch.full((moe.moe_window_bytes(S, K, H),), POISON, dtype=torch.uint8, device=DEV)
    lay = moe.moe_layout_dispatch(to_dev(idx), E, P, C, bf16_dev(x_bits), win, quant, src_rank,
                                  out=poisoned_layout(moe, S, K, E, P, C), path=path)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in lay._asdict().items()}, win.cpu().numpy().reshape(S * K, -1)


def check_layout_dispatch(moe, idx, x_bits, E, P, C, quant, src_rank, what, path=None):
    got, win = gpu_layout_dispatch(moe, idx, x_bits, E, P, C, quant, src_rank, path)
    ref = oracle.layout(idx, E, P, C)
    assert_layout_equal(got, ref, what)
    H = x_bits.shape[1]
    assert_window_equal(win, oracle.dispatch_slots(x_bits, ref["slot_idx"], quant, src_rank),
                        oracle.slot_geometry(H, quant), what)


@pytest.mark.parametrize("cfg,quant", [(1, 0), (1, 1), (2, 0), (2, 1), (2, 2), (3, 0)])
def test_layout_dispatch_workloads(moe, cfg, quant, layout_path):
    """One call for the layout and the pack: one kernel at workloads 1 and 2, the separate kernels
    at workload 3 (and everywhere with MOE_LAYOUT_MULTI)."""
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    note(f"layout_dispatch cfg{cfg} quant {quant} path={layout_path}")
    check_layout_dispatch(moe, inp["topk_idx"], inp["x"], w.E, w.P, w.C, quant, 5,
                          f"cfg{cfg} quant {quant}", layout_path)


FUSED_CASES = [
    # (S, K, H, E, P, C, quant, p_mask, p_bad, seed)
    (1, 1, 16, 1, 1, 1, 0, 0.0, 0.0, 31),
    (5, 3, 48, 6, 3, 2, 1, 0.3, 0.0, 32),
    (37, 4, 2064, 12, 4, 3, 2, 0.2, 0.1, 33),      # bad ids: status bit 0, no slot
    (300, 13, 1024, 512, 1, 7, 0, 0.1, 0.0, 34),   # E at its maximum, one rank
    (512, 8, 7168, 256, 8, 128, 0, 0.0, 0.0, 35),  # S*K = 4096: the largest one-kernel table
    (512, 8, 7168, 256, 8, 128, 1, 0.05, 0.0, 36),
    (513, 8, 1024, 256, 8, 128, 2, 0.0, 0.0, 37),  # one token more: separate kernels
    (4096, 1, 256, 16, 4, 1000, 1, 0.1, 0.0, 38),  # 4096 tokens over 256 pack workgroups
    (4096, 1, 256, 16, 4, 1000, 0, 0.1, 0.0, 39),
    (64, 8, 7168, 512, 256, 64, 1, 0.1, 0.05, 40),
    (128, 16, 16384, 64, 8, 128, 0, 0.0, 0.0, 41),  # largest H and K: row split in 2 parts
    (128, 16, 16384, 64, 8, 128, 2, 0.2, 0.0, 42),
    (200, 3, 4112, 9, 3, 7, 0, 0.0, 0.0, 43),       # ragged channels, H not a multiple of 512 B
    (256, 4, 2048, 32, 4, 128, 1, 0.1, 0.02, 44),   # S*K = 1024, fp8 with masked and bad ids
    (205, 5, 2048, 64, 8, 64, 0, 0.1, 0.0, 45),     # odd K, S*K = 1025
    (96, 4, 64, 16, 4, 3, 0, 1.0, 0.0, 44),         # everything masked: nothing written
]


@pytest.mark.parametrize("case", FUSED_CASES)
def test_layout_dispatch_tiny(moe, case, layout_path):
    S, K, H, E, P, C, quant, p_mask, p_bad, seed = case
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=p_mask, p_bad=p_bad)
    x = rng.standard_normal((S, H)).astype(np.float32) * 3
    x[0, :] = 0.0
    xb = f32_to_bf16_input(x)
    note(f"layout_dispatch tiny {case} path={layout_path}")
    check_layout_dispatch(moe, idx, xb, E, P, C, quant, seed, str(case), layout_path)


# ---------------------------------------------------------------- dispatch


@pytest.mark.parametrize("cfg", sorted(WORKLOADS))
def test_dispatch_workloads(moe, cfg):
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    slot = oracle.layout(inp["topk_idx"], w.E, w.P, w.C)["slot_idx"]
    note(f"dispatch cfg{cfg} {w.describe()}")
    win = gpu_dispatch(moe, inp["x"], slot, w.quant)
    ref = oracle.dispatch_slots(inp["x"], slot, w.quant, 0)
    assert_window_equal(win, ref, oracle.slot_geometry(w.H, w.quant), f"cfg{cfg}")


def test_dispatch_fp8_on_bf16_workload(moe):
    """The fp8 pack on the plain N(0,1) prefill rows as well."""
    w = WORKLOADS[3]
    inp = inputs(3)
    slot = oracle.layout(inp["topk_idx"], w.E, w.P, w.C)["slot_idx"]
    note("dispatch fp8 on cfg3 rows")
    win = gpu_dispatch(moe, inp["x"], slot, 1)
    assert_window_equal(win, oracle.dispatch_slots(inp["x"], slot, 1, 0),
                        oracle.slot_geometry(w.H, 1), "fp8 cfg3")


@pytest.mark.parametrize("cfg", [3, 4])
def test_dispatch_int8_workloads(moe, cfg):
    """INT8 dynamic quant (the pages' own quantised type) on the prefill and outlier rows."""
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    slot = oracle.layout(inp["topk_idx"], w.E, w.P, w.C)["slot_idx"]
    note(f"dispatch int8 cfg{cfg}")
    win = gpu_dispatch(moe, inp["x"], slot, 2)
    assert_window_equal(win, oracle.dispatch_slots(inp["x"], slot, 2, 0),
                        oracle.slot_geometry(w.H, 2), f"int8 cfg{cfg}")


TINY_DISPATCH = [
    # (S, K, H, E, P, quant, seed)
    (1, 1, 16, 1, 1, 0, 1),
    (1, 1, 16, 1, 1, 1, 2),
    (1, 1, 16, 1, 1, 2, 12),
    (9, 3, 48, 6, 3, 2, 13),
    (33, 5, 2064, 10, 5, 2, 14),
    (6, 16, 16384, 32, 4, 2, 15),
    (9, 3, 48, 6, 3, 1, 3),        # fp8 payload 48 B: 16-byte pad before the scale block
    (33, 5, 2064, 10, 5, 0, 4),    # H not a multiple of the workgroup's vector stride
    (33, 5, 2064, 10, 5, 1, 5),
    (6, 16, 16384, 32, 4, 0, 6),   # MOE_MAX_HIDDEN, K_MAX
    (6, 16, 16384, 32, 4, 1, 7),
    (70, 2, 1024, 4, 2, 1, 8),
]


@pytest.mark.parametrize("case", TINY_DISPATCH)
def test_dispatch_tiny(moe, case):
    S, K, H, E, P, quant, seed = case
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=0.2)
    x = rng.standard_normal((S, H)).astype(np.float32) * 4
    x[0, :] = 0.0  # an all-zero row: fp8 scale 0, codes 0
    if S > 2:
        x[1, 3] = 1e4  # an outlier
        x[2, :] = -0.0
    xb = f32_to_bf16_input(x)
    slot = oracle.layout(idx, E, P, 1)["slot_idx"]
    note(f"dispatch tiny {case}")
    win = gpu_dispatch(moe, xb, slot, quant, src_rank=seed)
    assert_window_equal(win, oracle.dispatch_slots(xb, slot, quant, seed),
                        oracle.slot_geometry(H, quant), str(case))


LARGE_DISPATCH = [
    # (S, K, H, E, P, p_mask, seed): bf16 windows of 16k+ slots with rows of 4096+ elements
    (2100, 8, 4096, 64, 8, 0.1, 91),
    (2300, 8, 7200, 40, 8, 0.05, 92),    # 900 vectors per row: a ragged last part
    (2049, 8, 16384, 256, 8, 0.0, 93),   # MOE_MAX_HIDDEN
    (1100, 16, 7168, 128, 16, 0.2, 94),  # K at its maximum
    (3001, 6, 4112, 48, 4, 0.1, 95),
]


@pytest.mark.parametrize("case", LARGE_DISPATCH)
def test_dispatch_large_shapes(moe, case):
    S, K, H, E, P, p_mask, seed = case
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=p_mask)
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32) * 2)
    slot = oracle.layout(idx, E, P, min(S, 128))["slot_idx"]
    note(f"dispatch large {case}")
    win = gpu_dispatch(moe, xb, slot, 0, src_rank=seed)
    assert_window_equal(win, oracle.dispatch_slots(xb, slot, 0, seed), oracle.slot_geometry(H, 0), str(case))


def test_dispatch_large_any_slot_table(moe):
    """A random permutation of the slots of a 16k-slot window, -1 pads and entries past S*K."""
    rng = np.random.default_rng(96)
    S, K, H = 2048, 8, 4096
    slot = np.full((S, K), -1, np.int32)
    keep = rng.random((S, K)) < 0.9
    n = int(keep.sum())
    slot[keep] = rng.permutation(n).astype(np.int32)
    far = (~keep) & (rng.random((S, K)) < 0.5)
    slot[far] = S * K + rng.integers(0, 1000, int(far.sum())).astype(np.int32)
    x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    note(f"dispatch large permuted slots: {n} used, {int(far.sum())} out of range")
    win = gpu_dispatch(moe, x, slot, 0, src_rank=4)
    ref = oracle.dispatch_slots(x, np.where(slot < S * K, slot, -1), 0, 4)
    assert_window_equal(win, ref, oracle.slot_geometry(H, 0), "large permuted")


def every_bf16_rows(amax_bits, H):
    """Rows that pass every finite bf16 value of magnitude <= amax through the quantiser with the
    row maximum amax: per amax, element 0 of each row is +-amax and the rest of the rows hold all
    such values (both signs, -0.0 included), zero-filled at the end."""
    finite = np.arange(1 << 16, dtype=np.uint32)
    finite = finite[(finite & 0x7F80) != 0x7F80].astype(np.uint16)
    mag = (finite.astype(np.uint32) << 16).view(np.float32)
    rows = []
    for i, ab in enumerate(amax_bits):
        amax = float((np.uint32(ab) << 16).view(np.float32))
        vals = finite[np.abs(mag) <= amax]
        per = H - 1
        for r0 in range(0, vals.size, per):
            row = np.zeros(H, np.uint16)
            row[0] = ab | (0x8000 if (r0 // per + i) % 2 else 0)
            chunk = vals[r0 : r0 + per]
            row[1 : 1 + chunk.size] = chunk
            rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("quant", [1, 2])
def test_dispatch_quant_every_bf16_value(moe, quant):
    """Every finite bf16 value under row maxima that put the scale on a power of two (amax 448 or
    127: the quotient is x itself), at the largest bf16, near the smallest scale of the reciprocal
    division (448 * 2^-90 and one bf16 step either side) and far below it (subnormal amax), and at
    random bf16 values. Codes and scales must equal the oracle's bit for bit."""
    top = 448.0 if quant == 1 else 127.0
    special = [top, top * 2.0 ** -90, top * 2.0 ** 60, 3.3895313892515355e38, 2.0 ** -133, 1e-30]
    bits = list(f32_to_bf16_input(np.array(special, np.float32)).astype(np.uint32))
    edge = int(f32_to_bf16_input(np.array([top * 2.0 ** -90], np.float32))[0])
    bits += [edge - 1, edge + 1]
    rng = np.random.default_rng(40 + quant)
    bits += list(rng.integers(0x0080, 0x7F7F, 10))
    H = 8192
    xb = every_bf16_rows([int(b) & 0x7FFF for b in bits], H)
    S = xb.shape[0]
    slot = np.arange(S, dtype=np.int32).reshape(S, 1)
    note(f"dispatch every bf16 value quant {quant}: S={S} H={H}")
    win = gpu_dispatch(moe, xb, slot, quant)
    assert_window_equal(win, oracle.dispatch_slots(xb, slot, quant, 0),
                        oracle.slot_geometry(H, quant), f"every bf16 quant {quant}")


@pytest.mark.parametrize("quant", [0, 1, 2])
def test_dispatch_any_slot_table(moe, quant):
    """moe_dispatch takes any table of distinct slots, not only a layout's: a random permutation of
    [0, N) over the valid entries, with -1 pads and entries at or past S*K, which are skipped."""
    rng = np.random.default_rng(81 + quant)
    S, K, H = 150, 5, 2064
    slot = np.full((S, K), -1, np.int32)
    keep = rng.random((S, K)) < 0.8
    n = int(keep.sum())
    slot[keep] = rng.permutation(n).astype(np.int32)
    far = (~keep) & (rng.random((S, K)) < 0.5)
    slot[far] = S * K + rng.integers(0, 1000, int(far.sum())).astype(np.int32)
    x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32) * 3)
    note(f"dispatch permuted slots quant {quant}: {n} used, {int(far.sum())} out of range")
    win = gpu_dispatch(moe, x, slot, quant, src_rank=9)
    ref = oracle.dispatch_slots(x, np.where(slot < S * K, slot, -1), quant, 9)
    assert_window_equal(win, ref, oracle.slot_geometry(H, quant), f"permuted quant {quant}")


def test_dispatch_bf16_copies_non_finite_bits(moe):
    """The bf16 pack is a byte copy: infinities and NaN payloads (quiet and signalling bit
    patterns) arrive unchanged."""
    rng = np.random.default_rng(78)
    S, K, H, E = 40, 4, 512, 8
    idx = random_tiny_routing(rng, S, K, E, p_mask=0.1)
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x7FFF, 0x8000], np.uint16)
    pick = rng.random((S, H)) < 0.05
    xb[pick] = rng.choice(specials, size=int(pick.sum()))
    slot = oracle.layout(idx, E, 2, 1)["slot_idx"]
    note("dispatch bf16 non-finite bits")
    win = gpu_dispatch(moe, xb, slot, 0, src_rank=1)
    assert_window_equal(win, oracle.dispatch_slots(xb, slot, 0, 1), oracle.slot_geometry(H, 0), "non-finite bf16")


# ---------------------------------------------------------------- dispatch with a workspace (planned pack)


def gpu_dispatch_ws(moe, x_bits, slot, quant, src_rank=0, ws_poison=0x5C):
    S, H = x_bits.shape
    K = slot.shape[1]
    win = torch.full((moe.moe_window_bytes(S, K, H),), POISON, dtype=torch.uint8, device=DEV)
    nws = moe.moe_dispatch_workspace_bytes(S, K, quant)
    ws = torch.full((max(nws, 16),), ws_poison, dtype=torch.uint8, device=DEV) if nws else None
    moe.moe_dispatch_ws(bf16_dev(x_bits), to_dev(slot), win, ws, quant, src_rank)
    torch.cuda.synchronize()
    return win.cpu().numpy().reshape(S * K, -1)


@pytest.mark.parametrize("cfg,quant", [(1, 0), (2, 0), (3, 0), (4, 1), (4, 0), (5, 0), (3, 2)])
def test_dispatch_ws_workloads(moe, cfg, quant):
    """moe_dispatch_ws on the workloads: the planned pack at workloads 3-5 in bf16, the token-order
    pack elsewhere; window bytes equal to the oracle's, nothing else written."""
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    slot = oracle.layout(inp["topk_idx"], w.E, w.P, w.C)["slot_idx"]
    note(f"dispatch_ws cfg{cfg} quant {quant}")
    win = gpu_dispatch_ws(moe, inp["x"], slot, quant, src_rank=2)
    assert_window_equal(win, oracle.dispatch_slots(inp["x"], slot, quant, 2), oracle.slot_geometry(w.H, quant),
                        f"ws cfg{cfg} quant {quant}")


PLANNED_DISPATCH = [
    # (S, K, H, E, P, p_mask, p_bad_slot, seed): bf16 tables of 8192+ entries take the planned pack
    (1024, 8, 7168, 256, 8, 0.0, 0.0, 101),    # S*K = 8192: the smallest planned table
    (1023, 8, 1024, 64, 8, 0.0, 0.0, 102),     # S*K = 8184: token order
    (8192, 1, 2048, 16, 4, 0.1, 0.0, 103),     # K = 1: chunks of 1024 tokens
    (3001, 3, 4112, 48, 4, 0.1, 0.02, 104),    # K = 3 (chunks of 256 tokens), ragged last chunk and part
    (600, 16, 7168, 128, 16, 0.2, 0.0, 105),   # K at its maximum: chunks of 64 tokens
    (2049, 8, 16384, 256, 8, 0.0, 0.0, 106),   # MOE_MAX_HIDDEN: 16 parts per row
    (1700, 5, 16, 40, 8, 0.3, 0.05, 107),      # smallest H: one part, mostly tail
    (9000, 8, 64, 256, 8, 1.0, 0.0, 108),      # everything masked: nothing written
]


@pytest.mark.parametrize("case", PLANNED_DISPATCH)
def test_dispatch_ws_planned_shapes(moe, case):
    """Planned-pack chunking at the edges: K in {1, 3, 5, 8, 16}, ragged chunks, masked entries and
    entries at or past S*K in the slot table, H from 16 to 16384."""
    S, K, H, E, P, p_mask, p_bad, seed = case
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=p_mask)
    slot = oracle.layout(idx, E, P, min(S, 128))["slot_idx"]
    far = (slot < 0) & (rng.random((S, K)) < p_bad * 10)
    slot = slot.copy()
    slot[far] = S * K + rng.integers(0, 1000, int(far.sum())).astype(np.int32)
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    note(f"dispatch_ws planned {case}")
    win = gpu_dispatch_ws(moe, xb, slot, 0, src_rank=seed)
    ref = oracle.dispatch_slots(xb, np.where(slot < S * K, slot, -1), 0, seed)
    assert_window_equal(win, ref, oracle.slot_geometry(H, 0), str(case))


def test_dispatch_ws_any_slot_table_and_reused_workspace(moe):
    """A random permutation of the slots (not a layout's order) through the planned pack, twice with
    the same workspace, the second time after the workspace was overwritten: identical windows."""
    rng = np.random.default_rng(109)
    S, K, H = 2048, 8, 4096
    slot = np.full((S, K), -1, np.int32)
    keep = rng.random((S, K)) < 0.9
    n = int(keep.sum())
    slot[keep] = rng.permutation(n).astype(np.int32)
    x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    ws = torch.full((moe.moe_dispatch_workspace_bytes(S, K),), 0x11, dtype=torch.uint8, device=DEV)
    ref = oracle.dispatch_slots(x, slot, 0, 4)
    geo = oracle.slot_geometry(H, 0)
    xd, sd = bf16_dev(x), to_dev(slot)
    for rep in range(2):
        win = torch.full((moe.moe_window_bytes(S, K, H),), POISON, dtype=torch.uint8, device=DEV)
        moe.moe_dispatch_ws(xd, sd, win, ws, 0, 4)
        torch.cuda.synchronize()
        note(f"dispatch_ws permuted slots, rep {rep}")
        assert_window_equal(win.cpu().numpy().reshape(S * K, -1), ref, geo, f"permuted rep {rep}")
        ws.fill_(0xEE)


# ---------------------------------------------------------------- layout + dispatch with a workspace


def gpu_layout_dispatch_ws(moe, idx, x_bits, E, P, C, quant, src_rank=0, path=None, ws=None, ws_poison=0x5C,
                           split=False):
    """moe_layout_dispatch_ws, or (split) moe_layout_ws then moe_dispatch_planned on the same workspace."""
    S, K = idx.shape
    H = x_bits.shape[1]
    path = 0 if path is None else path
    win = torch.full((moe.moe_window_bytes(S, K, H),), POISON, dtype=torch.uint8, device=DEV)
    if ws is None:
        nws = moe.moe_layout_dispatch_workspace_bytes(S, K, E, P, C, quant, path)
        ws = torch.full((nws,), ws_poison, dtype=torch.uint8, device=DEV) if nws else None
    out = poisoned_layout(moe, S, K, E, P, C)
    if split:
        lay = moe.moe_layout_ws(to_dev(idx), E, P, C, ws, quant, out=out, path=path)
        moe.moe_dispatch_planned(bf16_dev(x_bits), lay.slot_idx, win, ws, C, quant, src_rank)
    else:
        lay = moe.moe_layout_dispatch_ws(to_dev(idx), E, P, C, bf16_dev(x_bits), win, ws, quant, src_rank, out=out,
                                         path=path)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in lay._asdict().items()}, win.cpu().numpy().reshape(S * K, -1)


def check_layout_dispatch_ws(moe, idx, x_bits, E, P, C, quant, src_rank, what, path=None, ws=None, split=False):
    got, win = gpu_layout_dispatch_ws(moe, idx, x_bits, E, P, C, quant, src_rank, path, ws, split=split)
    ref = oracle.layout(idx, E, P, C)
    assert_layout_equal(got, ref, what)
    H = x_bits.shape[1]
    assert_window_equal(win, oracle.dispatch_slots(x_bits, ref["slot_idx"], quant, src_rank),
                        oracle.slot_geometry(H, quant), what)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("cfg,quant", [(1, 0), (2, 0), (3, 0), (3, 1), (4, 1), (5, 0), (5, 2)])
def test_layout_dispatch_ws_workloads(moe, cfg, quant, layout_path, split):
    """moe_layout_dispatch_ws (or moe_layout_ws + moe_dispatch_planned) on the workloads: the two-launch
    layout writing the pack's plan at workloads 3 and 5 in bf16 (one batch per channel at 3, two at
    5), the token-order pack in fp8 and int8."""
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    note(f"layout_dispatch_ws cfg{cfg} quant {quant} path={layout_path} split={split}")
    check_layout_dispatch_ws(moe, inp["topk_idx"], inp["x"], w.E, w.P, w.C, quant, 3,
                             f"ws cfg{cfg} quant {quant}", layout_path, split=split)


LAYOUT_DISPATCH_WS = [
    # (S, K, H, E, P, C, quant, p_mask, p_bad, seed)
    (4096, 8, 1024, 256, 8, 1, 0, 0.0, 0.0, 201),      # one channel of 32768 entries: plan kernel
    (4096, 8, 1024, 256, 8, 16, 0, 0.05, 0.01, 202),   # 2048 entries per channel: plan kernel
    (4096, 8, 1024, 256, 8, 32, 0, 0.05, 0.01, 203),   # 1024 entries per channel: one per group
    (4096, 8, 1024, 256, 8, 4096, 0, 0.1, 0.0, 204),   # a token per channel: 128 channels a group
    (3001, 3, 4112, 48, 4, 77, 0, 0.1, 0.02, 205),     # K = 3, ragged channels and row part
    (600, 16, 7168, 128, 16, 40, 0, 0.2, 0.0, 206),    # K = 16: 15 tokens per channel
    (2049, 8, 2048, 512, 128, 100, 0, 0.1, 0.05, 207),  # E at its maximum, bad ids (status 1)
    (1536, 8, 256, 384, 384, 96, 0, 0.0, 0.0, 208),    # P at its maximum
    (8192, 1, 2048, 16, 4, 8, 0, 0.1, 0.0, 209),       # K = 1, 1024 tokens per channel
    (1700, 5, 16, 40, 8, 33, 0, 0.3, 0.05, 210),       # smallest H
    (9000, 8, 64, 256, 8, 128, 0, 1.0, 0.0, 211),      # everything masked: nothing written
    (1000, 8, 1024, 64, 8, 128, 0, 0.0, 0.0, 212),     # S*K = 8000: token-order pack, two launches
    (2048, 8, 2048, 256, 8, 64, 2, 0.05, 0.01, 213),   # int8 codes
    (65536, 2, 64, 64, 8, 4096, 0, 0.0, 0.0, 214),     # maximum S and C
]


@pytest.mark.parametrize("case", LAYOUT_DISPATCH_WS)
def test_layout_dispatch_ws_shapes(moe, case):
    """The two-launch layout at its edges: one channel (several batches; the separate plan kernel),
    a token per channel, K in {1, 3, 5, 8, 16}, E and P at their maxima, bad and masked ids."""
    S, K, H, E, P, C, quant, p_mask, p_bad, seed = case
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=p_mask, p_bad=p_bad)
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    note(f"layout_dispatch_ws {case}")
    check_layout_dispatch_ws(moe, idx, xb, E, P, C, quant, seed, str(case), path=1, split=seed % 2 == 0)


def test_layout_ws_at_the_maxima(moe):
    """moe_layout_ws + moe_dispatch_planned at S = MOE_MAX_TOKENS, K = MOE_MAX_K, E = MOE_MAX_EXPERTS and
    C = MOE_MAX_CHANNELS (16 tokens a channel: the layout writes 64 groups of 4 channels per XCD list),
    with masked and bad ids: every layout output and the window equal to the oracle's."""
    rng = np.random.default_rng(301)
    S, K, E, P, C, H = 65536, 16, 512, 256, 4096, 16  # the header's MOE_MAX_* limits
    idx = random_tiny_routing(rng, S, K, E, p_mask=0.02, p_bad=0.001)
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    note("layout_ws at the maxima")
    check_layout_dispatch_ws(moe, idx, xb, E, P, C, 0, 5, "maxima", split=True)


def test_layout_dispatch_ws_reused_workspace(moe):
    """Two tables through one workspace, the second after the workspace was overwritten, and the
    first again: every output equal to the oracle's each time."""
    rng = np.random.default_rng(215)
    S, K, H, E, P, C = 2048, 8, 2048, 256, 8, 64
    ws = torch.full((moe.moe_layout_dispatch_workspace_bytes(S, K, E, P, C),), 0x11, dtype=torch.uint8,
                    device=DEV)
    tables = [random_tiny_routing(rng, S, K, E, p_mask=0.1), random_tiny_routing(rng, S, K, E, p_mask=0.0)]
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    for rep, idx in enumerate(tables + tables[:1]):
        note(f"layout_dispatch_ws reused workspace, rep {rep}")
        check_layout_dispatch_ws(moe, idx, xb, E, P, C, 0, rep, f"rep {rep}", ws=ws)
        ws.fill_(0xEE)


def test_dispatch_all_masked_writes_nothing(moe):
    S, K, H = 8, 4, 64
    slot = np.full((S, K), -1, np.int32)
    xb = f32_to_bf16_input(np.ones((S, H), np.float32))
    for quant in (0, 1, 2):
        win = gpu_dispatch(moe, xb, slot, quant)
        assert np.all(win == POISON)


# ---------------------------------------------------------------- unpack


def run_unpack(moe, lay_slot, x_bits, S, K, H, E, quant, n_dev):
    """Dispatch with the given slots, then unpack; outputs poisoned beforehand."""
    win = torch.full((moe.moe_window_bytes(S, K, H),), POISON, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(bf16_dev(x_bits), to_dev(lay_slot), win, quant, 7)
    rows = S * K
    ex = torch.full((rows, H if quant else 2 * H), POISON, dtype=torch.uint8, device=DEV)
    sc = torch.full((rows,), -1.0, dtype=torch.float32, device=DEV) if quant else None
    idx = torch.full((rows, 3), -7, dtype=torch.int32, device=DEV)
    moe.moe_unpack(win, n_dev, S, K, H, quant, out=(ex, sc, idx))
    torch.cuda.synchronize()
    return ex.cpu().numpy(), None if sc is None else sc.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("cfg,quant", [(3, 0), (4, 1), (4, 2), (5, 0)])
def test_unpack_workloads(moe, cfg, quant):
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    lay, ref = checked_layout(moe, inp["topk_idx"], w.E, w.P, w.C)
    slot = ref["slot_idx"]
    note(f"unpack cfg{cfg} quant {quant}")
    ex, sc, idx = run_unpack(moe, slot, inp["x"], w.S, w.K, w.H, w.E, quant, lay.expert_slot_base[w.E:])
    rex, ridx, rsc = oracle.unpack(oracle.dispatch_slots(inp["x"], slot, quant, 7), w.H, quant)
    n = rex.shape[0]
    assert np.array_equal(ex[:n], rex) and np.array_equal(idx[:n], ridx)
    if quant:
        assert np.array_equal(sc[:n].view(np.uint32), rsc.view(np.uint32))


def test_unpack_partial_and_empty(moe):
    """N below S*K (masked entries) leaves the rows past N untouched; N = 0 writes nothing."""
    rng = np.random.default_rng(21)
    S, K, E, P, H = 50, 4, 12, 4, 2064
    idx_tab = random_tiny_routing(rng, S, K, E, p_mask=0.4)
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    for quant in (0, 1, 2):
        lay, ref = checked_layout(moe, idx_tab, E, P, 3)
        slot = ref["slot_idx"]
        n = int(ref["expert_slot_base"][E])
        ex, sc, idx = run_unpack(moe, slot, xb, S, K, H, E, quant, lay.expert_slot_base[E:])
        rex, ridx, rsc = oracle.unpack(oracle.dispatch_slots(xb, slot, quant, 7), H, quant)
        assert np.array_equal(ex[:n], rex) and np.array_equal(idx[:n], ridx)
        assert np.all(ex[n:] == POISON) and np.all(idx[n:] == -7)
        if quant:
            assert np.array_equal(sc[:n], rsc) and np.all(sc[n:] == -1.0)
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    ex, sc, idx = run_unpack(moe, np.full((S, K), -1, np.int32), xb, S, K, H, E, 0, zero)
    assert np.all(ex == POISON) and np.all(idx == -7)


def run_unpack_padded(moe, lay, x_bits, S, K, H, E, quant, A, R):
    """Dispatch with the layout's slots, then the padded unpack into poisoned outputs."""
    win = torch.full((moe.moe_window_bytes(S, K, H),), POISON, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(bf16_dev(x_bits), lay.slot_idx, win, quant, 3)
    i32 = dict(dtype=torch.int32, device=DEV)
    out = moe.PaddedUnpacked(
        torch.full((R, H if quant else 2 * H), POISON, dtype=torch.uint8, device=DEV),
        torch.full((R,), -1.0, dtype=torch.float32, device=DEV) if quant else None,
        torch.full((R, 3), -7, **i32), torch.full((E + 1,), -7, **i32), torch.full((1,), -7, **i32))
    moe.moe_unpack_padded(win, lay.expert_slot_base, S, K, H, quant, A, R, out=out)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy() for t in out]


def assert_padded_equal(got, ref, what):
    ex, sc, idx, base, status = got
    rex, ridx, rsc, rbase, rtrunc = ref
    assert np.array_equal(base, rbase), what
    assert int(status[0]) == int(rtrunc), what
    assert np.array_equal(idx, ridx), what
    assert np.array_equal(ex, rex), what
    if rsc is not None:
        assert np.array_equal(sc.view(np.uint32), rsc.view(np.uint32)), what


@pytest.mark.parametrize("cfg,quant", [(1, 0), (2, 1), (3, 0), (4, 2)])
def test_unpack_padded_workloads(moe, cfg, quant):
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    lay, ref_lay = checked_layout(moe, inp["topk_idx"], w.E, w.P, w.C)
    slot = ref_lay["slot_idx"]
    esb = ref_lay["expert_slot_base"]
    regions = oracle.dispatch_slots(inp["x"], slot, quant, 3)
    # (alignment, rows relative to the aligned total): exact fit, extra padding rows, truncation
    cases = [(1, 0), (16, 37), (128, -1000)] if w.S * w.K > 4096 else \
        [(a, d) for a in (1, 16, 128) for d in (0, 37, -1000)]
    for A, d in cases:
        total = int(oracle.aligned_row_base(esb, A)[-1])
        R = max(1, total + d)
        note(f"unpack_padded cfg{cfg} quant {quant} A={A} R={R} (aligned total {total})")
        got = run_unpack_padded(moe, lay, inp["x"], w.S, w.K, w.H, w.E, quant, A, R)
        ref = oracle.unpack_padded(regions, esb, w.H, quant, A, R)
        assert_padded_equal(got, ref, f"cfg{cfg} A={A} R={R}")


@pytest.mark.parametrize("H", [48, 2064])  # 2064: 258 bf16 vectors, the last 256-vector part ragged
def test_unpack_padded_tiny_and_degenerate(moe, H):
    """Masked entries, empty experts, R = 1, alignment larger than every count."""
    rng = np.random.default_rng(33)
    S, K, E, P = 40, 3, 12, 4
    tab = random_tiny_routing(rng, S, K, E, p_mask=0.3)
    tab[:, :] = np.where(np.isin(tab, [2, 3]), -1, tab)  # experts 2 and 3 receive nothing
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    lay, ref_lay = checked_layout(moe, tab, E, P, 3)
    slot = ref_lay["slot_idx"]
    esb = ref_lay["expert_slot_base"]
    for quant in (0, 1):
        regions = oracle.dispatch_slots(xb, slot, quant, 3)
        for A, R in ((1, 1), (5, 64), (64, 1000), (7, int(esb[-1])), (3, 17)):
            note(f"unpack_padded tiny quant {quant} A={A} R={R}")
            got = run_unpack_padded(moe, lay, xb, S, K, H, E, quant, A, R)
            ref = oracle.unpack_padded(regions, esb, H, quant, A, R)
            assert_padded_equal(got, ref, f"tiny quant {quant} A={A} R={R}")
    empty, _ = checked_layout(moe, np.full((S, K), -1, np.int32), E, P, 3)
    got = run_unpack_padded(moe, empty, xb, S, K, H, E, 0, 8, 20)
    assert np.all(got[2] == -1) and not got[0].any() and np.all(got[3] == 0) and got[4][0] == 0


# ---------------------------------------------------------------- per-rank deduplicated dispatch


def gpu_rank_rows(moe, idx, E, P, C, path=None):
    t = to_dev(idx)
    lay, _ = checked_layout(moe, idx, E, P, C, path)
    S, K = idx.shape
    out = moe.RankRows(torch.full((S, K), -7, dtype=torch.int32, device=DEV),
                       torch.full((P + 1,), -7, dtype=torch.int32, device=DEV))
    moe.moe_rank_rows(t, lay, E, P, C, out=out)
    torch.cuda.synchronize()
    return lay, out


@pytest.mark.parametrize("cfg", sorted(WORKLOADS))
def test_rank_rows_workloads(moe, cfg, layout_path):
    w = WORKLOADS[cfg]
    idx = inputs(cfg)["topk_idx"]
    ref_rr, ref_base = oracle.rank_rows(idx, w.E, w.P)
    for C in sorted({w.C, 1, 3}):
        note(f"rank_rows cfg{cfg} C={C} path={layout_path}")
        _, out = gpu_rank_rows(moe, idx, w.E, w.P, C, layout_path)
        assert np.array_equal(out.rank_row_idx.cpu().numpy(), ref_rr), C
        assert np.array_equal(out.rank_token_base.cpu().numpy(), ref_base), C


@pytest.mark.parametrize("case", TINY_LAYOUTS)
def test_rank_rows_tiny(moe, case):
    S, K, E, P, C, p_mask, p_bad, seed = case
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=p_mask, p_bad=p_bad)
    note(f"rank_rows tiny {case}")
    _, out = gpu_rank_rows(moe, idx, E, P, C)
    ref_rr, ref_base = oracle.rank_rows(idx, E, P)
    assert np.array_equal(out.rank_row_idx.cpu().numpy(), ref_rr)
    assert np.array_equal(out.rank_token_base.cpu().numpy(), ref_base)


def dedup_dispatch(moe, x_bits, idx, E, P, C, H, quant=0):
    S, K = idx.shape
    t = to_dev(idx)
    lay, rr = gpu_rank_rows(moe, idx, E, P, C)
    win = torch.full((moe.moe_dedup_window_bytes(S, K, P, H),), POISON, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch_dedup(bf16_dev(x_bits), rr.rank_row_idx, t, E, P, win, quant=quant, src_rank=5)
    torch.cuda.synchronize()
    return lay, rr, win


def check_expansion(moe, win, rr, lay, ref_slot, x_bits, E, P, H, quant, prefill=None):
    """Expand the dedup rows and compare with the oracle's unpack of the K-fold window built from
    the oracle's slots ref_slot (lay is the HIP layout of the same table, already checked)."""
    S, K = lay.slot_idx.shape
    out = prefill
    got = moe.moe_expand_dedup(win, rr.rank_row_idx, lay.slot_idx, lay.expert_slot_base[E:], P, H, quant,
                               out=out)
    torch.cuda.synchronize()
    rex, ridx, rsc = oracle.unpack(oracle.dispatch_slots(x_bits, ref_slot, quant, 5), H, quant)
    n = rex.shape[0]
    ex = got.expand_x.view(torch.uint8).cpu().numpy().reshape(S * K, -1)
    assert np.array_equal(ex[:n], rex)
    assert np.array_equal(got.expand_idx.cpu().numpy()[:n], ridx)
    if quant:
        assert np.array_equal(got.expand_scales.cpu().numpy()[:n].view(np.uint32), rsc.view(np.uint32))
    return got, n


@pytest.mark.parametrize("cfg,quant", [(1, 0), (2, 0), (3, 0), (5, 0), (2, 1), (4, 1), (4, 2)])
def test_dispatch_dedup_workloads(moe, cfg, quant):
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    note(f"dispatch_dedup cfg{cfg} quant {quant} {w.describe()}")
    lay, rr, win = dedup_dispatch(moe, inp["x"], inp["topk_idx"], w.E, w.P, w.C, w.H, quant)
    ref_rr, _ = oracle.rank_rows(inp["topk_idx"], w.E, w.P)
    ref = oracle.dispatch_dedup(inp["x"], ref_rr, inp["topk_idx"], w.E, w.P, src_rank=5, quant=quant)
    geo = oracle.slot_geometry(w.H, quant)
    m = ref.shape[0]
    rows = win.view(-1, geo.slot_bytes).cpu().numpy()
    assert np.array_equal(rows[:m, : geo.tail_end], ref)
    assert np.all(rows[m:] == POISON)  # rows past M untouched
    # expansion to expert-major rows equals the K-fold unpack
    ref_slot = oracle.layout(inp["topk_idx"], w.E, w.P, w.C)["slot_idx"]
    check_expansion(moe, win, rr, lay, ref_slot, inp["x"], w.E, w.P, w.H, quant)


def test_dedup_tiny_masks_duplicates_and_bad_ids(moe):
    rng = np.random.default_rng(61)
    for S, K, E, P, C, H in ((45, 6, 12, 4, 5, 32), (17, 16, 32, 32, 17, 64), (100, 3, 8, 1, 7, 48)):
        tab = random_tiny_routing(rng, S, K, E, p_mask=0.3, p_bad=0.05)
        x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
        for quant in (0, 1, 2):
            note(f"dedup tiny S={S} K={K} E={E} P={P} C={C} H={H} quant {quant}")
            lay, rr, win = dedup_dispatch(moe, x, tab, E, P, C, H, quant)
            ref_rr, _ = oracle.rank_rows(tab, E, P)
            assert np.array_equal(rr.rank_row_idx.cpu().numpy(), ref_rr)
            geo = oracle.slot_geometry(H, quant)
            if (ref_rr >= 0).any():
                ref = oracle.dispatch_dedup(x, ref_rr, tab, E, P, src_rank=5, quant=quant)
                rows = win.view(-1, geo.slot_bytes).cpu().numpy()
                assert np.array_equal(rows[: ref.shape[0], : geo.tail_end], ref)
            width = H if quant else 2 * H
            pre = moe.Unpacked(torch.full((S * K, width), 0xCD, dtype=torch.uint8, device=DEV),
                               torch.full((S * K,), -2.0, dtype=torch.float32, device=DEV) if quant else None,
                               torch.full((S * K, 3), -3, dtype=torch.int32, device=DEV))
            ref_slot = oracle.layout(tab, E, P, C)["slot_idx"]
            got, n = check_expansion(moe, win, rr, lay, ref_slot, x, E, P, H, quant, prefill=pre)
            assert np.all(got.expand_idx.cpu().numpy()[n:] == -3)  # rows past N keep their contents
            assert np.all(got.expand_x.cpu().numpy()[n:] == 0xCD)


@pytest.mark.parametrize("S,K,E,P,C", [(65536, 2, 64, 8, 4096), (1024, 4, 384, 384, 1024)])
def test_dedup_at_maximum_tokens_and_ranks(moe, S, K, E, P, C):
    """S = MOE_MAX_TOKENS with C = MOE_MAX_CHANNELS, then P = MOE_MAX_RANKS (one expert per
    rank): rank rows, the deduplicated fp8 pack and its expansion against the oracle on a small
    hidden size."""
    rng = np.random.default_rng(62)
    H = 16
    tab = random_tiny_routing(rng, S, K, E, p_mask=0.1, p_bad=0.01)
    x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    note(f"dedup at S={S} K={K} E={E} P={P} C={C}")
    lay, rr, win = dedup_dispatch(moe, x, tab, E, P, C, H, 1)
    ref_rr, ref_base = oracle.rank_rows(tab, E, P)
    assert np.array_equal(rr.rank_row_idx.cpu().numpy(), ref_rr)
    assert np.array_equal(rr.rank_token_base.cpu().numpy(), ref_base)
    ref = oracle.dispatch_dedup(x, ref_rr, tab, E, P, src_rank=5, quant=1)
    geo = oracle.slot_geometry(H, 1)
    rows = win.view(-1, geo.slot_bytes).cpu().numpy()
    assert np.array_equal(rows[: ref.shape[0], : geo.tail_end], ref)
    check_expansion(moe, win, rr, lay, oracle.layout(tab, E, P, C)["slot_idx"], x, E, P, H, 1)


def test_unpack_padded_at_its_limits(moe):
    """expert_alignment = MOE_MAX_ALIGNMENT and out_rows = MOE_MAX_OUT_ROWS: with 16 non-empty
    experts the aligned blocks fill the output exactly; with 17 the last block is cut (flag set)."""
    rng = np.random.default_rng(63)
    A, R = 65536, 1048576
    for E, P in ((16, 4), (17, 17)):
        S, K, H = 96, 2, 16
        idx = np.stack([rng.permutation(E)[:K] for _ in range(S)]).astype(np.int32)
        idx[: E // K + 1] = np.arange(2 * (E // K + 1), dtype=np.int32).reshape(-1, 2) % E  # every expert used
        x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
        lay, ref_lay = checked_layout(moe, idx, E, P, 3)
        esb = ref_lay["expert_slot_base"]
        assert np.all(np.diff(esb) > 0)
        note(f"unpack_padded limits E={E} A={A} R={R}")
        got = run_unpack_padded(moe, lay, x, S, K, H, E, 1, A, R)
        regions = oracle.dispatch_slots(x, ref_lay["slot_idx"], 1, 3)
        ref = oracle.unpack_padded(regions, esb, H, 1, A, R)
        assert int(ref[4]) == (1 if E * A > R else 0)
        assert_padded_equal(got, ref, f"limits E={E}")


# ---------------------------------------------------------------- combine


@pytest.mark.parametrize("cfg", sorted(WORKLOADS))
def test_combine_workloads(moe, cfg):
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    slot = oracle.layout(inp["topk_idx"], w.E, w.P, w.C)["slot_idx"]
    note(f"combine cfg{cfg} {w.describe()}")
    eo = expert_out(cfg)
    got = gpu_combine(moe, eo, slot, inp["topk_weights"])
    ref = oracle.combine(eo, slot, inp["topk_weights"])
    assert_bf16_within_ulp(got, ref, f"cfg{cfg}")
    assert np.array_equal(got, ref), f"cfg{cfg}: within 1 ulp but not bit-exact"


TINY_COMBINE = [
    # (S, K, H, R, p_mask, seed)
    (1, 1, 16, 1, 0.0, 1),
    (17, 3, 48, 60, 0.3, 2),
    (40, 16, 2064, 700, 0.1, 3),
    (5, 8, 16384, 40, 0.2, 4),
    (64, 2, 1024, 128, 1.0, 5),  # everything masked -> +0.0
]


@pytest.mark.parametrize("case", TINY_COMBINE)
def test_combine_tiny(moe, case):
    S, K, H, R, p_mask, seed = case
    rng = np.random.default_rng(seed)
    slot = np.stack([rng.choice(R, size=K, replace=K > R) for _ in range(S)]).astype(np.int32)
    slot[rng.random((S, K)) < p_mask] = -1
    rows = f32_to_bf16_input(rng.standard_normal((R, H)).astype(np.float32) * 3)
    w = rng.standard_normal((S, K)).astype(np.float32)
    note(f"combine tiny {case}")
    got = gpu_combine(moe, rows, slot, w)
    ref = oracle.combine(rows, slot, w)
    assert_bf16_within_ulp(got, ref, str(case))
    assert np.array_equal(got, ref), f"{case}: within 1 ulp but not bit-exact"


def test_combine_non_finite_inputs(moe):
    """Infinities and NaNs in the rows and the weights: every result that is a number (finite or
    infinite) matches the oracle's IEEE fp32 reduction bit for bit; every NaN result is a NaN
    (its payload is not specified). Large finite rows and weights also overflow to infinity."""
    rng = np.random.default_rng(77)
    S, K, H, R = 96, 6, 256, 300
    slot = np.stack([rng.choice(R, size=K, replace=False) for _ in range(S)]).astype(np.int32)
    slot[rng.random((S, K)) < 0.1] = -1
    vals = rng.standard_normal((R, H)).astype(np.float32) * 3
    special = np.array([np.inf, -np.inf, np.nan, 3.0e38, -3.0e38], np.float32)
    pick = rng.random((R, H)) < 0.02
    vals[pick] = rng.choice(special, size=int(pick.sum()))
    rows = f32_to_bf16_input(vals)
    w = rng.standard_normal((S, K)).astype(np.float32)
    wpick = rng.random((S, K)) < 0.05
    w[wpick] = rng.choice(np.array([np.inf, -np.inf, np.nan, 1e30], np.float32), size=int(wpick.sum()))
    note("combine non-finite inputs")
    got = gpu_combine(moe, rows, slot, w)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.combine(rows, slot, w)
    ref_nan = np.isnan(oracle.bf16_bits_to_f32(ref))
    got_nan = np.isnan(oracle.bf16_bits_to_f32(got))
    assert ref_nan.any() and np.isinf(oracle.bf16_bits_to_f32(ref)).any(), "the inputs reach NaN and infinity"
    assert np.array_equal(got_nan, ref_nan), "NaN results differ in position"
    assert np.array_equal(got[~ref_nan], ref[~ref_nan]), "non-NaN results differ"


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_two_pass_combine_workloads(moe, cfg):
    """Scatter by the unpacked triples, then the staged reduction: staging rows and y bit for bit
    against the oracle's two passes (and so against the gather combine)."""
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    lay, ref_lay = checked_layout(moe, inp["topk_idx"], w.E, w.P, w.C)
    slot = ref_lay["slot_idx"]
    n = int(ref_lay["expert_slot_base"][w.E])
    win = torch.empty(moe.moe_window_bytes(w.S, w.K, w.H), dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(bf16_dev(inp["x"]), lay.slot_idx, win, 0, 0)
    un = moe.moe_unpack(win, lay.expert_slot_base[w.E:], w.S, w.K, w.H, 0)
    # the triples the scatter is given must be the oracle's (checked before they are used)
    _, ref_idx, _ = oracle.unpack(oracle.dispatch_slots(inp["x"], slot, 0, 0), w.H, 0)
    eo = expert_out(cfg)
    wts = to_dev(inp["topk_weights"])
    stride = -(-2 * w.H // 512) * 512  # the page's 512-byte rows
    staging = torch.full((w.S * w.K * stride,), POISON, dtype=torch.uint8, device=DEV)
    note(f"two-pass combine cfg{cfg} {w.describe()}")
    moe.moe_combine_scatter(bf16_dev(eo[: w.S * w.K]), un.expand_idx, lay.expert_slot_base[w.E:], w.S,
                            w.K, staging=staging, staging_stride_bytes=stride)
    y = moe.moe_combine_staged(staging, lay.slot_idx, wts, w.H, staging_stride_bytes=stride)
    torch.cuda.synchronize()
    assert np.array_equal(un.expand_idx.cpu().numpy()[:n], ref_idx)
    ref_stg = oracle.combine_scatter(eo, ref_idx, n, w.S, w.K)
    got_stg = staging.view(w.S * w.K, stride).cpu().numpy()[:, : 2 * w.H].view(np.uint16)
    live = (slot >= 0).reshape(-1)
    assert np.array_equal(got_stg[live], ref_stg[live])
    assert np.all(got_stg[~live].view(np.uint8) == POISON)  # masked positions never written
    ref_y = oracle.combine_staged(ref_stg, slot, inp["topk_weights"])
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ref_y)
    assert np.array_equal(ref_y, oracle.combine(eo, slot, inp["topk_weights"]))


def test_two_pass_combine_masked_and_partial(moe):
    """Masked entries and N below the row count: skipped rows move nothing; y still matches."""
    rng = np.random.default_rng(44)
    S, K, E, P, H = 70, 6, 10, 5, 272
    tab = random_tiny_routing(rng, S, K, E, p_mask=0.35)
    lay, ref_lay = checked_layout(moe, tab, E, P, 4)
    slot = ref_lay["slot_idx"]
    n = int((slot >= 0).sum())
    rows = f32_to_bf16_input(rng.standard_normal((S * K, H)).astype(np.float32))
    wts = rng.random((S, K)).astype(np.float32)
    idx = np.full((S * K, 3), -1, np.int32)
    for t, k in zip(*np.nonzero(slot >= 0)):
        idx[slot[t, k]] = (0, t, k)
    full = None
    for n_dev in (n, n // 2, 0):
        staging = torch.full((S * K, H), -7, dtype=torch.int16, device=DEV)
        nd = torch.tensor([n_dev], dtype=torch.int32, device=DEV)
        moe.moe_combine_scatter(bf16_dev(rows), to_dev(idx), nd, S, K, staging=staging)
        torch.cuda.synchronize()
        ref = oracle.combine_scatter(rows, idx, n_dev, S, K,
                                     staging=np.full((S * K, H), 0xFFF9, np.uint16))
        assert np.array_equal(staging.cpu().numpy().view(np.uint16), ref), n_dev
        if full is None:
            full = staging
    y = moe.moe_combine_staged(full, lay.slot_idx, to_dev(wts), H)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), oracle.combine(rows, slot, wts))


def test_combine_scatter_skips_out_of_range_triples(moe):
    """Rows inside [0, N) whose triple names a token or k outside [0, S) x [0, K) (or negative) are
    not moved; the others land at row t*K + k."""
    rng = np.random.default_rng(45)
    S, K, H = 40, 4, 64
    n = S * K
    rows = f32_to_bf16_input(rng.standard_normal((n, H)).astype(np.float32))
    idx = np.stack([np.zeros(n), np.repeat(np.arange(S), K), np.tile(np.arange(K), S)], axis=1).astype(np.int32)
    perm = rng.permutation(n)
    idx = idx[perm]  # rows in a shuffled order
    bad = rng.choice(n, 25, replace=False)
    for j, b in enumerate(bad):
        if j % 2 == 0:
            idx[b, 1] = (S, -1, S + 7)[j // 2 % 3]  # token out of range
        else:
            idx[b, 2] = (K, -1)[j // 2 % 2]  # k out of range
    staging = torch.full((n, H), -7, dtype=torch.int16, device=DEV)
    nd = torch.tensor([n], dtype=torch.int32, device=DEV)
    note("combine_scatter with out-of-range triples")
    moe.moe_combine_scatter(bf16_dev(rows), to_dev(idx), nd, S, K, staging=staging)
    torch.cuda.synchronize()
    ref = oracle.combine_scatter(rows, idx, n, S, K, staging=np.full((n, H), 0xFFF9, np.uint16))
    assert np.array_equal(staging.cpu().numpy().view(np.uint16), ref)
    assert (ref == 0xFFF9).all(axis=1).sum() >= 1  # some staging rows received nothing


def test_combine_from_window_round_trip(moe):
    """Identity experts: combine read straight from the bf16 window returns x (weights sum to 1)."""
    w = WORKLOADS[3]
    inp = inputs(3)
    x = bf16_dev(inp["x"])
    lay, ref_lay = checked_layout(moe, inp["topk_idx"], w.E, w.P, w.C)
    win = torch.empty(moe.moe_window_bytes(w.S, w.K, w.H), dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(x, lay.slot_idx, win, 0)
    wts = to_dev(inp["topk_weights"])
    y = moe.moe_combine(win, lay.slot_idx, wts, row_stride_bytes=moe.moe_slot_bytes(w.H),
                        expert_rows=w.S * w.K, hidden=w.H)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    slot = ref_lay["slot_idx"]
    regions = oracle.dispatch_slots(inp["x"], slot, 0, 0)
    n = regions.shape[0]
    assert np.array_equal(win.cpu().numpy().reshape(w.S * w.K, -1)[:n, : regions.shape[1]], regions)
    rows = np.ascontiguousarray(regions[:, : 2 * w.H]).view(np.uint16)
    assert np.array_equal(got, oracle.combine(rows, slot, inp["topk_weights"]))
    xr = oracle.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    assert np.all(np.abs(oracle.bf16_bits_to_f32(got) - xr) <= np.abs(xr) * 2.0**-7)


def test_combine_row_stride_and_expert_rows(moe):
    """Rows at a caller stride wider than 2H (here 2H + 528 bytes, filled with garbage between the
    rows), and expert_rows below the slot count: entries naming a row at or past expert_rows are
    skipped like pads, so y equals the oracle's combine with those entries set to -1."""
    rng = np.random.default_rng(71)
    S, K, H, E, P = 300, 6, 1040, 24, 4
    idx = random_tiny_routing(rng, S, K, E, p_mask=0.1)
    slot = oracle.layout(idx, E, P, 5)["slot_idx"]
    n = int((slot >= 0).sum())
    rows = f32_to_bf16_input(rng.standard_normal((n, H)).astype(np.float32))
    wts = rng.random((S, K)).astype(np.float32)
    stride = 2 * H + 528
    buf = rng.integers(0, 256, size=(n, stride), dtype=np.uint8)
    buf[:, : 2 * H] = rows.view(np.uint8).reshape(n, 2 * H)
    dev_buf = to_dev(buf.reshape(-1))
    for expert_rows in (n, n // 2, 0):
        note(f"combine stride {stride} expert_rows {expert_rows} of {n}")
        y = moe.moe_combine(dev_buf, to_dev(slot), to_dev(wts), row_stride_bytes=stride,
                            expert_rows=expert_rows, hidden=H)
        torch.cuda.synchronize()
        got = y.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.combine(rows, np.where(slot < expert_rows, slot, -1), wts)
        assert np.array_equal(got, ref), expert_rows


# ---------------------------------------------------------------- determinism


@pytest.mark.parametrize("cfg,quant,fused", [(3, 0, False), (3, 0, "ws"), (3, 0, "lws"), (5, 0, "lws"),
                                             (2, 0, False), (2, 0, True), (2, 1, True), (1, 2, True)])
def test_repeat_runs_are_byte_identical(moe, cfg, quant, fused):
    """Each kernel twice on identical inputs, outputs poisoned differently before each run: the
    three-launch layout (workload 3), the planned pack (workload 3, its workspace poisoned too), the
    two-launch layout with the pack from its plan (workloads 3 and 5, workspace poisoned), the
    single-launch layout (workload 2) and the one-kernel layout + pack (moe_layout_dispatch)."""
    w = WORKLOADS[cfg]
    inp = inputs(cfg)
    idx = to_dev(inp["topk_idx"])
    x = bf16_dev(inp["x"])
    eo = bf16_dev(expert_out(cfg))
    wts = to_dev(inp["topk_weights"])
    outs = []
    note(f"determinism cfg{cfg} quant {quant} fused {fused}")
    for poison in (0x00, 0xFF):
        lay = moe.empty_layout(w.S, w.K, w.E, w.P, w.C, DEV)
        for t in lay:
            t.view(torch.uint8).fill_(poison)
        win = torch.full((moe.moe_window_bytes(w.S, w.K, w.H),), poison, dtype=torch.uint8, device=DEV)
        if fused == "lws":
            ws = torch.full((moe.moe_layout_dispatch_workspace_bytes(w.S, w.K, w.E, w.P, w.C, quant),), poison,
                            dtype=torch.uint8, device=DEV)
            moe.moe_layout_ws(idx, w.E, w.P, w.C, ws, quant, out=lay)
            moe.moe_dispatch_planned(x, lay.slot_idx, win, ws, w.C, quant)
        elif fused == "ws":
            moe.moe_layout(idx, w.E, w.P, w.C, out=lay)
            ws = torch.full((moe.moe_dispatch_workspace_bytes(w.S, w.K, quant),), poison, dtype=torch.uint8,
                            device=DEV)
            moe.moe_dispatch_ws(x, lay.slot_idx, win, ws, quant)
        elif fused:
            moe.moe_layout_dispatch(idx, w.E, w.P, w.C, x, win, quant, out=lay)
        else:
            moe.moe_layout(idx, w.E, w.P, w.C, out=lay)
            moe.moe_dispatch(x, lay.slot_idx, win, quant)
        y = torch.full((w.S, w.H), float(poison), dtype=torch.bfloat16, device=DEV)
        moe.moe_combine(eo, lay.slot_idx, wts, y=y)
        torch.cuda.synchronize()
        g = oracle.slot_geometry(w.H, quant)
        regions = win.view(w.S * w.K, -1)[:, : g.tail_end].cpu().numpy()
        outs.append(([t.cpu().numpy() for t in lay], regions, y.view(torch.int16).cpu().numpy()))
    (l0, r0, y0), (l1, r1, y1) = outs
    for a, b in zip(l0, l1):
        assert np.array_equal(a, b)
    assert np.array_equal(r0, r1)
    assert np.array_equal(y0, y1)


def test_two_streams_at_once(moe):
    """Two independent steps enqueued on two streams so that their kernels can overlap: workload 2
    through the one-kernel layout + pack (fp8), workload 1 through the separate calls (bf16). The
    library keeps no state between calls, so each must match the oracle on its own inputs."""
    jobs = []
    for cfg, quant, fused in ((2, 1, True), (1, 0, False)):
        w = WORKLOADS[cfg]
        inp = inputs(cfg)
        eo_host = expert_out(cfg)
        jobs.append(dict(w=w, inp=inp, quant=quant, fused=fused, stream=torch.cuda.Stream(), eo_host=eo_host,
                         idx=to_dev(inp["topk_idx"]), x=bf16_dev(inp["x"]), eo=bf16_dev(eo_host),
                         wts=to_dev(inp["topk_weights"]),
                         lay=poisoned_layout(moe, w.S, w.K, w.E, w.P, w.C),
                         win=torch.full((moe.moe_window_bytes(w.S, w.K, w.H),), POISON, dtype=torch.uint8,
                                        device=DEV),
                         y=torch.empty((w.S, w.H), dtype=torch.bfloat16, device=DEV)))
    torch.cuda.synchronize()
    note("two streams: cfg2 fused fp8 and cfg1 separate bf16")
    for rep in range(3):
        for j in jobs:
            w = j["w"]
            with torch.cuda.stream(j["stream"]):
                if j["fused"]:
                    moe.moe_layout_dispatch(j["idx"], w.E, w.P, w.C, j["x"], j["win"], j["quant"], 0, out=j["lay"])
                else:
                    moe.moe_layout(j["idx"], w.E, w.P, w.C, out=j["lay"])
                    moe.moe_dispatch(j["x"], j["lay"].slot_idx, j["win"], j["quant"], 0)
                moe.moe_combine(j["eo"], j["lay"].slot_idx, j["wts"], y=j["y"])
    torch.cuda.synchronize()
    for j in jobs:
        w, inp = j["w"], j["inp"]
        ref = oracle.layout(inp["topk_idx"], w.E, w.P, w.C)
        got = {k: v.cpu().numpy() for k, v in j["lay"]._asdict().items()}
        assert_layout_equal(got, ref, w.name)
        win = j["win"].cpu().numpy().reshape(w.S * w.K, -1)
        assert_window_equal(win, oracle.dispatch_slots(inp["x"], ref["slot_idx"], j["quant"], 0),
                            oracle.slot_geometry(w.H, j["quant"]), w.name)
        y = j["y"].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(y, oracle.combine(j["eo_host"], ref["slot_idx"], inp["topk_weights"]))


def test_maximum_tokens_and_channels(moe):
    """S = MOE_MAX_TOKENS (65536) with C = MOE_MAX_CHANNELS (4096): layout, dispatch and combine
    against the oracle on a small hidden size."""
    rng = np.random.default_rng(77)
    S, K, H, E, P, C = 65536, 2, 16, 64, 8, 4096
    idx = random_tiny_routing(rng, S, K, E, p_mask=0.05)
    note(f"max tokens S={S} K={K} H={H} E={E} P={P} C={C}")
    got = gpu_layout(moe, idx, E, P, C)
    ref = oracle.layout(idx, E, P, C)
    assert_layout_equal(got, ref, "max tokens")
    x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    win = gpu_dispatch(moe, x, ref["slot_idx"], 0)
    assert_window_equal(win, oracle.dispatch_slots(x, ref["slot_idx"], 0, 0), oracle.slot_geometry(H, 0),
                        "max tokens")
    rows = f32_to_bf16_input(rng.standard_normal((S * K, H)).astype(np.float32))
    wts = rng.random((S, K)).astype(np.float32)
    y = gpu_combine(moe, rows, ref["slot_idx"], wts)
    assert np.array_equal(y, oracle.combine(rows, ref["slot_idx"], wts))


@pytest.mark.parametrize("cfg,quant,fused", [(2, 0, True), (2, 1, True), (1, 2, True), (3, 0, False), (3, 0, "ws"),
                                             (2, 0, "ws")])
def test_plans_match_the_oracle(moe, cfg, quant, fused):
    """Pre-validated calls (moe_plan_*, run by moe_plan_run) on fixed buffers, three seeded inputs
    copied into them one after the other: layout, window and y against the oracle each time."""
    w = WORKLOADS[cfg]
    S, K, H, E, P, C = w.S, w.K, w.H, w.E, w.P, w.C
    idx_s = torch.empty((S, K), dtype=torch.int32, device=DEV)
    x_s = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)
    eo_s = torch.empty((S * K, H), dtype=torch.bfloat16, device=DEV)
    wts_s = torch.empty((S, K), dtype=torch.float32, device=DEV)
    lay = moe.empty_layout(S, K, E, P, C, DEV)
    win = torch.empty(moe.moe_window_bytes(S, K, H), dtype=torch.uint8, device=DEV)
    y = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)
    if fused == "ws":
        nws = moe.moe_layout_dispatch_workspace_bytes(S, K, E, P, C, quant)
    else:
        nws = moe.moe_dispatch_workspace_bytes(S, K, quant)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV) if nws else None
    if fused == "ws":
        plans = [moe.plan_layout_ws(idx_s, E, P, C, lay, ws, quant),
                 moe.plan_dispatch_planned(x_s, lay.slot_idx, win, ws, C, quant, 6)]
    elif fused:
        plans = [moe.plan_layout_dispatch(idx_s, E, P, C, x_s, win, lay, quant, 6)]
    else:
        plans = [moe.plan_layout(idx_s, E, P, C, lay), moe.plan_dispatch_ws(x_s, lay.slot_idx, win, ws, quant, 6)]
    plans.append(moe.plan_combine(eo_s, lay.slot_idx, wts_s, y))
    for seed in (1, 2, 3):
        rng = np.random.default_rng(1000 * cfg + seed)
        idx = random_tiny_routing(rng, S, K, E, p_mask=0.05, p_bad=0.01)
        x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
        eo = f32_to_bf16_input(rng.standard_normal((S * K, H)).astype(np.float32))
        wts = rng.random((S, K)).astype(np.float32)
        idx_s.copy_(to_dev(idx))
        x_s.copy_(bf16_dev(x))
        eo_s.copy_(bf16_dev(eo))
        wts_s.copy_(to_dev(wts))
        win.fill_(POISON)
        torch.cuda.synchronize()
        for plan in plans:
            plan.run()
        torch.cuda.synchronize()
        note(f"plans cfg{cfg} quant {quant} fused {fused} seed {seed}")
        ref = oracle.layout(idx, E, P, C)
        assert_layout_equal({k: v.cpu().numpy() for k, v in lay._asdict().items()}, ref, f"plan seed {seed}")
        assert_window_equal(win.cpu().numpy().reshape(S * K, -1), oracle.dispatch_slots(x, ref["slot_idx"], quant, 6),
                            oracle.slot_geometry(H, quant), f"plan seed {seed}")
        got_y = y.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got_y, oracle.combine(eo, ref["slot_idx"], wts)), f"plan seed {seed}"


def test_python_layer_rejects_bad_window(moe):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    slot = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
    small = torch.empty(moe.moe_window_bytes(4, 2, 64) - 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="window"):
        moe.moe_dispatch(x, slot, small)


# ---------------------------------------------------------------- graph capture


@pytest.mark.parametrize("fused", [False, True, "lws"])
def test_step_replays_from_a_captured_graph(moe, fused):
    """layout -> dispatch -> combine (or moe_layout_dispatch -> combine, or moe_layout_ws ->
    moe_dispatch_planned -> combine on a table of 8192 entries) captured once in a HIP graph (the
    library allocates and synchronises nothing) and replayed on fresh inputs copied into the
    captured buffers; every replay must equal the eager result on the same inputs. Eager work runs
    between replays."""
    if fused == "lws":
        S, K, H, E, P, C = 1024, 8, 256, 64, 8, 32
    else:
        w = WORKLOADS[1]
        S, K, H, E, P, C = w.S, w.K, w.H, w.E, w.P, w.C
    lws = torch.empty(max(16, moe.moe_layout_dispatch_workspace_bytes(S, K, E, P, C)), dtype=torch.uint8,
                      device=DEV)
    x_s = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)
    idx_s = torch.empty((S, K), dtype=torch.int32, device=DEV)
    wts_s = torch.empty((S, K), dtype=torch.float32, device=DEV)
    eo_s = torch.empty((S * K, H), dtype=torch.bfloat16, device=DEV)
    lay_s = moe.empty_layout(S, K, E, P, C, DEV)
    win_s = torch.empty(moe.moe_window_bytes(S, K, H), dtype=torch.uint8, device=DEV)
    y_s = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)

    def load(seed):
        rng = np.random.default_rng(seed)
        idx = np.stack([rng.permutation(E)[:K] for _ in range(S)]).astype(np.int32)
        x_s.copy_(bf16_dev(f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))))
        idx_s.copy_(to_dev(idx))
        wts_s.copy_(to_dev(rng.random((S, K)).astype(np.float32)))
        eo_s.copy_(bf16_dev(f32_to_bf16_input(rng.standard_normal((S * K, H)).astype(np.float32))))

    def step():
        if fused == "lws":
            moe.moe_layout_ws(idx_s, E, P, C, lws, 0, out=lay_s)
            moe.moe_dispatch_planned(x_s, lay_s.slot_idx, win_s, lws, C, 0)
        elif fused:
            moe.moe_layout_dispatch(idx_s, E, P, C, x_s, win_s, 0, out=lay_s)
        else:
            moe.moe_layout(idx_s, E, P, C, out=lay_s)
            moe.moe_dispatch(x_s, lay_s.slot_idx, win_s, 0)
        moe.moe_combine(eo_s, lay_s.slot_idx, wts_s, y=y_s)

    def snapshot():
        tail = oracle.slot_geometry(H, 0).tail_end
        return ([t.cpu().numpy().copy() for t in lay_s],
                win_s.view(S * K, -1)[:, :tail].cpu().numpy().copy(),
                y_s.view(torch.int16).cpu().numpy().copy())

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        load(seed)
        torch.cuda.synchronize()
        step()  # eager reference on the same inputs
        torch.cuda.synchronize()
        ref = snapshot()
        for t in (*lay_s, win_s, y_s, lws):  # poison (the workspace too), then replay
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        note(f"graph replay seed {seed} fused {fused}")
        for a, b in zip(ref[0], got[0]):
            assert np.array_equal(a, b)
        assert np.array_equal(ref[1], got[1]) and np.array_equal(ref[2], got[2])
