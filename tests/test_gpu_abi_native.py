"""The C ABI from a native C++ program on the GPU (tests/c_abi/abi_gpu.cpp): hipMalloc'd buffers,
moe_layout -> moe_dispatch (or moe_layout_dispatch, or moe_layout_ws -> moe_dispatch_planned, directly
or as pre-validated plans) -> moe_combine through libmoe.so, no Python or torch in the process.
Its outputs are compared with the oracle bit for bit. The program is built with the library
(combine_moe_layout_02_amd/build.py)."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from conftest import ROOT
from workloads import WORKLOADS, draw_expert_out, f32_to_bf16_input, make_inputs, random_tiny_routing

pytestmark = pytest.mark.gpu

EXE = os.path.join(ROOT, "tests", "c_abi", "abi_gpu")


def _run_native(tmp_path, S, K, H, E, P, C, quant, inp, mode=0):
    assert os.path.exists(EXE), f"{EXE} is missing: run python combine_moe_layout_02_amd/build.py"
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([S, K, H, E, P, C, quant, mode], np.int32).tobytes())
        f.write(np.ascontiguousarray(inp["topk_idx"], np.int32).tobytes())
        f.write(np.ascontiguousarray(inp["x"], np.uint16).tobytes())
        f.write(np.ascontiguousarray(inp["topk_weights"], np.float32).tobytes())
        f.write(np.ascontiguousarray(inp["expert_out"], np.uint16).tobytes())
    print(f"native abi program: S={S} K={K} H={H} E={E} P={P} C={C} quant={quant} mode={mode}", flush=True)
    res = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    raw = dst.read_bytes()
    slot_bytes = oracle.slot_geometry(H, quant).slot_bytes
    off = 0
    status = int(np.frombuffer(raw, np.int32, 1, off)[0])
    off += 4
    slot = np.frombuffer(raw, np.int32, S * K, off).reshape(S, K)
    off += 4 * S * K
    win = np.frombuffer(raw, np.uint8, S * K * slot_bytes, off).reshape(S * K, slot_bytes)
    off += S * K * slot_bytes
    y = np.frombuffer(raw, np.uint16, S * H, off).reshape(S, H)
    assert off + 2 * S * H == len(raw)

    ref = oracle.layout(inp["topk_idx"], E, P, C)
    assert status == ref["status"]
    assert np.array_equal(slot, ref["slot_idx"])
    regions = oracle.dispatch_slots(inp["x"], ref["slot_idx"], quant, 0)
    tail = oracle.slot_geometry(H, quant).tail_end
    assert np.array_equal(win[: regions.shape[0], :tail], regions)
    assert np.array_equal(y, oracle.combine(inp["expert_out"], ref["slot_idx"], inp["topk_weights"]))


@pytest.mark.parametrize("cfg,quant,mode", [(1, 0, 0), (1, 1, 0), (2, 2, 0), (1, 0, 1), (2, 1, 1), (2, 0, 2), (1, 0, 3)])
def test_native_program_matches_oracle(tmp_path, cfg, quant, mode):
    w = WORKLOADS[cfg]
    _run_native(tmp_path, w.S, w.K, w.H, w.E, w.P, w.C, quant, make_inputs(w), mode)


@pytest.mark.parametrize("quant,mode", [(0, 2), (0, 3), (1, 2)])
def test_native_program_workspace_calls(tmp_path, quant, mode):
    """The workspace calls on a table of 8192 entries with 256 entries a channel, so the layout writes
    the planned pack's record lists (bf16), and in fp8 the token-order pack follows."""
    S, K, H, E, P, C = 1024, 8, 256, 64, 8, 32
    rng = np.random.Generator(np.random.PCG64(7200 + quant))
    inp = {
        "topk_idx": random_tiny_routing(rng, S, K, E, p_mask=0.05, p_bad=0.01),
        "x": f32_to_bf16_input(rng.standard_normal((S, H), dtype=np.float32)),
        "topk_weights": rng.random((S, K), dtype=np.float32),
        "expert_out": draw_expert_out(7201, S * K, H),
    }
    _run_native(tmp_path, S, K, H, E, P, C, quant, inp, mode)


def test_native_program_masked_and_bad_ids(tmp_path):
    """Masked (-1) and out-of-range ids: status bit 0 set, those entries get no slot and add
    nothing to y."""
    S, K, H, E, P, C = 200, 3, 48, 9, 3, 7
    rng = np.random.Generator(np.random.PCG64(7100))
    inp = {
        "topk_idx": random_tiny_routing(rng, S, K, E, p_mask=0.2, p_bad=0.1),
        "x": f32_to_bf16_input(rng.standard_normal((S, H), dtype=np.float32)),
        "topk_weights": rng.random((S, K), dtype=np.float32),
        "expert_out": draw_expert_out(7101, S * K, H),
    }
    _run_native(tmp_path, S, K, H, E, P, C, 0, inp)
    _run_native(tmp_path, S, K, H, E, P, C, 1, inp, mode=1)
