"""Compiles the decode kernel for gfx950 (no GPU needed) and checks its assembly."""
import os
import shutil
import subprocess

import pytest

from tests import asm_checks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_absorbed_amd", "csrc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    from decode_attention_absorbed_amd.build import HIP_FLAGS

    out = str(tmp_path_factory.mktemp("asm") / "mla_decode.s")
    flags = [f for f in HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "mla_decode.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def test_decode_kernels_present(asm):
    bodies = asm_checks.kernel_bodies(asm)
    # one page per tile / two pages per tile, each with the lazy and the
    # power-of-two rescale
    assert len(bodies) == 4
    for b in bodies:
        assert sum(t.startswith("v_mfma_f32_16x16x32_bf16") for t in b) >= 136


def test_no_valu_to_mfma_hazards(asm):
    for body in asm_checks.kernel_bodies(asm):
        assert asm_checks.mfma_hazards(body) == []


def test_no_mfma_result_to_valu_hazards(asm):
    for body in asm_checks.kernel_bodies(asm):
        assert asm_checks.mfma_result_hazards(body) == []


def test_async_query_loads_untouched_until_waited(asm):
    for body in asm_checks.kernel_bodies(asm):
        # the query rows: 32 c_kv chunks and 4 rope chunks per lane
        assert sum(t.startswith("global_load_dwordx4") for t in body) == 36
        assert asm_checks.async_load_violations(body) == []


def test_only_explicit_vmcnt_waits(asm):
    # 36 = query loads in flight (page ids landed), 18 = two tiles of copies
    # in flight (prologue), 9 = one tile (loop), 0 = drain
    for body in asm_checks.kernel_bodies(asm):
        waits = asm_checks.vmcnt_waits(body)
        counts = sorted({int(w.split("vmcnt(")[1].split(")")[0]) for w in waits})
        assert counts == [0, 9, 18, 36], waits


def test_accumulators_only_touched_by_inline_asm(asm):
    # the 256 output accumulators live in a0..a255, named only by inline asm
    assert asm_checks.compiler_agpr_uses(asm, asm_checks.DECODE_PREFIX) == []


def test_decode_kernels_do_not_spill(asm):
    res = {k: v for k, v in asm_checks.kernel_resources(asm).items() if k.startswith(asm_checks.DECODE_PREFIX)}
    assert len(res) == 4
    for name, r in res.items():
        # no VGPR spills and no scratch memory at all (spilled SGPRs go to
        # lanes of a VGPR, not to memory)
        assert r.get("vgpr_spill_count") == 0, (name, r)
        assert r.get("private_segment_fixed_size") == 0, (name, r)


def test_every_load_result_waited_for(asm):
    # in-order vmcnt model: no register of an outstanding load is touched
    for body in asm_checks.kernel_bodies(asm):
        assert asm_checks.pending_load_violations(body) == []


def test_no_sgpr_write_to_vmem_hazards(asm):
    # the copies and stores are inline asm with SGPR bases: no VALU write of
    # such an SGPR within 5 wait states before them (whole kernel bodies)
    for body in asm_checks.kernel_bodies(asm, whole=True):
        assert asm_checks.sgpr_vmem_hazards(body) == []


def test_no_mfma_destination_races(asm):
    # nothing but the next MFMA of the same accumulation chain touches an
    # inline-asm MFMA's result registers (VGPR or AGPR) within 19 wait states
    for body in asm_checks.kernel_bodies(asm, whole=True):
        assert asm_checks.mfma_dst_races(body) == []


def test_page_ids_not_loaded_by_vector_loads(asm):
    # one vector dword load (the piece's first 64 page ids, waited for
    # explicitly); pages further on come from scalar loads, never from a vector
    # load whose wait would drain the tile copies
    for body in asm_checks.kernel_bodies(asm):
        assert sum(t.startswith("global_load_dword ") for t in body) == 1


def test_no_store_data_hazards(asm):
    # every kernel of the library: the decode kernel's inline-asm stores and
    # the compiler's own stores in the combine kernels
    bodies = asm_checks.kernel_bodies(asm, prefix="_ZN3mla")
    assert len(bodies) >= 4
    for body in bodies:
        assert asm_checks.store_data_hazards(body) == []


# ---- the FP8 kernel ---------------------------------------------------------------------

FP8_PREFIX = "_ZN3mla12_GLOBAL__N_117decode_fp8_kernel"


@pytest.fixture(scope="module")
def asm_fp8(tmp_path_factory):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    from decode_attention_absorbed_amd.build import HIP_FLAGS

    out = str(tmp_path_factory.mktemp("asm8") / "mla_decode_fp8.s")
    flags = [f for f in HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "mla_decode_fp8.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def test_fp8_kernels_present(asm_fp8):
    bodies = asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX)
    assert len(bodies) == 3  # 1, 2 or 4 pages per 64-key tile
    for b in bodies:
        # 18 QK^T MFMAs per tile (prologue tile + loop) and 16 PV MFMAs per
        # tile (two loop variants), all on the scaled instruction
        assert sum(t.startswith("v_mfma_scale_f32_32x32x64_f8f6f4") for t in b) >= 36 + 32


def test_fp8_hazards(asm_fp8):
    for body in asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX):
        assert asm_checks.mfma_hazards(body) == []
        assert asm_checks.mfma_result_hazards(body) == []
        assert asm_checks.store_data_hazards(body) == []


def test_fp8_async_query_loads_untouched_until_waited(asm_fp8):
    for body in asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX):
        assert sum(t.startswith("global_load_dwordx4") for t in body) == 36
        assert asm_checks.async_load_violations(body) == []


def test_fp8_only_explicit_vmcnt_waits(asm_fp8):
    # the counts the FP8 kernel's source writes: 24/22/20 (prologue, query and
    # scale copies in flight), 10 (one tile of copies in flight), 0 (drain)
    for body in asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX):
        waits = asm_checks.vmcnt_waits(body)
        counts = sorted({int(w.split("vmcnt(")[1].split(")")[0]) for w in waits})
        assert counts == [0, 10, 20, 22, 24], waits


def test_fp8_every_load_result_waited_for(asm_fp8):
    for body in asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX):
        assert asm_checks.pending_load_violations(body) == []


def test_fp8_no_sgpr_write_to_vmem_hazards(asm_fp8):
    for body in asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX, whole=True):
        assert asm_checks.sgpr_vmem_hazards(body) == []


def test_fp8_no_mfma_destination_races(asm_fp8):
    for body in asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX, whole=True):
        assert asm_checks.mfma_dst_races(body) == []


def test_fp8_page_ids_not_loaded_by_vector_loads(asm_fp8):
    for body in asm_checks.kernel_bodies(asm_fp8, prefix=FP8_PREFIX):
        assert sum(t.startswith("global_load_dword ") for t in body) == 1


def test_fp8_accumulators_only_touched_by_inline_asm(asm_fp8):
    assert asm_checks.compiler_agpr_uses(asm_fp8, FP8_PREFIX) == []


def test_fp8_kernels_do_not_spill(asm_fp8):
    res = {k: v for k, v in asm_checks.kernel_resources(asm_fp8).items() if k.startswith(FP8_PREFIX)}
    assert len(res) == 3
    for name, r in res.items():
        # no VGPR spills and no scratch memory at all (spilled SGPRs go to
        # lanes of a VGPR, not to memory)
        assert r.get("vgpr_spill_count") == 0, (name, r)
        assert r.get("private_segment_fixed_size") == 0, (name, r)


# ---- the prolog / epilog projections -----------------------------------------------------

PROJ_PREFIX = "_ZN3mla12_GLOBAL__N_111proj_kernel"


@pytest.fixture(scope="module")
def asm_prolog(tmp_path_factory):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    from decode_attention_absorbed_amd.build import HIP_FLAGS

    out = str(tmp_path_factory.mktemp("asm") / "mla_prolog.s")
    flags = [f for f in HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "mla_prolog.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def test_projection_loads_issued_up_front(asm_prolog):
    """Absorption (bf16 and FP8 cache; 32- or 128-row chunks): 2 or 8 X loads +
    8 weight loads per lane; up-projection: 16 X + 16 weight loads (32-row
    chunks), 32 + 16 (64-row chunks, 64 outputs per workgroup) or 16 + 32
    (32-row chunks, 128 outputs); the first wait leaves the weights in flight,
    the second drains them before the MFMAs."""
    bodies = asm_checks.kernel_bodies(asm_prolog, prefix=PROJ_PREFIX, whole=True)
    assert len(bodies) == 7
    seen = set()
    for body in bodies:
        first = next(i for i, t in enumerate(body) if t.startswith("global_load_dwordx4"))
        run = 0
        for t in body[first:]:
            if not t.startswith("global_load_dwordx4"):
                if t.startswith(("v_", "s_")) and not t.startswith("s_waitcnt"):
                    continue
                break
            run += 1
        waits = [int(t.split("vmcnt(")[1].split(")")[0]) for t in body if t.startswith("s_waitcnt") and "vmcnt" in t]
        mfma = sum(t.startswith("v_mfma_f32_16x16x32_bf16") for t in body)
        seen.add((run, tuple(waits[:2]), mfma))
    assert seen == {(10, (8, 0), 8), (16, (8, 0), 8), (32, (16, 0), 16), (48, (16, 0), 16), (48, (32, 0), 32)}, seen


def test_projection_loads_untouched_until_waited(asm_prolog):
    for body in asm_checks.kernel_bodies(asm_prolog, prefix=PROJ_PREFIX, whole=True):
        assert asm_checks.pending_load_violations(body) == []


OPROJ_PREFIX = "_ZN3mla12_GLOBAL__N_112oproj_kernel"


def test_output_projection_loads(asm_prolog):
    """Per chunk and lane: X loads (32 or 64 query rows x 128 columns: 2 or 4;
    128 x 256: 16) + weight loads (128 output rows per workgroup: 2 x 4; 64:
    4 or 8); the first wait leaves the weights in flight; no register of a
    pending load is touched."""
    bodies = asm_checks.kernel_bodies(asm_prolog, prefix=OPROJ_PREFIX, whole=True)
    assert len(bodies) == 5
    seen = set()
    for body in bodies:
        n = sum(t.startswith("global_load_dwordx4") for t in body)
        waits = sorted({int(t.split("vmcnt(")[1].split(")")[0]) for t in body if t.startswith("s_waitcnt") and "vmcnt" in t})
        mfma = sum(t.startswith("v_mfma_f32_16x16x32_bf16") for t in body)
        seen.add((n, tuple(waits), mfma))
        assert asm_checks.pending_load_violations(body) == []
    assert seen == {(10, (0, 8), 16), (12, (0, 8), 32), (6, (0, 4), 8), (8, (0, 4), 16), (24, (0, 8), 64)}, seen
