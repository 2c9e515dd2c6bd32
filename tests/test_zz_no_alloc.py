"""The allocation-free ALL_GATHER_MATMUL (coc_allgather_matmul_noalloc),
called through the C ABI.  It is a variant of coc_allgather_matmul whose
gathered matrix and hand-over counters live in the library's static device
array, so its outputs must equal that entry point's bit for bit (the same
kernels walk k in the same order).  Checked on consecutive calls that reuse
the array, the later ones smaller than the first, over the one-launch
pipeline with the copy inside the matmul launch, the same with the copy as
its own launch, and the serial form; sizes past the array's limit are
refused before anything is enqueued."""
import pytest
import torch

import oracle
import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import synth
from tests._util import assert_bits_equal, assert_close, f64, log

pytestmark = pytest.mark.gpu

WID = 160
LIMIT = 64 << 20   # bytes of gathered rows the static array holds


def _case(world, rank, shard, k, n, dtype, seed):
    shards = [synth.normal(WID + seed, synth.T_PEER, r, (shard, k), 1.0, dtype).to("cuda") for r in range(world)]
    w = synth.normal(WID + seed, synth.T_W, 0, (k, n), 0.02, dtype).to("cuda")
    peers = [None if r == rank else shards[r] for r in range(world)]
    return shards, w, peers


def _check_against_plain(world, rank, shard, k, n, dtype, split, seed, oracle_check=False):
    log(f"no-alloc AG {dtype} world={world} rank={rank} m={world * shard} k={k} n={n} split={split}")
    shards, w, peers = _case(world, rank, shard, k, n, dtype, seed)
    y = torch.full((world * shard, n), float("nan"), dtype=w.dtype, device="cuda")
    got = tgc.allgather_matmul_noalloc(shards[rank], peers, w, rank, y=y, split=split)
    want = tgc.allgather_matmul(shards[rank], peers, w, rank, split=split)
    torch.cuda.synchronize()
    tgc.check_waits()
    assert got.data_ptr() == y.data_ptr()
    assert_bits_equal(got, want, f"no-alloc vs workspace all-gather matmul ({dtype}, split {split})")
    if oracle_check:
        ref = oracle.matmul(oracle.allgather([f64(s, dtype) for s in shards]), f64(w, dtype))
        assert_close(got, ref, dtype, "no-alloc y vs the oracle")


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    # the LLaMA2-70B TP8 gather: 8 shards of 512 x 8192 bf16 fill the array exactly;
    # the launch copies the rows itself
    _check_against_plain(8, 3, 512, 8192, 7168, "bf16", 4, 0)
    # smaller, reusing the array: fp16, another rank and split
    _check_against_plain(8, 6, 128, 512, 640, "f16", 8, 1, oracle_check=True)
    # smaller still, too small for the copy inside the matmul launch (a separate copy launch)
    _check_against_plain(4, 1, 64, 256, 256, "bf16", 2, 2, oracle_check=True)
    # the serial form (split 1) and a k that is not a multiple of 32
    _check_against_plain(2, 0, 32, 72, 128, "bf16", 1, 3, oracle_check=True)


def test_noalloc_refuses_sizes_past_its_limit():
    world, rank, k, n = 8, 0, 8192, 256
    shard = LIMIT // (2 * k * world) + 8           # m x k x 2 bytes just past the limit
    shards, w, peers = _case(world, rank, 8, k, n, "bf16", 4)
    y = torch.zeros((8 * world, n), dtype=torch.bfloat16, device="cuda")
    L = tgc.lib()
    pa = (tgc.coc.ctypes.c_void_p * world)(*[None if p is None else p.data_ptr() for p in peers])
    st = L.coc_allgather_matmul_noalloc(shards[rank].data_ptr(), pa, w.data_ptr(), y.data_ptr(), world, rank,
                                        shard * world, n, k, tgc.COC_BF16, 4, 0,
                                        torch.cuda.current_stream().cuda_stream)
    assert tgc.coc.STATUS[st] == "COC_ERR_WORKSPACE", tgc.coc.STATUS.get(st, st)
    assert "64" in L.coc_last_error().decode() or "bytes" in L.coc_last_error().decode()
    torch.cuda.synchronize()
    assert not y.any(), "a refused call wrote its output"
