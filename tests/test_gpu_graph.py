"""The hot path inside a HIP graph.  No entry point allocates, synchronizes or clears memory
with a memset, so a whole step -- resolve the new tokens' slots, write their rows, attend --
can be captured once and replayed.  Each replay rewrites the same rows at the same slots,
so every replay must reproduce the eager step's output bit for bit; eager calls run between
the replays, as a serving loop would interleave them."""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_80_amd as pkv
    pkv.load()


from gpu_util import DeviceCase  # noqa: E402

CASES = {
    "bf16 GQA decode, window": lambda: workloads.decode_case(5, 8, 32, 8, 128, "bf16", block_size=32, max_blocks=40,
                                                             len_range=(1, 1200), window=500, null_block=True),
    "append: bf16 GQA decode with its write fused in": lambda: workloads.decode_case(
        12, 8, 32, 8, 128, "bf16", block_size=64, max_blocks=40, len_range=(1, 2500), null_block=True),
    "int8 MHA decode": lambda: workloads.decode_case(6, 4, 16, 16, 128, "bf16", block_size=64, max_blocks=20,
                                                     len_range=(1, 1200), int8=True),
    "fp32 decode (partition kernels)": lambda: workloads.decode_case(7, 3, 8, 2, 128, "f32", block_size=16,
                                                                     max_blocks=50, len_range=(1, 700)),
    "fp32 decode (one 16-wave workgroup per sequence)": lambda: workloads.decode_case(
        13, 2, 4, 4, 128, "f32", block_size=128, max_blocks=4, len_range=(1, 512)),
    "MLA decode": lambda: workloads.decode_case(8, 3, 32, 1, 512, "bf16", block_size=64, max_blocks=20,
                                                len_range=(1, 1200), rope_dim=64, scale=576 ** -0.5),
    "chunked prefill": lambda: workloads.prefill_case(9, 3, 16, 4, 128, "bf16", cached=[100, 0, 700],
                                                      new=[60, 33, 128], block_size=64),
    "multi-token decode (stream split + combine)": lambda: workloads.prefill_case(
        10, 3, 16, 4, 128, "bf16", cached=[5000, 100, 3000], new=[4, 2, 3], block_size=128, null_block=True),
    "few-row prefill (key split + combine)": lambda: workloads.prefill_case(
        11, 3, 16, 4, 128, "bf16", cached=[5000, 100, 3000], new=[12, 9, 10], block_size=128, null_block=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_replays_in_a_graph(name):
    import paged_kv_cache_80_amd as pkv

    case = CASES[name]()
    d = DeviceCase(case)
    out_eager, _ = d.run()
    ref = out_eager.clone()

    slots = torch.empty(case.new_pos.size, dtype=torch.int32, device="cuda")
    out = torch.empty_like(ref)
    if case.kind == "decode":
        ws_bytes = pkv.paged_attn_decode_workspace(d.cache, case.B, case.H, case.max_blocks, case.scale, case.window,
                                                   pkv.PKV_BF16 if ref.dtype == torch.bfloat16 else pkv.PKV_F32)
    else:
        ws_bytes = pkv.paged_attn_prefill_workspace(d.cache, case.B, case.H, case.max_blocks, case.q.shape[0],
                                                    case.scale, case.window, pkv.PKV_BF16)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    if "split" in name:
        assert ws_bytes > 0, "this case takes the key split"
    if "16-wave" in name:
        assert ws_bytes == 0, "this case takes the whole-sequence workgroups"
    max_q = int(np.diff(case.cu_seqlens_q).max(initial=0)) if case.kind == "prefill" else 1

    def step():
        if name.startswith("append"):  # write and decode in one kernel
            pkv.paged_attn_decode_append(d.q, d.new_k, d.new_v, d.cache, d.block_table, d.seq_lens, case.scale,
                                         case.window, out=out, workspace=ws)
            return
        if name.startswith("bf16"):  # index resolution fused into the write
            pkv.kv_cache_write_at(d.block_table, d.new_batch_idx, d.new_pos, d.new_k, d.new_v, d.cache,
                                  k_rope=d.new_k_rope, slots_out=slots)
        else:
            pkv.pkv_resolve_slots(d.block_table, case.block_size, d.new_batch_idx, d.new_pos, slots_out=slots)
            pkv.kv_cache_write(slots, d.new_k, d.new_v, d.cache, k_rope=d.new_k_rope)
        if case.kind == "decode":
            pkv.paged_attn_decode(d.q, d.cache, d.block_table, d.seq_lens, case.scale, case.window,
                                  q_rope=d.q_rope, out=out, workspace=ws)
        else:
            pkv.paged_attn_prefill(d.q, d.cache, d.block_table, d.cu_seqlens_q, d.seq_lens, max_q, case.scale,
                                   case.window, q_rope=d.q_rope, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name}: replay {i} differs from the eager step"
        # eager work between replays, on the same cache
        d.attend()
        torch.cuda.synchronize()
