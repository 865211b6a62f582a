"""msa_decode_step_noalloc (the decode step in the library's static per-GPU
scratch, no workspace argument) against msa_decode_step with a caller
workspace, through the C ABI (needs an MI355X)."""
import pytest
import torch

from block_sparse_attention_03_amd import _lib as L
from block_sparse_attention_03_amd import inputs as gen
from block_sparse_attention_03_amd.pipeline import MsaStep

pytestmark = pytest.mark.gpu


def _noalloc_into(step):
    x = step.x
    out = torch.full_like(step.out, float("nan"))
    lse = torch.full_like(step.lse, float("nan"))
    sel = torch.full_like(step.sel, -7)
    L.msa_decode_step_noalloc(step.dims, x.q_idx, x.kidx_cache, x.q, x.k_cache, x.v_cache,
                              x.block_table, x.seq_lens, out, lse, sel)
    return out, lse, sel


def test_noalloc_decode_step_equals_the_workspace_form():
    """Calls in a row on one GPU's scratch: the 8 x 60,000 paged decode, then a
    smaller ragged batch, then rows past 8192 blocks (whose selection and page
    table also live in the scratch, with and without the selection output),
    then the 16-sequence ragged decode (several page slots per workgroup),
    then the first shape again.  Each equals msa_decode_step with its own
    workspace, bit for bit (out, lse, selection)."""
    cases = [gen.config(2),
             gen.MsaConfig("noalloc_small", [300, 1000, 4500], [1, 1, 1], 12, 3,
                           permute_pages=True, seed=91),
             gen.MsaConfig("noalloc_8300_blocks", [8300 * 128 - 5, 3000], [1, 1], 2, 1,
                           permute_pages=True, seed=92),
             # 128 flattened rows: several page slots per workgroup
             gen.config(5)]
    steps = []
    for cfg in cases:
        assert L.msa_decode_step_workspace_size(L.dims_for(cfg)) <= L.MSA_STATIC_SCRATCH_BYTES
        x = gen.make_inputs(cfg, device="cuda", poison_padding=True)
        ref = MsaStep(x, fused=True)
        ref.run()
        steps.append(ref)
    torch.cuda.synchronize()
    for i, k in enumerate([0, 1, 2, 3, 0]):
        ref = steps[k]
        print(f"[noalloc] call {i}: {cases[k].name}", flush=True)
        out, lse, sel = _noalloc_into(ref)
        torch.cuda.synchronize()
        assert torch.equal(out, ref.out), f"call {i}: out"
        assert torch.equal(lse, ref.lse), f"call {i}: lse"
        assert torch.equal(sel, ref.sel), f"call {i}: sel"
    # without the selection output (rows past 8192 blocks keep it in the scratch)
    ref = steps[2]
    print("[noalloc] no selection output", flush=True)
    x = ref.x
    out = torch.empty_like(ref.out)
    L.msa_decode_step_noalloc(ref.dims, x.q_idx, x.kidx_cache, x.q, x.k_cache, x.v_cache,
                              x.block_table, x.seq_lens, out, None, None)
    torch.cuda.synchronize()
    assert torch.equal(out, ref.out)


def test_noalloc_rejects_a_shape_past_the_scratch():
    """A batch whose decode-step scratch exceeds MSA_STATIC_SCRATCH_BYTES is
    refused before anything is launched; the outputs are left untouched."""
    cfg = gen.MsaConfig("noalloc_too_big", [300] * 700, [1] * 700, 16, 2, seed=93)
    d = L.dims_for(cfg)
    assert L.msa_decode_step_workspace_size(d) > L.MSA_STATIC_SCRATCH_BYTES
    x = gen.make_inputs(cfg, device="cuda")
    out = torch.zeros_like(x.q)
    with pytest.raises(L.MsaError) as e:
        L.msa_decode_step_noalloc(d, x.q_idx, x.kidx_cache, x.q, x.k_cache, x.v_cache,
                                  x.block_table, x.seq_lens, out, None, None)
    assert e.value.status == L.MSA_ERROR_WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()
