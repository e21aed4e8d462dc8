"""dspark_draft_block_noalloc, through the C ABI, against dspark_draft_block.

The no-allocation entry point runs the same kernels as the workspace entry
point, with the scratch its plan needs laid out in the library's static
device array, so its outputs must equal the workspace entry point's bit for
bit (the parity bar against the oracle is met by the workspace entry point's
own tests). Two calls in a row share the static array, the second with a
smaller input; a call whose plan needs more scratch than the array holds is
rejected before anything is enqueued.
"""

from __future__ import annotations

import pytest

from ancestral_draft_token_amd import inputs

from gpu_util import require_gpu, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def noalloc_outputs(p, rc_expected=0):
    """Run the no-allocation entry point on problem p's inputs into fresh outputs."""
    import torch
    from ancestral_draft_token_amd import dspark_draft_block_noalloc
    w = p.w
    tok = torch.full_like(p.tokens, -7)
    lg = torch.full_like(p.logits, 3.0)
    q = torch.full_like(p.q, 5.0)
    rc = dspark_draft_block_noalloc(p.base, p.base_dtype, p.E, p.W, p.prev, p.seed, p.offset, p.temperature,
                                    p.n_real, w.B, w.K, w.V, w.r, tok, lg, q, check=False)
    torch.cuda.synchronize()
    assert rc == rc_expected, rc
    return tok, lg, q


def same(p, outs, name):
    import torch
    tok, lg, q = outs
    assert torch.equal(tok, p.tokens), name
    assert torch.equal(lg, p.logits), name
    assert torch.equal(q, p.q), name
    say(f"noalloc equals the workspace entry point bit for bit: {name}")


def test_noalloc_equals_workspace_entry_twice_then_smaller():
    from ancestral_draft_token_amd import dspark_launch_plan
    cases = [
        ("b96 resident MFMA", inputs.large_padded()),
        ("b1 resident GEMV (smaller)", inputs.single_request()),
        ("b3 per-position plan (r=288)", inputs.tiny(B=3, K=3, r=288, fixed_seed=None, fixed_offset=None)),
        ("b5 ragged resident MFMA", inputs.tiny(B=5, K=3, V=1000, r=64, fixed_seed=None, fixed_offset=None)),
    ]
    for name, w in cases:
        say(f"noalloc case {name}: plan {dspark_launch_plan(w.B, w.K, w.V, w.r)}")
        p = run_gpu(w)
        same(p, noalloc_outputs(p), name)
        # and again: the array keeps the last call's contents, which must not matter
        same(p, noalloc_outputs(p), name + ", second call")
        del p


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """B=200 takes the per-position plan, whose partials need ~10 MB: rejected,
    nothing enqueued (the outputs keep their fill)."""
    import torch
    from ancestral_draft_token_amd import DSPARK_ERR_SCRATCH
    w = inputs.small_batch(B=200, K=2)
    say("noalloc rejection: B=200 K=2 V=200064")
    p = run_gpu(w)
    tok, lg, q = noalloc_outputs(p, rc_expected=DSPARK_ERR_SCRATCH)
    assert bool((tok == -7).all()) and bool((lg == 3.0).all()) and bool((q == 5.0).all())
    # a smaller call right after still works
    w2 = inputs.small_batch(B=8, K=2)
    p2 = run_gpu(w2)
    same(p2, noalloc_outputs(p2), "b8 after a rejected call")
    del p, p2
    torch.cuda.empty_cache()
