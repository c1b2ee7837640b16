"""Checkpoint/resume and KV rollback for the closed decoding loop, in the oracle (CPU).

The loop state between steps is what the pages' stationary batch keeps per request: the
paged cache with its page table, the context lengths (a rejected draft is rolled back by
not advancing the length, 「首次超越 AR 模型」 "實際部署：SGLang 整合"), the next drafts and the rows
they were drawn from.  Two properties follow and are checked here:
  * saving that state after k steps and resuming from the saved copy gives exactly the
    steps an uninterrupted run gives;
  * the slots of rejected drafts, left stale in the cache, change nothing: the next block
    overwrites them, and attention equals attention over a cache that never held them."""
import json

import numpy as np

import oracle
from oracle.verify import commit, verify

B, N, Hq, Hkv, D, V = 3, 3, 4, 2, 16, 64
R = 2 * N - 1
PAGE = 16


def u24(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


def initial_state(seed=5):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(3, 40, size=B).astype(np.int32)
    max_pages = 12
    perm = rng.permutation(B * max_pages).astype(np.int32)
    state = dict(
        k_pages=np.zeros((B * max_pages, Hkv, PAGE, D), np.float32),
        v_pages=np.zeros((B * max_pages, Hkv, PAGE, D), np.float32),
        page_table=perm.reshape(B, max_pages),
        ctx=ctx, drafts=np.full((B, N - 1), -1, np.int32),
        draft_rows=np.zeros((B, N - 1, V), np.float32))
    for b in range(B):
        for j in range(int(ctx[b])):
            p = state["page_table"][b, j // PAGE]
            state["k_pages"][p, :, j % PAGE] = rng.standard_normal((Hkv, D))
            state["v_pages"][p, :, j % PAGE] = rng.standard_normal((Hkv, D))
    return state, rng


def step(state, rng):
    """One step of the loop: fresh block rows, attention (appending the block), rows for
    verification from a synthetic model (a hot request's verify rows are its draft rows
    plus noise), verification, commit.  Returns the step's outputs."""
    q = rng.standard_normal((B, R, Hq, D)).astype(np.float32)
    kn = rng.standard_normal((B, R, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, R, Hkv, D)).astype(np.float32)
    out, state["k_pages"], state["v_pages"] = oracle.attention_step(
        q, kn, vn, state["k_pages"], state["v_pages"], state["page_table"], state["ctx"])
    logits = (rng.standard_normal((B, R, V)) * 2).astype(np.float32)
    hot = state["drafts"][:, 0] >= 0
    logits[hot, :N - 1] = state["draft_rows"][hot] + (rng.standard_normal((int(hot.sum()), N - 1, V)) * 0.4)
    u = u24(rng, (B, R))
    res = verify(logits, state["draft_rows"], state["drafts"], u, N)
    state["ctx"], state["drafts"], toks, cnt = commit(res["n_accept"], res["next_token"], res["sampled_ids"],
                                                     state["drafts"], state["ctx"], N)
    state["draft_rows"] = logits[:, N:].copy()
    return dict(out=out, n_accept=res["n_accept"], tokens=toks, counts=cnt, ctx=state["ctx"].copy())


def save(state, rng, path):
    np.savez(path, **state)
    with open(str(path) + ".rng.json", "w") as f:
        json.dump(rng.bit_generator.state, f)


def load(path):
    with np.load(str(path) + ".npz", allow_pickle=False) as z:
        state = {k: z[k].copy() for k in z.files}
    rng = np.random.default_rng()
    with open(str(path) + ".rng.json") as f:
        rng.bit_generator.state = json.load(f)
    return state, rng


def test_resume_from_checkpoint_equals_uninterrupted_run(tmp_path):
    state, rng = initial_state()
    straight = [step(state, rng) for _ in range(6)]
    state, rng = initial_state()
    first = [step(state, rng) for _ in range(3)]
    save(state, rng, tmp_path / "ckpt")
    del state, rng
    state, rng = load(tmp_path / "ckpt")
    resumed = first + [step(state, rng) for _ in range(3)]
    assert sum(int(s["n_accept"].sum()) for s in straight) > 0      # the loop accepted drafts
    for a, b in zip(straight, resumed):
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_rejected_slots_are_overwritten_and_change_nothing():
    state, rng = initial_state(seed=9)
    # run until some request rejected a draft: its slots past the new length are stale
    for _ in range(20):
        before = state["ctx"].copy()
        rec = step(state, rng)
        rolled = (before + R) > state["ctx"]
        if rolled.any():
            break
    assert rolled.any()
    # a cache that never held the rejected rows: the same pages with every slot past ctx zeroed
    clean_k, clean_v = state["k_pages"].copy(), state["v_pages"].copy()
    stale = 0
    for b in range(B):
        for j in range(int(state["ctx"][b]), clean_k.shape[0] // B * PAGE):
            p = state["page_table"][b, j // PAGE]
            stale += int(np.any(clean_k[p, :, j % PAGE] != 0))
            clean_k[p, :, j % PAGE] = 0
            clean_v[p, :, j % PAGE] = 0
    assert stale > 0, "the rejected rows were left in the cache"
    q = rng.standard_normal((B, R, Hq, D)).astype(np.float32)
    kn = rng.standard_normal((B, R, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, R, Hkv, D)).astype(np.float32)
    a, ka, va = oracle.attention_step(q, kn, vn, state["k_pages"], state["v_pages"], state["page_table"], state["ctx"])
    c, kc, vc = oracle.attention_step(q, kn, vn, clean_k, clean_v, state["page_table"], state["ctx"])
    assert np.array_equal(a, c)
    # every slot up to the end of the new block agrees; only stale slots past it differ
    for b in range(B):
        for j in range(int(state["ctx"][b]) + R):
            p = state["page_table"][b, j // PAGE]
            assert np.array_equal(ka[p, :, j % PAGE], kc[p, :, j % PAGE])
            assert np.array_equal(va[p, :, j % PAGE], vc[p, :, j % PAGE])
    assert rec["counts"].sum() > 0
