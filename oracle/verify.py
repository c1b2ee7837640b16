"""Oracle: vocab-wide verification of one ISD step.  (Test infrastructure.)

What it follows:
  * One forward both proposes and verifies: [MASK] positions propose new tokens from a
    proposal distribution q, clean ("introspective") positions re-check earlier tokens
    against the causal anchor distribution p (「首次超越 AR 模型」 "I-DLM 如何解決這些問題"; 「内省扩散语言模型」
    "1. 引言", contribution list; 「I-DLM – introspektive Diffusion Language Models」 "Inference & ISD").
  * A proposal x is accepted with probability min(1, p(x)/q(x)), which makes the emitted
    tokens follow the AR distribution (「首次超越 AR 模型」 "I-DLM 如何解決這些問題"; 「I-DLM – introspektive Diffusion Language Models」
    "Inference & ISD").  The pages do not print what happens on a rejection; the only
    completion that keeps that guarantee is the standard one, resampling from the
    normalised residual max(0, p - q) -- taken as the reading here.
  * Proposals are argmax ids of the proposal rows (「首次超越 AR 模型」 "實際部署：SGLang 整合",
    argmax proposal; 「I-DLM – introspektive Diffusion Language Models」 "Serving (SGLang)").
  * Temperature divides the logits (the pages' example request uses 1.0, 「首次超越 AR 模型」 "快速開始").

Layout of one request's rows: logits rows 0..N-2 are the anchors p_i that verify draft
d_i; rows N-1..2N-2 are the N proposal rows.  draft_logits row i is the distribution
q~_i that d_i was drawn from (the previous step's proposal row); without it the drafts
are argmax proposals and q~_i is one-hot on d_i.

Steps, per request (all float64):
  1. softmax of every row: z = l / T, lse = m + log(sum exp(z - m)), prob = exp(z - lse)
  2. argmax of each proposal row over the raw stored logits, lowest id on ties
  3. walk i = 0 .. N-2: P = p_i(d_i), Q = q~_i(d_i); a = 1 if P >= Q else P / Q;
     accept iff u_i < a; stop at the first rejection i*
  4. rejection: w = max(0, p_i* - q~_i*), u' = (u - a) / (1 - a), next token = inverse
     CDF of w at u' (if w sums to 0, of p_i* -- unreachable when d ~ q~)
  5. full acceptance: next token = inverse-CDF draw of proposal row 0 at u_{N-1}
  6. sampled_ids[j] = inverse-CDF draw of proposal row j at u_{N-1+j}
Inverse CDF: the smallest k with (w_0 + ... + w_k) > u * sum(w), ids ascending.

Cold requests.  After a rejection the new proposals were made after a token that was
then rejected, so the next step has no valid drafts (「I-DLM – introspektive Diffusion
Language Models」 "Inference & ISD": the step that cannot verify emits one exact token and
fresh proposals).  A request whose draft_ids[b][0] is negative is such a cold request:
no walk (n_accept 0, nothing accepted, P = Q = 0), and the next token is the inverse-CDF
draw of row 0 -- the anchor of the next position -- at u_0.  Its proposal rows and
samples are as for any request.

Every draw is also checked against the boundaries it was compared with: a draw whose
uniform lies within `eps` of one (in u-space) is flagged, since a correct
implementation in another precision may fall on either side of it.
"""
import numpy as np

from .stored import to_f64


def log_softmax_row(z):
    """(lse, prob) of one row of scaled logits."""
    m = np.max(z)
    lse = m + np.log(np.sum(np.exp(z - m)))
    return lse, np.exp(z - lse)


def argmax_lowest(raw):
    """Lowest index holding the maximum value."""
    return int(np.flatnonzero(raw == np.max(raw))[0])


def acceptance_probability(P, Q):
    """min(1, P/Q), with no division when P >= Q (covers Q == 0)."""
    return 1.0 if P >= Q else P / Q


def residual_weights(p, q):
    return np.maximum(0.0, p - q)


def residual_uniform(u, a):
    """Given a rejection (u >= a), (u - a)/(1 - a) is again uniform on [0, 1)."""
    return (u - a) / (1.0 - a)


def inverse_cdf(w, u):
    """(k, lo, hi): k = smallest index with cumsum(w)[k] > u * sum(w);
    lo, hi = cumulative fractions bounding k's interval.  If rounding leaves no such
    index, the largest index with w > 0."""
    c = np.cumsum(w)
    total = c[-1]
    k = int(np.searchsorted(c, u * total, side="right"))
    if k >= len(c):
        k = int(np.flatnonzero(w > 0)[-1])
    lo = (c[k - 1] if k > 0 else 0.0) / total
    return k, lo, c[k] / total


def expected_acceptance(anchor_logits, draft_logits, temperature=1.0):
    """Probability that a draft d ~ q~ passes the test u < min(1, p(d)/q~(d)):
    sum_d q~(d) min(1, p(d)/q~(d)) = sum_k min(p_k, q~_k), with p = softmax(anchor/T) and
    q~ = softmax(draft/T) of one row each.  This is the acceptance rate p of the
    tokens-per-forward formula for i.i.d. rows."""
    _, p = log_softmax_row(to_f64(anchor_logits) / float(temperature))
    _, q = log_softmax_row(to_f64(draft_logits) / float(temperature))
    return float(np.sum(np.minimum(p, q)))


def verify(logits, draft_logits, draft_ids, uniforms, N, temperature=1.0, eps=1e-6):
    """One verification step for B requests.  Returns a dict of NumPy arrays:

    n_accept [B], accept [B,N-1] uint8, next_token [B], argmax_ids [B,N],
    sampled_ids [B,N], p_draft / q_draft [B,N-1], row_lse [B, 2N-1 + N-1]
    (draft-row entries 0 without draft logits), and the near-threshold flags
    accept_flag [B,N-1], residual_flag [B], sample_flag [B,N]."""
    raw = to_f64(logits)
    B, R, V = raw.shape
    assert R == 2 * N - 1 and N >= 1
    T = float(temperature)
    assert T > 0
    z = raw / T
    zd = None if draft_logits is None else to_f64(draft_logits) / T
    u_all = np.asarray(uniforms, dtype=np.float32).astype(np.float64)
    d_all = np.asarray(draft_ids)

    res = dict(
        n_accept=np.zeros(B, np.int32), accept=np.zeros((B, N - 1), np.uint8),
        next_token=np.zeros(B, np.int32), argmax_ids=np.zeros((B, N), np.int32),
        sampled_ids=np.zeros((B, N), np.int32), p_draft=np.zeros((B, N - 1)),
        q_draft=np.zeros((B, N - 1)), row_lse=np.zeros((B, R + N - 1)),
        accept_flag=np.zeros((B, N - 1), bool), residual_flag=np.zeros(B, bool),
        sample_flag=np.zeros((B, N), bool), accept_prob=np.zeros((B, N - 1)))

    for b in range(B):
        probs = []
        for r in range(R):
            lse, pr = log_softmax_row(z[b, r])
            res["row_lse"][b, r] = lse
            probs.append(pr)
        dprobs = []
        if zd is not None:
            for i in range(N - 1):
                lse, pr = log_softmax_row(zd[b, i])
                res["row_lse"][b, R + i] = lse
                dprobs.append(pr)

        for j in range(N):                              # proposals and their samples
            res["argmax_ids"][b, j] = argmax_lowest(raw[b, N - 1 + j])
            u = u_all[b, N - 1 + j]
            k, lo, hi = inverse_cdf(probs[N - 1 + j], u)
            res["sampled_ids"][b, j] = k
            res["sample_flag"][b, j] = abs(u - lo) < eps or abs(u - hi) < eps

        if N > 1 and int(d_all[b, 0]) < 0:             # cold: one exact token from row 0
            u = u_all[b, 0]
            k, lo, hi = inverse_cdf(probs[0], u)
            res["next_token"][b] = k
            res["residual_flag"][b] = abs(u - lo) < eps or abs(u - hi) < eps
            continue

        rejected = None
        for i in range(N - 1):                          # the acceptance walk
            d = int(d_all[b, i])
            P = probs[i][d]
            Q = dprobs[i][d] if zd is not None else 1.0
            a = acceptance_probability(P, Q)
            res["p_draft"][b, i], res["q_draft"][b, i], res["accept_prob"][b, i] = P, Q, a
            if rejected is not None:
                continue
            u = u_all[b, i]
            res["accept_flag"][b, i] = abs(u - a) < eps
            if u < a:
                res["accept"][b, i] = 1
            else:
                rejected = (i, a, u)
        res["n_accept"][b] = N - 1 if rejected is None else rejected[0]

        if rejected is None:                            # bonus token from proposal row 0
            res["next_token"][b] = res["sampled_ids"][b, 0]
            res["residual_flag"][b] = res["sample_flag"][b, 0]
        else:
            i, a, u = rejected
            d = int(d_all[b, i])
            if zd is not None:
                qt = dprobs[i]
            else:
                qt = np.zeros(V)
                qt[d] = 1.0
            w = residual_weights(probs[i], qt)
            up = residual_uniform(u, a)
            if np.sum(w) > 0:
                k, lo, hi = inverse_cdf(w, up)
            else:
                k, lo, hi = inverse_cdf(probs[i], up)
            res["next_token"][b] = k
            # boundaries mapped back to u-space: u = a + (1 - a) * C / W
            res["residual_flag"][b] = (abs(u - (a + (1 - a) * lo)) < eps or
                                       abs(u - (a + (1 - a) * hi)) < eps)
    return res


def commit(n_accept, next_token, sampled_ids, draft_ids, ctx_lens, N):
    """State of every request after one step (the two-state chain of tokens per
    forward, 「I-DLM – introspektive Diffusion Language Models」 "Speedup Factor
    Explorer", with the slots of one strided block).

    The block held [c, d_1 .. d_{N-1}, MASK ..] (hot) or [c, MASK ..] (cold), c being the
    last committed token at position ctx_len.  The step keeps c and the n accepted
    drafts, so ctx_len grows by n + 1 and next_token becomes the new c.  The next step is
    hot -- drafts sampled_ids[1 .. N-1], drawn from the [MASK] rows -- when this step
    was cold or accepted every draft; otherwise those proposals followed a rejected
    token and the next step is cold (draft ids -1).

    Returns (ctx_lens', draft_ids', emitted tokens [B, N] padded with -1, count [B])."""
    n_accept = np.asarray(n_accept)
    draft_ids = np.asarray(draft_ids)
    B = len(n_accept)
    ctx = np.asarray(ctx_lens).astype(np.int64).copy()
    nxt = np.full((B, max(N - 1, 0)), -1, np.int32)
    out = np.full((B, N), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        cold = N > 1 and int(draft_ids[b, 0]) < 0
        n = 0 if cold else int(n_accept[b])
        toks = [int(t) for t in draft_ids[b, :n]] + [int(next_token[b])]
        out[b, :len(toks)] = toks
        cnt[b] = len(toks)
        ctx[b] += len(toks)
        if N > 1 and (cold or n == N - 1):
            nxt[b] = np.asarray(sampled_ids)[b, 1:N]
    return ctx.astype(np.int32), nxt, out, cnt
