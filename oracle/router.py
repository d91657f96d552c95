"""Router: top_k of E experts per token, renormalised weights.

[PE] "What does Paged Experts actually do?": an MoE layer sends each token to
top_k of its E experts (Qwen3-30B-A3B: 8 of 128). The routing itself is not
changed by paging ([PE] "Can paging change the model's outputs?").

Readings where the page is silent:
  * the top-k is taken on the float32 logits, compared as float32 (so that two
    different logits can never collapse into a tie through rounding of the
    probabilities); equal logits go to the smaller expert id; the ids are
    listed by descending logit, then ascending id;
  * the weights are the softmax over all E experts (float64), renormalised over
    the selected k so that they sum to one.
"""
import numpy as np


def topk_ids(logits_row, top_k):
    """Ids of the top_k largest float32 logits of one token; ties to the smaller id.

    Ordered by descending logit, then ascending id. Input must be finite.
    """
    z = np.asarray(logits_row, dtype=np.float32)
    if not np.all(np.isfinite(z)):
        raise ValueError("router logits must be finite")
    ids = np.arange(z.shape[0])
    # lexsort: last key is primary -> primary key -z (float32, exact), then id.
    order = np.lexsort((ids, -z))
    return order[:top_k].astype(np.int32)


def softmax64(logits_row):
    """Softmax over all E logits in float64."""
    z = np.asarray(logits_row, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def route(logits, top_k):
    """Route a batch: logits float32 [B, E] -> (ids int32 [B, k], weights float64 [B, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    B, E = logits.shape
    if not (1 <= top_k <= E):
        raise ValueError("need 1 <= top_k <= E")
    ids = np.zeros((B, top_k), dtype=np.int32)
    w = np.zeros((B, top_k), dtype=np.float64)
    for b in range(B):
        sel = topk_ids(logits[b], top_k)
        p = softmax64(logits[b])
        ps = p[sel]
        ids[b] = sel
        w[b] = ps / ps.sum()
    return ids, w
