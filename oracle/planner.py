"""Plain definitions of the serving planners (test infrastructure only; integer arithmetic).

* Concurrency and token capacity: the free memory divided by what one sequence (per-token bytes times
  context length), or one token, needs, rounded down ("Grouped Query Attention: Why 8 KV Heads Decide
  Your Batch Size", section "Why does GQA decide your batch size?").
* Tensor-parallel head sharding: attention is sharded by query head, rank r taking the r-th of tp equal
  contiguous slices; a rank must hold every KV head its query heads read, under the contiguous grouping
  h -> h // G.  When tp exceeds the KV head count, or does not divide it, some KV heads are held by
  several ranks (replication): "What breaks when num_kv_heads is smaller than your tensor-parallel
  degree?" of the same page, and "Grouped-Query Attention: How Sharing KV Heads Shrinks Inference
  Memory", section "Why not always go to one KV head?".
"""


def max_concurrency(free_bytes, per_token, ctx_len):
    if per_token * ctx_len == 0:
        return 0
    return free_bytes // (per_token * ctx_len)


def max_cached_tokens(free_bytes, per_token):
    return 0 if per_token == 0 else free_bytes // per_token


def tp_plan(num_q_heads, num_kv_heads, tp):
    """List of (q_begin, q_end, kv_begin, kv_end) per rank, half-open ranges; None when the query heads
    do not split evenly (tp must divide num_q_heads) or the head counts are invalid."""
    if tp <= 0 or num_kv_heads <= 0 or num_q_heads <= 0 or num_q_heads % num_kv_heads or num_q_heads % tp:
        return None
    G = num_q_heads // num_kv_heads
    per = num_q_heads // tp
    plan = []
    for r in range(tp):
        q0, q1 = r * per, (r + 1) * per
        heads = sorted({h // G for h in range(q0, q1)})      # every KV head read by the slice
        plan.append((q0, q1, heads[0], heads[-1] + 1))
    return plan


def kv_heads_held(plan):
    return sum(kv1 - kv0 for _, _, kv0, kv1 in plan)
