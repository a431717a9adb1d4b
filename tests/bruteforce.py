"""Scalar-loop restatement of one attention output element, for tiny inputs.

Independent of the oracle's vectorised code: plain Python floats, math.exp,
math.tanh and math.fsum, one key at a time.  Used only as a pin."""
import math


def attention_row(q, keys, values, pos, *, scale, window=0, cap=0.0, sink=None):
    """q: list[D]; keys/values: list of list[D] for positions 0..kv_len-1.
    Returns list[D]: sum_j w_j v_j with w the softmax over visible keys."""
    logits = []
    for j, k in enumerate(keys):
        if j > pos:
            continue
        if window and pos - j >= window:
            continue
        s = math.fsum(a * b for a, b in zip(q, k)) * scale
        if cap:
            s = cap * math.tanh(s / cap)
        logits.append((j, s))
    m = max([s for _, s in logits] + ([sink] if sink is not None else []))
    ws = [(j, math.exp(s - m)) for j, s in logits]
    z = math.fsum([w for _, w in ws] + ([math.exp(sink - m)] if sink is not None else []))
    D = len(q)
    return [math.fsum(w * values[j][d] for j, w in ws) / z for d in range(D)]
