"""Tri-axis token tags and greedy bit widths -- TEST INFRASTRUCTURE ONLY.

Plain Python loops written from the TriAxialKV page:
- key design 1: the tag space is temporal (current, turn_m1, turn_m2, older) x modal
  (text, image) x semantic role (inst, user, assistant, reasoning, tool_call, obs,
  delim), read in one pass from the chat template's special boundary tokens;
- key design 2: minimise sum_k D_k(b_k) over b_k in {2, 4} with sum_k N_k b_k at most
  B sum_k N_k: start every tag at 2 bits, rank tags by rho_k = (D_k(2) - D_k(4)) /
  (2 N_k), largest first, and upgrade until the target average width B is reached.

Only the tests may import this module; the library shares nothing with it.
"""
TEMPORAL = ("current", "turn_m1", "turn_m2", "older")
MODAL = ("text", "image")
SEMANTIC = ("inst", "user", "assistant", "reasoning", "tool_call", "obs", "delim")
EVENTS = ("system", "user", "assistant", "observation", "end", "think_begin", "think_end",
          "tool_call_begin", "tool_call_end", "image_begin", "image_end")


def tag_tokens(tokens, markers):
    """tokens: sequence of ints; markers: {token id: event name}.  Returns (list of
    (temporal, modal, semantic) names per token, number of user turns)."""
    role = "inst"             # before any marker: system prompt / tool specifications
    inside = set()            # open spans among "think", "tool_call", "image"
    turn = 0
    walked = []               # (turn, modal, semantic) per token
    for tok in tokens:
        event = markers.get(int(tok))
        if event is None:
            if "tool_call" in inside:
                semantic = "tool_call"
            elif "think" in inside:
                semantic = "reasoning"
            else:
                semantic = role
            modal = "image" if "image" in inside else "text"
            walked.append((turn, modal, semantic))
            continue
        # a boundary token is a delimiter of the template, text, of the current turn
        # unless it opens a new user turn
        if event in ("system", "user", "assistant", "observation", "end"):
            inside.clear()    # a new role (or the end of one) closes every open span
            if event == "user":
                turn += 1
            if event != "end":
                role = {"system": "inst", "user": "user", "assistant": "assistant",
                        "observation": "obs"}[event]
        elif event.endswith("_begin"):
            inside.add(event[: -len("_begin")])
        else:
            inside.discard(event[: -len("_end")])
        walked.append((turn, "text", "delim"))
    tags = []
    for t, modal, semantic in walked:
        back = turn - t
        temporal = TEMPORAL[back] if back < 3 else "older"
        tags.append((temporal, modal, semantic))
    return tags, turn


def tag_index(temporal, modal, semantic):
    return (TEMPORAL.index(temporal) * len(MODAL) + MODAL.index(modal)) * len(SEMANTIC) + SEMANTIC.index(semantic)


def allocate_bits(d2, d4, counts, budget):
    """Greedy widths: list of 2 / 4 per tag, and the average width reached."""
    n = len(counts)
    bits = [2] * n
    total = sum(int(c) for c in counts)
    gain = []                 # (rho, tag) for tags that hold tokens
    for k in range(n):
        if counts[k] > 0:
            gain.append(((float(d2[k]) - float(d4[k])) / (2.0 * float(counts[k])), k))
    # largest rho first; equal rho: smaller tag index first
    gain.sort(key=lambda rk: (-rk[0], rk[1]))
    spent = 2 * total
    for _, k in gain:
        if spent + 2 * int(counts[k]) > budget * total:
            break             # the first tag that would exceed the budget ends the walk
        spent += 2 * int(counts[k])
        bits[k] = 4
    return bits, (spent / total if total else 2.0)
