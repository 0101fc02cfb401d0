"""Plain fp64 CPU oracle for YaRN-scaled RoPE causal attention.

TEST INFRASTRUCTURE ONLY.  This package states, as directly as numpy allows,
what the attention hot path computes: the YaRN rotary frequencies and logit
temperature, the pairwise rotation, and dense causal softmax attention with
grouped-query heads (prefill), plus attention of one new query over a cache
(decode) and the log-sum-exp merge of partial results.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  The GPU library never imports, links or calls it,
and it shares no code, constants or helpers with the GPU library.

Sources (web pages about long-context attention, cited by title and section):
  * "LLM context window mechanics" (randomcommits.com) -- sections
    "The memory wall, quantified" and "The position wall: RoPE and
    interpolation".
  * "Long Context" (gunjandhanuka research hub) -- "Key math / How it works".
  * "Arch 03 -- Long Context" (brendanjameslynskey slide deck) -- the
    scaled-dot-product attention slide, the RoPE slide, the Position
    Interpolation slide, the NTK-aware slide, the YaRN slide and its steps
    table, and the ALiBi slide (for the causal visibility rule).
  * "Long context (engineering 100k+ tokens)" (askaiml academy) -- sections 1-2.
  * "Long-context models" (blog.ecitis.org) -- "Position enters attention",
    "Context parallelism distributes exact attention".

Parity status: every function here is pinned by the CPU tests in ``tests/``
(closed forms, invariants, brute force on tiny inputs, printed values).  The
pages print no worked YaRN frequency or attention value, so the YaRN table is
pinned by what the mathematics fixes: s = 1 gives plain RoPE, the pure
regions give exactly theta and theta/s, the region boundaries agree with their
closed form, and the ramp interior is pinned at constructed original lengths
that put a pair at a known turn count (half way from alpha to beta: the mean
of theta/s and theta; a quarter and three quarters of the way: the values
that fixes) and by its linearity in the original length.  Dynamic NTK is
pinned by its rule (no scaling below the training length) and by the NTK-aware
slide's worked base at eight times the training length.
"""

from . import freqs, rope, attention, bruteforce  # noqa: F401
