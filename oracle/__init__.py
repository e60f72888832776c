"""fp64 CPU oracle for the exact MoE-layer forward over a global expert cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product library never calls it, and it shares no code with the
HIP path: it reads the packed expert records and the element formats with its
own decoders, written from the format specifications.

What it follows (FreeToken pages; "explainer" = the frelia.link explainer page,
"architecture guide" = the freetoken.wiki page):
  * the output is the exact MoE output and routing is neither changed nor
    approximated; a split of the selected experts between places is summed
    and stays mathematically identical (explainer, "how" section);
  * one LRU expert cache in free device memory is shared by all MoE layers,
    the full expert pool lives in host memory (explainer, "how" section);
  * LRU means: at capacity, drop the entry unreferenced for longest
    (explainer, glossary);
  * layer shape 256 experts / 6 active / 43 layers (explainer, "why now").
The pages give no formula for the layer; the plain textbook reading is used:
softmax router scores, top-k with renormalised gates, SwiGLU experts,
gate-weighted sum.

Modules: ``formats`` (element decoders), ``record`` (packed-record parser),
``moe`` (routing, expert FFN, layer), ``lru`` (the slot-table state machine),
``mx`` (MXFP8 activation quantisation mirrored for the prefill path).
"""
