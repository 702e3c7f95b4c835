"""Plain, slow CPU oracle for Skiparse-2D sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library and does not
import it.

Sources.  All citations name a web page by its title and the section on it:

* "OSP-Next summary" -- the Chinese-language summary page of OSP-Next
  (paper.rainbus.top/paper/2605.28691), sections 核心方法 (core method),
  方法步骤详情 (method steps), 技术新颖性 (novelty), 局限与改进 (limitations).
* "OSP-Next abstract" -- the English abstract as shown on chatpaper.ai and
  thelatestinai.com.
* "OSP-Next review" -- the Korean review on blog.secrett2633.cloud, section
  "Key Terms & Definitions".

Modules:

* :mod:`oracle.skiparse_ref` -- any-resolution plan, the token-wise and
  group-wise rearrange as a closed-form gather map and as a literal
  pad/reshape/transpose, masked attention per subsequence (float64), brute
  force block-masked full attention, and sampled-row evaluation for full-size
  shapes.
* :mod:`oracle.skiparse_bwd` -- the gradients dQ, dK, dV of the same attention
  for an upstream dO (the chain rule through softmax attention, per
  subsequence), the per-query log-sum-exp, and sampled-row evaluators for
  full-size shapes.
* :mod:`oracle.block_ref` -- one fp8 attention block around the sparse
  attention (per-tensor e4m3 input, QKV projections, 3-axis rotary embedding,
  attention, output projection), every product in float64.
* :mod:`oracle.fp8_ref` -- OCP FP8 E4M3 codec from the format definition and the
  per-tensor amax scale rule.
* :mod:`oracle.cpu_baseline` -- the same algorithm in fp32 numpy/BLAS, timed
  as the CPU baseline.

Every function is pinned by ``-m "not gpu"`` tests against values the pages
and the mathematics fix (hand-derived golden maps, torch's pixel_unshuffle,
textbook softmax attention, closed forms, invariants; for the gradients:
finite differences of the forward oracle and torch's float64 autograd; for
the block: the rotary embedding as complex rotation, its relative-position
property, torch's linear layers with the codec bypassed).  No function here is
"parity unpinned".
"""
