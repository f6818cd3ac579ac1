"""Float64 CPU oracle for the verify step of speculative decoding.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The verify library (``draft_verify_sampling_amd``) never calls it, and
it shares no code with that library: it reads the stored input rows itself,
computes everything in float64 with plain numpy, one request at a time, in the
order the pages describe.

Pages followed (cited by title and section in each function):

* "第 13 篇：推理引擎一次猜几个字——草稿 + 验证" (zero-threshold inference-engine
  series, article 13): the greedy draft-then-verify loop (section ③, pseudocode),
  the history n-gram drafter (notes under ③), forward accounting (section ④).
* "投机解码:为什么一个字都不改" (course C13, lesson 3): accept with min(1, p/q),
  resample from norm(max(0, p - q)), the identity behind it, k+1 rows from one
  target forward with P = softmax(f / T), tokens per round = accepted + 1 and
  its closed form.
* "Speculative decoding explained" (opera24.net): greedy prefix verification
  on the fixed path ABCDEFG, its four-case table and its function contract.
* "Speculative Decoding II" (taking-lying-flat): EAGLE's tree verification
  (speculative sampling applied recursively at every node, as SpecInfer does),
  the EAGLE-2 dynamic tree and its worked example.

Pins (every public function is pinned by a CPU test against values the pages
print, closed forms, or brute force):

* ``chain.verify_greedy``       four-case table; forward accounting; greedy
                                 equals the sampled verify on one-hot rows;
                                 brute-force argmax on tiny rows.
* ``chain.greedy_path_verify``  four-case table and the disallowed inputs.
* ``chain.verify_sample``       the identity min(p,q) + (1-a) norm(max(0,p-q)) = p;
                                 exact law on V=8 by enumeration over drafts and
                                 exact integration over the uniforms; TV at
                                 sampling-noise level over 200,000 rounds;
                                 tokens-per-round closed form; alpha=0.8, k=1 ->
                                 1.8 exactly.
* edge readings of ``verify_sample``, ``verify_greedy`` and the three tree
  walks (tests/test_oracle_edges.py, hand-worked cases on one-hot rows):
  the end-token cut (inclusive, first occurrence only), the budget cut and
  the over-budget bit, the zero-residual fallback (chain: drawn from p_m with
  the fallback bit; tree: p unchanged for the next sibling), and the outputs
  and status bits of invalid requests (bad token, draft count, row range,
  tree shape).  The point-mass walk's fallback cannot occur in exact
  arithmetic (removing x from p leaves no mass only if p is the point mass
  on x, which is then always kept), so it has no hand case.
* ``chain.verify_sample(variant="resample_from_p")``  TV equal to the closed
                                 form 1/2 sum |min(p,q) - alpha p|.
* ``chain.naive_round``         acceptance = sum p q.
* ``chain.shard_pairs`` / ``combine_pairs``  the combined pairs of any column
                                 split equal the full row's (M, S) (1e-12).
* ``ngram.ngram_draft``         brute force over every window position on
                                 small contexts, hand cases.
* ``tree.verify_tree``          chain-as-tree equals ``verify_sample``; exact
                                 law on V=8 with i.i.d. sampled siblings.
* ``tree.verify_tree_greedy``   chain-as-tree equals ``verify_greedy``; equals
                                 ``verify_tree`` on one-hot target rows; every
                                 emitted token is the argmax of the previous
                                 kept node's row (brute force on small trees).
* ``tree.verify_tree_pointmass`` exact law on V=8 for fixed candidate sets
                                 (duplicates included): each emitted token
                                 follows the row it is drawn against; equals
                                 ``verify_tree`` when every draft row is one-hot
                                 at the node's single child.
* ``philox.philox4x64_10``      numpy's Philox bit generator (an independent
                                 implementation of the same published function)
                                 on many keys and counters, carries included.
* ``philox.philox_uniforms``    the slot-to-word mapping against those blocks;
                                 grid and range.
* ``tree_build``                the EAGLE-2 worked example (values, kept set,
                                 flattened order, positions); brute-force
                                 top-k; connectivity and ancestor-mask
                                 invariants on random rounds.
"""
from .rows import widen, FLAG_BAD_REQUEST, FLAG_BAD_TOKEN, FLAG_NONFINITE, \
    FLAG_OVER_BUDGET, FLAG_FALLBACK, FLAG_BAD_TREE, INVALID_FLAGS
from .chain import (verify_sample, verify_greedy, greedy_path_verify,
                    forward_accounting, naive_round, softmax_T, inverse_cdf,
                    shard_pairs, combine_pairs)
from .ngram import ngram_draft
from .tree import verify_tree, verify_tree_greedy, verify_tree_pointmass
from .philox import philox4x64_10, philox_uniforms
from .tree_build import DraftTree, topk_children, build_tree

__all__ = [
    "widen", "verify_sample", "verify_greedy", "greedy_path_verify",
    "forward_accounting", "naive_round", "softmax_T", "inverse_cdf", "shard_pairs", "combine_pairs",
    "ngram_draft", "verify_tree", "verify_tree_greedy", "verify_tree_pointmass",
    "philox4x64_10", "philox_uniforms", "DraftTree", "topk_children", "build_tree",
    "FLAG_BAD_REQUEST", "FLAG_BAD_TOKEN", "FLAG_NONFINITE", "FLAG_OVER_BUDGET",
    "FLAG_FALLBACK", "FLAG_BAD_TREE", "INVALID_FLAGS",
]
