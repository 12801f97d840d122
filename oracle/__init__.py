"""fp64 CPU oracle for exact multi-head attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written reference that the HIP kernels are
checked against.  It is not part of the product path: only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``exact_io_aware_09_amd`` (kernels, C-ABI
or binding) and imports nothing from it; both sides receive the same seeded
input tensors from the caller.

Modules
-------
attention      standard attention with S and P materialised (forward) and the
               explicit chain-rule backward, fp64.
sampled        the same definitions restricted to chosen query rows / key rows,
               streamed over query chunks so that no N x N matrix is ever held
               at long sequence lengths.
online_softmax running (max, sum) statistics, element-wise and block-wise, and
               the symmetric merge of two partial states.
tiled          the tiled forward (outer loop over K/V blocks, inner over Q
               blocks, normalised output kept between steps) and the
               recomputing backward, as fp64 models of the algorithm.
io_model       element counts of HBM traffic for standard and tiled attention
               and FLOP counts.
philox         the Philox4x32-10 counter-based generator (Salmon et al., SC 2011).
dropout        the 8-bit draws of every (query, key) pair, the keep masks, and
               attention with dropout on the softmax weights, forward and
               backward, fp64.
fp8            the OCP E4M3 format, block quantisation with power-of-two
               block scales, and attention of the quantised inputs, fp64.

Sources: "Lecture 8 . GPU Performance & FlashAttention" (CS324 notes,
semidirectx.com), "Stanford CS336 Lecture 5: GPUs" (chengshu blog, section 7)
and "FlashAttention and GPU memory" (world.lapla.si).  Each function names the
section, equation or exercise it follows.

Parity status: every function here is pinned by tests under ``tests/`` that do
not re-type its formula (page-printed worked examples, closed forms,
finite differences, invariants, a library routine on special cases).  The one
page example whose inputs are not printed (eight scores in blocks of two,
"FlashAttention and GPU memory" section 08) is parity unpinned and is not
used.
"""
