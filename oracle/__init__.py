"""CPU oracle for pipelined tile copy + elementwise (TEST INFRASTRUCTURE ONLY).

A plain, slow, obviously-correct reference written from the four pages on
asynchronous tile copies:

* "copy_async -> tma" (TVM TIRx docs): host-encoded tile descriptor, plan
  search, 128-byte swizzled shared layout;
* "elementwise -> smem" (TVM TIRx docs): ``[outer, threads, vec]`` partition
  and the elementwise op registry;
* "Add TMA support for circular buffering pass" (nvFuser PR #2833): the
  N-stage ring (prologue / main / epilogue) and its stage-index formulas;
* "copy_async -> ldgsts" (TVM TIRx docs): per-thread async vector copies and
  the vector-width / outer-count table.

Modules
-------
``swizzle``   XOR swizzles (32-, 64- and 128-byte modes) of stage-relative LDS
              byte offsets.
``plan``      descriptor encode, plan search (L1 -> L2 -> L3), partition.
``tiles``     LDS byte image of a tile (gather, swizzle, zero fill) and the
              tiled copy / elementwise data path built from it.
``ops``       the elementwise ops with IEEE-754 round-to-nearest-even results
              (exact fma via round-to-odd; sqrt and exp computed in binary32).
``ring``      the circular-buffer event schedule with per-wait counters.
``reference`` the plain definitions every result must equal (copy,
              elementwise, streamed fma, store with reduce-add, row sums).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
and imports nothing from it.

Parity pins: every function here is pinned by a ``-m "not gpu"`` test
against something other than itself (the pages' worked examples, closed
forms, exact rational arithmetic, libm, brute force).  No function is
"parity unpinned".
"""
