"""fp64 CPU oracle for paged decode attention. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything here. The HIP library never calls into this
package and this package never imports the HIP library or its binding; the
two sides share only the seeded input generators in ``workloads/``.

Contents (each function cites the passage of the pages it follows):
  numerics   bf16 bit patterns -> exact float64
  allocator  refcounted block pool with copy-on-write (pure Python)
  store      host model of the paged K/V pool and its gather
  attention  softmax(q K^T * scale) V over the gathered context (fp64)
  split      partition-local attention and the log-sum-exp merge (fp64)
  kvbytes    closed form for KV-cache bytes per token
  fp8        OCP E4M3 codec and the per-(token, KV head) quantiser
  tree       tree-structured verification: ancestor masks, visible positions
  spec       speculative decoding's accept / resample step (fixed-point draw)
  prefix_cache  radix prefix cache over the pool (match, insert, LRU reclaim)

Pins (tests marked ``not gpu``): brute-force scalar loops, torch's fp64
scaled_dot_product_attention on the never-paged K/V, the literal block tables
printed on the pages, the closed form's printed values, invariants (placement,
prefix sharing, one-token context, zero query, causal rows), torch's
float8_e4m3fn for the codec, parent-pointer walks for the tree masks, the
identity P(x) = p(x) for the accept / resample step, and planted mistakes
that the pins must catch. No function here is "parity unpinned".
"""
