"""CPU oracle for the Mixtral sparse mixture-of-experts layer forward and the
attention sub-block in front of it.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP kernels in ``sparse_mixture_experts_32_amd`` and imports nothing from
that package.

Modules
-------
``moe_oracle``  numpy float64 implementation of the layer, for every size.
``scalar``      pure-Python loops over the definition, for tiny shapes.
``swa_oracle``  float64 sliding-window grouped-query attention with the
                rolling-buffer cache and chunked prefill (the sub-block in
                front of the MoE).
"""
