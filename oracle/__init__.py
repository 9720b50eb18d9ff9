"""Float64 CPU oracle for paged grouped-query decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.
It shares no code, table or header with the HIP library: it reads the same
input bytes and computes the same quantities by their plain definitions, in
float64, slowly and obviously.

Modules
-------
``e4m3``            OCP FP8 E4M3 (``e4m3fn``) decode/encode and per-(block, head)
                    quantisation of K/V blocks.
``paged_attention`` the paged KV pool as bytes, the slot write, the gather, and
                    decode attention (full, split into partitions, LSE merge).
``bruteforce``      a pure-Python triple loop for tiny inputs, used only to pin
                    the numpy oracle.

Every function says which passage of the pages it follows.  The pages are
cited by title and section:

* "rvLLM: High-performance LLM inference in Rust" (github.com/arm64be/rvllm),
  section "CUDA Kernels" (PagedAttention V2: block-table indirection with
  online softmax; Reshape and Cache: writing the new K/V into the paged cache;
  FP8 KV Cache: E4M3 quantisation with per-head scaling).
* "rvllm - A Small LLM Inference Engine in Rust" (ermolushka.github.io),
  section "How it's put together" (a pool of fixed-size blocks, explicit
  write positions and read blocks; each KV head shared by a group of query
  heads; each running sequence contributes one new token per decode step).
* "LLM Serving Kernels" (marcoharuni/llm-serving-kernels), section "Projects"
  (project 04: page tables, GQA/MQA, online softmax; project 05: E4M3
  storage, page scales, fused dequantisation) and "Verified NVIDIA L4
  release" (FP8 KV storage saving).
"""
