"""fp64 CPU oracle for the PRISM matrix-function path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it. It shares no code with the HIP
library; the two meet only through the seeded input generators in
``workloads`` (which hold none of the method's arithmetic).

Sources (titles of the web pages the method is taken from):
  * "深度学习中的优化器之Shampoo算法原理与二阶优化机制" (idocdown blog on Shampoo),
    cited as [Shampoo blog] with its section numbers.
  * "PRISM：分布无关的自适应矩阵函数计算以加速神经网络训练" (euno.news summary of
    arXiv 2601.22137), cited as [PRISM summary].
  * "Sintesi Tecnica: PRISM" (gist.science synthesis of arXiv 2601.22137),
    cited as [PRISM synthesis] with its Part I / Part II headings.

Modules
  closed_form  -- the definitions: Shampoo statistics EMA, eigendecomposition
                  roots, SVD polar factor, preconditioned apply.
  prism        -- the step-by-step fp64 PRISM Newton-Schulz iteration (alpha fit
                  on a Gaussian sketch, coupled square root, chained inverse 4th
                  root, polar factor), used to pin alpha traces, iteration and
                  product counts.
  inv_newton   -- the coupled inverse Newton iteration for A^{-1/p} with the
                  PRISM coefficient (residual map 1 - (1 - xi) g^p, an objective
                  of degree 2p in alpha).
  shampoo_step -- a whole Shampoo step over a model's layers (block-diagonal
                  statistics, roots every k steps, momentum, adaptive rate,
                  convolution reshape), from the closed forms.
  interval     -- the [lo, hi] interval rule for the adaptive coefficient.
  eigen_model  -- the same iteration on a known spectrum (scalar map), an
                  independent route to iteration counts and alpha.
  philox       -- Philox4x32-10 counter-based generator and Box-Muller normals
                  that define the sketch matrices.

Parity status: every function here is pinned by tests/test_oracle_*.py against
closed forms, library routines of a different algorithm, brute force or
published test vectors.  The multiplication-count ratio quoted by the PRISM
summary's results table (about 2.2x for a 10^4 square root) is "parity
unpinned": the pages do not give the spectrum, degree or baseline behind it.
"""
