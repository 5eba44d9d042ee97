"""CPU oracle for the Q-Sparse inference hot path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the bench may
import or call anything in this package.  The product (the HIP library and
its Python binding) never does, and shares no code with it: no kernels, no
headers, no helpers, no constants.

Everything here is plain NumPy, written from the definitions on the pages,
in float64 wherever the result is floating point, except the quantisers,
whose results are integers that the pages define through IEEE binary32
rounding and which therefore use float32 arithmetic step by step.

Sources cited in the docstrings:

* "Q-Sparse news article" -- the zxwl-tech.com report on Q-Sparse (Microsoft
  Research Asia, July 2024), sections "Sparsification with the Top-K
  function", "60% activated parameters reach the same result" and "A new
  scaling law for inference";
* "Q-Sparse abstract" -- the arXiv 2407.10969 listing page (shd-paper.top),
  authors' English abstract;
* "Turbo Sparse summary" -- the blog.csdn.net summary of Turbo Sparse
  (SJTU, June 2024), Eq. 2 (dReLU), Eq. 3-4 (top-k% by magnitude before the
  down projection) and the per-layer zero-activation figure;
* "Q-Sparse aibase report" -- the aibase.com (pt) news item, section on the
  advantages of sparse activation.

Parity status of each function is stated in its docstring; the quantiser
formulas are missing from the pages (their images were lost), so
``absmax_quant_i8`` and ``ternarize`` follow the stated reading and their
parity to the paper's own formula is unpinned.
"""
from .qsparse import (  # noqa: F401
    magnitude, topk_select, block_topk_select, sparse_linear, relu2, relu2_glu, drelu, absmax_quant_i8,
    ternarize, unpack_ternary, i8t_linear, ffn_relu2, ffn_relu2_glu, ffn_drelu,
    ffn_relu2_down_from, ffn_drelu_down_from, ste_backward, sparse_linear_backward,
    moe_route, moe_drelu_ffn,
)
