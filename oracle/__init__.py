"""Plain fp64 CPU oracle of the E2Former-V2 node-centric attention layer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call, link or execute anything under oracle/.
The product path (atomistic_attention_amd, its HIP library) never does, and the
oracle imports nothing from the product path: the two share no code.

Parity status per function (what pins it to something other than itself is in
tests/test_oracle_*.py):
  so3.real_sh / real_sh_legendre  pinned: scipy complex harmonics, closed forms
  so3.cg_complex                  pinned: sympy, unitarity
  so3.paths                       pinned: the literal path lists at l_max 0..3
  so3.coupling_tensor             pinned: equivariance, dot/cross closed forms,
                                  sparsity rule of the explainer section 2.2, the
                                  closed-form EAAS table at l_max = 2 (odd paths too)
  so3.wigner_d                    pinned: D^1 = P R P^T, orthogonal, det 1, homomorphism
  so3.eaas_couple                 pinned: Proposition 4.3 (equals the full CG product)
  layer.neighbors                 pinned: scipy cKDTree (sets and K-nearest)
  layer.rbf_bias                  pinned: closed-form values of Gaussians and envelope,
                                  0 from the cutoff on (value and slope)
  layer.attention                 pinned: torch scaled_dot_product_attention (l_max = 0),
                                  one-neighbour and equal-logit special cases
  layer.layer_forward             pinned: rotation equivariance to 1e-10; per-degree
                                  W_V / W_O by distinct scalar weights per degree; a
                                  listed pair beyond the cutoff against a closed-form
                                  softmax
  stack.filter_rows               pinned: equals the brute-force search at the smaller cutoff
  stack.max_displacement2         pinned: exact dyadic displacements, strict threshold
  stack.StackState (rebuild rule) pinned: trajectories with known rebuild steps
  stack.stack_step / run_stack    pinned: topology reuse on a two-atom system, rotation
                                  equivariance of the whole stack to 1e-10
  backward.grad_h                 pinned: central finite differences of layer.layer_forward
                                  (directional and element-wise), forward equal to
                                  layer.layer_forward, one-neighbour and isolated-atom cases
  edge.solid_sh                   pinned: polynomial closed forms to l = 2, homogeneity, parity
  edge.edge_forward               pinned: invariance under a common translation, rotation
                                  equivariance (l_max 1..3), the l <= 1 paths by hand (dot
                                  and cross products), alpha from a closed-form bias
  backward.stack_grad_pos_h       pinned: central finite differences of the numpy layer
                                  composition over the stack's fixed lists
"""
from . import so3, layer, stack, backward, edge  # noqa: F401
