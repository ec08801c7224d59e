"""One update over a layer set, as the sequence of library calls.

Argument marshalling only: these functions fix the order and grouping of the
calls (which matrices share one launch, in which order) and issue them
through the binding; every step runs in liblogra's kernels.  The benchmark
times exactly this sequence, and the full-size parity tests run it.

For every selected matrix of every layer and every microbatch ("LoGRA: Scaling
LLM Reinforcement Learning with Low-Rank Gradient Sketches", §2.1-2.3):

  project     XAt = X A^T, written in the accumulate's packed operand form;
              one persistent launch per microbatch (or per group of
              microbatches whose inputs are stored one after another, which
              is one launch over their tokens) over all matrices of all
              layers, layers ascending and each layer's matrices in
              q, k, v, o, gate, up, down order, so the matrices that share an
              input (q, k, v; gate, up) are neighbours and are projected
              together, reading their input once
  accumulate  S += D^T XAt; one persistent launch per microbatch (or group)
              over all matrices, layers in reverse (the order a backward pass
              produces their derivatives)
  optimise    RowAdam of every sketch in one grouped call, writing the update
              in the merge's packed operand form
  step size   q over the context set and alpha = min(alpha_max, sqrt(delta/q)),
              both on the device
  merge       W <- round(W - eta alpha U A); one grouped launch per layer (or per
              group of layers)

Accessors are callables: key(l, kind), x(l, kind) and so on return the key or
tensor of matrix `kind` of layer `l` (for the microbatch being processed).
"""
from __future__ import annotations

from . import binding as B

KINDS = ("q", "k", "v", "o", "gate", "up", "down")
# the layer input each projection reads: q, k, v the attention input, gate and
# up the MLP input
SHARED_INPUT = {"q": "att", "k": "att", "v": "att", "o": "o", "gate": "mlp", "up": "mlp", "down": "down"}


def project(layers, kinds, key, x, planes, r, ws, stream=None):
    """One microbatch's projections of every matrix of `layers` (one launch)."""
    B.project_input_table([(key(l, kd), x(l, kd), None, planes(l, kd)) for l in layers for kd in kinds],
                          r, ws=ws, stream=stream)


def accumulate(layers, kinds, d, planes, s, r, ws, stream=None):
    """One microbatch's sketch accumulation for every matrix of `layers` (one launch)."""
    B.sketch_accumulate_table([(d(l, kd), planes(l, kd), s(l, kd)) for l in reversed(list(layers))
                               for kd in kinds], r, ws=ws, stream=stream)


def optimise(sketches, r, t, beta, eps, ws, stream=None):
    """RowAdam of every (S, v, packed update) in one grouped call (three launches)."""
    B.rowadam_packed_grouped(sketches, r, t, beta, eps, ws=ws, stream=stream)


def step_size(z, zdot, tau, delta, alpha_max, q, alpha, ws, stream=None):
    """q over the contexts into q, then alpha into alpha (both one-element device tensors)."""
    B.predicted_kl_q(z, zdot, tau, out=q, ws=ws, stream=stream)
    B.step_alpha_dev(q, delta, alpha_max, out=alpha, stream=stream)


def merge(layers, kinds, key, w, up, r, eta, alpha, mode, sr_seed, stream=None, per_launch=1):
    """W <- round(W - eta * alpha * U A) for every matrix, one grouped launch per `per_launch`
    layers; alpha is a one-element device tensor (or None for alpha = 1)."""
    layers = list(layers)
    for i in range(0, len(layers), per_launch):
        B.merge_grouped_packed([(key(l, kd), w(l, kd), up(l, kd)) for l in layers[i:i + per_launch]
                                for kd in kinds], r, eta, scale_dev=alpha, mode=mode, sr_seed=sr_seed,
                               stream=stream)
