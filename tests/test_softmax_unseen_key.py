"""The input that breaks a softmax shifted by a norm bound rather than by the
maximum logit, shown on the CPU with the oracle's own numbers.

The 129^3 decoder's queries of head h are Wq_h e, so they lie in the span of
the 51 columns of Wq_h (64 x 51). One token whose key gets a component of norm
400 along each head's unseen direction (orthogonal to that span) keeps every
logit within a few units of the others, but its key norm becomes ~400. The
bound B = ||q_h|| max_j ||k_hj|| (base-2 logit units, queries scaled by
log2(e)/8, inflated by 2^-8 for rounding) then exceeds the true maximum logit
t_max by more than 213 for every sampled query, so exp2(t + 64 - B) < 2^-149
for every token: a float32 softmax shifted by 64 - B has an all-zero row sum.
The GPU tests (test_gpu_dense.py, test_gpu_akvs.py) decode this K against the
oracle."""

import numpy as np

import vdm_workloads as W
from oracle import decoder as odec

LOG2E_8 = np.log2(np.e) / 8


def test_unseen_key_component_leaves_logits_and_inflates_the_bound():
    w = W.make(1)
    od = odec.Decoder.from_workload(w)
    K2 = W.with_unseen_key(od.K, w.weights["Wq"], w.H, token=7, norm=400.0)
    pts = W.gen.random_points(5, 1500)
    Q = od.q(pts) * LOG2E_8
    for h in range(w.H):
        c = slice(64 * h, 64 * h + 64)
        t_old = Q[:, c] @ od.K[:, c].T
        t_new = Q[:, c] @ K2[:, c].T
        # only token 7 changed, and its logits moved by bf16 rounding of the new
        # row only (the component itself is orthogonal to every query)
        assert np.array_equal(np.delete(t_new, 7, axis=1), np.delete(t_old, 7, axis=1))
        assert np.max(np.abs(t_new[:, 7] - t_old[:, 7])) < 4.0
        B = 1.00390625 * np.linalg.norm(Q[:, c], axis=1) * np.linalg.norm(K2[:, c], axis=1).max()
        gap = B - t_new.max(axis=1)
        assert gap.min() > 213.0, (h, gap.min())
    # the oracle's softmax (max-subtracted, float64) is unaffected: rows sum to 1
    P = odec.attention_probs(od.q(pts[:64]), K2, w.H)
    assert np.max(np.abs(P.sum(axis=-1) - 1.0)) < 1e-12


def test_unseen_directions_are_orthogonal_to_the_query_weights():
    w = W.make(1)
    U = W.gen.unseen_key_directions(w.weights["Wq"], w.H)
    for h in range(w.H):
        Wh = np.asarray(w.weights["Wq"], np.float64)[64 * h:64 * h + 64]
        assert abs(np.linalg.norm(U[h]) - 1) < 1e-12
        assert np.max(np.abs(Wh.T @ U[h])) < 1e-12
