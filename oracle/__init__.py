"""Plain fp64 CPU oracle for exact Lloyd k-means.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call this package.
The library under ``exact_means_clustering_amd/`` never imports it, and the
oracle imports nothing from the library: the two share no kernels, helpers,
tables or pre/post-processing.  Inputs reach both sides from ``datagen``.

What it computes follows "Flash-KMeans: Fast and Memory-Efficient Exact
K-Means" (abstract): the method keeps the k-means formulas unchanged and is
exact, so the oracle is the textbook Lloyd iteration written out in fp64 —
an assignment stage (nearest centroid in squared Euclidean distance) and a
centroid update stage (per-cluster mean).  Every function cites the passage
it follows and lists the readings taken where the pages are silent.

Parity pins (see tests/test_oracle_pins.py): exact rational brute force on
tiny inputs with planted exact ties, closed forms (K=1, K=N), planted
separated mixtures, per-iteration invariants (counts, means, minimality,
the rounding-penalised monotonicity bound) and textbook library routines
(scipy.cluster.vq, scikit-learn Lloyd, numpy/torch float rounding).
"""

from .fp64 import (  # noqa: F401
    FORMATS,
    round_to_format,
    decode,
    sq_dist_direct,
    assign,
    assign_top2,
    soft_assign,
    gauss_sum,
    seed_random,
    kmeanspp,
    update,
    inertia,
    lloyd,
    near_tie_report,
    centroid_rel_err,
)
