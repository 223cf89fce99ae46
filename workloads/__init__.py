"""Seeded synthetic inputs (trees, factors, gates, states, accepted paths); no verify or
commit arithmetic lives here."""
from .gen import (CONFIG_NAMES, Layer, Workload, best_first_from_marginals, best_first_tree, draft_marginals,
                  make_accept_inputs, make_marginals,
                  greedy_branch, make_config,
                  make_random, random_tree)

__all__ = ["CONFIG_NAMES", "Layer", "Workload", "best_first_from_marginals", "best_first_tree", "draft_marginals", "greedy_branch", "make_accept_inputs", "make_marginals",
           "make_config", "make_random", "random_tree"]
