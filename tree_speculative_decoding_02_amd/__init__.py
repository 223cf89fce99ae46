"""MI355X (gfx950) Bole tree verification and accepted-path commit for linear-recurrence
layers. The compute lives in libbole.so (HIP kernels behind the C ABI of include/bole.h);
``bole`` is its thin Python binding."""
from .bole import (bind_build_tree, bole_build_tree, bind_tree_accept, bole_tree_accept, bind_commit_path, bind_commit_path_layers, bind_tree_verify,
                   bind_tree_verify_lazy_commit, bind_tree_verify_lazy_commit_layers,
                   bind_tree_verify_layers, bole_commit_path, bole_commit_path_layers,
                   bole_tree_prepare, bole_tree_verify, bole_tree_verify_lazy_commit,
                   bole_tree_verify_lazy_commit_layers, bole_tree_verify_layers,
                   bole_tree_verify_naive, BoleError, MAX_TREE_NODES)

__all__ = ["bind_build_tree", "bole_build_tree", "bind_tree_accept", "bole_tree_accept", "bind_commit_path", "bind_commit_path_layers", "bind_tree_verify",
           "bind_tree_verify_lazy_commit", "bind_tree_verify_lazy_commit_layers",
           "bind_tree_verify_layers", "bole_commit_path", "bole_commit_path_layers",
           "bole_tree_prepare", "bole_tree_verify", "bole_tree_verify_lazy_commit",
           "bole_tree_verify_lazy_commit_layers", "bole_tree_verify_layers",
           "bole_tree_verify_naive", "BoleError", "MAX_TREE_NODES"]
