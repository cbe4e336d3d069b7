"""MI355X-native fused Gaussian-mixture EM E-step (HIP for gfx950 behind a C-ABI).

Importing the package loads nothing native; ``soft_clustering_gmm_amd.gmm``
loads the HIP library on first use and fails loudly when it is missing.
"""
