"""MI355X-native fused EM step for diagonal-covariance Gaussian mixtures.

The compute path is the HIP library ``libgmm_em.so`` (built from ``csrc/``)
behind a C ABI; ``gmm_em_amd.ops`` is its thin Python binding. Importing this
package loads nothing; importing ``gmm_em_amd.ops`` loads the library and
fails loudly if it has not been built.
"""
