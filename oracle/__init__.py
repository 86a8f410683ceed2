"""CPU oracle (float64) for the pre-norm dilated Conv1d block and Conv1d+GroupNorm.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg may import this package. The HIP library and
its Python binding never import or call it.
"""
from .reference import (batch_stats, bn_eval_relu, conv1d_k3_padded,  # noqa: F401
                        conv_groupnorm, conv_output_length, group_norm, prenorm_block,
                        prenorm_block_points, prenorm_block_train, relu_conv_residual,
                        running_stats_update, zero_pad_time)
