"""CPU oracle for greedy IoU NMS -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls anything in it, and it imports nothing from the GPU library.

Contents:
  * ``c_nms``        -- ctypes front-end of ``nms_oracle.c`` (the oracle proper).
  * ``np_nms``       -- a second, independent implementation in numpy float32.
  * ``certify``      -- checks a kept list against the three properties that
                        characterise the greedy result uniquely.
  * ``brute_force``  -- subset enumeration for tiny inputs.
  * ``mask_rows``    -- the suppression bitmask by its definition.
  * ``c_matrix_nms`` -- Matrix NMS (Gaussian decay) through the C oracle.
  * ``np_matrix_nms``-- the same, as the naive matrix formulation in numpy.
"""
from .reference import (  # noqa: F401
    ORACLE_STATUS, OracleError, build_c_oracle, c_nms, c_pair_iou, np_nms, np_iou_pairs,
    stable_order, groups_of, certify, brute_force, mask_rows, iou_row_f32,
    c_matrix_nms, np_matrix_nms,
)
