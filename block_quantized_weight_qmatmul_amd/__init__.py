"""Block-quantized weight mat-vec (Q4_0 / Q8_0, expert-indexed) for MI355X.

The compute lives in HIP kernels behind the C ABI of include/qmv.h
(``libqmv.so``); ``qmv`` is its thin Python binding.
"""
from .qmv import (QMV_EALIGN, QMV_EHIP, QMV_EINVAL, QMV_EUNSUPPORTED, QMV_OK, QMV_Q4_0, QMV_Q8_0, QmvError,
                  qmv_batch, qmv_id, qmv_q4_0, qmv_q8_0)

__all__ = ["qmv_q4_0", "qmv_q8_0", "qmv_id", "qmv_batch", "QmvError", "QMV_OK", "QMV_EINVAL", "QMV_EALIGN",
           "QMV_EUNSUPPORTED", "QMV_EHIP", "QMV_Q4_0", "QMV_Q8_0"]
