"""CPU oracle for the ragged verify + acceptance path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The HIP library never calls it and it never calls the HIP library: the two share no
kernels, helpers, constants or tables.  The only code both sides consume is the seeded
input generator in ``workloads/``, which contains none of the method's arithmetic.

Every function here is the plain, slow definition of one step of the path, in float64
NumPy (float32 only where a step is defined in float32 so that integer decisions can be
reproduced bit for bit), with one Python loop per request.

Sources (web pages; cited by title and section, never by a line of any copy):

* [SGL]   "DFlash 到 DSpark in SGLang：解码提速 4.3×，以及 DeepSeek-V4 支持"
          (yichizhang.dev, AI-Infra-Visualized, lesson "dspark-speculative-decoding").
          Sections used: "Background", "DSpark：sequential head 加验证预算",
          "Confidence scheduler 与 verify 模式", "Ragged verify under full CUDA graphs".
* [CSDN]  the devpress.csdn.net (awstech) article on DSpark in SGLang, sections
          "2. DSpark如何实现真正的动态验证预算", "3. 可变长度验证的工程实现挑战",
          "4. 零开销调度如何隐藏计算成本" (the additive step-cost model T(bs, K)),
          "5. 可观测性：理解修剪下的真实性能" (the cap-accept verify mode).
* [NOTES] "DSpark：投机解码与生产级 Serving 学习笔记" (sorenprojections.com),
          sections "02 · Speculative Decoding", "05 · Core Innovation A"
          (semi-autoregressive generation, the Markov head), "07 · Confidence Head",
          "08 · Core Innovation B", "09 · End-to-End Cycle".

Pins: each function is checked in ``tests/test_oracle_pins.py``,
``tests/test_oracle_calibration.py`` and ``tests/test_oracle_markov.py`` against values
the pages print (``tests/golden/``), closed forms, special cases that reduce to a library
routine, and brute force on tiny inputs.  Parity unpinned: that the Sequential Temperature Scaling fit in
``calibration.py`` is the one the pages' authors ran (no page prints fitted temperatures;
the estimator itself is pinned by its single-position special case, by recovery of known
temperatures and by optimality).
"""

from .scheduling import confidence_from_head, survival, schedule_windows
from .packing import pack_ragged
from .attention import verify_attention
from .calibration import sts_fit, ece, log_prefix_survival
from .markov import markov_sample
from .acceptance import (softmax64, inverse_cdf, accept_request, accept_request_capped,
                         accept_and_commit, confidence_labels)

__all__ = [
    "confidence_from_head",
    "survival",
    "schedule_windows",
    "pack_ragged",
    "verify_attention",
    "softmax64",
    "inverse_cdf",
    "accept_request",
    "accept_request_capped",
    "accept_and_commit",
    "confidence_labels",
    "sts_fit",
    "ece",
    "log_prefix_survival",
    "markov_sample",
]
