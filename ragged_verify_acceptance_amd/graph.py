"""HIP-graph capture of the verify path's library calls.

The SGLang integration of confidence-scheduled verification (the devpress.csdn.net article
on DSpark in SGLang, section "3. 可变长度验证的工程实现挑战"; the yichizhang.dev lesson,
section "Ragged verify under full CUDA graphs") packs the ragged windows and rounds the row
count up to the nearest captured tier, one graph per tier, because its kernels take the
tier as a launch shape.  Here every launch of the path has a
shape fixed by (B, gamma, max_rows) alone: the packed row count M and its tier are written
and read on the device.  One graph per batch shape therefore replays every tier, and the
host never reads M back to pick a graph.

The capture goes through ``torch.cuda.CUDAGraph`` (a hipGraph on ROCm), which records the
library's launches on the capture stream; the library allocates nothing and records no
memset or host synchronisation, so its calls are capturable as they are.
"""

from __future__ import annotations

from typing import Callable

import torch


class CallGraph:
    """Captures ``fn`` (a sequence of library calls on the current stream) once and replays it.

    Every buffer ``fn`` touches must stay alive and keep its address while the graph is in
    use; arguments are frozen at capture time, data is read at replay time.  ``fn`` runs once
    eagerly on a side stream before the capture (first-call set-up stays out of the graph),
    so its side effects happen once more than the replays: callers that mutate state
    (the commit advances context_lens) restore it before each replay.
    """

    def __init__(self, fn: Callable[[], None], warmup: bool = True):
        self.fn = fn
        self.graph = torch.cuda.CUDAGraph()
        if warmup:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph):
            fn()
        torch.cuda.synchronize()

    def replay(self) -> None:
        self.graph.replay()
