"""MI355X (gfx950) compressed attention of DeepSeek-V4: C4A/C128A compressors,
indexer top-k and sparse MQA with a learned sink, behind the C ABI of
libcsa.so (include/csa.h).  `binding` holds the entry points; `path` runs one
whole pass; `workloads` draws seeded synthetic inputs."""
__all__ = ["binding", "path", "workloads", "build"]
