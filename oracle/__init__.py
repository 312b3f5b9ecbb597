"""CPU fp64 oracle for the Cosmos 3 Mixture-of-Transformers joint-attention
hot path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the library (``include/``,
``multimodal_diffusion_transformer_amd/``) and never imports it; the only
common module is ``workloads`` (seeded inputs and the data format of a
segment list, no arithmetic of the method).

Sources (the pages, by title and section):

* "Cosmos 3 方法原理全解" (Cosmos 3 method explained), cnblogs:
  §2 the packed sequence S = [S_AR, S_DM] and its fixed DM order;
  §3 the two MoT "rooms" and the joint-attention equations O_AR / O_DM;
  §4.1 latent shapes of the video tokenizer;
  §5 the 3D mRoPE coordinates, Δt = 6/TPS and the AR→DM time gap of 15000;
  §6.3 the rectified-flow path x_σ = σε + (1-σ)x0, v* = ε - x0, and the
  flow shift of the noise level;
  §7.2 the Euler update x_next = x + (σ_next - σ)·v and the CFG combination
  v = v_base + w (v_cond - v_base); §7.3 the generation loop;
  §12.1 the recommended steps, guidance and shift per model and mode;
  §12.4 the model table (grouped Q / KV heads).
* "NVIDIA 发布 Cosmos 3 系列四个开放权重世界模型" (news page on four new
  checkpoints), section "流式生成如何工作" (how streaming generation works):
  temporal-causal chunk attention against a key/value cache.

Where the pages leave a step open, the reading taken is stated in the module
that uses it.  Every function here is pinned by a CPU test in ``tests/``
against values the pages print, closed forms, invariants or brute force; none
is "parity unpinned" except the end-to-end free-running chain of
``oracle.denoiser`` (see its docstring).
"""
from . import (layout, mask, mrope, attention, projection, euler, denoiser, streaming,  # noqa: F401
               schedule, cfg)
