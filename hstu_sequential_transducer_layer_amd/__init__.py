"""HSTU sequential-transducer layer forward for AMD MI355X (gfx950).

The layer (pointwise SiLU attention with relative position/time bias over
jagged sequences, LayerNorm, U gate, output projection) runs in hand-written
HIP kernels behind the C ABI of libhstu.so (include/hstu.h).  Submodules:

  _lib      ctypes binding of the C ABI (argument marshalling only)
  layer     device helpers: workload -> tensors, stacks of layers
  synth     seeded synthetic workloads
  build_lib hipcc build of libhstu.so
"""

__all__ = ["_lib", "layer", "synth", "build_lib"]
