"""MI355X (gfx950) implementation of the Key-Value Means attention layer's
chunk-parallel prefill and decode.

The compute lives in libkvm.so (hand-written HIP kernels behind the C ABI in
include/kvm.h); this package only binds it for PyTorch tensors.
"""
from .kvm import (DTYPE, KVM_E_CAPACITY, KVM_E_HIP, KVM_E_INVALID_ARG, KVM_E_STATE, KVM_E_WORKSPACE,
                  KVM_FLAG_NO_MERGE_GATE, KVM_FLAG_NO_SINK_PROTECT, KVM_FLAG_NO_VALUE_NORM, KVM_FLAG_TRACE, KVM_OK,
                  SCHED, KvmConfig, KvmError, KvmState, library, prefill_noalloc, project_in, project_out, schedule,
                  workspace_bytes)

__all__ = ["KvmConfig", "KvmState", "KvmError", "library", "schedule", "workspace_bytes", "prefill_noalloc", "project_in", "project_out",
           "SCHED", "DTYPE",
           "KVM_OK", "KVM_E_INVALID_ARG", "KVM_E_WORKSPACE", "KVM_E_CAPACITY", "KVM_E_STATE", "KVM_E_HIP",
           "KVM_FLAG_TRACE", "KVM_FLAG_NO_VALUE_NORM", "KVM_FLAG_NO_SINK_PROTECT", "KVM_FLAG_NO_MERGE_GATE"]
