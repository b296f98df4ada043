// Host-side launchers of the libswasink kernels.  Each enqueues on `s` and
// returns the launch status; argument validation happens before, in abi.hip.
#pragma once

#include "common.h"

namespace swa {

// Shape-general vector-ALU kernels (fp32 or bf16 I/O, head_dim 64 or 128).
hipError_t launch_generic_prefill(const PrefillArgs& a, bool bf16_io, hipStream_t s);
hipError_t launch_generic_decode(const DecodeArgs& a, bool bf16_io, hipStream_t s);
hipError_t launch_generic_sparse(const SparseArgs& a, bool bf16_io, hipStream_t s);

// Matrix-core kernels: bf16 I/O, head_dim 128, query heads per KV head a multiple of 8.
// Sliding window of at most 128 keys, whole window held in registers.
hipError_t launch_swa_window_mfma(const PrefillArgs& a, hipStream_t s);
// Any window (or none) with online softmax over key chunks; used for global
// attention and for windows longer than 128.
hipError_t launch_online_mfma(const PrefillArgs& a, hipStream_t s);
// Ring decode, window 128, 1 <= T <= 4.
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s);

// Backward (gradients of O): delta, dq, dk/dv, dsink in stream order.
hipError_t launch_backward(const BackwardArgs& a, bool bf16_io, hipStream_t s);
// Matrix-core dq and dk/dv (bf16, head_dim 128, window <= 128, groups of 8k heads);
// needs delta in the workspace.
bool backward_mfma_supported(const BackwardArgs& a, bool bf16_io);
hipError_t launch_backward_mfma(const BackwardArgs& a, hipStream_t s);

// Rotary embedding in place (bf16 / fp32, head_dim 64 / 128), and the ring append of
// accepted tokens (keys rotated on the way in when a.rope_pos is set).
hipError_t launch_rope(const RopeArgs& a, bool bf16_io, hipStream_t s);
hipError_t launch_ring_append(const AppendArgs& a, bool bf16_io, hipStream_t s);

// Token-level top-k selection and the sparse decode over selected + recent keys.
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s);
bool sparse_mfma_supported(const SparseArgs& a, bool bf16_io);
hipError_t launch_sparse_decode(const SparseArgs& a, bool bf16_io, hipStream_t s);

// Compute units of the current device (cached per device).
hipError_t device_cu_count(int* out);

bool swa_window_mfma_supported(const PrefillArgs& a, bool bf16_io);
bool online_mfma_supported(const PrefillArgs& a, bool bf16_io);
bool decode_mfma_supported(const DecodeArgs& a, bool bf16_io);

}  // namespace swa
