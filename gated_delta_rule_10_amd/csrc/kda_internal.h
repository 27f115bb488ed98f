// kda_internal.h -- host-side launchers shared between the libkda sources.
// Every launcher assumes its arguments were validated by kda_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Decode (one loop kernel, one workgroup per (row, head)): the plain step, the
// fused step (front end + step + output norm) and the speculative-decode
// verification with replay.
hipError_t launch_recurrent_step(const kda_recurrent_step_args &a, hipStream_t stream);
hipError_t launch_fused_decode_step(const kda_fused_step_args &a, hipStream_t stream);
hipError_t launch_spec_verify(const kda_spec_verify_args &v, hipStream_t stream);

// State pool copy/convert/zero.
hipError_t launch_state_io(kda_state_op op, const void *src, kda_dtype src_dtype,
                           int32_t src_slots, void *dst, kda_dtype dst_dtype,
                           int32_t dst_slots, const int32_t *indices, int32_t count,
                           int32_t num_heads, hipStream_t stream);

// Chunked prefill plan, computed on the host from sizes only.
struct ChunkPlan {
  int32_t num_seqs = 0;
  int32_t heads = 0;
  int64_t total_tokens = 0;
  bool varlen = false;
  int32_t segments = 1;          // segments per sequence (1 = no split)
  bool seg_front = false;        // segment 0 takes two shares of the chunks
  int64_t max_chunks = 0;        // chunks of the longest sequence
  // workspace layout (byte offsets)
  size_t order_off = 0, order_bytes = 0;      // int32 [N] longest-first sequence order
  size_t seg_state_off = 0, seg_state_bytes = 0;  // fp32 segment M / S~ / S_in buffers
  // balanced schedule of equal-length chains: workgroups, chunks per
  // workgroup, and the hand-over states + flags
  int64_t ho_workers = 0, ho_len = 0, ho_rounds = 0;
  size_t ho_off = 0, ho_bytes = 0;
  size_t total_bytes = 0;
};

kda_status plan_chunk_fwd(const kda_chunk_fwd_args &a, ChunkPlan *plan);

// The per-GPU scratch buffer of kda_chunk_fwd_no_alloc: its size, and its device
// address on the current device (looked up on the first call per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t no_alloc_scratch(void **addr);
hipError_t launch_chunk_fwd(const kda_chunk_fwd_args &a, const ChunkPlan &plan,
                            hipStream_t stream);

// Balanced schedule of C equal chains of n chunks on U compute units: whether
// the prefill uses it, and if so its runs (ho_len, ho_workers, ho_rounds).
bool balanced_schedule_applies(int64_t C, int64_t n, int U, ChunkPlan *pl);

// The per-GPU status word (KDA_DEVICE_* bits) and the polls a tail workgroup of
// the balanced schedule makes before giving up on its hand-over flag.
constexpr int32_t kDefaultHandoffPolls = 1 << 22;
hipError_t device_status_word(uint32_t **addr);
hipError_t read_device_status(hipStream_t stream, bool clear, uint32_t *bits);
int32_t handoff_poll_limit();
void set_handoff_poll_limit(int32_t polls);

// Chunked backward: workspace size and the three launches.
size_t chunk_bwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t heads);
size_t chunk_bwd_min_workspace_bytes(const kda_chunk_bwd_args &a);
hipError_t launch_chunk_bwd(const kda_chunk_bwd_args &a, int64_t total_tokens, int64_t max_sub,
                            hipStream_t stream);

}  // namespace kda
