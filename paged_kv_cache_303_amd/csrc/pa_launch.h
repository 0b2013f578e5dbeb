// Internal launch interface between the C ABI entry points (pa_api.cpp) and
// the kernel translation units.  Arguments here are already validated.
#pragma once

#include <stdint.h>

#include "../../include/pa.h"

// KV heads (one wave each) per decode workgroup, at most.
#ifndef PA_WAVES_PER_GROUP
#define PA_WAVES_PER_GROUP 2
#endif

namespace pa {

struct DecodeArgs {
  const void* q;               // [num_q_tokens, num_q_heads, head_dim]
  const void* k_pool;          // [num_blocks, block_size, num_kv_heads, head_dim]
  const void* v_pool;
  const float* k_scale;        // fp8 pools: [num_blocks, block_size, num_kv_heads] scales
  const float* v_scale;        //   (nullptr for fp32 / bf16 pools)
  const int32_t* block_tables; // [num_seqs, max_blocks]
  const int32_t* seq_lens;     // [num_seqs]
  const int32_t* cu_q_lens;    // [num_seqs + 1] or nullptr (one query per sequence)
  void* out;                   // final output (pa_decode)
  float* part_o;               // partial outputs (pa_decode_split)
  float* part_lse;
  float scale_log2;            // scale * log2(e)
  int32_t num_seqs;
  int32_t num_q_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;               // pa_dtype
  int32_t num_blocks;
  int32_t block_size;
  int32_t log2_bs;
  int32_t max_blocks;
  int32_t partition_size;      // tokens per partition (split) or 0 (single pass)
  int32_t max_partitions;
  int32_t waves_per_group;     // KV heads (= waves) per workgroup
  int32_t* queue;              // split: work-queue counters in the caller's workspace
};

struct ReduceArgs {
  void* out;
  float* lse_out;
  const float* part_o;
  const float* part_lse;
  const int32_t* cu_q_lens;
  const int32_t* seq_lens;
  int32_t out_dtype;
  int32_t max_partitions;
  int32_t partition_size;
  int32_t num_seqs;
  int32_t num_q_tokens;
  int32_t num_q_heads;
  int32_t head_dim;
};

// Workspace of the balanced streaming decode (inside the caller's workspace).
struct StreamArgs {
  float* part_o;       // [num_slices, 2, num_q_heads, head_dim]
  float* part_lse;     // [num_slices, 2, num_q_heads]
  int32_t* seq_slices; // [num_seqs, 4]: first and last slice holding the sequence's
                       // tiles (-1: no key), whether the first slice begins with an
                       // earlier sequence, 0
  int32_t num_slices;  // equal slices of the batch's (sequence, tile) work (at most)
};

// Sequences the streaming decode handles per launch (its LDS holds two ints
// per sequence); larger batches use the grid kernel.
constexpr int32_t kStreamMaxSeqs = 4096;
size_t stream_lds_bytes(int32_t num_seqs);

// Cached device facts (pa_devinfo.cpp): the calling thread's current device,
// its compute-unit count, and how many workgroups of `kernel` (threads per
// workgroup, dynamic LDS bytes) one compute unit holds at once.
pa_status current_device(int* dev);
pa_status device_cus(int dev, int* cus);
pa_status resident_per_cu(int dev, const void* kernel, int threads, size_t lds, int* per_cu);

// Returns PA_OK, PA_ERR_UNSUPPORTED (no instance for the shape) or PA_ERR_HIP.
// Single-pass grid decode (one workgroup per sequence and KV-head group).
pa_status launch_decode(const DecodeArgs& a, void* stream);
// Number of slices = workgroups of the streaming kernel resident on the
// current device at once / KV-head groups.
pa_status stream_slices(const DecodeArgs& a, int32_t* num_slices);
pa_status launch_decode_stream(const DecodeArgs& a, const StreamArgs& s, void* stream);
// The library's own device scratch for the balanced decode (pa_decode_noalloc):
// kScratchBytes on every device, its address on the current device.
constexpr size_t kScratchBytes = (size_t)8 << 20;
pa_status scratch_buffer(void** ptr);
// Split first pass: one persistent launch over a work list of decode
// partitions and (bf16, head_dim <= 128) matrix-core prefill row tiles;
// writes partition p of every single-query sequence's query, and for every
// query of a multi-query sequence its two partitions (keys before and from
// the split point of half the cached context), or partition 0 with all its
// keys when that split point is 0.
constexpr int32_t kSplitMaxSeqs = 8192;  // sequences per launch (LDS prefix sums)
constexpr int32_t kSplitQueueInts = 16;  // work-queue counters the control block reserves
pa_status launch_split(const DecodeArgs& a, void* stream);
pa_status launch_reduce(const ReduceArgs& a, void* stream);
pa_status launch_kv_write(const pa_kv_layout& l, void* k_pool, void* v_pool, const void* k_new,
                          const void* v_new, const int32_t* slots, int32_t num_tokens,
                          void* stream);
// Quantizing cache write into e4m3 pools (bf16 new tokens).
pa_status launch_kv_write_fp8(const pa_kv_layout& l, void* k_pool, void* v_pool, float* k_scale,
                              float* v_scale, const void* k_new, const void* v_new,
                              const int32_t* slots, int32_t num_tokens, void* stream);
// dst_pool[dst] = src_pool[src] between two pools of the same layout (one may be
// pinned host memory); l.num_blocks is the destination's block count.
pa_status launch_swap_blocks(const pa_kv_layout& l, void* dst_k, void* dst_v, const void* src_k,
                             const void* src_v, int32_t src_num_blocks, const int32_t* pairs,
                             int32_t num_pairs, void* stream);
pa_status launch_copy_blocks(const pa_kv_layout& l, void* k_pool, void* v_pool,
                             const int32_t* pairs, int32_t num_pairs, void* stream);

}  // namespace pa
