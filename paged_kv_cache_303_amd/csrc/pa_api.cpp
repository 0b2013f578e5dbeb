// C ABI entry points of libpa.so for the device calls: argument validation,
// launch parameters, error reporting.  Kernels live in pa_decode.hip and
// pa_cache.hip; the host block pool in pa_pool.cpp.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/pa.h"
#include "pa_error.h"
#include "pa_launch.h"

namespace pa {
namespace {
thread_local std::string g_last_error;
}

pa_status fail(pa_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

namespace {

bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }
int32_t log2i(int32_t x) {
  int32_t r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Bytes of one pool element.
int64_t elt_bytes(int32_t dtype) { return dtype == PA_BF16 ? 2 : (dtype == PA_FP8 ? 1 : 4); }

// Checks the pool layout; `what` names the calling entry point.
pa_status check_layout(const pa_kv_layout* l, const char* what) {
  if (!l) return fail(PA_ERR_INVALID_ARG, "%s: layout is NULL", what);
  if (l->num_blocks <= 0 || l->block_size <= 0 || l->num_kv_heads <= 0 || l->head_dim <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: layout sizes must be positive", what);
  if (l->dtype != PA_F32 && l->dtype != PA_BF16 && l->dtype != PA_FP8)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d is not PA_F32, PA_BF16 or PA_FP8", what,
                l->dtype);
  if (l->dtype == PA_FP8 && l->head_dim < 64)
    return fail(PA_ERR_UNSUPPORTED, "%s: fp8 pools need head_dim >= 64", what);
  if (!pow2(l->block_size) || l->block_size > 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d is not a power of two <= 256", what,
                l->block_size);
  if (l->head_dim != 32 && l->head_dim != 64 && l->head_dim != 128 && l->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {32, 64, 128, 256}", what,
                l->head_dim);
  const int64_t rows = (int64_t)l->num_blocks * l->block_size;
  if (rows > (int64_t)INT32_MAX + 1)
    return fail(PA_ERR_INVALID_ARG, "%s: num_blocks*block_size exceeds the int32 slot range", what);
  const int64_t block_bytes =
      (int64_t)l->block_size * l->num_kv_heads * l->head_dim * elt_bytes(l->dtype);
  if (block_bytes > (int64_t)1 << 30)
    return fail(PA_ERR_UNSUPPORTED, "%s: one block exceeds 1 GiB", what);
  return PA_OK;
}

pa_status check_heads(const pa_kv_layout* l, int32_t num_q_heads, const char* what) {
  if (num_q_heads <= 0 || num_q_heads % l->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %d is not a positive multiple of num_kv_heads %d",
                what, num_q_heads, l->num_kv_heads);
  const int32_t g = num_q_heads / l->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PA_ERR_UNSUPPORTED, "%s: query heads per KV head %d not in {1, 2, 4, 8}", what, g);
  return PA_OK;
}

// KV heads handled by one workgroup (one wave each): the largest divisor of
// num_kv_heads that is at most PA_WAVES_PER_GROUP.
int32_t waves_per_group(int32_t num_kv_heads) {
  for (int32_t w = PA_WAVES_PER_GROUP; w > 1; --w)
    if (num_kv_heads % w == 0) return w;
  return 1;
}

pa_status launch_status(pa_status st, const char* what) {
  if (st == PA_ERR_UNSUPPORTED) return fail(st, "%s: no kernel instance for this shape", what);
  if (st == PA_ERR_HIP) return fail(st, "%s: kernel launch failed", what);
  return st;
}

}  // namespace
}  // namespace pa

using pa::fail;

static pa_status fill_decode_args(const char* what, const pa_kv_layout* layout, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, int32_t max_blocks,
                                  const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t num_q_heads, float scale, pa::DecodeArgs* a) {
  if (pa_status st = pa::check_layout(layout, what)) return st;
  if (pa_status st = pa::check_heads(layout, num_q_heads, what)) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_seqs < 0", what);
  if (max_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq must be > 0", what);
  if ((int64_t)max_blocks * layout->block_size > (int64_t)INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq*block_size overflows int32", what);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", what);
  if (num_seqs > 0 && (!q || !k_pool || !v_pool || !block_tables || !seq_lens))
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", what);
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->k_scale = nullptr;
  a->v_scale = nullptr;
  a->block_tables = block_tables;
  a->seq_lens = seq_lens;
  a->cu_q_lens = nullptr;
  a->out = nullptr;
  a->part_o = nullptr;
  a->part_lse = nullptr;
  a->scale_log2 = scale * 1.44269504088896340736f;
  a->num_seqs = num_seqs;
  a->num_q_tokens = num_seqs;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = layout->num_kv_heads;
  a->head_dim = layout->head_dim;
  a->dtype = layout->dtype;
  a->num_blocks = layout->num_blocks;
  a->block_size = layout->block_size;
  a->log2_bs = pa::log2i(layout->block_size);
  a->max_blocks = max_blocks;
  a->partition_size = 0;
  a->max_partitions = 1;
  a->waves_per_group = pa::waves_per_group(layout->num_kv_heads);
  a->queue = nullptr;
  return PA_OK;
}

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct StreamLayout {
  int32_t slices = 0;
  size_t o_bytes = 0, lse_bytes = 0, cum_bytes = 0;
  size_t total() const { return o_bytes + lse_bytes + cum_bytes; }
};

StreamLayout stream_layout_for(const pa::DecodeArgs& a, int32_t slices) {
  StreamLayout sl;
  sl.slices = slices;
  sl.o_bytes = align256((size_t)slices * 2 * a.num_q_heads * a.head_dim * sizeof(float));
  sl.lse_bytes = align256((size_t)slices * 2 * a.num_q_heads * sizeof(float));
  sl.cum_bytes = align256((size_t)a.num_seqs * 4 * sizeof(int32_t));
  return sl;
}

// Workspace of the balanced path for these arguments (slices = 0: the batch
// is too large for it and the grid kernel runs instead).
pa_status stream_layout(const pa::DecodeArgs& a, StreamLayout* sl) {
  *sl = StreamLayout();
  if (a.num_seqs <= 0 || a.num_seqs > pa::kStreamMaxSeqs) return PA_OK;
  int32_t slices = 0;
  const pa_status st = pa::stream_slices(a, &slices);
  if (st != PA_OK) return st;
  *sl = stream_layout_for(a, slices);
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return pa::g_last_error.c_str(); }

const char* pa_version(void) { return "libpa 0.1 gfx950"; }

pa_status pa_kv_write(const pa_kv_layout* layout, void* k_pool, void* v_pool, const void* k_new,
                      const void* v_new, const int32_t* slot_mapping, int32_t num_tokens,
                      void* stream) {
  const char* what = "pa_kv_write";
  if (pa_status st = pa::check_layout(layout, what)) return st;
  if (layout->dtype == PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 pools are written by pa_kv_write_fp8", what);
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_tokens < 0", what);
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", what);
  return pa::launch_status(
      pa::launch_kv_write(*layout, k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens, stream),
      what);
}

pa_status pa_copy_blocks(const pa_kv_layout* layout, void* k_pool, void* v_pool,
                         const int32_t* pairs, int32_t num_pairs, void* stream) {
  const char* what = "pa_copy_blocks";
  if (pa_status st = pa::check_layout(layout, what)) return st;
  if (layout->dtype == PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 pools (codes and scales) use pa_copy_blocks_fp8",
                what);
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_pairs < 0", what);
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !pairs) return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", what);
  const int64_t block_bytes = (int64_t)layout->block_size * layout->num_kv_heads *
                              layout->head_dim * pa::elt_bytes(layout->dtype);
  if ((int64_t)num_pairs * ((block_bytes + 16383) / 16384) > (int64_t)INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: too many pairs for one launch", what);
  return pa::launch_status(
      pa::launch_copy_blocks(*layout, k_pool, v_pool, pairs, num_pairs, stream), what);
}

pa_status pa_decode_workspace_size(const pa_kv_layout* layout, int32_t num_seqs,
                                   int32_t num_q_heads, size_t* bytes) {
  const char* what = "pa_decode_workspace_size";
  if (!bytes) return fail(PA_ERR_INVALID_ARG, "%s: bytes is NULL", what);
  *bytes = 0;
  pa::DecodeArgs a;
  const void* dummy = (const void*)16;
  if (pa_status st = fill_decode_args(what, layout, dummy, dummy, dummy, (const int32_t*)dummy, 1,
                                      (const int32_t*)dummy, num_seqs, num_q_heads, 1.f, &a))
    return st;
  StreamLayout sl;
  if (pa_status st = stream_layout(a, &sl))
    return fail(st, "%s: cannot query the device occupancy", what);
  *bytes = sl.total();
  return PA_OK;
}

}  // extern "C"

// pa_decode / pa_decode_fp8 / pa_decode_noalloc after their own argument
// checks; max_slices > 0 caps the balanced path's slices (its workspace).
static pa_status decode_launch(const char* what, pa::DecodeArgs& a, void* out, void* workspace,
                               size_t workspace_bytes, void* stream, int32_t max_slices = 0) {
  if (a.num_seqs == 0) return PA_OK;
  if (!out) return fail(PA_ERR_INVALID_ARG, "%s: out is NULL", what);
  a.out = out;
  if (workspace != nullptr) {
    StreamLayout sl;
    if (pa_status st = stream_layout(a, &sl))
      return fail(st, "%s: cannot query the device occupancy", what);
    if (max_slices > 0 && sl.slices > max_slices) sl = stream_layout_for(a, max_slices);
    if (sl.slices > 0) {
      if (workspace_bytes < sl.total())
        return fail(PA_ERR_INVALID_ARG, "%s: workspace of %zu bytes < %zu needed", what,
                    workspace_bytes, sl.total());
      if (((uintptr_t)workspace & 255) != 0)
        return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", what);
      char* ws = (char*)workspace;
      pa::StreamArgs s;
      s.part_o = (float*)ws;
      s.part_lse = (float*)(ws + sl.o_bytes);
      s.seq_slices = (int32_t*)(ws + sl.o_bytes + sl.lse_bytes);
      s.num_slices = sl.slices;
      return pa::launch_status(pa::launch_decode_stream(a, s, stream), what);
    }
  }
  return pa::launch_status(pa::launch_decode(a, stream), what);
}

extern "C" {

pa_status pa_decode(const pa_kv_layout* layout, void* out, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "pa_decode";
  pa::DecodeArgs a;
  if (pa_status st = fill_decode_args(what, layout, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                                      &a))
    return st;
  if (layout->dtype == PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 pools need their scales: use pa_decode_fp8", what);
  return decode_launch(what, a, out, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(const pa_kv_layout* layout, void* out, const void* q,
                            const void* k_pool, const void* v_pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, float scale, void* stream) {
  const char* what = "pa_decode_noalloc";
  pa::DecodeArgs a;
  if (pa_status st = fill_decode_args(what, layout, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                                      &a))
    return st;
  if (layout->dtype == PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 pools are decoded by pa_decode_fp8", what);
  if (num_seqs == 0) return PA_OK;
  StreamLayout sl;
  if (pa_status st = stream_layout(a, &sl))
    return fail(st, "%s: cannot query the device occupancy", what);
  if (sl.slices == 0)  // the balanced path does not apply: the grid kernel needs no scratch
    return decode_launch(what, a, out, nullptr, 0, stream);
  // as many slices as the device holds at once, or as fit in the scratch
  int32_t slices = sl.slices;
  while (slices > 0 && stream_layout_for(a, slices).total() > pa::kScratchBytes)
    slices = stream_layout_for(a, slices).total() / 2 > pa::kScratchBytes ? slices / 2
                                                                            : slices - 1;
  if (slices < 1)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: one slice of these sizes needs %zu bytes of scratch, more than the "
                "library's %zu; use pa_decode with a workspace",
                what, stream_layout_for(a, 1).total(), pa::kScratchBytes);
  void* scratch = nullptr;
  if (pa::scratch_buffer(&scratch) != PA_OK)
    return fail(PA_ERR_HIP, "%s: cannot find the scratch array on this device", what);
  return decode_launch(what, a, out, scratch, pa::kScratchBytes, stream, slices);
}

pa_status pa_decode_fp8(const pa_kv_layout* layout, void* out, const void* q,
                        const void* k_pool, const void* v_pool, const float* k_scale,
                        const float* v_scale, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_q_heads, float scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const char* what = "pa_decode_fp8";
  pa::DecodeArgs a;
  if (pa_status st = fill_decode_args(what, layout, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                                      &a))
    return st;
  if (layout->dtype != PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: layout dtype must be PA_FP8", what);
  if (num_seqs > 0 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARG, "%s: NULL scale pool", what);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return decode_launch(what, a, out, workspace, workspace_bytes, stream);
}

pa_status pa_kv_write_fp8(const pa_kv_layout* layout, void* k_pool, void* v_pool,
                          float* k_scale, float* v_scale, const void* k_new, const void* v_new,
                          const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
  const char* what = "pa_kv_write_fp8";
  if (pa_status st = pa::check_layout(layout, what)) return st;
  if (layout->dtype != PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: layout dtype must be PA_FP8", what);
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_tokens < 0", what);
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_scale || !v_scale || !k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", what);
  return pa::launch_status(pa::launch_kv_write_fp8(*layout, k_pool, v_pool, k_scale, v_scale,
                                                   k_new, v_new, slot_mapping, num_tokens,
                                                   stream),
                           what);
}

pa_status pa_swap_blocks(const pa_kv_layout* dst_layout, void* dst_k, void* dst_v,
                         const void* src_k, const void* src_v, int32_t src_num_blocks,
                         const int32_t* pairs, int32_t num_pairs, void* stream) {
  const char* what = "pa_swap_blocks";
  // any block shape (the scale pools of fp8 caches have head_dim 1)
  if (!dst_layout) return fail(PA_ERR_INVALID_ARG, "%s: layout is NULL", what);
  if (dst_layout->num_blocks <= 0 || dst_layout->block_size <= 0 ||
      dst_layout->num_kv_heads <= 0 || dst_layout->head_dim <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: layout sizes must be positive", what);
  if (dst_layout->dtype != PA_F32 && dst_layout->dtype != PA_BF16 && dst_layout->dtype != PA_FP8)
    return fail(PA_ERR_UNSUPPORTED, "%s: unknown dtype %d", what, dst_layout->dtype);
  if ((int64_t)dst_layout->block_size * dst_layout->num_kv_heads * dst_layout->head_dim *
          pa::elt_bytes(dst_layout->dtype) % 4 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: a block must be a multiple of 4 bytes", what);
  if (src_num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "%s: src_num_blocks must be > 0", what);
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_pairs < 0", what);
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", what);
  const int64_t block_bytes = (int64_t)dst_layout->block_size * dst_layout->num_kv_heads *
                              dst_layout->head_dim * pa::elt_bytes(dst_layout->dtype);
  if ((int64_t)num_pairs * ((block_bytes + 16383) / 16384) > (int64_t)INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: too many pairs for one launch", what);
  return pa::launch_status(pa::launch_swap_blocks(*dst_layout, dst_k, dst_v, src_k, src_v,
                                                  src_num_blocks, pairs, num_pairs, stream),
                           what);
}

pa_status pa_copy_blocks_fp8(const pa_kv_layout* layout, void* k_pool, void* v_pool,
                             float* k_scale, float* v_scale, const int32_t* pairs,
                             int32_t num_pairs, void* stream) {
  const char* what = "pa_copy_blocks_fp8";
  if (pa_status st = pa::check_layout(layout, what)) return st;
  if (layout->dtype != PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: layout dtype must be PA_FP8", what);
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_pairs < 0", what);
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_scale || !v_scale || !pairs)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", what);
  const int64_t block_bytes =
      (int64_t)layout->block_size * layout->num_kv_heads * layout->head_dim;
  if ((int64_t)num_pairs * ((block_bytes + 16383) / 16384) > (int64_t)INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: too many pairs for one launch", what);
  // the codes, then the scales as a pool of float32 rows of num_kv_heads
  if (pa_status st = pa::launch_status(
          pa::launch_copy_blocks(*layout, k_pool, v_pool, pairs, num_pairs, stream), what))
    return st;
  pa_kv_layout sc = *layout;
  sc.head_dim = 1;
  sc.dtype = PA_F32;
  return pa::launch_status(
      pa::launch_copy_blocks(sc, k_scale, v_scale, pairs, num_pairs, stream), what);
}

}  // extern "C"

namespace {

// Workspace of the split path: partial outputs, partial lse values and the
// work-queue counters, each 256-byte aligned.  false if a size is out of range.
bool split_layout(int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim,
                  int32_t max_partitions, pa_split_layout* l) {
  if (num_q_tokens < 0 || num_q_heads <= 0 || head_dim <= 0 || max_partitions <= 0) return false;
  const uint64_t rows = (uint64_t)num_q_tokens * (uint64_t)num_q_heads * (uint64_t)max_partitions;
  if (rows > ((uint64_t)1 << 40) / (uint64_t)head_dim) return false;
  const size_t o_bytes = align256((size_t)(rows * (uint64_t)head_dim * sizeof(float)));
  const size_t lse_bytes = align256((size_t)(rows * sizeof(float)));
  l->part_o_offset = 0;
  l->part_lse_offset = o_bytes;
  l->control_offset = o_bytes + lse_bytes;
  l->total_bytes = o_bytes + lse_bytes + 256;
  return true;
}

// The partial buffers of a split workspace, after checking its size and alignment.
pa_status split_buffers(const char* what, const void* workspace, size_t workspace_bytes,
                        int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim,
                        int32_t max_partitions, float** part_o, float** part_lse,
                        int32_t** control) {
  pa_split_layout l;
  if (!split_layout(num_q_tokens, num_q_heads, head_dim, max_partitions, &l))
    return fail(PA_ERR_INVALID_ARG, "%s: workspace sizes out of range", what);
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "%s: workspace is NULL", what);
  if (((uintptr_t)workspace & 255) != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", what);
  if (workspace_bytes < l.total_bytes)
    return fail(PA_ERR_INVALID_ARG, "%s: workspace of %zu bytes < %zu needed", what,
                workspace_bytes, l.total_bytes);
  char* ws = (char*)workspace;
  *part_o = (float*)(ws + l.part_o_offset);
  *part_lse = (float*)(ws + l.part_lse_offset);
  if (control) *control = (int32_t*)(ws + l.control_offset);
  return PA_OK;
}

}  // namespace

// pa_decode_split / pa_decode_split_fp8 after their own argument checks.
static pa_status split_launch(const char* what, const pa_kv_layout* layout, pa::DecodeArgs& a,
                              void* workspace, size_t workspace_bytes, int32_t max_partitions,
                              int32_t partition_size, const int32_t* cu_q_lens,
                              int32_t num_q_tokens, int32_t max_blocks_per_seq, void* stream) {
  if (num_q_tokens < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_q_tokens < 0", what);
  if (!cu_q_lens && num_q_tokens != a.num_seqs)
    return fail(PA_ERR_INVALID_ARG,
                "%s: without cu_q_lens num_q_tokens (%d) must equal num_seqs (%d)", what,
                num_q_tokens, a.num_seqs);
  if (cu_q_lens && a.num_seqs == 0 && num_q_tokens != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: query tokens without sequences", what);
  if (a.num_seqs > pa::kSplitMaxSeqs)
    return fail(PA_ERR_UNSUPPORTED, "%s: more than %d sequences in one call", what,
                pa::kSplitMaxSeqs);
  if (partition_size <= 0 || partition_size % 16 != 0 || partition_size % layout->block_size != 0)
    return fail(PA_ERR_INVALID_ARG,
                "%s: partition_size %d must be a positive multiple of 16 and of block_size %d",
                what, partition_size, layout->block_size);
  if (max_partitions <= 0 || max_partitions > 65535)
    return fail(PA_ERR_INVALID_ARG, "%s: max_partitions must be in [1, 65535]", what);
  if ((int64_t)max_partitions * partition_size < (int64_t)max_blocks_per_seq * layout->block_size)
    return fail(PA_ERR_INVALID_ARG,
                "%s: max_partitions*partition_size (%lld) < max_blocks_per_seq*block_size (%lld)",
                what, (long long)max_partitions * partition_size,
                (long long)max_blocks_per_seq * layout->block_size);
  if (cu_q_lens && max_partitions < 2)
    return fail(PA_ERR_INVALID_ARG,
                "%s: with cu_q_lens (prefill chunks have two partitions) max_partitions must be >= 2",
                what);
  if ((int64_t)num_q_tokens * max_partitions * layout->num_kv_heads > (int64_t)INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: too many (query, partition, KV head) units", what);
  if (num_q_tokens == 0) return PA_OK;
  float *part_o = nullptr, *part_lse = nullptr;
  int32_t* control = nullptr;
  if (pa_status st = split_buffers(what, workspace, workspace_bytes, num_q_tokens, a.num_q_heads,
                                   a.head_dim, max_partitions, &part_o, &part_lse, &control))
    return st;
  a.cu_q_lens = cu_q_lens;
  a.num_q_tokens = num_q_tokens;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.queue = control;
  a.partition_size = partition_size;
  a.max_partitions = max_partitions;
  return pa::launch_status(pa::launch_split(a, stream), what);
}

extern "C" {

pa_status pa_split_workspace_layout(int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_partitions, pa_split_layout* layout) {
  const char* what = "pa_split_workspace_layout";
  if (!layout) return fail(PA_ERR_INVALID_ARG, "%s: layout is NULL", what);
  if (!split_layout(num_q_tokens, num_q_heads, head_dim, max_partitions, layout))
    return fail(PA_ERR_INVALID_ARG, "%s: sizes out of range", what);
  return PA_OK;
}

size_t pa_split_workspace_bytes(int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_partitions) {
  pa_split_layout l;
  if (!split_layout(num_q_tokens, num_q_heads, head_dim, max_partitions, &l)) return 0;
  return l.total_bytes;
}

pa_status pa_decode_split(const pa_kv_layout* layout, void* workspace, size_t workspace_bytes,
                          int32_t max_partitions, int32_t partition_size, const void* q,
                          const int32_t* cu_q_lens, int32_t num_q_tokens, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, float scale, void* stream) {
  const char* what = "pa_decode_split";
  pa::DecodeArgs a;
  if (pa_status st = fill_decode_args(what, layout, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                                      &a))
    return st;
  if (layout->dtype == PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 pools need their scales: use pa_decode_split_fp8",
                what);
  return split_launch(what, layout, a, workspace, workspace_bytes, max_partitions,
                      partition_size, cu_q_lens, num_q_tokens, max_blocks_per_seq, stream);
}

pa_status pa_decode_split_fp8(const pa_kv_layout* layout, void* workspace,
                              size_t workspace_bytes, int32_t max_partitions,
                              int32_t partition_size, const void* q, const int32_t* cu_q_lens,
                              int32_t num_q_tokens, const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                              float scale, void* stream) {
  const char* what = "pa_decode_split_fp8";
  pa::DecodeArgs a;
  if (pa_status st = fill_decode_args(what, layout, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                                      &a))
    return st;
  if (layout->dtype != PA_FP8)
    return fail(PA_ERR_INVALID_ARG, "%s: layout dtype must be PA_FP8", what);
  if (num_seqs > 0 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARG, "%s: NULL scale pool", what);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return split_launch(what, layout, a, workspace, workspace_bytes, max_partitions,
                      partition_size, cu_q_lens, num_q_tokens, max_blocks_per_seq, stream);
}

pa_status pa_reduce(void* out, int32_t out_dtype, float* lse_out, const void* workspace,
                    size_t workspace_bytes, int32_t max_partitions, int32_t partition_size,
                    const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_tokens, int32_t num_q_heads, int32_t head_dim, void* stream) {
  const char* what = "pa_reduce";
  if (out_dtype != PA_F32 && out_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: out_dtype %d is not PA_F32 or PA_BF16", what, out_dtype);
  if (num_seqs < 0 || num_q_tokens < 0 || num_q_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: bad sizes", what);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {32, 64, 128, 256}", what, head_dim);
  if (partition_size <= 0 || max_partitions <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: partition_size and max_partitions must be > 0", what);
  if (!cu_q_lens && num_q_tokens != num_seqs)
    return fail(PA_ERR_INVALID_ARG, "%s: without cu_q_lens num_q_tokens must equal num_seqs", what);
  if (num_q_tokens == 0) return PA_OK;
  if (num_seqs == 0) return fail(PA_ERR_INVALID_ARG, "%s: query tokens without sequences", what);
  if (!out || !seq_lens) return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", what);
  float *part_o = nullptr, *part_lse = nullptr;
  if (pa_status st = split_buffers(what, workspace, workspace_bytes, num_q_tokens, num_q_heads,
                                   head_dim, max_partitions, &part_o, &part_lse, nullptr))
    return st;
  pa::ReduceArgs a;
  a.out = out;
  a.lse_out = lse_out;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.cu_q_lens = cu_q_lens;
  a.seq_lens = seq_lens;
  a.out_dtype = out_dtype;
  a.max_partitions = max_partitions;
  a.partition_size = partition_size;
  a.num_seqs = num_seqs;
  a.num_q_tokens = num_q_tokens;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  return pa::launch_status(pa::launch_reduce(a, stream), what);
}

}  // extern "C"
