// Slot-mapped cache writes, whole-block copies (copy-on-write) and the
// log-sum-exp merge of split-sequence partitions, for gfx950.
//
// * kv_write ("19.2 KV Cache 系统化管理" §19.2.3, write_slot): token t's keys
//   and values for all KV heads, one contiguous row of num_kv_heads*head_dim
//   elements, go to pool row slot_mapping[t] (the flat slot
//   physical*block_size + offset is exactly the pool row index).  One
//   workgroup per token, 16-byte lanes.
// * copy_blocks (same page, §19.2.2): pool[dst] = pool[src], K and V; a block
//   is one contiguous span of block_size rows.  Workgroups stride over
//   (pair, 16 KiB chunk) so a handful of pairs still fills the chip.
// * kv_write_fp8 (same page, §19.2.4): the quantizing write into e4m3 pools
//   with one scale per (token, KV head).
// * reduce: the partitions of one query head are merged with weights
//   exp(lse_p - L), L = log sum_p exp(lse_p) -- the online-softmax rescale of
//   §19.2.3 applied once per partition.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void kv_write_kernel(char* __restrict__ kp, char* __restrict__ vp,
                                                       const char* __restrict__ kn,
                                                       const char* __restrict__ vn,
                                                       const int32_t* __restrict__ slots,
                                                       int64_t row_bytes, int64_t num_rows) {
  const int t = blockIdx.x;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_rows) return;
  const int64_t n16 = row_bytes >> 4;
  const uint4* sk = (const uint4*)(kn + (int64_t)t * row_bytes);
  const uint4* sv = (const uint4*)(vn + (int64_t)t * row_bytes);
  uint4* dk = (uint4*)(kp + s * row_bytes);
  uint4* dv = (uint4*)(vp + s * row_bytes);
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) {
    const uint4 a = sk[i];
    const uint4 b = sv[i];
    dk[i] = a;
    dv[i] = b;
  }
}

// Quantizing write into e4m3 pools ("19.2 KV Cache 系统化管理" §19.2.4: every
// token's vector is scaled on its own).  One wave per (token, KV head, K|V):
// the row's absmax across the wave, scale = absmax / 448, codes of x / scale
// (IEEE float32 division, clamped to +-448) by the hardware's nearest-even
// conversion; lane i handles the value pairs 2i + 128k.  A zero row gets
// scale 0 and zero codes.
__global__ __launch_bounds__(64) void kv_write_fp8_kernel(
    uint8_t* __restrict__ kp, uint8_t* __restrict__ vp, float* __restrict__ ks,
    float* __restrict__ vs, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const int32_t* __restrict__ slots, int32_t num_kv_heads, int32_t head_dim, int32_t log2_bs,
    int64_t num_rows) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_rows) return;
  const int lane = threadIdx.x;
  const uint16_t* x = (is_v ? vn : kn) + ((int64_t)t * num_kv_heads + h) * head_dim;
  uint8_t* dst = (is_v ? vp : kp) + (s * num_kv_heads + h) * head_dim;
  float amax = 0.f;
  for (int d = 2 * lane; d < head_dim; d += 2 * kWave) {
    const uint32_t pair = *(const uint32_t*)(x + d);
    amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(pair)), fabsf(bf16_hi(pair))));
  }
  amax = reduce_levels<0, 6>(amax, OpMax());
  const float scale = __fdiv_rn(amax, 448.f);
  for (int d = 2 * lane; d < head_dim; d += 2 * kWave) {
    const uint32_t pair = *(const uint32_t*)(x + d);
    uint32_t codes = 0;
    if (scale > 0.f) {
      const float a = fminf(fmaxf(__fdiv_rn(bf16_lo(pair), scale), -448.f), 448.f);
      const float b = fminf(fmaxf(__fdiv_rn(bf16_hi(pair), scale), -448.f), 448.f);
      codes = f32x2_to_fp8(a, b);
    }
    *(uint16_t*)(dst + d) = (uint16_t)codes;
  }
  if (lane == 0)
    (is_v ? vs : ks)[fp8_scale_index(s >> log2_bs, (int)(s & ((1 << log2_bs) - 1)), h,
                                     num_kv_heads, log2_bs)] = scale;
}

constexpr int64_t kCopyChunk = 16384;  // bytes per workgroup

// Bytes [lo, hi) of one K block and one V block.  Blocks whose size is a
// multiple of 16 bytes (every K/V pool) go in 16-byte lanes; others (the fp8
// scale pools hold block_size * kv_heads float32 values, so a block may be 8
// bytes, and its start only 4-byte aligned) go in 4-byte words.
__device__ __forceinline__ void copy_span(char* __restrict__ dk, char* __restrict__ dv,
                                          const char* __restrict__ sk,
                                          const char* __restrict__ sv, int64_t lo, int64_t hi,
                                          bool words16) {
  if (words16) {
    const int64_t n16 = (hi - lo) >> 4;
    const uint4* a = (const uint4*)(sk + lo);
    const uint4* b = (const uint4*)(sv + lo);
    uint4* c = (uint4*)(dk + lo);
    uint4* d = (uint4*)(dv + lo);
    for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) {
      const uint4 x = a[i];
      const uint4 y = b[i];
      c[i] = x;
      d[i] = y;
    }
    return;
  }
  const int64_t n4 = (hi - lo) >> 2;
  const uint32_t* a = (const uint32_t*)(sk + lo);
  const uint32_t* b = (const uint32_t*)(sv + lo);
  uint32_t* c = (uint32_t*)(dk + lo);
  uint32_t* d = (uint32_t*)(dv + lo);
  for (int64_t i = threadIdx.x; i < n4; i += blockDim.x) {
    const uint32_t x = a[i];
    const uint32_t y = b[i];
    c[i] = x;
    d[i] = y;
  }
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ kp, char* __restrict__ vp,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t block_bytes, int32_t num_blocks,
                                                          int64_t chunks_per_block) {
  const int64_t pair = blockIdx.x / chunks_per_block;
  const int64_t chunk = blockIdx.x % chunks_per_block;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  copy_span(kp + dst * block_bytes, vp + dst * block_bytes, kp + src * block_bytes,
            vp + src * block_bytes, chunk * kCopyChunk, min((chunk + 1) * kCopyChunk, block_bytes),
            (block_bytes & 15) == 0);
}

// One wave per (query token, query head); kReduceWaves heads per workgroup.
// Lane l owns dims [VEC l, VEC l + VEC) of the row (VEC = max(D / 64, 1)) and
// the weight exp(lse_p - m) of partition p = l (per 64 partitions).  The
// row's first two partitions and its first 64 lse values are requested at
// once, before the query's partition count is known (they lie inside the
// row's slots whatever that count is, and are used only below it): a query
// of a prefill chunk has at most two partitions, so it needs no other load.
// Further partitions are loaded 8 or 16 rows at a time, all in flight
// together, and summed in partition order with the weights read from their
// lanes.
constexpr int kReduceWaves = 4;

template <int VEC>
__device__ __forceinline__ void reduce_query(const ReduceArgs& a, int j, int h, int lane) {
  constexpr int kReduceBatch = VEC >= 4 ? 8 : 16;  // rows in flight per lane
  const int D = a.head_dim;
  const int64_t row = (int64_t)j * a.num_q_heads + h;
  const float* lse = a.part_lse + row * a.max_partitions;
  const float* po = a.part_o + row * a.max_partitions * D;
  const int d0 = lane * VEC;
  const bool active = d0 < D;  // (head_dim 32: the upper half of the wave idles)
  auto load = [&](int p, float (&v)[VEC]) {
    const float* src = po + (int64_t)p * D + d0;
    if constexpr (VEC == 4) {
      const float4 x = active ? *(const float4*)src : make_float4(0.f, 0.f, 0.f, 0.f);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else if constexpr (VEC == 2) {
      const float2 x = active ? *(const float2*)src : make_float2(0.f, 0.f);
      v[0] = x.x; v[1] = x.y;
    } else {
      v[0] = active ? *src : 0.f;
    }
  };
  // rows p0 .. p0 + kReduceBatch - 1 of the n partitions (those past n are not read)
  auto load_batch = [&](int p0, int n, float (&v)[kReduceBatch][VEC]) {
#pragma unroll
    for (int i = 0; i < kReduceBatch; ++i) {
      if (p0 + i < n) {
        load(p0 + i, v[i]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[i][e] = 0.f;
      }
    }
  };
  // ---- requested before the partition count: partitions 0 and 1, lse[lane]
  float pre[2][VEC];
  load(0, pre[0]);
  if (a.max_partitions > 1) {
    load(1, pre[1]);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) pre[1][e] = 0.f;
  }
  const float lse_lane = lane < a.max_partitions ? lse[lane] : -INFINITY;

  // ---- the query's sequence and partition count ------------------------------
  int q_first = j, q_len = 1, len = 0;
  if (a.cu_q_lens != nullptr) {
    // the last b with cu_q_lens[b] <= j: each round reads 64 entries at once
    // (one per lane) and keeps the span between the last two that qualify;
    // the last round (one entry per lane) also reads each candidate's next
    // entry and length, so the sequence is known when the round ends
    int lo = 0, n = a.num_seqs;  // b in [lo, lo + n)
    for (;;) {
      const int step = (n + kWave - 1) / kWave;
      const int i = lo + lane * step;
      const bool in = lane * step < n;
      const int ci = in ? a.cu_q_lens[i] : 0;
      int cn = 0, sl = 0;
      if (step == 1 && in) {
        cn = a.cu_q_lens[i + 1];
        sl = a.seq_lens[i];
      }
      const int k = 63 - __builtin_clzll(__ballot(in && ci <= j) | 1ull);  // last that qualifies
      if (step == 1) {
        q_first = __builtin_amdgcn_readlane(ci, k);
        q_len = __builtin_amdgcn_readlane(cn, k) - q_first;
        len = max(__builtin_amdgcn_readlane(sl, k), 0);
        break;
      }
      lo += k * step;
      n = min(step, n - k * step);
    }
  } else {
    len = max(a.seq_lens[j], 0);
  }
  const int key_end = len - q_len + (j - q_first) + 1;
  // a decode query has ceil(key_end / P) partitions; each query of a prefill
  // chunk (q_len > 1) has two split at half the cached context (in 32-key
  // tiles), or one when that half is empty
  int nparts = 0;
  if (key_end > 0) {
    if (q_len > 1) nparts = 32 * (((len - q_len + 31) / 32) / 2) > 0 ? 2 : 1;
    else nparts = (key_end + a.partition_size - 1) / a.partition_size;
  }
  nparts = min(nparts, a.max_partitions);

  // ---- weights exp(lse_p - m), their sum, the weighted rows ------------------
  float m = lane < nparts ? lse_lane : -INFINITY;
  for (int p = lane + kWave; p < nparts; p += kWave) m = fmaxf(m, lse[p]);
  m = reduce_levels<0, 6>(m, OpMax());
  float wsum = lane < nparts ? __expf(lse_lane - m) : 0.f;
  for (int p = lane + kWave; p < nparts; p += kWave) wsum += __expf(lse[p] - m);
  wsum = reduce_levels<0, 6>(wsum, OpSum());
  const float inv = nparts > 0 ? 1.f / wsum : 0.f;

  float o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.f;
  for (int pc = 0; pc < nparts; pc += kWave) {
    const int n = min(kWave, nparts - pc);
    const float wl = lane < n ? __expf((pc == 0 ? lse_lane : lse[pc + lane]) - m) : 0.f;
    auto weight = [&](int p) {  // p is wave-uniform
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), p));
    };
    int p = 0;
    if (pc == 0) {  // partitions 0 and 1: already loaded
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (i < n) {
          const float w = weight(i);
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = fmaf(w, pre[i][e], o[e]);
        }
      }
      p = 2;
    }
    for (; p < n; p += kReduceBatch) {
      float v[kReduceBatch][VEC];
      load_batch(pc + p, pc + n, v);
#pragma unroll
      for (int i = 0; i < kReduceBatch; ++i) {
        if (p + i < n) {
          const float w = weight(p + i);
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = fmaf(w, v[i][e], o[e]);
        }
      }
    }
  }
  if (active) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float x = o[e] * inv;
      if (a.out_dtype == PA_BF16)
        ((__bf16*)a.out)[row * D + d0 + e] = (__bf16)x;
      else
        ((float*)a.out)[row * D + d0 + e] = x;
    }
  }
  if (a.lse_out != nullptr && lane == 0)
    a.lse_out[row] = nparts > 0 ? m + __logf(wsum) : -INFINITY;
}

__global__ __launch_bounds__(kReduceWaves * kWave) void reduce_kernel(ReduceArgs a) {
  const int j = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int h = blockIdx.y * kReduceWaves + threadIdx.x / kWave;
  if (h >= a.num_q_heads) return;
  switch (a.head_dim) {
    case 256: reduce_query<4>(a, j, h, lane); break;
    case 128: reduce_query<2>(a, j, h, lane); break;
    default: reduce_query<1>(a, j, h, lane); break;  // 32, 64
  }
}

// Block copies between two pools (swap out to / in from pinned host memory,
// which the GPU reads and writes through the same pointers; preemption in
// "LLM 推理引擎的内存管理与调度" §9 and "19.2 KV Cache 系统化管理" §19.2.6):
// dst_pool[pair.dst] = src_pool[pair.src], K and V, 16 KiB chunks per
// workgroup; pairs with an id out of range are skipped.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    char* __restrict__ dk, char* __restrict__ dv, const char* __restrict__ sk,
    const char* __restrict__ sv, const int32_t* __restrict__ pairs, int64_t block_bytes,
    int32_t dst_blocks, int32_t src_blocks, int64_t chunks_per_block) {
  const int64_t pair = blockIdx.x / chunks_per_block;
  const int64_t chunk = blockIdx.x % chunks_per_block;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  copy_span(dk + dst * block_bytes, dv + dst * block_bytes, sk + src * block_bytes,
            sv + src * block_bytes, chunk * kCopyChunk, min((chunk + 1) * kCopyChunk, block_bytes),
            (block_bytes & 15) == 0);
}

inline int64_t elt_size(int32_t dtype) {
  return dtype == PA_BF16 ? 2 : (dtype == PA_FP8 ? 1 : 4);
}

}  // namespace

pa_status launch_kv_write(const pa_kv_layout& l, void* k_pool, void* v_pool, const void* k_new,
                          const void* v_new, const int32_t* slots, int32_t num_tokens,
                          void* stream) {
  if (num_tokens == 0) return PA_OK;
  const int64_t row_bytes = (int64_t)l.num_kv_heads * l.head_dim * elt_size(l.dtype);
  const int64_t num_rows = (int64_t)l.num_blocks * l.block_size;
  const int threads = row_bytes >= 4096 ? 256 : (row_bytes >= 2048 ? 128 : 64);
  hipLaunchKernelGGL(kv_write_kernel, dim3(num_tokens), dim3(threads), 0, (hipStream_t)stream,
                     (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new, slots,
                     row_bytes, num_rows);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_kv_write_fp8(const pa_kv_layout& l, void* k_pool, void* v_pool, float* k_scale,
                              float* v_scale, const void* k_new, const void* v_new,
                              const int32_t* slots, int32_t num_tokens, void* stream) {
  if (num_tokens == 0) return PA_OK;
  const int64_t num_rows = (int64_t)l.num_blocks * l.block_size;
  int log2_bs = 0;  // block_size is a power of two (checked by the caller)
  while ((1 << log2_bs) < l.block_size) ++log2_bs;
  hipLaunchKernelGGL(kv_write_fp8_kernel, dim3(num_tokens, l.num_kv_heads, 2), dim3(kWave), 0,
                     (hipStream_t)stream, (uint8_t*)k_pool, (uint8_t*)v_pool, k_scale, v_scale,
                     (const uint16_t*)k_new, (const uint16_t*)v_new, slots, l.num_kv_heads,
                     l.head_dim, log2_bs, num_rows);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_swap_blocks(const pa_kv_layout& l, void* dst_k, void* dst_v, const void* src_k,
                             const void* src_v, int32_t src_num_blocks, const int32_t* pairs,
                             int32_t num_pairs, void* stream) {
  if (num_pairs == 0) return PA_OK;
  const int64_t block_bytes =
      (int64_t)l.block_size * l.num_kv_heads * l.head_dim * elt_size(l.dtype);
  const int64_t chunks = (block_bytes + kCopyChunk - 1) / kCopyChunk;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((uint32_t)(num_pairs * chunks)), dim3(256), 0,
                     (hipStream_t)stream, (char*)dst_k, (char*)dst_v, (const char*)src_k,
                     (const char*)src_v, pairs, block_bytes, l.num_blocks, src_num_blocks, chunks);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_copy_blocks(const pa_kv_layout& l, void* k_pool, void* v_pool,
                             const int32_t* pairs, int32_t num_pairs, void* stream) {
  if (num_pairs == 0) return PA_OK;
  const int64_t block_bytes =
      (int64_t)l.block_size * l.num_kv_heads * l.head_dim * elt_size(l.dtype);
  const int64_t chunks = (block_bytes + kCopyChunk - 1) / kCopyChunk;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)(num_pairs * chunks)), dim3(256), 0,
                     (hipStream_t)stream, (char*)k_pool, (char*)v_pool, pairs, block_bytes,
                     l.num_blocks, chunks);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_reduce(const ReduceArgs& a, void* stream) {
  if (a.num_q_tokens == 0) return PA_OK;
  const dim3 grid(a.num_q_tokens, (a.num_q_heads + kReduceWaves - 1) / kReduceWaves);
  hipLaunchKernelGGL(reduce_kernel, grid, dim3(kReduceWaves * kWave), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
