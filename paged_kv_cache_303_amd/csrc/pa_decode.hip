// Paged decode attention on gfx950: block-table gather, QK, online softmax,
// PV -- single pass (final output) or one partition per workgroup (partials
// for the log-sum-exp reduce).
//
// What it computes ("19.2 KV Cache 系统化管理" §19.2.3, paged_attention): for
// one query token, walk the request's keys in logical order through its block
// table (logical block t / block_size -> physical block, row t % block_size;
// "LLM 推理引擎的内存管理与调度" §3), and fold them into a running maximum m,
// a running sum l of exp(s - m) and a running weighted sum of values, both
// rescaled by exp(m_old - m_new) whenever the maximum grows; divide at the end.
// The unit folded at once is a tile of 16 tokens instead of one block.
//
// Work decomposition (one workgroup = one query token x a group of KV heads x
// one partition; one wave per KV head):
//   * The wave serves the G = num_q_heads/num_kv_heads query heads that share
//     its KV head, so every K/V byte is read once per KV head (grouped-query
//     attention) and used G times.
//   * Loads are 16 bytes per lane and row-contiguous: a token row of one KV
//     head (head_dim elements) is read by LPR = head_dim*elt/16 neighbouring
//     lanes, TPI = 64/LPR rows per load instruction, NI instructions per tile.
//   * QK: each lane takes partial dot products over its 16-byte chunk for the
//     G heads (v_dot2_f32_bf16 for bfloat16) and the LPR lanes of a row are
//     summed with DPP row operations -- no LDS.  After that every lane holds
//     the full scores of its own tokens, exactly the tokens whose V chunk it
//     loaded, so PV needs no exchange either.
//   * Softmax runs in the log2 domain (scores carry scale*log2(e)); the tile
//     maximum crosses token groups with DPP / v_permlane{16,32}_swap.
//   * Masked tokens (past the partition end) load a clamped in-range row and
//     get probability exactly 0, so the NaN-poisoned tails of partly filled
//     blocks never reach the sums.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kMaxWaves = 8;  // workgroup = up to 8 KV heads

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
};
template <>
struct Elt<uint16_t> {  // bfloat16 bit patterns
  static constexpr int kVec = 8;
};

// Lane layout for (element type, head_dim, query heads per KV head):
//   CPL  16-byte chunks of a row per lane (2 halves the row reduction and the
//        redundant exponentials; 1 when G is large, to bound accumulators)
//   LPR  lanes per token row, TPI rows per load instruction
//   NI   load instructions (of CPL chunks each) per tile, TT tokens per tile
#ifndef PA_GROUP_MAJOR
#define PA_GROUP_MAJOR 0  // 1: KV-head groups vary fastest in the grid
#endif
#ifndef PA_TILE_TOKENS
#define PA_TILE_TOKENS 32  // target tokens per tile (per wave, per KV head)
#endif
#ifndef PA_MAX_TILE_LOADS
#define PA_MAX_TILE_LOADS 8  // 16-byte loads per lane per tile (K or V), hot shapes
#endif

template <typename T, int D, int G, bool UNIFORM = true>
struct Shape {
  static constexpr int VEC = Elt<T>::kVec;
  static constexpr int CHUNKS = D / VEC;
  static constexpr int CPL = (CHUNKS >= 8 && G <= 4) ? 2 : 1;
  static constexpr int LPR = CHUNKS / CPL;
  static constexpr int TPI = kWave / LPR;
  // Loads per lane per tile (K or V; two tiles are in registers at a time):
  // the bf16 shapes with small G get the full budget, the others half of it
  // so that accumulators and both tiles stay in 256 VGPRs without spilling.
  static constexpr int MAX_LOADS =
      (sizeof(T) == 2 && G <= 4 && D <= 128 && UNIFORM) ? PA_MAX_TILE_LOADS
      : (G >= 8 ? PA_MAX_TILE_LOADS / 4 : PA_MAX_TILE_LOADS / 2);
  static constexpr int NI0 = (PA_TILE_TOKENS / TPI) < 1 ? 1 : (PA_TILE_TOKENS / TPI);
  static constexpr int NI = (NI0 * CPL > MAX_LOADS) ? (MAX_LOADS / CPL < 1 ? 1 : MAX_LOADS / CPL) : NI0;
  static constexpr int TT = NI * TPI;
  // Tiles start at multiples of 16 plus multiples of TT, so every load
  // instruction starts on a multiple of TPI (needed by the UNIFORM lookup).
  static_assert(LPR * CPL * VEC == D && LPR <= kWave && (16 % TPI) == 0 && NI >= 1,
                "unsupported lane layout");
};

// Lazy rescaling: the running maximum m (log2 domain) is only moved when a
// tile's maximum exceeds it by more than this, so probabilities stay below
// 2^kLazy and the O(G*D) rescale of the accumulators is rare.  The result
// is independent of m up to rounding (acc and l carry the same factor).
constexpr float kLazy = 8.0f;

// UNIFORM: the rows of one load instruction always share a block (the block
// size is a multiple of TPI), so block-table entries are wave-uniform scalar
// loads; otherwise every lane looks its block up.
template <typename T, int D, int G, bool SPLIT, bool UNIFORM>
__global__ __launch_bounds__(kMaxWaves * kWave) void decode_kernel(DecodeArgs a) {
  using S = Shape<T, D, G, UNIFORM>;
  constexpr int VEC = S::VEC;
  constexpr int CPL = S::CPL;
  constexpr int LPR = S::LPR;
  constexpr int LOG_LPR = ilog2(LPR);
  constexpr int TPI = S::TPI;
  constexpr int NI = S::NI;
  constexpr int TT = S::TT;
  constexpr bool BF16 = sizeof(T) == 2;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tg = lane / LPR;  // which row of a load instruction
  const int c = lane % LPR;   // first 16-byte chunk of this lane (then c + LPR, ...)
#if PA_GROUP_MAJOR
  const int j = blockIdx.y;   // query token
  const int kvh = blockIdx.x * a.waves_per_group + wave;
#else
  const int j = blockIdx.x;   // query token
  const int kvh = blockIdx.y * a.waves_per_group + wave;
#endif
  // Partitions run last-first so the long sequences' tails start early.
  const int part = (int)gridDim.z - 1 - (int)blockIdx.z;

  // --- query token -> sequence, position, key range -------------------------
  int b = j, q_first = j, q_len = 1;
  if (a.cu_q_lens != nullptr) {
    int lo = 0, hi = a.num_seqs - 1;  // last b with cu[b] <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_q_lens[mid] <= j) lo = mid; else hi = mid - 1;
    }
    b = lo;
    q_first = a.cu_q_lens[b];
    q_len = a.cu_q_lens[b + 1] - q_first;
  }
  const int cap = a.max_blocks << a.log2_bs;
  const int len = min(max(a.seq_lens[b], 0), cap);
  const int key_end = len - q_len + (j - q_first) + 1;  // keys 0 .. position
  int start = 0, end = key_end;
  if constexpr (SPLIT) {
    if (q_len > 1) {
      if (part != 0) return;  // multi-query sequences: one partition
    } else {
      start = part * a.partition_size;
      end = min(key_end, start + a.partition_size);
    }
    if (start >= end) return;  // this partition holds no key
  }
  const int h0 = kvh * G;
  if constexpr (!SPLIT) {
    if (end <= 0) {  // no key: zero row
      if (tg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int k = 0; k < CPL; ++k)
            *(uint4*)((T*)a.out + ((int64_t)j * a.num_q_heads + h0 + g) * D +
                      (c + k * LPR) * VEC) = make_uint4(0, 0, 0, 0);
      }
      return;
    }
  }

  // --- query: this lane's chunks of each of the G heads ------------------------
  // Scores are kept unscaled; scale*log2(e) is applied inside the exponent's
  // fma (bf16) or folded into the fp32 query.  Requires scale > 0.
  const T* qrow = (const T*)a.q + ((int64_t)j * a.num_q_heads + h0) * D;
  uint4 qraw[G][CPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int k = 0; k < CPL; ++k)
      qraw[g][k] = *(const uint4*)(qrow + (int64_t)g * D + (c + k * LPR) * VEC);
  float qf[G][CPL][4];
  if constexpr (!BF16) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        qf[g][k][0] = __uint_as_float(qraw[g][k].x) * a.scale_log2;
        qf[g][k][1] = __uint_as_float(qraw[g][k].y) * a.scale_log2;
        qf[g][k][2] = __uint_as_float(qraw[g][k].z) * a.scale_log2;
        qf[g][k][3] = __uint_as_float(qraw[g][k].w) * a.scale_log2;
      }
  }
  const float qk_scale = BF16 ? a.scale_log2 : 1.0f;

  // --- addressing --------------------------------------------------------------
  const uint32_t row_bytes = (uint32_t)a.num_kv_heads * D * sizeof(T);
  const int64_t block_bytes = (int64_t)row_bytes << a.log2_bs;
  const uint32_t lane_col = (uint32_t)(kvh * D + c * VEC) * sizeof(T);
  constexpr uint32_t kChunkStride = LPR * 16;  // bytes between a lane's chunks
  const char* kp = (const char*)a.k_pool;
  const char* vp = (const char*)a.v_pool;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  const int bs_mask = (1 << a.log2_bs) - 1;
  const int nb_max = a.num_blocks - 1;

  float m_run[G], l_run[G], acc[G][CPL][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[g][k][e] = 0.f;
  }

  // Physical block of each load instruction of the tile starting at t0.  In
  // UNIFORM mode these are wave-uniform scalar loads.  Rows are clamped to
  // end-1, so a tile past the end still addresses valid (written) rows.
  auto lookup = [&](int t0, int (&ph)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (UNIFORM) {
        ph[i] = bt[min(t0 + i * TPI, end - 1) >> a.log2_bs];
      } else {
        ph[i] = bt[min(t0 + i * TPI + tg, end - 1) >> a.log2_bs];
      }
    }
  };

  struct Tile {
    uint4 k[NI][CPL];
    uint4 v[NI][CPL];
  };
  // Gather the K and V rows of the tile at t0 through the block table.
  auto issue = [&](Tile& tl, int t0, const int (&ph)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = min(t0 + i * TPI + tg, end - 1);  // clamp rows past the end
      const int phys = min(max(ph[i], 0), nb_max);
      uint32_t off;
      if constexpr (UNIFORM) {
        // the TPI rows of this instruction lie in one block: the block of its
        // first (clamped) row.
        const int blk0 = min(t0 + i * TPI, end - 1) >> a.log2_bs;
        off = (uint32_t)(tok - (blk0 << a.log2_bs)) * row_bytes + lane_col;
      } else {
        off = (uint32_t)(tok & bs_mask) * row_bytes + lane_col;
      }
      const char* kb = kp + phys * block_bytes + off;
      const char* vb = vp + phys * block_bytes + off;
#pragma unroll
      for (int k = 0; k < CPL; ++k) tl.k[i][k] = *(const uint4*)(kb + k * kChunkStride);
#pragma unroll
      for (int k = 0; k < CPL; ++k) tl.v[i][k] = *(const uint4*)(vb + k * kChunkStride);
    }
  };

  auto compute = [&](const Tile& tl, int t0) {
    // ---- scores: partial dots over the lane's chunks, then sum the row -----
    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          if constexpr (BF16) {
            d = dot2_bf16(qraw[g][k].x, tl.k[i][k].x, d);
            d = dot2_bf16(qraw[g][k].y, tl.k[i][k].y, d);
            d = dot2_bf16(qraw[g][k].z, tl.k[i][k].z, d);
            d = dot2_bf16(qraw[g][k].w, tl.k[i][k].w, d);
          } else {
            d = fmaf(qf[g][k][0], __uint_as_float(tl.k[i][k].x), d);
            d = fmaf(qf[g][k][1], __uint_as_float(tl.k[i][k].y), d);
            d = fmaf(qf[g][k][2], __uint_as_float(tl.k[i][k].z), d);
            d = fmaf(qf[g][k][3], __uint_as_float(tl.k[i][k].w), d);
          }
        }
        s[i][g] = reduce_levels<0, LOG_LPR>(d, OpSum());
      }
    }
    if (t0 + TT > end) {  // tail tile: rows past the end get probability 0
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool valid = (t0 + i * TPI + tg) < end;
#pragma unroll
        for (int g = 0; g < G; ++g) s[i][g] = valid ? s[i][g] : -INFINITY;
      }
    }

    // ---- online softmax (log2 domain), lazily rescaled ------------------------
    float mt[G];
    bool move = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = s[0][g];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[i][g]);
      mt[g] = reduce_groups<LOG_LPR>(mx, OpMax()) * qk_scale;
      move |= mt[g] > m_run[g] + kLazy;
    }
    if (move) {  // same outcome on every lane of the wave
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m_new = fmaxf(m_run[g], mt[g]);
        const float alpha = fast_exp2(m_run[g] - m_new);
        m_run[g] = m_new;
        l_run[g] *= alpha;
#pragma unroll
        for (int k = 0; k < CPL; ++k)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[g][k][e] *= alpha;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = fast_exp2(fmaf(s[i][g], qk_scale, -m_run[g]));
        l_run[g] += p;
        s[i][g] = p;
      }
    }

    // ---- PV --------------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        float v[VEC];
        if constexpr (BF16) {
          v[0] = bf16_lo(tl.v[i][k].x); v[1] = bf16_hi(tl.v[i][k].x);
          v[2] = bf16_lo(tl.v[i][k].y); v[3] = bf16_hi(tl.v[i][k].y);
          v[4] = bf16_lo(tl.v[i][k].z); v[5] = bf16_hi(tl.v[i][k].z);
          v[6] = bf16_lo(tl.v[i][k].w); v[7] = bf16_hi(tl.v[i][k].w);
        } else {
          v[0] = __uint_as_float(tl.v[i][k].x); v[1] = __uint_as_float(tl.v[i][k].y);
          v[2] = __uint_as_float(tl.v[i][k].z); v[3] = __uint_as_float(tl.v[i][k].w);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[g][k][e] = fmaf(s[i][g], v[e], acc[g][k][e]);
      }
    }
  };

  // Software pipeline: the loads of tile t+1 are in flight while tile t is
  // computed (two register tiles, A and B).  They are issued unconditionally
  // -- past the end they re-read the clamped last row -- so the wait before
  // each compute is always "all but the newest tile's loads".
  int ph[NI];
  lookup(start, ph);
  Tile ta, tb;
  issue(ta, start, ph);
  lookup(start + TT, ph);
  for (int t0 = start;;) {
    issue(tb, t0 + TT, ph);
    lookup(t0 + 2 * TT, ph);
    compute(ta, t0);
    t0 += TT;
    if (t0 >= end) break;
    issue(ta, t0 + TT, ph);
    lookup(t0 + 2 * TT, ph);
    compute(tb, t0);
    t0 += TT;
    if (t0 >= end) break;
  }

  // --- combine the token groups and write ---------------------------------------
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = reduce_groups<LOG_LPR>(l_run[g], OpSum());
#pragma unroll
    for (int k = 0; k < CPL; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[g][k][e] = reduce_groups<LOG_LPR>(acc[g][k][e], OpSum());
    const float inv = 1.f / l;
    const int h = h0 + g;
    if (tg == 0) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int col = (c + k * LPR) * VEC;
        if constexpr (SPLIT) {
          float* po = a.part_o + (((int64_t)j * a.num_q_heads + h) * a.max_partitions + part) * D + col;
#pragma unroll
          for (int e = 0; e < VEC; e += 4)
            *(float4*)(po + e) = make_float4(acc[g][k][e] * inv, acc[g][k][e + 1] * inv,
                                             acc[g][k][e + 2] * inv, acc[g][k][e + 3] * inv);
        } else {
          T* o = (T*)a.out + ((int64_t)j * a.num_q_heads + h) * D + col;
          if constexpr (BF16) {
            uint4 w;
            w.x = pack_bf16x2(acc[g][k][0] * inv, acc[g][k][1] * inv);
            w.y = pack_bf16x2(acc[g][k][2] * inv, acc[g][k][3] * inv);
            w.z = pack_bf16x2(acc[g][k][4] * inv, acc[g][k][5] * inv);
            w.w = pack_bf16x2(acc[g][k][6] * inv, acc[g][k][7] * inv);
            *(uint4*)o = w;
          } else {
            *(float4*)o = make_float4(acc[g][k][0] * inv, acc[g][k][1] * inv,
                                      acc[g][k][2] * inv, acc[g][k][3] * inv);
          }
        }
      }
      if constexpr (SPLIT) {
        if (c == 0)
          a.part_lse[((int64_t)j * a.num_q_heads + h) * a.max_partitions + part] =
              (m_run[g] + __log2f(l)) * 0.69314718055994530942f;
      }
    }
  }
}

template <typename T, int D, int G>
pa_status launch_typed(const DecodeArgs& a, bool split, hipStream_t stream) {
  const int groups = a.num_kv_heads / a.waves_per_group;
#if PA_GROUP_MAJOR
  const dim3 grid(groups, a.num_q_tokens, split ? a.max_partitions : 1);
#else
  const dim3 grid(a.num_q_tokens, groups, split ? a.max_partitions : 1);
#endif
  const dim3 block(a.waves_per_group * kWave);
  const bool uniform = (1 << a.log2_bs) >= Shape<T, D, G>::TPI;
  if (split) {
    if (uniform)
      hipLaunchKernelGGL((decode_kernel<T, D, G, true, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<T, D, G, true, false>), grid, block, 0, stream, a);
  } else {
    if (uniform)
      hipLaunchKernelGGL((decode_kernel<T, D, G, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<T, D, G, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <typename T, int D>
pa_status dispatch_g(const DecodeArgs& a, bool split, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_typed<T, D, 1>(a, split, s);
    case 2: return launch_typed<T, D, 2>(a, split, s);
    case 4: return launch_typed<T, D, 4>(a, split, s);
    case 8: return launch_typed<T, D, 8>(a, split, s);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <typename T>
pa_status dispatch_d(const DecodeArgs& a, bool split, hipStream_t s) {
  switch (a.head_dim) {
    case 32: return dispatch_g<T, 32>(a, split, s);
    case 64: return dispatch_g<T, 64>(a, split, s);
    case 128: return dispatch_g<T, 128>(a, split, s);
    case 256: return dispatch_g<T, 256>(a, split, s);
    default: return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace

pa_status launch_decode(const DecodeArgs& a, bool split, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.dtype == PA_BF16) return dispatch_d<uint16_t>(a, split, s);
  if (a.dtype == PA_F32) return dispatch_d<float>(a, split, s);
  return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
