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

// Tokens per tile: 16 (8 for fp32 head_dim 256, to bound registers).
template <typename T, int D>
constexpr int tile_instrs() {
  constexpr int vec = Elt<T>::kVec;
  constexpr int lpr = D / vec;
  constexpr int tpi = kWave / lpr;
  constexpr int ni = 16 / tpi;
  return ni > 8 ? 8 : (ni < 1 ? 1 : ni);
}

// UNIFORM: the rows of one load instruction always share a block (the block
// size is a multiple of TPI), so block-table entries are wave-uniform scalar
// loads; otherwise every lane looks its block up.
template <typename T, int D, int G, bool SPLIT, bool UNIFORM>
__global__ __launch_bounds__(kMaxWaves * kWave) void decode_kernel(DecodeArgs a) {
  constexpr int VEC = Elt<T>::kVec;
  constexpr bool BF16 = sizeof(T) == 2;
  constexpr int LPR = D / VEC;           // lanes per token row
  constexpr int LOG_LPR = ilog2(LPR);
  constexpr int TPI = kWave / LPR;       // token rows per load instruction
  constexpr int NI = tile_instrs<T, D>();
  constexpr int TT = NI * TPI;           // tokens per tile
  static_assert(LPR * VEC == D && LPR <= kWave, "row must fit a wave");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int tg = lane / LPR;  // which row of a load instruction
  const int c = lane % LPR;   // which 16-byte chunk of the row
  const int j = blockIdx.x;   // query token
  const int kvh = blockIdx.y * a.waves_per_group + wave;
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
        for (int g = 0; g < G; ++g) {
          uint4* o = (uint4*)((T*)a.out + ((int64_t)j * a.num_q_heads + h0 + g) * D + c * VEC);
          *o = make_uint4(0, 0, 0, 0);
        }
      }
      return;
    }
  }

  // --- query vectors: this lane's 16-byte chunk of each of the G heads -------
  const T* qrow = (const T*)a.q + ((int64_t)j * a.num_q_heads + h0) * D + c * VEC;
  uint4 qraw[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qraw[g] = *(const uint4*)(qrow + (int64_t)g * D);
  float qf[G][VEC];  // fp32 path: query pre-multiplied by scale*log2(e)
  if constexpr (!BF16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      qf[g][0] = __uint_as_float(qraw[g].x) * a.scale_log2;
      qf[g][1] = __uint_as_float(qraw[g].y) * a.scale_log2;
      qf[g][2] = __uint_as_float(qraw[g].z) * a.scale_log2;
      qf[g][3] = __uint_as_float(qraw[g].w) * a.scale_log2;
    }
  }

  // --- addressing --------------------------------------------------------------
  const uint32_t row_bytes = (uint32_t)a.num_kv_heads * D * sizeof(T);
  const int64_t block_bytes = (int64_t)row_bytes << a.log2_bs;
  const uint32_t lane_col = (uint32_t)(kvh * D + c * VEC) * sizeof(T);
  const char* kp = (const char*)a.k_pool;
  const char* vp = (const char*)a.v_pool;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  const int bs_mask = (1 << a.log2_bs) - 1;
  const int nb_max = a.num_blocks - 1;

  float m_run[G], l_run[G], acc[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
  }

  // Physical block of each load instruction of the tile starting at t0; in
  // UNIFORM mode these are wave-uniform scalar loads, fetched one tile ahead
  // so their latency hides behind the previous tile's arithmetic.
  auto lookup = [&](int t0, int (&ph)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (UNIFORM) {
        const int blk = min(t0 + i * TPI, end - 1) >> a.log2_bs;
        ph[i] = bt[blk];
      } else {
        ph[i] = bt[min(t0 + i * TPI + tg, end - 1) >> a.log2_bs];
      }
    }
  };
  int ph[NI];
  lookup(start, ph);

  for (int t0 = start; t0 < end; t0 += TT) {
    // ---- gather K and V rows of the tile through the block table ----------
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tok = min(t0 + i * TPI + tg, end - 1);  // clamp masked rows
      const int phys = min(max(ph[i], 0), nb_max);
      uint32_t off;
      if constexpr (UNIFORM) {
        // tiles start at multiples of TT (a multiple of TPI), so the TPI rows
        // of this instruction lie in one block: the block of its first row.
        const int blk0 = min(t0 + i * TPI, end - 1) >> a.log2_bs;
        off = (uint32_t)(tok - (blk0 << a.log2_bs)) * row_bytes + lane_col;
      } else {
        off = (uint32_t)(tok & bs_mask) * row_bytes + lane_col;
      }
      kr[i] = *(const uint4*)(kp + phys * block_bytes + off);
      vr[i] = *(const uint4*)(vp + phys * block_bytes + off);
    }
    if (t0 + TT < end) lookup(t0 + TT, ph);

    // ---- scores: partial dot over the lane's chunk, then sum the row -------
    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d;
        if constexpr (BF16) {
          d = dot2_bf16(qraw[g].x, kr[i].x, 0.f);
          d = dot2_bf16(qraw[g].y, kr[i].y, d);
          d = dot2_bf16(qraw[g].z, kr[i].z, d);
          d = dot2_bf16(qraw[g].w, kr[i].w, d);
        } else {
          d = qf[g][0] * __uint_as_float(kr[i].x);
          d = fmaf(qf[g][1], __uint_as_float(kr[i].y), d);
          d = fmaf(qf[g][2], __uint_as_float(kr[i].z), d);
          d = fmaf(qf[g][3], __uint_as_float(kr[i].w), d);
        }
        s[i][g] = reduce_levels<0, LOG_LPR>(d, OpSum());
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool valid = (t0 + i * TPI + tg) < end;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float sc = BF16 ? s[i][g] * a.scale_log2 : s[i][g];
        s[i][g] = valid ? sc : -INFINITY;
      }
    }

    // ---- online softmax (log2 domain) ----------------------------------------
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mt = s[0][g];
#pragma unroll
      for (int i = 1; i < NI; ++i) mt = fmaxf(mt, s[i][g]);
      mt = reduce_groups<LOG_LPR>(mt, OpMax());
      if (mt > m_run[g]) {  // same outcome on every lane of the wave
        const float alpha = fast_exp2(m_run[g] - mt);
        m_run[g] = mt;
        l_run[g] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] *= alpha;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float p = fast_exp2(s[i][g] - m_run[g]);
        l_run[g] += p;
        s[i][g] = p;
      }
    }

    // ---- PV --------------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float v[VEC];
      if constexpr (BF16) {
        v[0] = bf16_lo(vr[i].x); v[1] = bf16_hi(vr[i].x);
        v[2] = bf16_lo(vr[i].y); v[3] = bf16_hi(vr[i].y);
        v[4] = bf16_lo(vr[i].z); v[5] = bf16_hi(vr[i].z);
        v[6] = bf16_lo(vr[i].w); v[7] = bf16_hi(vr[i].w);
      } else {
        v[0] = __uint_as_float(vr[i].x); v[1] = __uint_as_float(vr[i].y);
        v[2] = __uint_as_float(vr[i].z); v[3] = __uint_as_float(vr[i].w);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = fmaf(s[i][g], v[e], acc[g][e]);
      }
    }
  }

  // --- combine the token groups and write ---------------------------------------
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = reduce_groups<LOG_LPR>(l_run[g], OpSum());
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[g][e] = reduce_groups<LOG_LPR>(acc[g][e], OpSum());
    const float inv = 1.f / l;
    const int h = h0 + g;
    if (tg == 0) {
      if constexpr (SPLIT) {
        float* po = a.part_o + (((int64_t)j * a.num_q_heads + h) * a.max_partitions + part) * D +
                    c * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          *(float4*)(po + e) =
              make_float4(acc[g][e] * inv, acc[g][e + 1] * inv, acc[g][e + 2] * inv,
                          acc[g][e + 3] * inv);
        if (c == 0) {
          a.part_lse[((int64_t)j * a.num_q_heads + h) * a.max_partitions + part] =
              (m_run[g] + __log2f(l)) * 0.69314718055994530942f;
        }
      } else {
        T* o = (T*)a.out + ((int64_t)j * a.num_q_heads + h) * D + c * VEC;
        if constexpr (BF16) {
          uint4 w;
          w.x = pack_bf16x2(acc[g][0] * inv, acc[g][1] * inv);
          w.y = pack_bf16x2(acc[g][2] * inv, acc[g][3] * inv);
          w.z = pack_bf16x2(acc[g][4] * inv, acc[g][5] * inv);
          w.w = pack_bf16x2(acc[g][6] * inv, acc[g][7] * inv);
          *(uint4*)o = w;
        } else {
          *(float4*)o = make_float4(acc[g][0] * inv, acc[g][1] * inv, acc[g][2] * inv,
                                    acc[g][3] * inv);
        }
      }
    }
  }
}

template <typename T, int D, int G>
pa_status launch_typed(const DecodeArgs& a, bool split, hipStream_t stream) {
  const int groups = a.num_kv_heads / a.waves_per_group;
  const dim3 grid(a.num_q_tokens, groups, split ? a.max_partitions : 1);
  const dim3 block(a.waves_per_group * kWave);
  constexpr int kTpi = kWave * Elt<T>::kVec / D;
  const bool uniform = (1 << a.log2_bs) >= kTpi;
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
