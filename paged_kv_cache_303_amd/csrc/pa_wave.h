// Per-wave tile machinery of the paged decode on gfx950 (WaveCtx): block-table
// gather, QK, online softmax and PV for one KV head and the G query heads
// that share it.  Used by the decode kernels (pa_decode.hip) and by the
// persistent split kernel (pa_split.hip).
//
// What it computes ("19.2 KV Cache 系统化管理" §19.2.3, paged_attention): for
// one query token, walk the request's keys in logical order through its block
// table (logical block t / block_size -> physical block, row t % block_size;
// "LLM 推理引擎的内存管理与调度" §3), and fold them into a running maximum m,
// a running sum l of exp(s - m) and a running weighted sum of values, both
// rescaled by exp(m_old - m_new) when the maximum grows; divide at the end.
// The unit folded at once is a tile of TT tokens instead of one block.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace wave {


constexpr int kMaxWaves = 8;  // workgroup = up to 8 KV heads

// Index of the wave in its workgroup, as a scalar: the compiler cannot tell
// that threadIdx.x / 64 is the same on every lane of a wave, and values
// derived from it would otherwise live in vector registers and turn the
// branches on them into exec-masked code.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

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
template <>
struct Elt<uint8_t> {  // e4m3 codes, one fp32 scale per (token, KV head)
  static constexpr int kVec = 16;
};

#ifndef PA_TILE_TOKENS
#define PA_TILE_TOKENS 16  // target tokens per tile (per wave, per KV head)
#endif
#ifndef PA_FP8_TILE_TOKENS
#define PA_FP8_TILE_TOKENS 32  // the same for e4m3 pools (half the bytes per row)
#endif
#ifndef PA_BF16_PAIR_PV
#define PA_BF16_PAIR_PV 1  // bf16 PV two rows at a time with v_dot2_f32_bf16
#endif
#ifndef PA_FP8_QREG_MAX_G
#define PA_FP8_QREG_MAX_G 8
#endif
#ifndef PA_FP8_QREG_MAX_D
#define PA_FP8_QREG_MAX_D 256  // fp8 with G <= 4: the query as bfloat16 pairs in registers up to this head size
#endif
#ifndef PA_FP8_MFMA_QK
#define PA_FP8_MFMA_QK 1  // fp8 scores on the matrix cores (see Shape::MQK_OK; 2: every shape)
#endif
#ifndef PA_MAX_CPL
#define PA_MAX_CPL 2  // 16-byte chunks of a row per lane, at most
#endif
#ifndef PA_MAX_TILE_LOADS
#define PA_MAX_TILE_LOADS 8  // 16-byte loads per lane per tile (K or V), hot shapes
#endif

// Lane layout for (element type, head_dim, query heads per KV head):
//   CPL  16-byte chunks of a row per lane (2 halves the row reduction and the
//        redundant exponentials; 1 when G is large, to bound accumulators)
//   LPR  lanes per token row, TPI rows per load instruction
//   NI   load instructions (of CPL chunks each) per tile, TT tokens per tile
template <typename T, int D, int G, bool UNIFORM = true, int TILE = 0>
struct Shape {
  static constexpr int VEC = Elt<T>::kVec;
  static constexpr int CHUNKS = D / VEC;
  // (fp8: one chunk of 16 codes per lane already needs 16 accumulators per head)
  static constexpr int CPL = (CHUNKS >= 8 && G <= 4 && PA_MAX_CPL >= 2 && sizeof(T) > 1) ? 2 : 1;
  static constexpr int LPR = CHUNKS / CPL;
  static constexpr int TPI = kWave / LPR;
  // Loads per lane per tile (K or V; two tiles are in registers at a time):
  // the bf16 shapes with small G get the full budget, the others less, so
  // that accumulators and both tiles stay in 256 VGPRs without spilling.
  static constexpr int MAX_LOADS =
      (sizeof(T) <= 2 && G <= 4 && D <= 128 && UNIFORM) ? PA_MAX_TILE_LOADS
      : (G >= 8 ? PA_MAX_TILE_LOADS / 4 : PA_MAX_TILE_LOADS / 2);
  // target tokens per tile: TILE if given, else the default of the type
  static constexpr int TILE_TOKENS =
      TILE > 0 ? TILE : (sizeof(T) == 1 ? PA_FP8_TILE_TOKENS : PA_TILE_TOKENS);
  static constexpr int NI0 = (TILE_TOKENS / TPI) < 1 ? 1 : (TILE_TOKENS / TPI);
  static constexpr int NI = (NI0 * CPL > MAX_LOADS) ? (MAX_LOADS / CPL < 1 ? 1 : MAX_LOADS / CPL) : NI0;
  static constexpr int TT = NI * TPI;
  // fp8 scores on the matrix cores (WaveCtx::MQK) where they pay: with 8
  // heads a KV head or head_dim 256 (MI355X, balanced decode at batch 128:
  // G = 8, D = 128 3.5 against 2.2 TB/s; G = 4, D = 256 4.7 against 4.4);
  // at G <= 4, D <= 128 the vector-unit scores are faster (4.4 against 4.0).
  // Its K loads cover 16 keys an instruction, so it needs blocks of at least
  // 16 keys for the uniform (one block per instruction) lookup.
  static constexpr bool MQK_OK = PA_FP8_MFMA_QK && sizeof(T) == 1 && G <= 8 &&
                                 (D == 64 || D == 128 || D == 256) && TT % 16 == 0 &&
                                 (G >= 8 || D >= 256 || PA_FP8_MFMA_QK >= 2);
  // keys a block must hold for the UNIFORM kernels
  static constexpr int UKEYS = MQK_OK && TPI < 16 ? 16 : TPI;
  // Ranges start at multiples of 16 (partitions) or of TT (slices), plus
  // multiples of TT, so every load instruction starts on a multiple of TPI
  // (needed by the UNIFORM lookup).
  static_assert(LPR * CPL * VEC == D && LPR <= kWave && (16 % TPI) == 0 && NI >= 1,
                "unsupported lane layout");
};

// Lazy rescaling: the running maximum m (log2 domain) is only moved when a
// tile's maximum exceeds it by more than this, so probabilities stay below
// 2^kLazy and the O(G*D) rescale of the accumulators is rare.  The result
// is independent of m up to rounding (acc and l carry the same factor).
constexpr float kLazy = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;

// Per-wave state and tile machinery for one KV head and its G query heads.
// UNIFORM: the rows of one load instruction always share a block (the block
// size is a multiple of TPI), so block-table entries are wave-uniform scalar
// loads; otherwise every lane looks its block up.
template <typename T, int D, int G, bool UNIFORM, int TILE = 0>
struct WaveCtx {
  using S = Shape<T, D, G, UNIFORM, TILE>;
  static constexpr int VEC = S::VEC, CPL = S::CPL, LPR = S::LPR, LOG_LPR = ilog2(S::LPR);
  static constexpr int TPI = S::TPI, NI = S::NI, TT = S::TT;
  static constexpr bool BF16 = sizeof(T) == 2;
  // fp8 pools: e4m3 codes with one fp32 scale per (token, KV head) for K and
  // V; the query and the output are bfloat16
  static constexpr bool FP8 = sizeof(T) == 1;
  static constexpr uint32_t kChunkStride = LPR * 16;  // bytes between a lane's chunks
  static constexpr int QW = FP8 ? 2 : 1;  // 16-byte pieces of one chunk of the bf16 query
  // fp8 scores on the matrix cores: S = Q K^T with v_mfma_f32_16x16x32_bf16
  // per group of 16 keys (query heads as the 16 rows, G of them real; keys
  // as the columns; 32 dims a step).  Lane l loads 16 codes of key l % 16 --
  // bytes 64 ii + 16 (l / 16) of the row for K load ii of the group -- and
  // feeds codes 8h .. 8h+7 of that load, converted exactly to bfloat16, to
  // step 2 ii + h; the query's rows are laid out the same way, once per
  // sequence.  Scores come back with key l % 16 in lane l and heads
  // 4 (l / 16) + r in its four registers; the softmax runs there, and each
  // lane then fetches the weights of its V rows for the vector-unit PV.
  static constexpr bool MQK = S::MQK_OK && UNIFORM;
  static constexpr int KG = TT / 16;  // 16-key groups per tile
  static constexpr int LPK = D / 64;  // K loads per group (64 codes per 16 lanes)
  static constexpr int NU = D / 32;   // matrix steps per group
  // fp8 scores on the vector units: the query in registers as bfloat16 pairs
  // (qp) up to PA_FP8_QREG_MAX_G heads and PA_FP8_QREG_MAX_D dims, else in
  // LDS like the other types
  static constexpr bool QREG = FP8 && !MQK && G <= PA_FP8_QREG_MAX_G && D <= PA_FP8_QREG_MAX_D;

  struct Tile {
    uint4 k[NI][CPL];
    uint4 v[NI][CPL];
    float ks[FP8 ? NI : 1], vs[FP8 ? NI : 1];  // fp8: scales of the lane's rows
  };

  // The current query lives in LDS, not registers: [G][CPL][LPR] 16-byte
  // chunks per wave (fp32: pre-scaled), read back once per tile; the lanes
  // of one chunk column read the same address (broadcast).  (fp8: registers,
  // see qp and qa.)
  static constexpr int kQChunks = QREG ? 1 : G * CPL * LPR * QW;

  const DecodeArgs& a;
  uint4* qs;  // this wave's kQChunks chunks in LDS
  int lane, tg, c, kvh;
  uint32_t row_bytes, lane_col;
  int64_t block_bytes;
  int nb_max, bs_mask;
  float qk_scale;
  float m_run[G], l_run[G], acc[G][CPL][VEC];
  // fp8: the current query's 16 dims of this lane's chunk, per head, as 8
  // bfloat16 pairs (held in registers for the whole sequence: each K chunk is
  // converted once per tile to bfloat16 pairs, exactly -- every e4m3 value is
  // a bfloat16 value -- and dotted with all G heads by v_dot2_f32_bf16)
  uint32_t qp[QREG ? G : 1][QREG ? 8 : 1];
  // MQK: the query as the matrix operand (row lane % 16 < G, else zero), per
  // step, and the lane's partial softmax sums of heads 4 (lane / 16) + r
  u32x4_t qa[MQK ? NU : 1];
  float lq[4];

  __device__ WaveCtx(const DecodeArgs& args, int kv_head, uint4* q_lds)
      : a(args), qs(q_lds), kvh(kv_head) {
    lane = threadIdx.x & (kWave - 1);
    tg = lane / LPR;
    c = lane % LPR;
    row_bytes = (uint32_t)a.num_kv_heads * D * sizeof(T);
    block_bytes = (int64_t)row_bytes << a.log2_bs;
    lane_col = (uint32_t)(kvh * D + c * VEC) * sizeof(T);
    nb_max = a.num_blocks - 1;
    bs_mask = (1 << a.log2_bs) - 1;
    qk_scale = (BF16 || FP8) ? a.scale_log2 : 1.0f;  // fp32 queries are pre-scaled
  }

  // Query token j's chunks of the G heads into LDS; scores stay unscaled and
  // scale*log2(e) goes into the exponent's fma (bf16) or into the fp32 query.
  __device__ void load_query(int j) {
    if constexpr (MQK) {
      const int row = lane & 15;
      const uint16_t* qrow =
          (const uint16_t*)a.q + ((int64_t)j * a.num_q_heads + kvh * G + min(row, G - 1)) * D;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int dim = 64 * (u >> 1) + 16 * (lane >> 4) + 8 * (u & 1);
        const uint4 v = *(const uint4*)(qrow + dim);
        qa[u] = row < G ? u32x4_t{v.x, v.y, v.z, v.w} : u32x4_t{0u, 0u, 0u, 0u};
      }
      return;
    }
    if constexpr (QREG) {  // bf16 query: every lane keeps its chunk's 16 dims per head
      const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)j * a.num_q_heads + kvh * G) * D;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int h = 0; h < QW; ++h) {
          const uint4 v = *(const uint4*)(qrow + (int64_t)g * D + c * VEC + h * 8);
          qp[g][4 * h] = v.x;
          qp[g][4 * h + 1] = v.y;
          qp[g][4 * h + 2] = v.z;
          qp[g][4 * h + 3] = v.w;
        }
      return;
    }
    if constexpr (FP8) {  // bf16 query in LDS: a chunk's 16 dims are two 16-byte pieces
      const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)j * a.num_q_heads + kvh * G) * D;
      if (tg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int h = 0; h < QW; ++h)
            qs[((g * CPL) * LPR + c) * QW + h] =
                *(const uint4*)(qrow + (int64_t)g * D + c * VEC + h * 8);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      return;
    }
    const T* qrow = (const T*)a.q + ((int64_t)j * a.num_q_heads + kvh * G) * D;
    if (tg == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          uint4 v = *(const uint4*)(qrow + (int64_t)g * D + (c + k * LPR) * VEC);
          if constexpr (!BF16) {
            v.x = __float_as_uint(__uint_as_float(v.x) * a.scale_log2);
            v.y = __float_as_uint(__uint_as_float(v.y) * a.scale_log2);
            v.z = __float_as_uint(__uint_as_float(v.z) * a.scale_log2);
            v.w = __float_as_uint(__uint_as_float(v.w) * a.scale_log2);
          }
          qs[(g * CPL + k) * LPR + c] = v;
        }
    }
    // the wave's own LDS writes must land before its reads (no other wave
    // touches this region)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  __device__ void reset() {
#pragma unroll
    for (int r = 0; r < 4; ++r) lq[r] = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_run[g] = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][k][e] = 0.f;
    }
  }

  // Physical block of each load instruction of the tile at token t0 of the
  // sequence whose table row is bt (keys < end).  Rows are clamped to end-1,
  // so a tile past the end still addresses a written row.
  __device__ void lookup(const int32_t* bt, int t0, int end, int (&ph)[NI]) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (UNIFORM) {
        // scalar loads: a vector load here would be waited for together with
        // the tile loads issued before it, draining the pipeline
        ph[i] = bt[min(t0 + i * TPI, end - 1) >> a.log2_bs];
      } else {
        ph[i] = bt[min(t0 + i * TPI + tg, end - 1) >> a.log2_bs];
      }
    }
  }

  // Gather the K and V rows of the tile at t0 through the block table.
  //
  // UNIFORM: instruction i reads rows t0 + i*TPI .. +TPI-1 of the block that
  // holds its first row (clamped to the range's last block), so the block
  // base is wave-uniform (scalar registers) and every lane adds the same
  // loop-invariant offset (tg rows down, its chunk across): no per-tile
  // vector address arithmetic.  Rows at or past `end` stay inside that
  // allocated block -- memory-safe -- and compute() masks them (their bytes
  // may be unwritten NaN poison).  Otherwise each lane looks up its own row,
  // clamped to end-1.
  __device__ void issue(Tile& tl, int t0, int end, const int (&ph)[NI]) const {
    const char* kp = (const char*)a.k_pool;
    const char* vp = (const char*)a.v_pool;
    if constexpr (UNIFORM) {
      // buffer loads: descriptor of the block (scalar), row offset (scalar),
      // lane offset (one loop-invariant vector register)
      const uint32_t lane_off = (uint32_t)tg * row_bytes + lane_col;
      if constexpr (MQK) {
        // K: group kg = keys t0 + 16 kg + (lane & 15), in the block of V
        // instruction 16 kg / TPI (blocks hold >= 16 keys, groups are aligned)
        const uint32_t k_off =
            (uint32_t)(lane & 15) * row_bytes + (uint32_t)(kvh * D + 16 * (lane >> 4));
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
          const int phys = min(max(ph[16 * kg / TPI], 0), nb_max);
          const int r0 = (t0 + 16 * kg) & bs_mask;
          const __amdgpu_buffer_rsrc_t kr =
              buffer_rsrc(kp + phys * block_bytes, (uint32_t)block_bytes);
#pragma unroll
          for (int ii = 0; ii < LPK; ++ii)
            tl.k[kg * LPK + ii][0] = buffer_load16_nt(kr, k_off + 64 * ii, (uint32_t)r0 * row_bytes);
          tl.ks[kg] = a.k_scale[fp8_scale_index(phys, r0 + (lane & 15), kvh, a.num_kv_heads,
                                                a.log2_bs)];
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int phys = min(max(ph[i], 0), nb_max);
          const uint32_t row = (uint32_t)((t0 + i * TPI) & bs_mask) * row_bytes;
          const __amdgpu_buffer_rsrc_t vr =
              buffer_rsrc(vp + phys * block_bytes, (uint32_t)block_bytes);
          tl.v[i][0] = buffer_load16_nt(vr, lane_off, row);
          tl.vs[i] = a.v_scale[fp8_scale_index(phys, ((t0 + i * TPI) & bs_mask) + tg, kvh,
                                               a.num_kv_heads, a.log2_bs)];
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int phys = min(max(ph[i], 0), nb_max);
        const int64_t blk = phys * block_bytes;
        const uint32_t row = (uint32_t)((t0 + i * TPI) & bs_mask) * row_bytes;
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kp + blk, (uint32_t)block_bytes);
        const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vp + blk, (uint32_t)block_bytes);
#pragma unroll
        for (int k = 0; k < CPL; ++k) tl.k[i][k] = buffer_load16_nt(kr, lane_off + k * kChunkStride, row);
#pragma unroll
        for (int k = 0; k < CPL; ++k) tl.v[i][k] = buffer_load16_nt(vr, lane_off + k * kChunkStride, row);
        if constexpr (FP8) {  // this lane's row: tg rows into the instruction's rows
          const int64_t si = fp8_scale_index(phys, ((t0 + i * TPI) & bs_mask) + tg, kvh,
                                             a.num_kv_heads, a.log2_bs);
          tl.ks[i] = a.k_scale[si];
          tl.vs[i] = a.v_scale[si];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int tok = min(t0 + i * TPI + tg, end - 1);  // clamp rows past the end
        const int phys = min(max(ph[i], 0), nb_max);
        const uint32_t off = (uint32_t)(tok & bs_mask) * row_bytes + lane_col;
        const char* kb = kp + phys * block_bytes + off;
        const char* vb = vp + phys * block_bytes + off;
#pragma unroll
        for (int k = 0; k < CPL; ++k) tl.k[i][k] = load16_nt(kb + k * kChunkStride);
#pragma unroll
        for (int k = 0; k < CPL; ++k) tl.v[i][k] = load16_nt(vb + k * kChunkStride);
        if constexpr (FP8) {
          const int64_t si =
              fp8_scale_index(phys, tok & bs_mask, kvh, a.num_kv_heads, a.log2_bs);
          tl.ks[i] = a.k_scale[si];
          tl.vs[i] = a.v_scale[si];
        }
      }
    }
  }

  // MQK scores and softmax of the tile at t0 (keys < end): afterwards s[i][g]
  // holds the weight of this lane's V row i for head g, as in dot_softmax.
  __device__ void mqk_softmax(const Tile& tl, int t0, int end, bool tail, float (&s)[NI][G]) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const int hsel = lane >> 4;  // heads 4 hsel + r of this lane's scores
    f32x4_t sc[KG];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      sc[kg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint4 w = tl.k[kg * LPK + (u >> 1)][0];
        const uint32_t lo = (u & 1) ? w.z : w.x, hi = (u & 1) ? w.w : w.y;
        const u32x4_t kb = {
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false)),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true))};
        sc[kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[u]),
                                                        __builtin_bit_cast(bf16x8_t, kb), sc[kg],
                                                        0, 0, 0);
      }
    }
    // the key's K scale; keys past the end (NaN-poisoned codes or scales
    // possible) get -inf by a bit select
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      const bool valid = !tail || (t0 + 16 * kg + (lane & 15)) < end;
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[kg][r] = select_bits(valid, sc[kg][r] * tl.ks[kg], -INFINITY);
    }
    // ---- online softmax (log2 domain), lazily rescaled ------------------------
    constexpr int R = G < 4 ? G : 4;  // score registers that hold real heads
    float mt[G];
    bool move = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mx = sc[0][r];
#pragma unroll
      for (int kg = 1; kg < KG; ++kg) mx = fmaxf(mx, sc[kg][r]);
      mx = reduce_levels<0, 4>(mx, OpMax());
#pragma unroll
      for (int hb = 0; 4 * hb + r < G; ++hb) {
        const int g = 4 * hb + r;
        mt[g] = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 16 * hb)) *
                qk_scale;
        move |= mt[g] > m_run[g] + kLazy;
      }
    }
    if (__builtin_amdgcn_readfirstlane((int)move)) {  // mt and m_run are uniform
      float alpha[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m_new = fmaxf(m_run[g], mt[g]);
        alpha[g] = fast_exp2(m_run[g] - m_new);
        m_run[g] = m_new;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][0][e] *= alpha[g];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) lq[r] *= (G > 4 && hsel == 1) ? alpha[(4 + r) % G] : alpha[r];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float m = (G > 4 && hsel == 1) ? m_run[(4 + r) % G] : m_run[r];
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        const float p = fast_exp2(fmaf(sc[kg][r], qk_scale, -m));
        lq[r] += p;
        sc[kg][r] = p;
      }
    }
    // ---- each lane's V rows: key i TPI + tg of the tile, from lane key % 16
    // (+ 16 per four heads) of its group's scores
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int key = i * TPI + tg;
      constexpr int kTPI = TPI;
      const int kg = (i * kTPI) / 16;  // the same for every lane (TPI divides 16)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int src = (key & 15) + 16 * (g >> 2);
        // (the element is copied out first: this compiler's __builtin_bit_cast
        // of a vector element reads element 0)
        const float x = sc[kg][g & 3];
        s[i][g] = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, x)));
      }
    }
  }

  // Fold the tile at t0 (keys < end) into the running softmax state.
  __device__ void compute(const Tile& tl, int t0, int end) {
    float s[NI][G];
    const bool tail = t0 + TT > end;
    if constexpr (MQK) {
      mqk_softmax(tl, t0, end, tail, s);
    } else {
      dot_softmax(tl, t0, end, tail, s);
    }
    pv(tl, t0, end, tail, s);
  }

  // Scores on the vector units (partial dots over the lane's chunks, summed
  // over the row's lanes) and the online softmax: afterwards s[i][g] holds the
  // weight of this lane's row i for head g.
  __device__ void dot_softmax(const Tile& tl, int t0, int end, bool tail, float (&s)[NI][G]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) s[i][g] = 0.f;
    if constexpr (QREG) {  // each chunk of 16 codes converted once, dotted with every head
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        uint32_t kb[8];
        fp8x16_to_bf16x2(tl.k[i][0], kb);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d = dot2_bf16(qp[g][e], kb[e], d);
          s[i][g] = d;
        }
      }
    } else if constexpr (FP8) {  // query from LDS, one head at a time
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint4 q0 = qs[((g * CPL) * LPR + c) * QW];
        const uint4 q1 = qs[((g * CPL) * LPR + c) * QW + 1];
        const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        float qg[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qg[2 * e] = bf16_lo(qw[e]);
          qg[2 * e + 1] = bf16_hi(qw[e]);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          float kf[16];
          fp8x16_to_f32(tl.k[i][0], kf);
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) d = fmaf(qg[e], kf[e], d);
          s[i][g] = d;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G && !FP8; ++g) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const uint4 qv = qs[(g * CPL + k) * LPR + c];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          float d = s[i][g];
          if constexpr (BF16) {
            d = dot2_bf16(qv.x, tl.k[i][k].x, d);
            d = dot2_bf16(qv.y, tl.k[i][k].y, d);
            d = dot2_bf16(qv.z, tl.k[i][k].z, d);
            d = dot2_bf16(qv.w, tl.k[i][k].w, d);
          } else {
            d = fmaf(__uint_as_float(qv.x), __uint_as_float(tl.k[i][k].x), d);
            d = fmaf(__uint_as_float(qv.y), __uint_as_float(tl.k[i][k].y), d);
            d = fmaf(__uint_as_float(qv.z), __uint_as_float(tl.k[i][k].z), d);
            d = fmaf(__uint_as_float(qv.w), __uint_as_float(tl.k[i][k].w), d);
          }
          s[i][g] = d;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) s[i][g] = reduce_levels<0, LOG_LPR>(s[i][g], OpSum());
    if constexpr (FP8) {  // the row's K scale (rows past the end are selected away below)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g) s[i][g] *= tl.ks[i];
    }
    if (tail) {  // rows past the end get probability 0
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool valid = (t0 + i * TPI + tg) < end;
#pragma unroll
        for (int g = 0; g < G; ++g) s[i][g] = select_bits(valid, s[i][g], -INFINITY);
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
    if (__builtin_amdgcn_readfirstlane((int)move)) {  // same on every lane: make it scalar
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

  }

  // PV of the tile at t0 with the weights s of this lane's rows.
  __device__ void pv(const Tile& tl, int t0, int end, bool tail, const float (&s)[NI][G]) {
    if constexpr ((QREG || MQK) && NI % 2 == 0) {
      // Two rows at a time, i and i + 1 (same lane, same dims): each dim's two
      // codes become one bfloat16 pair, and each head's two weights
      // p * v_scale one pair rounded to bfloat16, so that v_dot2_f32_bf16
      // adds both rows' terms at once.  Masked rows may hold NaN poison: their
      // scale and codes are zeroed (code 0 is +0) before any arithmetic.
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        const bool va = !(UNIFORM && tail) || (t0 + i * TPI + tg) < end;
        const bool vb = !(UNIFORM && tail) || (t0 + (i + 1) * TPI + tg) < end;
        const float sa = select_bits(va, tl.vs[i], 0.f);
        const float sb = select_bits(vb, tl.vs[i + 1], 0.f);
        uint32_t vp[16];  // dim e: (row i, row i + 1)
        fp8x16_pairs_to_bf16x2(mask_words(va, tl.v[i][0]), mask_words(vb, tl.v[i + 1][0]), vp);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t wpair = pack_bf16x2(s[i][g] * sa, s[i + 1][g] * sb);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[g][0][e] = dot2_bf16(wpair, vp[e], acc[g][0][e]);
        }
      }
      return;
    }
    if constexpr (BF16 && NI % 2 == 0 && PA_BF16_PAIR_PV) {
      // Two rows at a time, i and i + 1 (same lane, same dims): each dim's two
      // values form one bfloat16 pair and each head's two weights one pair
      // rounded to bfloat16, so that v_dot2_f32_bf16 adds both rows' terms
      // at once (half the multiply-adds of the fp32 form, and no unpacking).
      // Masked rows may hold NaN poison: their bits are zeroed first.
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        const bool va = !(UNIFORM && tail) || (t0 + i * TPI + tg) < end;
        const bool vb = !(UNIFORM && tail) || (t0 + (i + 1) * TPI + tg) < end;
        uint32_t wp[G];
#pragma unroll
        for (int g = 0; g < G; ++g) wp[g] = pack_bf16x2(s[i][g], s[i + 1][g]);
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const uint4 a4 = mask_words(va, tl.v[i][k]);
          const uint4 b4 = mask_words(vb, tl.v[i + 1][k]);
          const uint32_t aw[4] = {a4.x, a4.y, a4.z, a4.w};
          const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
          uint32_t vp[8];  // dim 2m + h: (row i, row i + 1)
#pragma unroll
          for (int m2 = 0; m2 < 4; ++m2) {
            vp[2 * m2] = __builtin_amdgcn_perm(bw[m2], aw[m2], 0x05040100u);
            vp[2 * m2 + 1] = __builtin_amdgcn_perm(bw[m2], aw[m2], 0x07060302u);
          }
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[g][k][e] = dot2_bf16(wp[g], vp[e], acc[g][k][e]);
        }
      }
      return;
    }
    if constexpr (FP8) {  // p * (code * scale): the row's V scale goes into p
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        // masked rows may hold NaN poison: zero their scale and codes (code 0
        // is +0) before any arithmetic, never multiply them
        const bool valid = !(UNIFORM && tail) || (t0 + i * TPI + tg) < end;
        const float vsc = select_bits(valid, tl.vs[i], 0.f);
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          float vf[16];
          fp8x16_to_f32(mask_words(valid, tl.v[i][k]), vf);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pv = s[i][g] * vsc;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[g][k][e] = fmaf(pv, vf[e], acc[g][k][e]);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        // masked rows may hold NaN poison: zero their bits before unpacking,
        // never multiply them
        const uint4 vw = mask_words(!(UNIFORM && tail) || (t0 + i * TPI + tg) < end, tl.v[i][k]);
        float v[VEC];
        if constexpr (BF16) {
          v[0] = bf16_lo(vw.x); v[1] = bf16_hi(vw.x);
          v[2] = bf16_lo(vw.y); v[3] = bf16_hi(vw.y);
          v[4] = bf16_lo(vw.z); v[5] = bf16_hi(vw.z);
          v[6] = bf16_lo(vw.w); v[7] = bf16_hi(vw.w);
        } else {
          v[0] = __uint_as_float(vw.x); v[1] = __uint_as_float(vw.y);
          v[2] = __uint_as_float(vw.z); v[3] = __uint_as_float(vw.w);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[g][k][e] = fmaf(s[i][g], v[e], acc[g][k][e]);
      }
    }
  }

  // Fold the keys [start, end) of the sequence with table row bt, pipelined:
  // the loads of tile t+1 are in flight while tile t is computed (two register
  // tiles).  Loads are issued unconditionally -- past the end they re-read the
  // clamped last row -- so each compute waits for exactly one older tile.
  // Requires start < end.
  __device__ void run(const int32_t* bt, int start, int end) {
    int ph[NI];
    lookup(bt, start, end, ph);
    Tile ta, tb;
    issue(ta, start, end, ph);
    lookup(bt, start + TT, end, ph);
    for (int t0 = start;;) {
      issue(tb, t0 + TT, end, ph);
      lookup(bt, t0 + 2 * TT, end, ph);
      compute(ta, t0, end);
      t0 += TT;
      if (t0 >= end) break;
      issue(ta, t0 + TT, end, ph);
      lookup(bt, t0 + 2 * TT, end, ph);
      compute(tb, t0, end);
      t0 += TT;
      if (t0 >= end) break;
    }
  }

  // Sum the token groups: afterwards lanes with tg == 0 hold the full acc of
  // their chunks and every lane the full l.
  __device__ void combine(float (&l)[G]) {
    if constexpr (MQK) {  // sums of the 16 key lanes of each head's registers
#pragma unroll
      for (int r = 0; r < (G < 4 ? G : 4); ++r) {
        const float t = reduce_levels<0, 4>(lq[r], OpSum());
#pragma unroll
        for (int hb = 0; 4 * hb + r < G; ++hb)
          l_run[4 * hb + r] =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 16 * hb));
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] = MQK ? l_run[g] : reduce_groups<LOG_LPR>(l_run[g], OpSum());
#pragma unroll
      for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][k][e] = reduce_groups<LOG_LPR>(acc[g][k][e], OpSum());
    }
  }

  // Normalised output of query j (dtype T) -- after combine().
  __device__ void store_out(void* out, int j, const float (&l)[G]) const {
    if (tg != 0) return;
    if constexpr (FP8) {  // bf16 output, 16 dims a chunk
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float inv = 1.f / l[g];
        uint16_t* o = (uint16_t*)out + ((int64_t)j * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          const int col = (c + k * LPR) * VEC;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float* x = &acc[g][k][8 * h];
            uint4 w;
            w.x = pack_bf16x2(x[0] * inv, x[1] * inv);
            w.y = pack_bf16x2(x[2] * inv, x[3] * inv);
            w.z = pack_bf16x2(x[4] * inv, x[5] * inv);
            w.w = pack_bf16x2(x[6] * inv, x[7] * inv);
            *(uint4*)(o + col + 8 * h) = w;
          }
        }
      }
      return;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float inv = 1.f / l[g];
      T* o = (T*)out + ((int64_t)j * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int col = (c + k * LPR) * VEC;
        if constexpr (BF16) {
          uint4 w;
          w.x = pack_bf16x2(acc[g][k][0] * inv, acc[g][k][1] * inv);
          w.y = pack_bf16x2(acc[g][k][2] * inv, acc[g][k][3] * inv);
          w.z = pack_bf16x2(acc[g][k][4] * inv, acc[g][k][5] * inv);
          w.w = pack_bf16x2(acc[g][k][6] * inv, acc[g][k][7] * inv);
          *(uint4*)(o + col) = w;
        } else {
          *(float4*)(o + col) = make_float4(acc[g][k][0] * inv, acc[g][k][1] * inv,
                                            acc[g][k][2] * inv, acc[g][k][3] * inv);
        }
      }
    }
  }

  // Partial (o, lse) of head h = kvh*G + g at o_row(h) / lse_at(h) -- after combine().
  template <class ORow, class LseAt>
  __device__ void store_partial(ORow o_row, LseAt lse_at, const float (&l)[G]) const {
    if (tg != 0) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int h = kvh * G + g;
      const float inv = 1.f / l[g];
      float* po = o_row(h);
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int col = (c + k * LPR) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          *(float4*)(po + col + e) = make_float4(acc[g][k][e] * inv, acc[g][k][e + 1] * inv,
                                                 acc[g][k][e + 2] * inv, acc[g][k][e + 3] * inv);
      }
      if (c == 0) *lse_at(h) = (m_run[g] + __log2f(l[g])) * kLn2;
    }
  }

  __device__ void store_zero(void* out, int j) const {
    if (tg != 0) return;
    if constexpr (FP8) {  // bf16 output
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < CPL; ++k)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *(uint4*)((uint16_t*)out + ((int64_t)j * a.num_q_heads + kvh * G + g) * D +
                      (c + k * LPR) * VEC + 8 * h) = make_uint4(0, 0, 0, 0);
      return;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int k = 0; k < CPL; ++k)
        *(uint4*)((T*)out + ((int64_t)j * a.num_q_heads + kvh * G + g) * D +
                  (c + k * LPR) * VEC) = make_uint4(0, 0, 0, 0);
  }
};

// Query token j -> (sequence, number of query tokens of that sequence, first
// query token of the sequence), binary search over cu_q_lens.
__device__ __forceinline__ void locate(const DecodeArgs& a, int j, int& b, int& q_len,
                                       int& q_first) {
  b = j;
  q_first = j;
  q_len = 1;
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
}

// (dtype, head_dim, G) -> template instance: f.template operator()<T, D, G>().
template <class F>
inline pa_status dispatch(const DecodeArgs& a, F&& f) {
  const int g = a.num_q_heads / a.num_kv_heads;
  auto by_g = [&](auto t, auto d) -> pa_status {
    using T = decltype(t);
    constexpr int Dv = decltype(d)::value;
    switch (g) {
      case 1: return f.template operator()<T, Dv, 1>();
      case 2: return f.template operator()<T, Dv, 2>();
      case 4: return f.template operator()<T, Dv, 4>();
      case 8: return f.template operator()<T, Dv, 8>();
      default: return PA_ERR_UNSUPPORTED;
    }
  };
  auto by_d = [&](auto t) -> pa_status {
    switch (a.head_dim) {
      case 32:
        // fp8 rows of 32 codes would put 32 tokens in one load instruction,
        // more than the 16-token alignment of partitions and slices
        if constexpr (sizeof(decltype(t)) == 1) return PA_ERR_UNSUPPORTED;
        else return by_g(t, std::integral_constant<int, 32>());
      case 64: return by_g(t, std::integral_constant<int, 64>());
      case 128: return by_g(t, std::integral_constant<int, 128>());
      case 256: return by_g(t, std::integral_constant<int, 256>());
      default: return PA_ERR_UNSUPPORTED;
    }
  };
  if (a.dtype == PA_BF16) return by_d(uint16_t());
  if (a.dtype == PA_F32) return by_d(float());
  if (a.dtype == PA_FP8) return by_d(uint8_t());
  return PA_ERR_UNSUPPORTED;
}

}  // namespace wave
}  // namespace pa
