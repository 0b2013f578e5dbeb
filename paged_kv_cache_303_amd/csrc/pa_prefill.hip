// Chunked-prefill attention tile on the matrix cores (gfx950 MFMA), bf16.
//
// What it computes ("LLM 推理引擎的内存管理与调度" §8, chunked prefill; the
// attention itself as in "19.2 KV Cache 系统化管理" §19.2.3): a sequence of
// len cached keys whose last q_len tokens are queries (a prefill chunk).
// Query j of the chunk sits at position len - q_len + j and attends to keys
// 0 .. that position through the sequence's block table (causal,
// bottom-right aligned).  Keys are cut into the split layout's partitions
// (partition p = keys [p*P, (p+1)*P)); for query token j, head h and each
// partition p holding keys it sees: part_o[j][h][p][:] = o_p,
// part_lse[j][h][p] = ln(sum exp(scale * q.k)) over the partition, which
// pa_reduce merges like any other query's partitions.
//
// Work item: (tile of 16 * kPfWaves query rows, partition, KV head) of a
// sequence with q_len > 1.  A query row is a (token, query head) pair of the
// G heads sharing the KV head, so rows = q_len * G, and 128 rows (8 waves)
// are 128 / G tokens; each wave owns 16 rows.  Every K/V tile gathered into
// LDS serves all rows of the workgroup, so the row tile sets how often a
// partition's K/V is re-read: 8 waves read it half as often as 4, and a
// 512-token chunk after 4096 cached tokens took 104 us instead of 145.  The workgroups are persistent
// (two per compute unit at 8 waves, all resident): each counts
// the items of every sequence (prefix sums in LDS) and takes items
// blockIdx.x, blockIdx.x + gridDim.x, ...; consecutive items are row tiles
// of one (partition, head), so workgroups running together read the same
// K/V rows.  Keys go in tiles of 32:
//   * the workgroup gathers the tile's K rows into LDS ([key][dim]) and its V
//     rows transposed ([dim][key]), through the block table;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (16 keys x 16 rows per
//     instruction, 32 dims of the contraction per instruction): each lane
//     then holds 8 scores of one query row, which are also the 8 values the
//     A operand of P V needs for that row when the P V contraction runs over
//     the keys in the same order (V^T is read in that order), so P stays in
//     registers;
//   * online softmax per row in the log2 domain with lazy rescaling (the
//     running max moves only when a tile's exceeds it by more than 8), the
//     causal and partition masks by position, probabilities rounded to bf16;
//   * O += P V with the same MFMA, 32 keys of the tile per step;
//   * the next tile's K/V rows are loaded into registers while the current
//     one is computed.
// MFMA operand layout (16x16x32): lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16] for e < 8, and D[4 (l / 16) + i][l % 16] for
// i < 4.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Staging registers of the K/V gathers.  A native vector type: copies of
// HIP's struct uint4 between global memory, a local array and LDS are
// memcpys that stay in private (scratch) memory, whose store makes every
// prefetch load wait at once.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef PA_PF_WAVES
#define PA_PF_WAVES 8
#endif
#ifndef PA_PF_BLOCKS_PER_CU
#define PA_PF_BLOCKS_PER_CU 2
#endif
constexpr int kPfWaves = PA_PF_WAVES;   // waves per workgroup (16 query rows each)
constexpr int kPfRows = 16 * kPfWaves;  // query rows per workgroup
constexpr int kPfKeys = 32;             // keys per tile (a multiple of 32)
constexpr int kPad = 8;                 // bf16 elements of padding per LDS row
constexpr float kLn2Pf = 0.69314718055994530942f;
constexpr float kPfLazy = 8.0f;  // running-max slack (log2 units) before a rescale
constexpr int kPrefillMaxSeqs = 1024;   // sequences per launch (LDS prefix sums)
constexpr int kPfMaxBlocks = 1024;      // block ids of one partition staged in LDS
constexpr int kPfBlocksPerCu = PA_PF_BLOCKS_PER_CU;  // persistent workgroups per compute unit

__device__ __forceinline__ f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int D, int G>
__global__ __launch_bounds__(kPfWaves * kWave) void prefill_mfma_kernel(
    DecodeArgs a, const int32_t* __restrict__ block_tables) {
  constexpr int KC = D / 32;  // 32-dim slices of the QK contraction
  constexpr int DB = D / 16;  // 16-dim column blocks of O
  constexpr int CPR = D / 8;  // 16-byte chunks per K/V row
  constexpr int KS = D + kPad;        // LDS row stride of K (elements)
  constexpr int VS = kPfKeys + kPad;  // LDS row stride of V^T
  constexpr int NCH = kPfKeys * CPR;                          // 16-byte chunks of K per tile
  constexpr int NLD = (NCH + kPfWaves * kWave - 1) / (kPfWaves * kWave);  // per thread
  constexpr int NCHV = kPfKeys / 2 * CPR;                     // key-pair chunks of V per tile
  constexpr int NLDV = (NCHV + kPfWaves * kWave - 1) / (kPfWaves * kWave);
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kPfKeys * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VS];
  __shared__ int wcum[kPrefillMaxSeqs + 1];  // prefix sums of work items per sequence
  __shared__ int blk_lds[kPfMaxBlocks];      // physical blocks of the item's key range

  const int B = a.num_seqs;
  const int H = a.num_kv_heads;
  const int P = a.partition_size;
  const int cap = a.max_blocks << a.log2_bs;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // ---- items per sequence: row tiles x partitions x KV heads ----------------
  auto items_of = [&](int q_len, int len) {
    if (q_len <= 1 || len <= 0) return 0;
    return (q_len * G + kPfRows - 1) / kPfRows * ((len + P - 1) / P) * H;
  };
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const int q_len = a.cu_q_lens[i + 1] - a.cu_q_lens[i];
    wcum[i + 1] = items_of(q_len, min(max(a.seq_lens[i], 0), cap));
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    int carry = 0;
    if (lane == 0) wcum[0] = 0;
    for (int base = 0; base < B; base += kWave) {
      const int i = base + lane;
      int x = i < B ? wcum[i + 1] : 0;  // inclusive scan across the wave
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
      }
      if (i < B) wcum[i + 1] = carry + x;
      carry += __shfl(x, kWave - 1, kWave);
    }
  }
  __syncthreads();
  const int total = __builtin_amdgcn_readfirstlane(wcum[B]);

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = B - 1;  // sequence: the last b with wcum[b] <= item
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(wcum[mid]) <= item) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int q_first = a.cu_q_lens[b];
    const int q_len = a.cu_q_lens[b + 1] - q_first;
    const int len = min(max(a.seq_lens[b], 0), cap);
    const int ntiles = (q_len * G + kPfRows - 1) / kPfRows;
    const int nparts = (len + P - 1) / P;
    int rem = item - __builtin_amdgcn_readfirstlane(wcum[b]);
    const int tile = rem % ntiles;
    rem /= ntiles;
    const int part = rem % nparts;
    const int kvh = rem / nparts;

    const int rows_total = q_len * G;
    const int row0 = tile * kPfRows;
    const int pos_base = len - q_len;  // position of the chunk's first query
    const int last_tok = min(q_len - 1, (row0 + kPfRows - 1) / G);
    const int k_lo = part * P;
    const int k_hi = min(k_lo + P, pos_base + last_tok + 1);  // keys of this item
    if (k_lo >= k_hi) continue;  // no row of the tile reaches this partition

    const int32_t* bt = block_tables + (int64_t)b * a.max_blocks;
    const int bs_mask = (1 << a.log2_bs) - 1;
    const int64_t row_bytes = (int64_t)H * D * 2;
    const int64_t block_bytes = row_bytes << a.log2_bs;
    const char* kp = (const char*)a.k_pool + (int64_t)kvh * D * 2;
    const char* vp = (const char*)a.v_pool + (int64_t)kvh * D * 2;

    // ---- Q fragments (A operand): row l % 16 of this wave, 8 dims per slice --
    const int ra = min(row0 + 16 * w + (lane & 15), rows_total - 1);
    const uint16_t* qrow = (const uint16_t*)a.q +
                           ((int64_t)(q_first + ra / G) * a.num_q_heads + kvh * G + ra % G) * D;
    uint4 qf[KC];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) qf[kk] = *(const uint4*)(qrow + 8 * (lane >> 4) + 32 * kk);

    // Scores are computed transposed, S^T = K Q^T (K as the A operand, Q as
    // B): lane l then holds the scores of one query row, l % 16, for keys
    // 4 (l / 16) + i and 16 + 4 (l / 16) + i of the tile (i < 4) -- exactly
    // the 8 contraction values the A operand of P V needs for that row, if
    // the P V contraction runs over the keys in that order (V^T is read
    // with the same order).  So P never leaves registers, and the softmax
    // state is one row per lane (m, l), shared by the 4 lanes l % 16 == row.
    const int rq = min(row0 + 16 * w + (lane & 15), rows_total - 1);  // this lane's row
    const int lim = min(pos_base + rq / G, k_hi - 1);  // last key the row sees here
    const int wave_last = pos_base + min(q_len - 1, (row0 + 16 * w + 15) / G);

    float m = -INFINITY, l = 0.f;
    f32x4 o[DB];  // O rows 4 (l / 16) + i, dim 16 db + l % 16
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the item's block ids (clamped) into LDS, so the tile gathers below do
    // not wait for a table lookup before their K/V loads
    const int blk0 = k_lo >> a.log2_bs;
    const int nblk = ((min(k_lo + P, len) - 1) >> a.log2_bs) - blk0 + 1;  // <= kPfMaxBlocks
    __syncthreads();  // the previous item's readers are done with blk_lds
    for (int i = threadIdx.x; i < nblk; i += blockDim.x)
      blk_lds[i] = min(max(bt[blk0 + i], 0), a.num_blocks - 1);
    __syncthreads();

    // K/V rows of keys k0 .. k0+31 (clamped to the item's last key) into
    // registers.  K: chunk ci = (key, 16-byte column), 16 lanes per 256-byte
    // row.  V: pair-chunk cv = (key pair kp = cv % 16, column dc = cv / 16),
    // both rows of the pair, so that each dim's two values pack into one
    // 32-bit LDS store of the transposed tile.
    u32x4 kreg[NLD], vreg[NLDV][2];
    auto row_off = [&](int key) {
      const int kk = min(key, k_hi - 1);  // keys past the item's range are masked
      const int phys = blk_lds[(kk >> a.log2_bs) - blk0];
      return phys * block_bytes + (int64_t)(kk & bs_mask) * row_bytes;
    };
    auto gather = [&](int k0) {
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int ci = min((int)threadIdx.x + n * kPfWaves * kWave, NCH - 1);
        kreg[n] = *(const u32x4*)(kp + row_off(k0 + ci / CPR) + (ci % CPR) * 16);
      }
#pragma unroll
      for (int n = 0; n < NLDV; ++n) {
        const int cv = min((int)threadIdx.x + n * kPfWaves * kWave, NCHV - 1);
        const int kp2 = 2 * (cv % (kPfKeys / 2)), dc = cv / (kPfKeys / 2);
        vreg[n][0] = *(const u32x4*)(vp + row_off(k0 + kp2) + dc * 16);
        vreg[n][1] = *(const u32x4*)(vp + row_off(k0 + kp2 + 1) + dc * 16);
      }
    };
    gather(k_lo);
    for (int k0 = k_lo; k0 < k_hi; k0 += kPfKeys) {
      // ---- registers -> LDS: K as [key][dim], V transposed as [dim][key] ----
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int ci = threadIdx.x + n * kPfWaves * kWave;
        if (NCH % (kPfWaves * kWave) != 0 && ci >= NCH) continue;
        *(u32x4*)(k_lds + (ci / CPR) * KS + (ci % CPR) * 8) = kreg[n];
      }
#pragma unroll
      for (int n = 0; n < NLDV; ++n) {
        const int cv = threadIdx.x + n * kPfWaves * kWave;
        if (NCHV % (kPfWaves * kWave) != 0 && cv >= NCHV) continue;
        const int kp2 = 2 * (cv % (kPfKeys / 2)), dc = cv / (kPfKeys / 2);
        const uint32_t r0[4] = {vreg[n][0].x, vreg[n][0].y, vreg[n][0].z, vreg[n][0].w};
        const uint32_t r1[4] = {vreg[n][1].x, vreg[n][1].y, vreg[n][1].z, vreg[n][1].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // dims 2q and 2q+1 of the chunk
          *(uint32_t*)(vt_lds + (dc * 8 + 2 * q) * VS + kp2) = (r0[q] & 0xFFFFu) | (r1[q] << 16);
          *(uint32_t*)(vt_lds + (dc * 8 + 2 * q + 1) * VS + kp2) =
              (r0[q] >> 16) | (r1[q] & 0xFFFF0000u);
        }
      }
      __syncthreads();
      if (k0 + kPfKeys < k_hi) gather(k0 + kPfKeys);  // in flight during the compute

      if (k0 <= wave_last) {  // this wave has rows that see some key of the tile
        // ---- S^T = K Q^T for the tile's 16-key blocks ----------------------
        constexpr int NB = kPfKeys / 16;  // 16-key blocks; pairs of them feed one P V step
        f32x4 st[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          st[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KC; ++kk) {
            const uint4 kf =
                *(const uint4*)(k_lds + (nb * 16 + (lane & 15)) * KS + 8 * (lane >> 4) + 32 * kk);
            st[nb] = mfma(kf, qf[kk], st[nb]);
          }
        }
        // ---- online softmax of this lane's row (log2 domain), lazy rescale --
        float x[NB * 4];
        float mx = -INFINITY;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + nb * 16 + 4 * (lane >> 4) + i;
            const float v = key <= lim ? st[nb][i] * a.scale_log2 : -INFINITY;
            x[nb * 4 + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = reduce_levels<4, 6>(mx, OpMax());  // the 4 lanes of the row
        // move the running max only when the tile's exceeds it by more than
        // kPfLazy (probabilities then stay below 2^kPfLazy); the rescale of
        // O needs each row's factor in the accumulator layout
        const bool move = mx > m + kPfLazy;
        if (__builtin_amdgcn_readfirstlane((int)(__ballot(move) != 0))) {
          const float m_new = move ? mx : m;
          const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - m_new);
          m = m_new;
          l *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * (lane >> 4) + i, kWave);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db][i] *= ai;
          }
        }
        float sum = 0.f;
        uint32_t pk[NB * 2];  // P as bf16 pairs, contraction order (block, i)
#pragma unroll
        for (int e = 0; e < NB * 4; e += 2) {
          const float p0 = m == -INFINITY ? 0.f : (float)(__bf16)fast_exp2(x[e] - m);
          const float p1 = m == -INFINITY ? 0.f : (float)(__bf16)fast_exp2(x[e + 1] - m);
          sum += p0 + p1;
          pk[e / 2] = (uint32_t)bf16_bits(p0) | ((uint32_t)bf16_bits(p1) << 16);
        }
        l += reduce_levels<4, 6>(sum, OpSum());
        // ---- O += P V: one MFMA step per pair of 16-key blocks; V^T rows read
        //      in the same key order (keys 4g..4g+3, then 16+4g..16+4g+3) -------
#pragma unroll
        for (int h = 0; h < NB / 2; ++h) {
          const uint4 pf = make_uint4(pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint16_t* vrow =
                vt_lds + (db * 16 + (lane & 15)) * VS + 32 * h + 4 * (lane >> 4);
            const uint2 v0 = *(const uint2*)vrow;
            const uint2 v1 = *(const uint2*)(vrow + 16);
            o[db] = mfma(pf, make_uint4(v0.x, v0.y, v1.x, v1.y), o[db]);
          }
        }
      }
      __syncthreads();  // the next tile overwrites K, V^T
    }

    // ---- normalise and store this partition of each row that has keys in it --
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = 4 * (lane >> 4) + i;  // lane holding row `src`'s m and l
      const float li = __shfl(l, src, kWave), mi = __shfl(m, src, kWave);
      const int rc = row0 + 16 * w + src;
      if (rc >= rows_total || pos_base + rc / G < k_lo) continue;
      const int64_t jh = (int64_t)(q_first + rc / G) * a.num_q_heads + kvh * G + rc % G;
      const float inv = 1.f / li;
      float* po = a.part_o + (jh * a.max_partitions + part) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) po[db * 16 + (lane & 15)] = o[db][i] * inv;
      if ((lane & 15) == 0)
        a.part_lse[jh * a.max_partitions + part] = (mi + __log2f(li)) * kLn2Pf;
    }
  }
}

template <int D>
pa_status launch_d(const DecodeArgs& a, hipStream_t stream) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return PA_ERR_HIP;
  const dim3 grid((uint32_t)(cus * kPfBlocksPerCu));
  const dim3 block(kPfWaves * kWave);
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: hipLaunchKernelGGL((prefill_mfma_kernel<D, 1>), grid, block, 0, stream, a, a.block_tables); break;
    case 2: hipLaunchKernelGGL((prefill_mfma_kernel<D, 2>), grid, block, 0, stream, a, a.block_tables); break;
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<D, 4>), grid, block, 0, stream, a, a.block_tables); break;
    case 8: hipLaunchKernelGGL((prefill_mfma_kernel<D, 8>), grid, block, 0, stream, a, a.block_tables); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

bool prefill_mfma_supported(const DecodeArgs& a) {
  const int g = a.num_kv_heads > 0 ? a.num_q_heads / a.num_kv_heads : 0;
  return a.dtype == PA_BF16 && a.cu_q_lens != nullptr && a.num_seqs <= kPrefillMaxSeqs &&
         a.partition_size / a.block_size + 1 <= kPfMaxBlocks &&
         (a.head_dim == 32 || a.head_dim == 64 || a.head_dim == 128 || a.head_dim == 256) &&
         (g == 1 || g == 2 || g == 4 || g == 8);
}

pa_status launch_prefill_mfma(const DecodeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (a.head_dim) {
    case 32: return launch_d<32>(a, s);
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    case 256: return launch_d<256>(a, s);
    default: return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace pa

