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
// Work item: (tile of 64 query rows, partition, KV head) of a sequence with
// q_len > 1.  A query row is a (token, query head) pair of the G heads
// sharing the KV head, so rows = q_len * G and 64 rows = 64 / G tokens; each
// of the 4 waves owns 16 rows.  The workgroups are persistent: each counts
// the items of every sequence (prefix sums in LDS) and takes items
// blockIdx.x, blockIdx.x + gridDim.x, ...; consecutive items are row tiles
// of one (partition, head), so workgroups running together read the same
// K/V rows.  Keys go in tiles of 32:
//   * the workgroup gathers the tile's K rows into LDS ([key][dim]) and its V
//     rows transposed ([dim][key]), through the block table;
//   * S = Q K^T with v_mfma_f32_16x16x32_bf16 (16 rows x 16 keys per
//     instruction, 32 dims of the contraction per instruction);
//   * online softmax per row in the log2 domain (running max, rescale of the
//     running sum and of O when it moves), causal mask by position;
//   * P is rounded to bf16 and staged through LDS into the A-operand layout,
//     then O += P V with the same MFMA (K = the tile's 32 keys);
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

constexpr int kPfWaves = 4;             // waves per workgroup
constexpr int kPfRows = 16 * kPfWaves;  // query rows per workgroup
constexpr int kPfKeys = 32;             // keys per tile
constexpr int kPad = 8;                 // bf16 elements of padding per LDS row
constexpr float kLn2Pf = 0.69314718055994530942f;
constexpr int kPrefillMaxSeqs = 1024;   // sequences per launch (LDS prefix sums)
constexpr int kPfMaxBlocks = 1024;      // block ids of one partition staged in LDS
constexpr int kPfBlocksPerCu = 4;       // persistent workgroups per compute unit

__device__ __forceinline__ f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int G>
__global__ __launch_bounds__(kPfWaves * kWave) void prefill_mfma_kernel(
    DecodeArgs a, const int32_t* __restrict__ block_tables) {
  constexpr int KC = D / 32;  // 32-dim slices of the QK contraction
  constexpr int DB = D / 16;  // 16-dim column blocks of O
  constexpr int CPR = D / 8;  // 16-byte chunks per K/V row
  constexpr int KS = D + kPad;        // LDS row stride of K (elements)
  constexpr int VS = kPfKeys + kPad;  // LDS row stride of V^T
  constexpr int PS = kPfKeys + kPad;  // LDS row stride of P
  constexpr int NCH = kPfKeys * CPR;                          // 16-byte chunks of K per tile
  constexpr int NLD = (NCH + kPfWaves * kWave - 1) / (kPfWaves * kWave);  // per thread
  constexpr int NCHV = kPfKeys / 2 * CPR;                     // key-pair chunks of V per tile
  constexpr int NLDV = (NCHV + kPfWaves * kWave - 1) / (kPfWaves * kWave);
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kPfKeys * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VS];
  __shared__ __attribute__((aligned(16))) uint16_t p_lds[kPfWaves][16 * PS];
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

    // rows this lane holds in the accumulator layout, and the last key each sees
    int lim[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rc = min(row0 + 16 * w + 4 * (lane >> 4) + i, rows_total - 1);
      lim[i] = min(pos_base + rc / G, k_hi - 1);
    }
    const int wave_last = pos_base + min(q_len - 1, (row0 + 16 * w + 15) / G);

    float m[4], l[4];
    f32x4 o[DB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.f;
    }
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
    uint4 kreg[NLD], vreg[NLDV][2];
    auto row_off = [&](int key) {
      const int kk = min(key, k_hi - 1);  // keys past the item's range are masked
      const int phys = blk_lds[(kk >> a.log2_bs) - blk0];
      return phys * block_bytes + (int64_t)(kk & bs_mask) * row_bytes;
    };
    auto gather = [&](int k0) {
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int ci = min((int)threadIdx.x + n * kPfWaves * kWave, NCH - 1);
        kreg[n] = *(const uint4*)(kp + row_off(k0 + ci / CPR) + (ci % CPR) * 16);
      }
#pragma unroll
      for (int n = 0; n < NLDV; ++n) {
        const int cv = min((int)threadIdx.x + n * kPfWaves * kWave, NCHV - 1);
        const int kp2 = 2 * (cv % (kPfKeys / 2)), dc = cv / (kPfKeys / 2);
        vreg[n][0] = *(const uint4*)(vp + row_off(k0 + kp2) + dc * 16);
        vreg[n][1] = *(const uint4*)(vp + row_off(k0 + kp2 + 1) + dc * 16);
      }
    };
    gather(k_lo);
    for (int k0 = k_lo; k0 < k_hi; k0 += kPfKeys) {
      // ---- registers -> LDS: K as [key][dim], V transposed as [dim][key] ----
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int ci = threadIdx.x + n * kPfWaves * kWave;
        if (NCH % (kPfWaves * kWave) != 0 && ci >= NCH) continue;
        *(uint4*)(k_lds + (ci / CPR) * KS + (ci % CPR) * 8) = kreg[n];
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
        // ---- S = Q K^T for two 16-key blocks ------------------------------
        f32x4 s[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          s[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KC; ++kk) {
            const uint4 kf =
                *(const uint4*)(k_lds + (nb * 16 + (lane & 15)) * KS + 8 * (lane >> 4) + 32 * kk);
            s[nb] = mfma(qf[kk], kf, s[nb]);
          }
        }
        // ---- online softmax per row (log2 domain), causal + partition mask --
        float p[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float mx = -INFINITY;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int key = k0 + nb * 16 + (lane & 15);
            const float x = key <= lim[i] ? s[nb][i] * a.scale_log2 : -INFINITY;
            p[nb][i] = x;
            mx = fmaxf(mx, x);
          }
          mx = reduce_levels<0, 4>(mx, OpMax());  // across the 16 key lanes
          const float m_new = fmaxf(m[i], mx);
          const bool none = m_new == -INFINITY;  // row sees no key yet
          const float alpha = none ? 1.f : fast_exp2(m[i] - m_new);
          m[i] = m_new;
          float sum = 0.f;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            // bf16 probabilities: the same values enter the sum and P V
            const float pr = none ? 0.f : (float)(__bf16)fast_exp2(p[nb][i] - m_new);
            p[nb][i] = pr;
            sum += pr;
          }
          sum = reduce_levels<0, 4>(sum, OpSum());
          l[i] = l[i] * alpha + sum;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db][i] *= alpha;
        }
        // ---- P (bf16) into the A-operand layout through LDS -----------------
        uint16_t* pw = p_lds[w];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pw[(4 * (lane >> 4) + i) * PS + nb * 16 + (lane & 15)] = bf16_bits(p[nb][i]);
        wave_lds_sync();
        const uint4 pf = *(const uint4*)(pw + (lane & 15) * PS + 8 * (lane >> 4));
        // ---- O += P V --------------------------------------------------------
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint4 vf =
              *(const uint4*)(vt_lds + (db * 16 + (lane & 15)) * VS + 8 * (lane >> 4));
          o[db] = mfma(pf, vf, o[db]);
        }
      }
      __syncthreads();  // the next tile overwrites K, V^T
    }

    // ---- normalise and store this partition of each row that has keys in it --
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rc = row0 + 16 * w + 4 * (lane >> 4) + i;
      if (rc >= rows_total || pos_base + rc / G < k_lo) continue;
      const int64_t jh = (int64_t)(q_first + rc / G) * a.num_q_heads + kvh * G + rc % G;
      const float inv = 1.f / l[i];
      float* po = a.part_o + (jh * a.max_partitions + part) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) po[db * 16 + (lane & 15)] = o[db][i] * inv;
      if ((lane & 15) == 0)
        a.part_lse[jh * a.max_partitions + part] = (m[i] + __log2f(l[i])) * kLn2Pf;
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

