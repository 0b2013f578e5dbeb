// Split-sequence paged attention in one persistent launch (pa_decode_split).
//
// What it computes: the first pass of split-sequence attention.  A sequence
// with one query token (a decode step) has its keys cut into partitions of P
// tokens, and every partition p is summarised by (o_p, lse_p): the
// softmax-weighted mean of its values and the log of its sum of exponentials
// -- the running max / running sum state of "19.2 KV Cache 系统化管理"
// §19.2.3 with one partition as the unit.  A sequence with several query
// tokens is a chunk of a prefill ("LLM 推理引擎的内存管理与调度" §8): its
// query i sits at position len - q_len + i and sees keys 0 .. position
// (causal, bottom-right aligned).  Each of its queries has two partitions
// split at h = 32 * floor(ceil(ctx / 32) / 2), ctx = len - q_len the cached
// context before the chunk: keys [0, h) and [h, position]; or one partition
// with all its keys when h is 0.  pa_reduce merges the summaries.
//
// One launch holds a work list that mixes both kinds of work:
//   * decode items: 8 (query token, partition, KV head) units, one per wave,
//     each run by the vector-unit tile machinery of pa_wave.h (HBM-bound);
//   * prefill items (bf16, head_dim <= 128): 128 query rows x one partition
//     x one KV head, on the matrix cores (compute-bound); a query row is a
//     (token, query head) pair of the G heads sharing the KV head.
// Workgroups are persistent (as many as the device holds at once) and drain
// eight work queues, one per XCD, through atomic counters in the caller's
// workspace; each claims its next item while it runs the current one, and
// one whose own queue is empty reads all the counters at once and takes from
// a queue with work left.  Work items are laid out in blocks of eight (one
// item per queue) and prefill blocks are spread evenly among decode blocks,
// so that while some compute units run matrix-core tiles the others keep the
// memory system busy.  The last workgroup to finish returns the counters to
// zero for the next call.
//
// Prefill item (8 waves): wave w takes row block w % 4 (32 rows) and key half
// w / 4 of the item's key range, in tiles of 32 keys.  Per step the workgroup
// brings the two halves' K and V tiles into LDS (each K/V byte loaded once
// serves 128 rows): with LDS-direct loads as [key][dim] for blocks of at
// least 4 keys (V^T then read with transposing LDS reads), otherwise through
// registers, K as [key][dim] and V transposed as [dim][key]; each wave then
// computes
//   S^T = K Q^T            v_mfma_f32_32x32x16_bf16, K from LDS, Q in registers
//   online softmax         per row, in registers, log2 domain, lazy rescale
//   O^T += V^T P^T         the same MFMA, V^T from LDS, P^T in registers
// Lane l holds row l % 32 in every one of these layouts (S^T and O^T as the
// D operand: row l % 32, 16 keys or dims per lane; P^T as the B operand), so
// the softmax state and the rescale never leave the lane and P needs no
// exchange: the 16 scores a lane holds are exactly its B-operand values for
// the two 16-key halves of the tile once the V^T columns are stored in the
// matching key order (within each 16 keys, key bits 2 and 3 swapped).  At the
// end the two key halves of each row block are merged through LDS.
//
// MFMA operand layout (32x32x16): lane l holds A[l % 32][8 (l / 32) + e] and
// B[8 (l / 32) + e][l % 32] for e < 8, and D[8 (r / 4) + 4 (l / 32) + r % 4]
// [l % 32] in accumulator r < 16.
#include <type_traits>
#include "pa_wave.h"

namespace pa {
namespace {
using namespace wave;

constexpr int kSplitWaves = 8;     // waves per workgroup
constexpr int kQueues = 8;         // work queues (one per XCD)
static_assert(kQueues + 1 <= kSplitQueueInts, "queue and finish counters fit the control block");
constexpr int kPfRowBlocks = 4;    // 32-row blocks per prefill item
constexpr int kPfKeySplit = 2;     // key halves per prefill item
constexpr int kPfRows = 32 * kPfRowBlocks;
constexpr int kPfTile = 32;        // keys per tile
constexpr int kPfPad = 8;          // bf16 elements of padding per LDS row
constexpr float kPfLazy = 8.0f;    // running-max slack (log2 units) before a rescale
constexpr float kLn2Split = 0.69314718055994530942f;
// s_waitcnt operand: vector-memory count 0, the other counters unconstrained
// (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;  // LDS / scalar-memory count 0, the others unconstrained
constexpr int kWaitLgkmMask = 0xF0FF;  // AND-ed into a vmcnt wait: lgkmcnt 0 as well
constexpr int vm_wait(int n) {  // vmcnt n (< 64), the other counters unconstrained
  return 0x0F70 | (n & 15) | ((n >> 4) << 14);
}

#ifndef PA_PF_DMA
#define PA_PF_DMA 1  // prefill tiles through LDS-direct loads (blocks of >= 4 keys)
#endif
#ifndef PA_SPLIT_ORDER
#define PA_SPLIT_ORDER 0  // 0: prefill blocks spread among decode blocks; 1: decode first
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// LDS of one prefill step: the K tiles [key][dim] and transposed V tiles
// [dim][key] of the key halves.
template <int D>
struct PfTiles {
  uint16_t k[kPfKeySplit][kPfTile][D + kPfPad];
  uint16_t vt[kPfKeySplit][D][kPfTile + kPfPad];
};
// The same with LDS-direct loads: K and V both [key][dim], unpadded rows
// whose 16-byte chunks are swizzled by key; three of them in flight.
template <int D>
struct PfDmaTiles {
  uint16_t k[kPfKeySplit][kPfTile][D];
  uint16_t v[kPfKeySplit][kPfTile][D];
};
constexpr int kPfStages = 3;  // tile buffers (rows loaded two steps ahead)
// The merge of key halves after the loop reuses the same LDS: per row block,
// m and l of the lane's row and the lane's D/2 accumulators.
template <int D>
constexpr size_t pf_merge_bytes() {
  return (size_t)kPfRowBlocks * kWave * (D / 2 + 4) * sizeof(float);
}
template <typename T, int D, int G, bool MFMA>
constexpr size_t split_lds_bytes() {
  constexpr size_t q = (size_t)kSplitWaves * WaveCtx<T, D, G, true>::kQChunks * 16;
  constexpr size_t qn = (size_t)kSplitWaves * WaveCtx<T, D, G, false>::kQChunks * 16;
  size_t m = q > qn ? q : qn;
  if constexpr (MFMA) {  // two tile buffers (staged and computed alternately), or the merge
    m = m > 2 * sizeof(PfTiles<D>) ? m : 2 * sizeof(PfTiles<D>);
#if PA_PF_DMA
    m = m > kPfStages * sizeof(PfDmaTiles<D>) ? m : kPfStages * sizeof(PfDmaTiles<D>);
#endif
    m = m > pf_merge_bytes<D>() ? m : pf_merge_bytes<D>();
  }
  return m;
}

// Position of key k (0..31) in a stored V^T row: bits 2 and 3 swapped, so
// that the 8 keys a lane contributes to one 16-key MFMA step are adjacent.
__device__ __forceinline__ int vt_quad_slot(int quad) {  // quad = k / 4, 0..7
  return (quad & 4) | ((quad & 1) << 1) | ((quad >> 1) & 1);
}

// LDS swizzles of the register-staged tile (XOR of a row's 16-byte chunk
// index by bits of the row), spreading the tile stores, whose lanes write rows
// 16 apart, over more banks; the MFMA operand reads stay 16-byte contiguous.
// (Counters still show bank conflicts on about half of this tile's LDS
// cycles; the LDS-direct tile below has none.)
__device__ __forceinline__ int k_chunk(int key, int chunk) {  // K row `key`
  return chunk ^ (((key >> 4) & 1) << 1);
}
__device__ __forceinline__ int vt_chunk(int dim, int chunk) {  // V^T row `dim`, 8 keys a chunk
  return chunk ^ ((dim >> 4) & 3);
}

// Split point of a prefill chunk's keys: half of its cached context, in
// whole 32-key tiles (0: one partition).
__device__ __forceinline__ int prefill_split(int len, int q_len) {
  const int tiles = (len - q_len + kPfTile - 1) / kPfTile;
  return kPfTile * (tiles / 2);
}

// One prefill item: rows [r0, r0 + 128) of a chunk (q_first, q_len, len), KV
// head kvh, keys [k_lo, k_hi) (partition `part`; rows see keys up to their
// position).  QUAD: blocks hold at least 4 keys, so every aligned key quad
// lies in one block.
template <int D, int G, bool QUAD>
__device__ void prefill_item(const DecodeArgs& a, const int32_t* __restrict__ bt, char* lds,
                             int q_first, int q_len, int len, int r0, int part, int k_lo,
                             int k_hi, int kvh) {
  constexpr int KC = D / 16;   // 16-dim MFMA steps of the QK contraction
  constexpr int DB = D / 32;   // 32-dim blocks of O^T
  constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  constexpr int UH = 8 * CPR;  // load units per key half: (key quad, column chunk)
  constexpr int NU = kPfKeySplit * UH;  // units per step, each loaded for K and for V
  static_assert(2 * NU <= kSplitWaves * kWave, "one K or V unit per thread");
  PfTiles<D>* tiles = reinterpret_cast<PfTiles<D>*>(lds);  // two buffers

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_id();
  const int rb = w % kPfRowBlocks, kh = w / kPfRowBlocks;
  const int H = a.num_kv_heads;
  const int rows_total = q_len * G;
  const int pos_base = len - q_len;
  const int ntiles = (k_hi - k_lo + kPfTile - 1) / kPfTile;
  const int bs_mask = (1 << a.log2_bs) - 1;
  static_assert(Shape<uint16_t, D, G>::TPI >= 4, "UNIFORM must imply blocks of >= 4 keys");
  const int64_t row_bytes = (int64_t)H * D * 2;
  const int64_t block_bytes = row_bytes << a.log2_bs;
  auto h_lo = [&](int h) { return h * ntiles / kPfKeySplit; };  // first tile of half h
  auto h_cnt = [&](int h) { return h_lo(h + 1) - h_lo(h); };
  const int nsteps = h_cnt(kPfKeySplit - 1);  // the last half has the most tiles

  // ---- this wave's rows: Q as the B operand, 8 dims per lane per MFMA -----
  const int rw0 = r0 + 32 * rb;
  const int row = min(rw0 + (lane & 31), rows_total - 1);
  const int lim = pos_base + row / G;  // last key this lane's row sees
  const int wave_first = pos_base + min(rw0, rows_total - 1) / G;
  const int wave_last = pos_base + min(rw0 + 31, rows_total - 1) / G;
  const uint16_t* qrow = (const uint16_t*)a.q +
                         ((int64_t)(q_first + row / G) * a.num_q_heads + kvh * G + row % G) * D;
  u32x4_t qf[KC];
#pragma unroll
  for (int kk = 0; kk < KC; ++kk) qf[kk] = *(const u32x4_t*)(qrow + 16 * kk + 8 * (lane >> 5));

  float m = -INFINITY, l = 0.f;  // row state (m shared by lanes l, l ^ 32; l partial)
  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // ---- gathers: thread = (K or V, unit (key half, key quad qd, 16-byte chunk dc))
  // Two register stages: the rows of step s + 2 are loaded while step s is
  // computed, and the block-table entries of a step are loaded one step
  // before its gathers (raw, clamped where used), so that no load waits on
  // another in the loop.  Every thread issues the same loads on every step
  // (a half with fewer steps, or a thread beyond the units, re-reads a valid
  // row and stores nothing), which keeps the in-order load counter exact.
  // Workgroups walk the tiles of each half from different starts (any order
  // gives the same softmax), so that the workgroups of one XCD do not all
  // request the same lines at once.
  const int rot = blockIdx.x / kQueues;
  const bool is_v = (tid / NU) & 1;
  const bool storer = tid < 2 * NU;
  const int u = tid % NU;
  // With 64 or more units per half a wave's units share their half, so its
  // tiles are wave-uniform and the table entries can be scalar loads (counted
  // apart from the vector loads in flight); blocks of >= 4 keys put a 32-key
  // tile in at most 8 consecutive table entries.
  constexpr bool SCALAR = QUAD && UH % kWave == 0;
  const int uh = SCALAR ? __builtin_amdgcn_readfirstlane(u / UH) : u / UH;
  // K units take a row's chunks on neighbouring lanes (each load instruction
  // reads whole 128-byte lines, which the cache takes in one access per line);
  // V units take neighbouring quads, so that the transposed stores below fall
  // in different LDS banks.
  const int uqd = is_v ? (u % UH) & 7 : (u % UH) / CPR;
  const int udc = is_v ? (u % UH) >> 3 : (u % UH) % CPR;
  const char* pool = (const char*)(is_v ? a.v_pool : a.k_pool) + (int64_t)kvh * D * 2 + udc * 16;
  auto tile_of = [&](int h, int s) { return h_lo(h) + (s + rot) % max(h_cnt(h), 1); };
  auto key_of = [&](int s, int i) {
    return max(min(k_lo + tile_of(uh, s) * kPfTile + 4 * uqd + i, k_hi - 1), 0);
  };
  u32x4_t buf[2][4];
  int ph[2][SCALAR ? 8 : 4];
  const int tile_blocks = max(kPfTile >> a.log2_bs, 1);
  // table-entry slot of step s: s % 2, a compile-time argument so that the
  // entries stay in registers
  auto lookup = [&](int s, auto slot) {
    constexpr int sl = decltype(slot)::value;
    if constexpr (SCALAR) {
      // the entries of the tile's blocks (entries past the table row repeat
      // the row's last one; their keys are masked)
      const int b0 = (k_lo + tile_of(uh, s) * kPfTile) >> a.log2_bs;
      const int last = min(tile_blocks, a.max_blocks - b0) - 1;
#pragma unroll
      for (int j = 0; j < 8; ++j) ph[sl][j] = bt[b0 + min(j, last)];
    } else {
      // with QUAD a key quad lies in one block, otherwise each key looks its block up
      ph[sl][0] = bt[key_of(s, 0) >> a.log2_bs];
      if constexpr (!QUAD) {
#pragma unroll
        for (int i = 1; i < 4; ++i) ph[sl][i] = bt[key_of(s, i) >> a.log2_bs];
      }
    }
  };
  auto gather = [&](int s, auto slot, u32x4_t (&r)[4]) {
    constexpr int sl = decltype(slot)::value;
    int quad_block = 0;
    if constexpr (SCALAR) {  // this lane's quad: entry j of the tile's blocks
      const int b0 = (k_lo + tile_of(uh, s) * kPfTile) >> a.log2_bs;
      const int j = min((key_of(s, 0) >> a.log2_bs) - b0, 7);
      // a select tree on the bits of j (the entries are wave-uniform)
      const int* e = ph[sl];
      const int t0 = j & 1 ? e[1] : e[0], t1 = j & 1 ? e[3] : e[2];
      const int t2 = j & 1 ? e[5] : e[4], t3 = j & 1 ? e[7] : e[6];
      const int u0 = j & 2 ? t1 : t0, u1 = j & 2 ? t3 : t2;
      quad_block = j & 4 ? u1 : u0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int entry = SCALAR ? quad_block : ph[sl][QUAD ? 0 : i];
      const int phys = min(max(entry, 0), a.num_blocks - 1);
      r[i] = *(const u32x4_t*)(pool + (int64_t)phys * block_bytes +
                               (uint32_t)((key_of(s, i) & bs_mask) * (uint32_t)row_bytes));
    }
  };
  auto stage = [&](int s, const u32x4_t (&r)[4], PfTiles<D>& tl) {  // registers -> LDS
    if (!storer || s >= h_cnt(uh)) return;
    if (!is_v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * uqd + i;
        *(u32x4_t*)&tl.k[uh][key][k_chunk(key, udc) * 8] = r[i];
      }
      return;
    }
    // V^T: dim 8 dc + 2c + h of the four keys as one 8-byte row segment
    const int slot = vt_quad_slot(uqd);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t sel = h ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(r[1][c], r[0][c], sel);
        const uint32_t hi = __builtin_amdgcn_perm(r[3][c], r[2][c], sel);
        const int dim = udc * 8 + 2 * c + h;
        *(uint2*)&tl.vt[uh][dim][vt_chunk(dim, slot >> 1) * 8 + (slot & 1) * 4] =
            make_uint2(lo, hi);
      }
    }
  };

  // Step s: compute from tile buffer s % 2 while the rows of step s + 1 are
  // stored into the other buffer (loaded two steps before), then gather step
  // s + 3 into the registers just freed and look up step s + 4; one barrier.
  auto compute = [&](int s, const PfTiles<D>& tl) {
    if (s >= h_cnt(kh)) return;
    const int k0 = k_lo + tile_of(kh, s) * kPfTile;
    if (k0 > wave_last) return;  // no row of this wave sees the tile
    // ---- S^T = K Q^T ------------------------------------------------------
    // Every fragment read is issued before the first product, so that the
    // reads overlap one another rather than each waiting alone (where the
    // registers allow: the per-key table entries of small blocks take some).
    f32x16_t st;
#pragma unroll
    for (int r2 = 0; r2 < 16; ++r2) st[r2] = 0.f;
    auto k_frag = [&](int kk) {
      const int key = lane & 31;
      return *(const u32x4_t*)&tl.k[kh][key][k_chunk(key, 2 * kk + (lane >> 5)) * 8];
    };
    u32x4_t kf[KC];
    if constexpr (QUAD) {
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) kf[kk] = k_frag(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) st = mfma32(QUAD ? kf[kk] : k_frag(kk), qf[kk], st);
    auto v_frag = [&](int h, int db) {
      const int dim = 32 * db + (lane & 31);
      return *(const u32x4_t*)&tl.vt[kh][dim][vt_chunk(dim, 2 * h + (lane >> 5)) * 8];
    };
    // the V^T fragments, read while the softmax below runs
    u32x4_t vf[2][DB];
    if constexpr (QUAD) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[h][db] = v_frag(h, db);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- online softmax of the lane's row (log2 domain) ----------------------
    // Scores stay unscaled until the exponent: scale*log2(e) > 0 keeps the
    // order, so the maximum is taken on raw scores and p = 2^(s*c - m).
    const float c = a.scale_log2;
    float x[16];
#pragma unroll
    for (int r2 = 0; r2 < 16; ++r2) x[r2] = st[r2];
    if (__builtin_amdgcn_readfirstlane((int)(k0 + kPfTile - 1 > wave_first))) {
      // some key of the tile lies past some row's position (the diagonal or
      // the range's end): key 8 (r / 4) + 4 (l / 32) + r % 4 of the tile
      const int room = lim - k0 - 4 * (lane >> 5);
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2)
        x[r2] = 8 * (r2 >> 2) + (r2 & 3) <= room ? x[r2] : -INFINITY;
    }
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int r2 = 2; r2 < 16; r2 += 2) mx = fmaxf(mx, fmaxf(x[r2], x[r2 + 1]));
    mx = level_step<5>(mx, OpMax()) * c;  // the row's other 16 keys sit in lane l ^ 32
    const bool move = mx > m + kPfLazy;
    if (__builtin_amdgcn_readfirstlane((int)(__ballot(move) != 0))) {
      const float m_new = move ? mx : m;
      const float alpha = m_new == m ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) o[db][r2] *= alpha;
    }
    // probabilities rounded to bf16 for the P V product; l sums the rounded
    // values (a dot2 with (1, 1) adds both halves of a pair exactly)
    uint32_t pk[8];
    const float mm = m == -INFINITY ? 0.f : m;  // a row with no key yet: every p is 0
#pragma unroll
    for (int r2 = 0; r2 < 16; r2 += 2) {
      const float p0 = fast_exp2(fmaf(x[r2], c, -mm));
      const float p1 = fast_exp2(fmaf(x[r2 + 1], c, -mm));
      const bf16x2_t pb = __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t);
      pk[r2 / 2] = __builtin_bit_cast(uint32_t, pb);
      l = dot2_bf16(pk[r2 / 2], 0x3F803F80u, l);
    }
    // ---- O^T += V^T P^T, 16 keys per step --------------------------------------
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t pf = {pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mfma32(QUAD ? vf[h][db] : v_frag(h, db), pf, o[db]);
    }
  };

  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  auto step = [&](int s, auto slot, const PfTiles<D>& cur, PfTiles<D>& next,
                  u32x4_t (&r)[4]) {  // slot: s % 2
    using Other = std::integral_constant<int, 1 - decltype(slot)::value>;
    compute(s, cur);
    stage(s + 1, r, next);  // r holds the rows of step s + 1
    if constexpr (SCALAR) {
      // scalar loads complete out of order: a use waits for all of them, so
      // the gathers are addressed before the next entries are requested
      gather(s + 3, Other{}, r);
      lookup(s + 4, slot);
    } else {
      // vector loads complete in order: the entries go first so that the
      // next step's gathers need not wait for this step's
      lookup(s + 4, slot);
      gather(s + 3, Other{}, r);  // in flight during the next two computes
    }
    __syncthreads();
  };

  lookup(0, Slot0{});
  lookup(1, Slot1{});
  // Wait for the query and the first table entries here: the loop keeps
  // gathers in flight across its compute, and the compiler cannot otherwise
  // prove these loads are done on every path into it (it would wait on the
  // gathers before each MFMA instead).
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  gather(0, Slot0{}, buf[0]);
  gather(1, Slot1{}, buf[1]);
  lookup(2, Slot0{});  // (two entry slots: step s's lookup reuses step s - 2's)
  stage(0, buf[0], tiles[0]);
  lookup(3, Slot1{});
  gather(2, Slot0{}, buf[0]);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {  // an odd count ends with an idle step
    step(s, Slot0{}, tiles[0], tiles[1], buf[1]);
    step(s + 1, Slot1{}, tiles[1], tiles[0], buf[0]);
  }

  // ---- merge the two key halves of each row block --------------------------------
  l = level_step<5>(l, OpSum());  // the row's sum over both lanes (l, l ^ 32)
  float* sp = reinterpret_cast<float*>(lds) + rb * kWave * (D / 2 + 4);
  __syncthreads();  // every wave is done with the tiles
  if (kh == 1) {
    sp[lane] = m;
    sp[kWave + lane] = l;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(float4*)&sp[2 * kWave + ((db * 4 + r4) * kWave + lane) * 4] =
            make_float4(o[db][4 * r4], o[db][4 * r4 + 1], o[db][4 * r4 + 2], o[db][4 * r4 + 3]);
  }
  __syncthreads();
  if (kh == 0) {
    const float m2 = sp[lane], l2 = sp[kWave + lane];
    const float mn = fmaxf(m, m2);
    const float a1 = m == mn ? 1.f : fast_exp2(m - mn);
    const float a2 = m2 == mn ? 1.f : fast_exp2(m2 - mn);
    l = l * a1 + l2 * a2;
    const int rr = rw0 + (lane & 31);
    if (rr < rows_total) {
      const int64_t jh = (int64_t)(q_first + rr / G) * a.num_q_heads + kvh * G + rr % G;
      const float inv = 1.f / l;
      float* po = a.part_o + (jh * a.max_partitions + part) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 v = *(const float4*)&sp[2 * kWave + ((db * 4 + r4) * kWave + lane) * 4];
          *(float4*)&po[32 * db + 8 * r4 + 4 * (lane >> 5)] =
              make_float4((o[db][4 * r4] * a1 + v.x * a2) * inv,
                          (o[db][4 * r4 + 1] * a1 + v.y * a2) * inv,
                          (o[db][4 * r4 + 2] * a1 + v.z * a2) * inv,
                          (o[db][4 * r4 + 3] * a1 + v.w * a2) * inv);
        }
      if (lane < 32) a.part_lse[jh * a.max_partitions + part] = (mn + __log2f(l)) * kLn2Split;
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill item with LDS-direct gathers (blocks of at least 4 keys).  Same work
// and arithmetic as prefill_item; only the way K and V reach LDS differs:
//   * Every K/V row goes from HBM straight into LDS with a 16-byte
//     global_load_lds per lane (one instruction fills 1 KiB: 512 / D rows),
//     so no register staging and no LDS stores.  Rows are unpadded; their
//     16-byte chunks are XOR-swizzled by key through the choice of source
//     address (LDS position p of row k holds chunk p ^ f(k)).
//   * V stays [key][dim]; the V^T operand of O^T += V^T P^T is read with the
//     transposing ds_read_b64_tr_b16 (within 16 lanes, lane j receives
//     element j % 4 of the 8-byte reads of lanes j / 4 + 4 e, e < 4), two
//     reads per 8 keys.
//   * Three tile buffers: step s is computed from buffer s % 3 while the
//     rows of steps s + 1 and s + 2 land in the other two.
// Counters on the 512-token chunk: no LDS bank conflicts (the register-staged
// tile below has them on about half of its LDS cycles) and the same or
// slightly better time.
// ---------------------------------------------------------------------------
// Chunk positions, for an LDS of 64 four-byte banks (16 lanes of a 16-byte
// read, or 32 lanes of an 8-byte read, are served together): the K reads of
// 16 consecutive keys and the transposed V reads of 4 consecutive keys x 32
// bytes (two 16-lane groups at once) each touch every bank once.
template <int D>
__device__ __forceinline__ int k_pos(int key, int c) {
  constexpr int CPR = D / 8;
  return c ^ ((key * CPR / 16) & (CPR - 1));
}
template <int D>
__device__ __forceinline__ int v_pos(int key, int c) {
  return c ^ (D == 128 ? 4 * (key & 3) : D == 64 ? 4 * ((key >> 1) & 1) : 0);
}
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int D, int G>
__device__ void prefill_item_dma(const DecodeArgs& a, const int32_t* __restrict__ bt, char* lds,
                                 int q_first, int q_len, int len, int r0, int part, int k_lo,
                                 int k_hi, int kvh) {
  constexpr int KC = D / 16;           // 16-dim MFMA steps of the QK contraction
  constexpr int DB = D / 32;           // 32-dim blocks of O^T
  constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
  constexpr int RPI = 512 / D;         // rows per load instruction (1 KiB)
  constexpr int NIS = 2 * kPfTile * kPfKeySplit / RPI;  // instructions per step (K and V)
  constexpr int IPW = NIS / kSplitWaves;                 // per wave
  static_assert(IPW >= 1 && NIS % kSplitWaves == 0, "whole instructions per wave");
  PfDmaTiles<D>* tiles = reinterpret_cast<PfDmaTiles<D>*>(lds);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = wave_id();
  const int rb = w % kPfRowBlocks, kh = w / kPfRowBlocks;
  const int H = a.num_kv_heads;
  const int rows_total = q_len * G;
  const int pos_base = len - q_len;
  const int ntiles = (k_hi - k_lo + kPfTile - 1) / kPfTile;
  const int bs_mask = (1 << a.log2_bs) - 1;
  const int64_t row_bytes = (int64_t)H * D * 2;
  const int64_t block_bytes = row_bytes << a.log2_bs;
  auto h_lo = [&](int h) { return h * ntiles / kPfKeySplit; };  // first tile of half h
  auto h_cnt = [&](int h) { return h_lo(h + 1) - h_lo(h); };
  const int nsteps = h_cnt(kPfKeySplit - 1);  // the last half has the most tiles

  // ---- this wave's rows: Q as the B operand, 8 dims per lane per MFMA -----
  const int rw0 = r0 + 32 * rb;
  const int row = min(rw0 + (lane & 31), rows_total - 1);
  const int lim = pos_base + row / G;  // last key this lane's row sees
  const int wave_first = pos_base + min(rw0, rows_total - 1) / G;
  const int wave_last = pos_base + min(rw0 + 31, rows_total - 1) / G;
  const uint16_t* qrow = (const uint16_t*)a.q +
                         ((int64_t)(q_first + row / G) * a.num_q_heads + kvh * G + row % G) * D;
  u32x4_t qf[KC];
#pragma unroll
  for (int kk = 0; kk < KC; ++kk) qf[kk] = *(const u32x4_t*)(qrow + 16 * kk + 8 * (lane >> 5));

  float m = -INFINITY, l = 0.f;  // row state (m shared by lanes l, l ^ 32; l partial)
  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // ---- the wave's loads: instructions g = IPW w + j, rows [RPI g', RPI g' + RPI)
  // of (K or V, half); with these sizes one wave always serves one (K or V, half).
  const int g0 = IPW * w;
  const bool is_v = g0 >= NIS / 2;
  const int lh = (g0 % (NIS / 2)) / (NIS / 4);  // the wave's key half
  const int key_base = (g0 % (NIS / 4)) * RPI;  // first key of its first instruction
  const int row_in = lane / CPR, pos = lane % CPR;
  const char* pool = (const char*)(is_v ? a.v_pool : a.k_pool) + (int64_t)kvh * D * 2;
  const int rot = blockIdx.x / kQueues;
  auto tile_of = [&](int h, int s) { return h_lo(h) + (s + rot) % max(h_cnt(h), 1); };
  const int tile_blocks = max(kPfTile >> a.log2_bs, 1);
  int ph[2][8];  // table entries of the half's tile, per step parity
  auto lookup = [&](int s, auto slot) {
    constexpr int sl = decltype(slot)::value;
    const int b0 = (k_lo + tile_of(lh, s) * kPfTile) >> a.log2_bs;
    const int last = min(tile_blocks, a.max_blocks - b0) - 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) ph[sl][j] = bt[b0 + min(j, last)];
  };
  auto load = [&](int s, auto slot, PfDmaTiles<D>& tl) {
    constexpr int sl = decltype(slot)::value;
    const int t0 = k_lo + tile_of(lh, s) * kPfTile;
    const int b0 = t0 >> a.log2_bs;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int key = key_base + j * RPI + row_in;  // within the tile
      const int tk = max(min(t0 + key, k_hi - 1), 0);
      const int e = min((tk >> a.log2_bs) - b0, 7);
      const int* ee = ph[sl];
      const int t_0 = e & 1 ? ee[1] : ee[0], t_1 = e & 1 ? ee[3] : ee[2];
      const int t_2 = e & 1 ? ee[5] : ee[4], t_3 = e & 1 ? ee[7] : ee[6];
      const int u_0 = e & 2 ? t_1 : t_0, u_1 = e & 2 ? t_3 : t_2;
      const int phys = min(max(e & 4 ? u_1 : u_0, 0), a.num_blocks - 1);
      const int c = is_v ? v_pos<D>(key, pos) : k_pos<D>(key, pos);
      const char* src = pool + (int64_t)phys * block_bytes +
                        (uint32_t)((tk & bs_mask) * (uint32_t)row_bytes) + c * 16;
      uint16_t* dst = is_v ? &tl.v[lh][key_base + j * RPI][0] : &tl.k[lh][key_base + j * RPI][0];
      const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(
          (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dst);
      // Written out rather than through the builtin: the compiler would treat
      // the pending LDS writes as aliasing every later LDS read and wait for
      // all of them (the next steps' rows included) before each compute.  The
      // waits are explicit instead (barrier_keep_loads, the prologue and the
      // end of the loop), and no other vector-memory access is issued in the
      // loop, so the counter holds only these loads.
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src), "s"(lds_addr)
                   : "memory", "m0");
    }
  };

  // QK of tile s into st (false: the wave has nothing to do for tile s)
  auto qk = [&](int s, const PfDmaTiles<D>& tl, f32x16_t& st) -> bool {
    if (s >= h_cnt(kh)) return false;
    const int k0 = k_lo + tile_of(kh, s) * kPfTile;
    if (k0 > wave_last) return false;  // no row of this wave sees the tile
    // ---- S^T = K Q^T ------------------------------------------------------
#pragma unroll
    for (int r2 = 0; r2 < 16; ++r2) st[r2] = 0.f;
    u32x4_t kf[KC];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int key = lane & 31;
      kf[kk] = *(const u32x4_t*)&tl.k[kh][key][k_pos<D>(key, 2 * kk + (lane >> 5)) * 8];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) st = mfma32(kf[kk], qf[kk], st);
    return true;
  };
  // softmax and PV of tile s, from its scores st
  auto softmax_pv = [&](int s, const f32x16_t& st, const PfDmaTiles<D>& tl) {
    const int k0 = k_lo + tile_of(kh, s) * kPfTile;
    // the V^T fragments (transposing reads), read while the softmax below runs
    u32x4_t vf[2][DB];
    {
      const int gq = lane >> 4, i = lane & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          uint32_t wv[4];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int key = 16 * h + 8 * r + 4 * (gq >> 1) + (i >> 2);
            const int dim = 32 * db + 16 * (gq & 1) + 4 * (i & 3);
            const uint16_t* p = &tl.v[kh][key][v_pos<D>(key, dim >> 3) * 8 + (dim & 4)];
            const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4_t __attribute__((address_space(3)))*)p);
            wv[2 * r] = (uint32_t)(uint16_t)x[0] | ((uint32_t)(uint16_t)x[1] << 16);
            wv[2 * r + 1] = (uint32_t)(uint16_t)x[2] | ((uint32_t)(uint16_t)x[3] << 16);
          }
          vf[h][db] = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- online softmax of the lane's row (log2 domain) ----------------------
    const float c = a.scale_log2;
    float x[16];
#pragma unroll
    for (int r2 = 0; r2 < 16; ++r2) x[r2] = st[r2];
    if (__builtin_amdgcn_readfirstlane((int)(k0 + kPfTile - 1 > wave_first))) {
      const int room = lim - k0 - 4 * (lane >> 5);
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2)
        x[r2] = 8 * (r2 >> 2) + (r2 & 3) <= room ? x[r2] : -INFINITY;
    }
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int r2 = 2; r2 < 16; r2 += 2) mx = fmaxf(mx, fmaxf(x[r2], x[r2 + 1]));
    mx = level_step<5>(mx, OpMax()) * c;
    const bool move = mx > m + kPfLazy;
    if (__builtin_amdgcn_readfirstlane((int)(__ballot(move) != 0))) {
      const float m_new = move ? mx : m;
      const float alpha = m_new == m ? 1.f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) o[db][r2] *= alpha;
    }
    uint32_t pk[8];
    const float mm = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int r2 = 0; r2 < 16; r2 += 2) {
      const float p0 = fast_exp2(fmaf(x[r2], c, -mm));
      const float p1 = fast_exp2(fmaf(x[r2 + 1], c, -mm));
      const bf16x2_t pb = __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t);
      pk[r2 / 2] = __builtin_bit_cast(uint32_t, pb);
      l = dot2_bf16(pk[r2 / 2], 0x3F803F80u, l);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t pf = {pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mfma32(vf[h][db], pf, o[db]);
    }
  };

  // The workgroup barrier of the loop: this wave's LDS accesses and its rows
  // of the next step (all but its last IPW loads) are complete, then every
  // wave meets.  __syncthreads would also wait for the rows just requested
  // (they are LDS writes), which would leave nothing in flight.
  auto barrier_keep_loads = [&]() {
    __builtin_amdgcn_s_waitcnt(vm_wait(IPW) & kWaitLgkmMask);
    asm volatile("s_barrier" ::: "memory");
  };
  // Step s: compute tile s from buffer s % 3; request the table entries of
  // step s + 3 and the rows of step s + 2 (into buffer (s + 2) % 3, last read
  // in step s - 1); wait for this wave's rows of step s + 1, then one barrier
  // makes every wave's rows of step s + 1 visible.  (Running the vector work
  // of key half 1 one tile behind, so that the two waves of a SIMD alternate
  // between matrix and vector work, was measured slower: 94 against 83 us
  // for the 512-token chunk.)
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  auto step = [&](int s, auto slot, int bc) {  // slot: s % 2, bc: s % 3
    using Other = std::integral_constant<int, 1 - decltype(slot)::value>;
    const PfDmaTiles<D>& cur = tiles[bc];
    f32x16_t st;
    if (qk(s, cur, st)) softmax_pv(s, st, cur);
    lookup(s + 3, Other{});
    load(s + 2, slot, tiles[(bc + 2) % kPfStages]);
    barrier_keep_loads();
  };

  lookup(0, Slot0{});
  lookup(1, Slot1{});
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the query
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  load(0, Slot0{}, tiles[0]);
  lookup(2, Slot0{});
  load(1, Slot1{}, tiles[1]);
  barrier_keep_loads();
  int bc = 0;  // s % 3
  for (int s = 0; s < nsteps; s += 2) {  // an odd count ends with an idle step
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    step(s, Slot0{}, bc);
    bc = bc == kPfStages - 1 ? 0 : bc + 1;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    step(s + 1, Slot1{}, bc);
    bc = bc == kPfStages - 1 ? 0 : bc + 1;
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the rows requested past the last step

  // ---- merge the two key halves of each row block --------------------------------
  l = level_step<5>(l, OpSum());
  float* sp = reinterpret_cast<float*>(lds) + rb * kWave * (D / 2 + 4);
  __syncthreads();  // every wave is done with the tiles
  if (kh == 1) {
    sp[lane] = m;
    sp[kWave + lane] = l;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(float4*)&sp[2 * kWave + ((db * 4 + r4) * kWave + lane) * 4] =
            make_float4(o[db][4 * r4], o[db][4 * r4 + 1], o[db][4 * r4 + 2], o[db][4 * r4 + 3]);
  }
  __syncthreads();
  if (kh == 0) {
    const float m2 = sp[lane], l2 = sp[kWave + lane];
    const float mn = fmaxf(m, m2);
    const float a1 = m == mn ? 1.f : fast_exp2(m - mn);
    const float a2 = m2 == mn ? 1.f : fast_exp2(m2 - mn);
    l = l * a1 + l2 * a2;
    const int rr = rw0 + (lane & 31);
    if (rr < rows_total) {
      const int64_t jh = (int64_t)(q_first + rr / G) * a.num_q_heads + kvh * G + rr % G;
      const float inv = 1.f / l;
      float* po = a.part_o + (jh * a.max_partitions + part) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 v = *(const float4*)&sp[2 * kWave + ((db * 4 + r4) * kWave + lane) * 4];
          *(float4*)&po[32 * db + 8 * r4 + 4 * (lane >> 5)] =
              make_float4((o[db][4 * r4] * a1 + v.x * a2) * inv,
                          (o[db][4 * r4 + 1] * a1 + v.y * a2) * inv,
                          (o[db][4 * r4 + 2] * a1 + v.z * a2) * inv,
                          (o[db][4 * r4 + 3] * a1 + v.w * a2) * inv);
        }
      if (lane < 32) a.part_lse[jh * a.max_partitions + part] = (mn + __log2f(l)) * kLn2Split;
    }
  }
}

// Inclusive-to-exclusive prefix sums of cnt[1..n] in place (cnt[0] = 0), by
// one wave.
__device__ void wave_scan(int* cnt, int n, int lane) {
  int carry = 0;
  if (lane == 0) cnt[0] = 0;
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    int x = i < n ? cnt[i + 1] : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(x, d, kWave);
      if (lane >= d) x += y;
    }
    if (i < n) cnt[i + 1] = carry + x;
    carry += __shfl(x, kWave - 1, kWave);
  }
}

// The last b with cum[b] <= t (cum in LDS, non-decreasing, cum[0] = 0 <= t).
__device__ __forceinline__ int find_seq(const int* cum, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(cum[mid]) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Prefill blocks before work block beta (of nb blocks, nbp of them prefill).
__device__ __forceinline__ int prefill_blocks_before(int beta, int nb, int nbp) {
#if PA_SPLIT_ORDER == 1
  return max(0, beta - (nb - nbp));
#else
  return (int)((int64_t)beta * nbp / nb);
#endif
}

// UNIFORM: blocks hold at least as many keys as one load instruction of the
// decode tiles covers (at least 4), so table lookups are per instruction and
// per key quad.
template <typename T, int D, int G, bool UNIFORM>
__global__ __launch_bounds__(kSplitWaves * kWave, 1) void split_kernel(
    DecodeArgs a, const int32_t* __restrict__ block_tables) {
  constexpr bool MFMA = sizeof(T) == 2 && D <= 128;
  using W = WaveCtx<T, D, G, UNIFORM>;
  __shared__ __attribute__((aligned(16))) char lds[split_lds_bytes<T, D, G, MFMA>()];
  __shared__ int item_lds;
  extern __shared__ int cum[];  // [2][num_seqs + 1]: decode units, prefill (tile, partition)s
  const int B = a.num_seqs;
  int* dcum = cum;
  int* pcum = cum + B + 1;
  const int H = a.num_kv_heads;
  const int P = a.partition_size;
  const int cap = a.max_blocks << a.log2_bs;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = wave_id();

  // ---- work queues ----------------------------------------------------------------
  // ctrl[q]: claims made on queue q (item block index); ctrl[kQueues]: finished
  // workgroups.  Thread 0 claims the next item of its current queue while the
  // workgroup runs the current one (the first claim already here, in flight
  // with the loads of the per-sequence work below).  When that queue is
  // spent, wave 0 reads every counter at once (one lane per queue) and claims
  // from the first queue after its own that still has blocks, until none has.
  int* ctrl = a.queue;
  const int home = blockIdx.x % kQueues;
  auto claim = [&](int q) {
    return __hip_atomic_fetch_add(&ctrl[q], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  int q_cur = home;
  int next = -1;  // thread 0: the claim in flight on q_cur
  if (threadIdx.x == 0) next = claim(q_cur);

  // ---- work per sequence ------------------------------------------------------------
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int q_len = a.cu_q_lens ? a.cu_q_lens[b + 1] - a.cu_q_lens[b] : 1;
    const int len = min(max(a.seq_lens[b], 0), cap);
    int du = 0, pt = 0;
    if (q_len == 1) {
      du = (len + P - 1) / P;  // decode partitions
    } else if (q_len > 1 && len > 0) {
      const int nparts = prefill_split(len, q_len) > 0 ? 2 : 1;
      if (MFMA) pt = (q_len * G + kPfRows - 1) / kPfRows * nparts;  // (row tile, partition)
      else du = q_len * nparts;  // one unit per (query token, partition)
    }
    dcum[b + 1] = du;
    pcum[b + 1] = pt;
  }
  __syncthreads();
  if (w == 0) wave_scan(dcum, B, lane);
  if (w == 1) wave_scan(pcum, B, lane);
  __syncthreads();
  const int nd_wave = __builtin_amdgcn_readfirstlane(dcum[B]) * H;  // decode wave units
  const int nd = (nd_wave + kSplitWaves - 1) / kSplitWaves;          // decode items
  const int np = __builtin_amdgcn_readfirstlane(pcum[B]) * H;         // prefill items
  const int nbd = (nd + kQueues - 1) / kQueues, nbp = (np + kQueues - 1) / kQueues;
  const int nb = nbd + nbp;  // blocks of kQueues items; queue q holds position q of each

  // ---- work queues: claims as set up above ------------------------------------------
  for (;;) {
    if (w == 0) {
      int item = -1;
      if (lane == 0 && next >= 0 && next < nb) item = next * kQueues + q_cur;
      item = __builtin_amdgcn_readfirstlane(item);
      while (item < 0) {
        // this queue is spent: find one with blocks left
        const int q = (home + 1 + lane) % kQueues;
        const int seen = lane < kQueues - 1
                             ? __hip_atomic_load(&ctrl[q], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : nb;
        const uint64_t left = __ballot(seen < nb);
        if (left == 0) break;
        q_cur = (home + 1 + __builtin_ctzll(left)) % kQueues;
        int mth = 0;
        if (lane == 0) mth = claim(q_cur);
        mth = __builtin_amdgcn_readfirstlane(mth);
        if (mth < nb) item = mth * kQueues + q_cur;
      }
      if (lane == 0) item_lds = item;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(item_lds);
    if (item < 0) break;
    q_cur = item % kQueues;
    if (threadIdx.x == 0) next = claim(q_cur);  // in flight while this item runs
    const int beta = item / kQueues, pos = item % kQueues;
    const int before = prefill_blocks_before(beta, nb, nbp);
    const bool is_prefill = prefill_blocks_before(beta + 1, nb, nbp) > before;
    if (is_prefill) {
      if constexpr (MFMA) {
        const int pi = before * kQueues + pos;
        if (pi < np) {
          const int tau = pi / H, kvh = pi % H;  // heads vary fastest: one head per queue
          const int b = find_seq(pcum, B, tau);
          const int q_first = a.cu_q_lens[b];
          const int q_len = a.cu_q_lens[b + 1] - q_first;
          const int len = min(max(a.seq_lens[b], 0), cap);
          const int hsplit = prefill_split(len, q_len);
          const int nparts = hsplit > 0 ? 2 : 1;
          const int local = tau - __builtin_amdgcn_readfirstlane(pcum[b]);
          const int r0 = (local / nparts) * kPfRows, part = local % nparts;
          const int last_row = min(r0 + kPfRows - 1, q_len * G - 1);
          const int k_end = len - q_len + last_row / G + 1;  // keys the tile's rows see
          const int k_lo = part == 1 ? hsplit : 0;
          const int k_hi = nparts == 2 && part == 0 ? hsplit : k_end;
#if PA_PF_DMA
          if constexpr (UNIFORM)
            prefill_item_dma<D, G>(a, block_tables + (int64_t)b * a.max_blocks, lds, q_first,
                                   q_len, len, r0, part, k_lo, k_hi, kvh);
          else
#endif
          prefill_item<D, G, UNIFORM>(a, block_tables + (int64_t)b * a.max_blocks, lds, q_first,
                                      q_len, len, r0, part, k_lo, k_hi, kvh);
        }
      }
    } else {
      const int di = (beta - before) * kQueues + pos;
      const int wi = di * kSplitWaves + w;
      if (di < nd && wi < nd_wave) {
        const int u = wi / H, kvh = wi % H;
        const int b = find_seq(dcum, B, u);
        const int local = u - __builtin_amdgcn_readfirstlane(dcum[b]);
        const int q_first = a.cu_q_lens ? a.cu_q_lens[b] : b;
        const int q_len = a.cu_q_lens ? a.cu_q_lens[b + 1] - q_first : 1;
        const int len = min(max(a.seq_lens[b], 0), cap);
        int j, p, start, end;
        if (q_len == 1) {  // decode partition `local`
          j = q_first;
          p = local;
          start = p * P;
          end = min(len, start + P);
        } else {  // a prefill query on the vector units: one of its partitions
          const int hsplit = prefill_split(len, q_len);
          const int nparts = hsplit > 0 ? 2 : 1;
          j = q_first + local / nparts;
          p = local % nparts;
          const int key_end = len - q_len + local / nparts + 1;
          start = p == 1 ? hsplit : 0;
          end = nparts == 2 && p == 0 ? hsplit : key_end;
        }
        if (start < end) {
          W wc(a, kvh, reinterpret_cast<uint4*>(lds) + w * W::kQChunks);
          wc.load_query(j);
          wc.reset();
          wc.run(block_tables + (int64_t)b * a.max_blocks, start, end);
          float l[G];
          wc.combine(l);
          const int64_t base = (int64_t)j * a.num_q_heads;
          wc.store_partial(
              [&](int h) { return a.part_o + ((base + h) * a.max_partitions + p) * D; },
              [&](int h) { return a.part_lse + (base + h) * a.max_partitions + p; }, l);
        }
      }
    }
    __syncthreads();  // LDS reuse and item_lds before the next claim
  }
  // The last workgroup out returns the counters to zero for the next call.
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(&ctrl[kQueues], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {
      for (int q = 0; q <= kQueues; ++q)
        __hip_atomic_store(&ctrl[q], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename T, int D, int G>
pa_status launch_split_t(const DecodeArgs& a, hipStream_t stream) {
  const bool uniform = (1 << a.log2_bs) >= Shape<T, D, G>::UKEYS;
  const void* k = uniform ? (const void*)split_kernel<T, D, G, true>
                          : (const void*)split_kernel<T, D, G, false>;
  const size_t lds = (size_t)2 * (a.num_seqs + 1) * sizeof(int);
  const int threads = kSplitWaves * kWave;
  int dev = 0, cus = 0, per_cu = 0;
  if (current_device(&dev) != PA_OK || device_cus(dev, &cus) != PA_OK ||
      resident_per_cu(dev, k, threads, lds, &per_cu) != PA_OK)
    return PA_ERR_HIP;
  if (per_cu < 1) return PA_ERR_UNSUPPORTED;
  const dim3 grid((uint32_t)(cus * per_cu));
  if (uniform)
    hipLaunchKernelGGL((split_kernel<T, D, G, true>), grid, dim3(threads), lds, stream, a,
                       a.block_tables);
  else
    hipLaunchKernelGGL((split_kernel<T, D, G, false>), grid, dim3(threads), lds, stream, a,
                       a.block_tables);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

pa_status launch_split(const DecodeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  return dispatch(a, [&]<typename T, int D, int G>() { return launch_split_t<T, D, G>(a, s); });
}

}  // namespace pa
