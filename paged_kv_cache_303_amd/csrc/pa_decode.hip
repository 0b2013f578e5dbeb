// Paged decode attention on gfx950: block-table gather, QK, online softmax,
// PV.  Three kernels share one per-wave tile machinery (WaveCtx):
//   * decode_kernel        grid of (query token, KV-head group, partition):
//                          single pass (final output) or one fixed partition
//                          per workgroup (partials for the log-sum-exp reduce)
//   * decode_stream_kernel persistent and load-balanced: every workgroup takes
//                          an equal, contiguous slice of all (sequence, tile)
//                          work, finishes the sequences that lie inside its
//                          slice and leaves (o, lse) partials for cut ones
//   * stream_fixup_kernel  merges the cut sequences' partials; zero rows for
//                          sequences without keys
//
// What it computes ("19.2 KV Cache 系统化管理" §19.2.3, paged_attention): for
// one query token, walk the request's keys in logical order through its block
// table (logical block t / block_size -> physical block, row t % block_size;
// "LLM 推理引擎的内存管理与调度" §3), and fold them into a running maximum m,
// a running sum l of exp(s - m) and a running weighted sum of values, both
// rescaled by exp(m_old - m_new) when the maximum grows; divide at the end.
// The unit folded at once is a tile of TT tokens instead of one block.
//
// Per wave (one KV head):
//   * The wave serves the G = num_q_heads/num_kv_heads query heads that share
//     its KV head, so every K/V byte is read once per KV head and used G times.
//   * Loads are 16 bytes per lane and row-contiguous: a token row of one KV
//     head is read by LPR neighbouring lanes (CPL chunks each), TPI rows per
//     load instruction, NI instructions per tile.
//   * QK: partial dot products over the lane's chunks (v_dot2_f32_bf16 for
//     bfloat16), summed over the LPR lanes of a row with DPP row operations;
//     every lane then holds the full scores of the tokens whose V chunks it
//     loaded, so PV needs no exchange.
//   * Softmax in the log2 domain, lazily rescaled; the tile maximum crosses
//     token groups with DPP / v_permlane{16,32}_swap.
//   * Software pipeline: the next tile's loads are in flight while the current
//     tile is computed.  Rows past a range's end are clamped to its last row
//     and get probability exactly 0, so NaN-poisoned tails never reach sums.
#include <map>
#include <mutex>
#include <type_traits>

#include "pa_wave.h"

namespace pa {
namespace {
using namespace wave;

// ---------------------------------------------------------------------------
// Grid kernel (single pass, one query token per sequence): blockIdx.x =
// sequence * groups + KV-head group (groups vary fastest, so the heads of one
// block are read at about the same time).
// ---------------------------------------------------------------------------
template <typename T, int D, int G, bool UNIFORM>
__global__ __launch_bounds__(kMaxWaves * kWave) void decode_kernel(
    DecodeArgs a, const int32_t* __restrict__ block_tables) {
  const int groups = a.num_kv_heads / a.waves_per_group;
  const int b = blockIdx.x / groups;
  const int kvh = (blockIdx.x % groups) * a.waves_per_group + wave_id();
  const int cap = a.max_blocks << a.log2_bs;
  const int end = min(max(a.seq_lens[b], 0), cap);  // keys 0 .. len-1
  using W = WaveCtx<T, D, G, UNIFORM>;
  __shared__ uint4 q_lds[kMaxWaves][W::kQChunks];
  W w(a, kvh, q_lds[wave_id()]);
  if (end <= 0) {
    w.store_zero(a.out, b);
    return;
  }
  w.load_query(b);
  w.reset();
  w.run(block_tables + (int64_t)b * a.max_blocks, 0, end);
  float l[G];
  w.combine(l);
  w.store_out(a.out, b, l);
}

// ---------------------------------------------------------------------------
// Balanced streaming decode (one query token per sequence).
//
// The batch's work is laid end to end -- sequence b contributes its tiles,
// tiles(b) = ceil(len_b / TT), plus a fixed restart cost (kSeqCost units) --
// and cut into R equal slices, one per workgroup slot that is resident on the
// device at once (at most one per unit); the KV-head groups of a slice are
// consecutive workgroups.  A workgroup computes the prefix sums cum[] of the
// units in LDS, walks its slice, writes the output of every sequence whose
// tiles lie wholly inside the slice, and stores (o, lse) for a sequence that
// the slice cuts: slot 0 if it is the slice's first sequence, slot 1 if it is
// its last.  stream_fixup_kernel merges the cut sequences.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t slice_start(int64_t r, int64_t T, int64_t R) {
  return r * T / R;
}

// An LDS value every lane reads at the same address, moved to a scalar register.
__device__ __forceinline__ int uniform_lds(const int* p) { return __builtin_amdgcn_readfirstlane(*p); }

// Work units of a sequence in the balanced decode's static slicing: its tiles
// plus the cost of the pipeline restart at every sequence a slice holds
// (query load, first block-table lookups and gathers, and the final
// cross-lane combine and store), a fixed number of tokens' worth of tiles:
// PA_SEQ_COST_TOKENS for bf16 and fp32 pools, PA_FP8_SEQ_COST_TOKENS for fp8.
// Per-wave timestamps on MI355X put one restart at 5-7 us.  On the batch-256
// GQA decode with 32-token tiles, 96 tokens beats 64 for bf16 (the kv_write +
// decode step 0.2845 -> 0.2825 ms, median of three pairs) while fp8 is
// fastest at 64 (0.1708 against 0.1720 ms at 96); 32 and 128 are slower for
// both.  The extra units come first: sequence b occupies units
// [cum[b], cum[b+1]), its tiles are the last tiles(b) of them, and an empty
// sequence has none.
#ifndef PA_SEQ_COST_TOKENS
#define PA_SEQ_COST_TOKENS 96
#endif
#ifndef PA_FP8_SEQ_COST_TOKENS
#define PA_FP8_SEQ_COST_TOKENS 64
#endif
// Restart cost in units of TT-token tiles.
template <typename T, int TT>
constexpr int seq_cost_tiles() {
  return ((sizeof(T) == 1 ? PA_FP8_SEQ_COST_TOKENS : PA_SEQ_COST_TOKENS) + TT - 1) / TT;
}

// Prefix sums of work units per sequence into LDS: ends[b] = len_b (clamped
// to the table's capacity), cum[b] = units of sequences 0..b-1 (TT tokens a
// tile).  Every thread loads lengths (one memory round trip), wave 0 scans.
// Ends with a workgroup barrier.
template <int TT, int kSeqCost>
__device__ void tile_prefix(const DecodeArgs& a, int* cum, int* ends) {
  const int B = a.num_seqs;
  const int cap = a.max_blocks << a.log2_bs;
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const int len = min(max(a.seq_lens[i], 0), cap);
    const int tiles = (len + TT - 1) / TT;
    ends[i] = len;
    cum[i + 1] = tiles > 0 ? tiles + kSeqCost : 0;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int carry = 0;
    if (lane == 0) cum[0] = 0;
    for (int base = 0; base < B; base += kWave) {
      const int i = base + lane;
      int x = i < B ? cum[i + 1] : 0;  // inclusive scan across the wave
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
      }
      if (i < B) cum[i + 1] = carry + x;
      carry += __shfl(x, kWave - 1, kWave);
    }
  }
  __syncthreads();
}

// The last b with cum[b] <= t (cum in LDS, non-decreasing, cum[0] = 0 <= t).
__device__ __forceinline__ int seq_of_tile(const int* cum, int B, int64_t t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uniform_lds(&cum[mid]) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The streaming kernel runs workgroups of at most kStreamWaves waves and may
// take a whole SIMD per wave (its launch bounds allow 512 VGPRs), so its
// tiles are twice as deep as the grid kernel's for bf16 and fp32: 16 KiB of
// K/V in flight per wave.  On MI355X one deep wave per SIMD beats two
// shallow ones that share it, one of which the hardware serves measurably
// slower (batch-256 GQA decode: 0.2935 -> 0.2880 ms).
constexpr int kStreamWaves = 2;
static_assert(PA_WAVES_PER_GROUP <= kStreamWaves, "stream workgroups hold at most 2 waves");
#ifndef PA_FP8_STREAM_TILE
#define PA_FP8_STREAM_TILE 32
#endif
template <typename T>
constexpr int stream_tile() {
  return sizeof(T) == 1 ? PA_FP8_STREAM_TILE : 2 * PA_TILE_TOKENS;
}

// block_tables is a separate __restrict__ argument: nothing the kernel stores
// can alias it, so its wave-uniform lookups stay scalar loads after stores.
template <typename T, int D, int G, bool UNIFORM>
__global__ __launch_bounds__(kStreamWaves * kWave, 1) void decode_stream_kernel(
    DecodeArgs a, StreamArgs s, const int32_t* __restrict__ block_tables) {
  using W = WaveCtx<T, D, G, UNIFORM, stream_tile<T>()>;
  constexpr int TT = W::TT;
  extern __shared__ int lds[];
  const int B = a.num_seqs;
  int* cum = lds;            // [B + 1]
  int* ends = lds + B + 1;   // [B]
  const int groups = a.num_kv_heads / a.waves_per_group;
  const int r = blockIdx.x / groups;
  const int kvh = (blockIdx.x % groups) * a.waves_per_group + wave_id();

  constexpr int kSeqCost = seq_cost_tiles<T, TT>();
  tile_prefix<TT, kSeqCost>(a, cum, ends);
  const int64_t total = uniform_lds(&cum[B]);
  // slices actually used: at most one per tile, so none is empty
  const int64_t R = min((int64_t)s.num_slices, total);
  if (blockIdx.x == 0) {
    // for the merge kernel, per sequence: the slices holding its first and
    // last tile (the largest r with slice_start(r) <= t), and whether the
    // first of them begins before the sequence's units, i.e. with tiles of
    // an earlier sequence (partial slot 1)
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
      const int64_t u0 = cum[i], u1 = cum[i + 1];
      int4 v = make_int4(-1, -1, 0, 0);
      if (u0 < u1) {
        const int64_t first = u0 + kSeqCost;  // unit of the first tile
        const int64_t r1 = ((first + 1) * R - 1) / total;
        const int64_t r2 = (u1 * R - 1) / total;
        v = make_int4((int)r1, (int)r2, slice_start(r1, total, R) < u0 ? 1 : 0, 0);
      }
      ((int4*)s.seq_slices)[i] = v;
    }
  }
  if (r >= R) return;
  const int64_t t_begin = slice_start(r, total, R);
  const int64_t t_end = slice_start(r + 1, total, R);

  const int b_first = seq_of_tile(cum, B, t_begin);  // first sequence of the slice

  __shared__ uint4 q_lds[kMaxWaves][W::kQChunks];
  W w(a, kvh, q_lds[wave_id()]);
  for (int b = b_first; b < B; ++b) {
    const int c_lo = uniform_lds(&cum[b]);
    const int c_hi = uniform_lds(&cum[b + 1]);
    const int t_lo = c_hi > c_lo ? c_lo + kSeqCost : c_lo;  // unit of the first tile
    const int64_t seg_lo = max(t_begin, (int64_t)t_lo);
    const int64_t seg_hi = min(t_end, (int64_t)c_hi);
    if (seg_lo < seg_hi) {
      const int start = (int)(seg_lo - t_lo) * TT;
      const int stop = min(uniform_lds(&ends[b]), (int)(seg_hi - t_lo) * TT);
      w.load_query(b);
      w.reset();
      w.run(block_tables + (int64_t)b * a.max_blocks, start, stop);
      float l[G];
      w.combine(l);
      if (seg_lo == t_lo && seg_hi == c_hi) {
        w.store_out(a.out, b, l);
      } else {
        const int slot = (b == b_first) ? 0 : 1;
        const int64_t base = ((int64_t)r * 2 + slot) * a.num_q_heads;
        w.store_partial([&](int h) { return s.part_o + (base + h) * D; },
                        [&](int h) { return s.part_lse + base + h; }, l);
      }
    }
    if (c_hi >= t_end) break;
  }
}

// Merge the partials of every sequence cut by slice boundaries; zero rows for
// sequences without keys.  One wave per (sequence, head), kFixupWaves heads
// per workgroup.  The sequence's slice range comes precomputed from the
// streaming kernel, so the partial rows of its first kPre slices are loaded
// together with the lse values (one memory round trip); lane k handles the
// k-th slice's weight, every lane its columns of the weighted sum.
constexpr int kFixupWaves = 4;
constexpr int kPre = 8;

__global__ __launch_bounds__(kFixupWaves * kWave) void stream_fixup_kernel(DecodeArgs a,
                                                                          StreamArgs s) {
  const int b = blockIdx.x;
  const int h = blockIdx.y * kFixupWaves + wave_id();
  if (h >= a.num_q_heads) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int D = a.head_dim;
  const bool bf16 = a.dtype != PA_F32;  // bf16 output for bf16 and fp8 pools
  const int64_t row = (int64_t)b * a.num_q_heads + h;
  const int4 sv = ((const int4*)s.seq_slices)[b];
  const int r1 = __builtin_amdgcn_readfirstlane(sv.x);
  const int r2 = __builtin_amdgcn_readfirstlane(sv.y);
  const bool first_cut = __builtin_amdgcn_readfirstlane(sv.z) != 0;
  if (r1 < 0) {  // no key: zero row
    for (int d = lane; d < D; d += kWave) {
      if (bf16) ((uint16_t*)a.out)[row * D + d] = 0;
      else ((float*)a.out)[row * D + d] = 0.f;
    }
    return;
  }
  if (r1 == r2) return;  // wholly inside one slice: already written
  const int nseg = r2 - r1 + 1;
  // partial row of slice r1 + k (slot 1 if the slice began with an earlier sequence)
  auto seg_index = [&](int k) -> int {
    const int slot = (k == 0 && first_cut) ? 1 : 0;
    return ((r1 + k) * 2 + slot) * a.num_q_heads + h;
  };
  // rows of the first kPre slices (slices past the sequence re-read slice 0's
  // row and get weight 0 below)
  float pre[kPre][4];
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    const float* po = s.part_o + (int64_t)seg_index(q < nseg ? q : 0) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) pre[q][i] = lane + i * kWave < D ? po[lane + i * kWave] : 0.f;
  }
  float m = -INFINITY;
  for (int k = lane; k < nseg; k += kWave) m = fmaxf(m, s.part_lse[seg_index(k)]);
  m = reduce_levels<0, 6>(m, OpMax());
  float den = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};  // dims lane + 64 * i
  for (int k0 = 0; k0 < nseg; k0 += kWave) {
    const int k = k0 + lane;
    const bool valid = k < nseg;
    const int idx = seg_index(valid ? k : 0);
    const float wgt = valid ? __expf(s.part_lse[idx] - m) : 0.f;
    den += wgt;
    const int n = min(kWave, nseg - k0);
    int q0 = 0;
    if (k0 == 0) {  // the preloaded rows (weight 0 past the sequence)
#pragma unroll
      for (int q = 0; q < kPre; ++q) {
        const float wq = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wgt), q));
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = fmaf(wq, pre[q][i], o[i]);
      }
      q0 = kPre;
    }
    // the rest, four slices at a time so that their rows load together;
    // slots past the sequence read row 0 and select the value away
    for (; q0 < n; q0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u;  // <= 63: n <= 64 and q0 is a multiple of 4
        const bool used = q < n;
        const float wq = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wgt), q));
        const int iq = __builtin_amdgcn_readlane(idx, q);
        const float* po = s.part_o + (int64_t)(used ? iq : 0) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (lane + i * kWave < D) {
            const float x = po[lane + i * kWave];
            o[i] = used ? fmaf(wq, x, o[i]) : o[i];
          }
      }
    }
  }
  den = reduce_levels<0, 6>(den, OpSum());
  const float inv = 1.f / den;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + i * kWave;
    if (d < D) {
      if (bf16) ((__bf16*)a.out)[row * D + d] = (__bf16)(o[i] * inv);
      else ((float*)a.out)[row * D + d] = o[i] * inv;
    }
  }
}

// Keys a block must hold for the UNIFORM kernels.
template <typename T, int D, int G>
constexpr int tpi() {
  return Shape<T, D, G>::UKEYS;
}

template <typename T, int D, int G>
pa_status launch_grid(const DecodeArgs& a, hipStream_t stream) {
  const int groups = a.num_kv_heads / a.waves_per_group;
  const dim3 grid((uint32_t)((int64_t)a.num_seqs * groups));
  const dim3 block(a.waves_per_group * kWave);
  if ((1 << a.log2_bs) >= tpi<T, D, G>())
    hipLaunchKernelGGL((decode_kernel<T, D, G, true>), grid, block, 0, stream, a,
                       a.block_tables);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, G, false>), grid, block, 0, stream, a,
                       a.block_tables);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <typename T, int D, int G>
pa_status stream_per_cu(const DecodeArgs& a, int dev, int* per_cu) {
  const size_t lds = stream_lds_bytes(a.num_seqs);
  const int threads = a.waves_per_group * kWave;
  const void* k = (1 << a.log2_bs) >= tpi<T, D, G>()
                      ? (const void*)decode_stream_kernel<T, D, G, true>
                      : (const void*)decode_stream_kernel<T, D, G, false>;
  return resident_per_cu(dev, k, threads, lds, per_cu);
}

template <typename T, int D, int G>
pa_status launch_stream(const DecodeArgs& a, const StreamArgs& s, hipStream_t stream) {
  const int groups = a.num_kv_heads / a.waves_per_group;
  const dim3 grid((uint32_t)((int64_t)s.num_slices * groups));
  const dim3 block(a.waves_per_group * kWave);
  const size_t lds = stream_lds_bytes(a.num_seqs);
  if ((1 << a.log2_bs) >= tpi<T, D, G>())
    hipLaunchKernelGGL((decode_stream_kernel<T, D, G, true>), grid, block, lds, stream, a, s,
                       a.block_tables);
  else
    hipLaunchKernelGGL((decode_stream_kernel<T, D, G, false>), grid, block, lds, stream, a, s,
                       a.block_tables);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  const dim3 fgrid(a.num_seqs, (a.num_q_heads + kFixupWaves - 1) / kFixupWaves);
  hipLaunchKernelGGL(stream_fixup_kernel, fgrid, dim3(kFixupWaves * kWave), 0, stream, a, s);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

size_t stream_lds_bytes(int32_t num_seqs) { return (size_t)(2 * num_seqs + 1) * sizeof(int); }

// Scratch of pa_decode_noalloc: the balanced decode's workspace (partial rows,
// partial lse values, per-sequence slice records) in a library-owned array,
// one copy per device, held until the process ends.  Nothing in it has to
// start at zero: the streaming kernel writes every entry the merge reads.
// In host code `scratch` only names the symbol; its device address on the
// current device comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) char scratch[kScratchBytes];

pa_status scratch_buffer(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> by_device;
  int dev = 0;
  if (current_device(&dev) != PA_OK) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_device.find(dev);
  if (it == by_device.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    it = by_device.emplace(dev, p).first;
  }
  *ptr = it->second;
  return PA_OK;
}

pa_status launch_decode(const DecodeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  return dispatch(a, [&]<typename T, int D, int G>() { return launch_grid<T, D, G>(a, s); });
}

pa_status stream_slices(const DecodeArgs& a, int32_t* num_slices) {
  int dev = 0, cus = 0, per_cu = 0;
  if (current_device(&dev) != PA_OK || device_cus(dev, &cus) != PA_OK) return PA_ERR_HIP;
  const pa_status st = dispatch(
      a, [&]<typename T, int D, int G>() { return stream_per_cu<T, D, G>(a, dev, &per_cu); });
  if (st != PA_OK) return st;
  if (per_cu < 1) return PA_ERR_UNSUPPORTED;
  // slices = workgroups resident at once, shared out among the KV-head groups
  const int groups = a.num_kv_heads / a.waves_per_group;
  const int64_t n = (int64_t)per_cu * cus / groups;
  *num_slices = (int32_t)(n < 1 ? 1 : n);
  return PA_OK;
}

pa_status launch_decode_stream(const DecodeArgs& a, const StreamArgs& sa, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  return dispatch(a, [&]<typename T, int D, int G>() { return launch_stream<T, D, G>(a, sa, s); });
}

}  // namespace pa
