// Pooled key/value index and block selection for block-sparse prefill
// ("Porting FlashPrefill V2 to Apple silicon for faster prefill", Part I:
// Compress keys before the heavy work; A cheap map of where the attention
// lives; The algorithm starts here).
//
// Both kernels reproduce a fixed fp64 evaluation order so that their outputs
// are bit-identical to a sequential reference:
//   pooled mean  = fp32( (((0 + k_t0) + k_t0+1) + ...) / n )     keys in increasing order
//   pooled score = ((0 + q_0 kbar_0) + q_1 kbar_1) + ...            dims in increasing order
// Every product of a bf16 and an fp32 value is exact in fp64, so fma and
// mul+add give the same bits.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"

namespace pa {

// ---------------------------------------------------------------------------
// build_pooled_index: one lane owns 8 adjacent columns (of the n_kv*d columns
// of a token row) of one key block, and walks the block's tokens in order.
// A wave reads 64 x 16 contiguous bytes per token: coalesced, HBM-bound.
// grid = (ceil(cols8 / 64), blocks b_first .. nb-1, 2 [K, V]), block = 64. The
// pooled arrays hold pool_ld block rows per KV head.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) pool_kernel(const uint16_t* __restrict__ K,
                                                  const uint16_t* __restrict__ V, int T,
                                                  int cols8, int d, int block, int b_first,
                                                  int pool_ld, float* __restrict__ Kp,
                                                  float* __restrict__ Vp) {
  const int c8 = blockIdx.x * 64 + threadIdx.x;
  if (c8 >= cols8) return;
  const int b = b_first + (int)blockIdx.y;
  const uint16_t* X = blockIdx.z ? V : K;
  float* P = blockIdx.z ? Vp : Kp;
  const int t0 = b * block;
  const int t1 = min(t0 + block, T);
  const u32x4* src = reinterpret_cast<const u32x4*>(X) + (size_t)t0 * cols8 + c8;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  const int n = t1 - t0;
  int t = 0;
  for (; t + 8 <= n; t += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + (size_t)(t + u) * cols8);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += (double)__uint_as_float(v[u][w] << 16);
        acc[2 * w + 1] += (double)__uint_as_float(v[u][w] & 0xFFFF0000u);
      }
    }
  }
  for (; t < n; ++t) {
    u32x4 v = src[(size_t)t * cols8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += (double)__uint_as_float(v[w] << 16);
      acc[2 * w + 1] += (double)__uint_as_float(v[w] & 0xFFFF0000u);
    }
  }
  const double dn = (double)n;
  const int col = c8 * 8;
  const int g = col / d, dd = col % d;
  float out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (float)(acc[e] / dn);
  float4* dst = reinterpret_cast<float4*>(P + ((size_t)g * pool_ld + b) * d + dd);
  dst[0] = make_float4(out[0], out[1], out[2], out[3]);
  dst[1] = make_float4(out[4], out[5], out[6], out[7]);
}

hipError_t launch_pool(const uint16_t* K, const uint16_t* V, int T, int n_kv, int d, int block,
                       int b_first, float* K_pool, float* V_pool, int pool_ld, hipStream_t stream) {
  const int cols8 = n_kv * d / 8;
  const int nb = (T + block - 1) / block;
  if (b_first >= nb) return hipSuccess;   // nothing new to pool
  dim3 grid((cols8 + 63) / 64, nb - b_first, 2);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(64), 0, stream, K, V, T, cols8, d, block, b_first,
                     pool_ld, K_pool, V_pool);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// select_blocks: one workgroup of 4 waves per (KV head g, query block j), or
// several sharing its voter tiles when the pairs are too few to fill the chip
// (their votes are merged by select_merge_kernel; see launch_select). A voter
// tile is 256 voters (64 per wave): the 128 rows x 4 query heads of a block at
// B = 128 in two tiles. Two workgroups share a CU (80 KB of LDS each), so one
// stages and waits on its loads while the other scores. Candidates are staged into LDS as fp16 in chunks of 256
// (head dim 128) or 512 (64); when all of a block's candidates fit in one chunk
// they are staged once and serve both passes of every voter tile.
//
// Voters are the (row, query head) pairs of block j in this chunk; candidates
// are the blocks b < j. The result must equal the fixed-order fp64 rule
//   vote(i, b)  <=>  fl64(r_ib - M_i) > theta,  M_i = max_b r_ib,
// for every voter, bit for bit. Evaluating every r_ib in fp64 costs 2 d flops
// per pair on the fp64 vector units; instead the kernel
//
//  1. filters on the fp16 matrix cores: k' = fp16(kbar), q' = fp16(q) (round
//     to nearest even, subnormals kept: both checked on the device), and
//     r'_ib = q'_i.k'_b accumulated in fp32 by v_mfma_f32_32x32x16_f16 (fp16
//     products are exact in fp32). A bf16 q in fp16's normal range converts
//     exactly; below it, and for kbar, each element moves by at most
//     2^-11 |x| + 2^-25. With A = sum_d |q_d||kbar_d| <= |q|_2 |kbar|_2
//     (Cauchy-Schwarz):
//        conversions: <= 2^-11 A + 2^-25 sqrt(d) (|q| + |kbar|) (1 + 2^-11)
//        fp32 accumulation of d+1 terms in any order, each step rounding by
//        at most 2^-23 (also covers truncating adders): <= gamma_129 (1+2^-11) A
//        the fp64 reference itself: <= 128 * 2^-53 A
//     so |r' - r64| <= 5.04e-4 A + 3.4e-7 (|q| + |kbar|). The kernel takes
//     E = 6e-4 max|q| max|kbar| + 1e-6 (max|q| + max|kbar| + 1) over the
//     wave's voters and the candidates (the margin absorbs the fp32 norms and
//     comparisons). Then |(r' - M') - (r - M)| <= 2E, so a pair whose filtered
//     gap lies more than 2E (+ 2^-22 |theta|) from theta is decided;
//  2. lists the other pairs as ambiguous, and every pair whose filtered score
//     lies within 2E of its voter's filtered max (near-max pairs): the exact
//     max M_i is attained at one of those;
//  3. re-evaluates in fp64 in the reference order the near-max pairs of the
//     voters with ambiguous pairs (their max gives M_i exactly) and the
//     ambiguous pairs, in one round, one pair per thread as a sequential fp64
//     fma chain over d; then each ambiguous pair is tested against theta.
// If a list overflows, or magnitudes leave the range where the bound holds
// (|q| or |kbar| above 65504, where fp16 would overflow), the voter tile is redone exactly
// in fp64 for all pairs. alpha = 0 (theta = -inf) keeps every visible block.
// Votes are ORed into a per-block bit mask in LDS, compacted in ascending
// order, and the diagonal block appended.
//
// MFMA orientation: A = kbar (32 candidates x 16 dims, LDS), B = Q^T (16 dims x
// 32 voters, registers). Accumulator element i of lane l is candidate
// 8(i/4) + 4(l/32) + i%4 against voter l%32, so a voter's max lives in lanes l
// and l^32; a lane's vote bits for its 16 candidates are ORed over the 32
// voters of each half-wave with DPP row operations.
// ---------------------------------------------------------------------------
constexpr int SEL_WAVES = 8;
constexpr int SEL_NG = 1;                // groups of 32 voters per wave
constexpr int SEL_VW = 32 * SEL_NG;      // voters per wave
constexpr int SEL_THREADS = SEL_WAVES * 64;
constexpr int SEL_VT = SEL_WAVES * SEL_VW;   // voters per tile
constexpr int SEL_WPE = 8 / SEL_NG / 2;  // waves per SIMD: two workgroups per CU
constexpr int SEL_MAX_NB = 8192;
constexpr int SEL_AMB_CAP = 1536;        // ambiguous pairs per voter tile (the fp16 band at 1K candidates)
constexpr int SEL_JOB_CAP = 512;         // exact max evaluations per voter tile
constexpr int SEL_P2G = 4;               // pass 2: slices of 32 candidates per list flush
constexpr int SEL_NEAR_W = 2 * SEL_VW;   // near-max pairs per wave and voter tile (at least one per voter)
// candidates per LDS chunk: 64 KB of fp16 rows
template <int D> struct SelGeo { static constexpr int CH = 32768 / D; };
constexpr float SEL_ERR = 6.0e-4f;
constexpr float SEL_ABS = 1.0e-6f;
constexpr float SEL_MAG = 65504.f;   // largest finite fp16

// Staged candidates in LDS: D/64 parts of [CH rows][64 dims] (rows of 128 bytes;
// dims 64p .. 64p+63 in part p), the 16-byte chunk c of row r at chunk position
// c ^ sel_swz(r). An MFMA operand read takes one chunk of 16 consecutive rows per
// 256-byte group of lanes; with two rows per 256-byte bank line of the 64-bank LDS,
// the swizzle gives the 8 even and the 8 odd rows distinct bank groups.
__device__ __forceinline__ int sel_swz(int row) { return (row >> 1) & 7; }

// halves offset of chunk c of candidate row r in the staged array
template <int D>
__device__ __forceinline__ int sel_pos(int r, int c) {
  return (c >> 3) * (SelGeo<D>::CH * 64) + r * 64 + (((c & 7) ^ sel_swz(r)) * 8);
}

// Workgroup barrier after this wave's LDS writes have completed, leaving its
// global loads in flight (the query loads of the voter tile keep arriving while
// the staged candidates are published).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A 16-byte load through a buffer resource over base[0 .. range): offsets at or
// past the range read as zeros without touching memory. (Kept outside the
// templates: hipcc's host pass drops kernel stubs when the buffer-resource type
// appears inside templated device code.)
__device__ __forceinline__ u32x4 buffer_load16(const void* base, uint32_t range, uint32_t voff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, range, 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// The thread id, opaque to the optimiser: addresses derived from it where the
// scoring loops are not are formed afresh there rather than held in registers
// through those loops.
__device__ __forceinline__ int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// All ones if the wave-uniform x is non-zero, else 0, on the scalar unit (a
// plain C++ test of the upper half of a 64-bit ballot becomes a 64-bit vector
// compare)
__device__ __forceinline__ uint32_t ones_if_nonzero(uint32_t x) {
  uint32_t r;
  asm("s_cmp_lg_u32 %1, 0\n\ts_cselect_b32 %0, -1, 0" : "=s"(r) : "s"(x) : "scc");
  return r;
}

// r = q.kbar in fp64, dims in increasing order (each product is exact in fp64)
template <int D>
__device__ __forceinline__ double dot_exact(const uint16_t* __restrict__ q, const float* __restrict__ kb) {
  double acc = 0.0;
#pragma unroll 1
  for (int d0 = 0; d0 < D; d0 += 8) {
    const u32x4 qv = *reinterpret_cast<const u32x4*>(q + d0);
    const float4 k0 = *reinterpret_cast<const float4*>(kb + d0);
    const float4 k1 = *reinterpret_cast<const float4*>(kb + d0 + 4);
    const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fma((double)__uint_as_float(qv[w] << 16), (double)kv[2 * w], acc);
      acc = __builtin_fma((double)__uint_as_float(qv[w] & 0xFFFF0000u), (double)kv[2 * w + 1], acc);
    }
  }
  return acc;
}

// bits of positions [a, b) inside the 32-position word starting at lo
__device__ __forceinline__ uint32_t range_bits(int lo, int a, int b) {
  const int s0 = max(a - lo, 0), e0 = min(b - lo, 32);
  if (s0 >= e0) return 0u;
  const uint32_t upto = e0 == 32 ? 0xFFFFFFFFu : ((1u << e0) - 1u);
  return upto & ~((1u << s0) - 1u);
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}

// order-preserving map of doubles to unsigned integers (for an LDS atomic max)
__device__ __forceinline__ unsigned long long dkey(double x) {
  const unsigned long long b = __double_as_longlong(x);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}
__device__ __forceinline__ double dval(unsigned long long k) {
  return __longlong_as_double((k >> 63) ? (k & ~(1ull << 63)) : ~k);
}

// Selection path counters of this device (pa_select_path_counts): voter tiles
// scored; tiles whose ambiguous pairs were listed once and decided in fp64;
// tiles relisted group by group (pass 2); tiles decided in fp64 pair by pair.
__device__ unsigned long long g_sel_paths[4];

template <int D>
struct SelShared {
  struct {
    uint16_t kh[SelGeo<D>::CH * D];   // fp16 candidates (layout: sel_pos)
  } k;
  unsigned long long mxkey[SEL_VT];        // exact max (as dkey) of voters with ambiguous pairs
  uint32_t amb[SEL_AMB_CAP];               // (voter << 16) | block
  uint32_t jobs[SEL_JOB_CAP];              // pairs whose exact score enters a max
  uint32_t nearl[SEL_WAVES * SEL_NEAR_W];  // near-max pairs, (voter << 16) | block, a part per wave
  uint32_t ncnt[SEL_WAVES];                // entries in each wave's part
  uint32_t flagw[SEL_MAX_NB / 32];
  uint32_t wsum[SEL_WAVES];
  uint8_t va[SEL_VT];                      // voter has ambiguous pairs
  float red[SEL_WAVES];
  uint32_t amb_cnt, job_cnt;
  uint32_t overflow;
  // pass 2 only, last (the fields above keep their offsets)
  uint32_t pcnt[2];                        // list counts, alternating by slice group
  float2 thr[SEL_VT];                      // per voter (tA, tY) of pass 1
};

// r = q.kbar in fp64, dims in increasing order, with each quarter of both rows
// loaded before its fmas (four rounds of loads in flight instead of sixteen)
template <int D>
__device__ __forceinline__ double dot_exact_prefetched(const uint16_t* __restrict__ q,
                                                       const float* __restrict__ kb) {
  constexpr int H = D / 4;
  double acc = 0.0;
#pragma unroll 1
  for (int h = 0; h < 4; ++h) {
    u32x4 qv[H / 8];
    float4 kv[H / 4];
#pragma unroll
    for (int c = 0; c < H / 8; ++c) qv[c] = *reinterpret_cast<const u32x4*>(q + h * H + 8 * c);
#pragma unroll
    for (int c = 0; c < H / 4; ++c) kv[c] = *reinterpret_cast<const float4*>(kb + h * H + 4 * c);
#pragma unroll
    for (int c = 0; c < H / 8; ++c) {
      const float k8[8] = {kv[2 * c].x, kv[2 * c].y, kv[2 * c].z, kv[2 * c].w,
                           kv[2 * c + 1].x, kv[2 * c + 1].y, kv[2 * c + 1].z, kv[2 * c + 1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = __builtin_fma((double)__uint_as_float(qv[c][w] << 16), (double)k8[2 * w], acc);
        acc = __builtin_fma((double)__uint_as_float(qv[c][w] & 0xFFFF0000u), (double)k8[2 * w + 1], acc);
      }
    }
  }
  return acc;
}

// Exact fp64 scores of the listed pairs, one pair per thread: the max jobs
// (jobs[0 .. njob), whose results raise their voters' exact max) and the
// ambiguous pairs (amb[0 .. namb)), each of which votes if its exact score
// clears theta against its voter's exact max once every job has landed (in one
// round when the two lists fit the workgroup's threads, else jobs first).
template <int D>
__device__ __forceinline__ void exact_pairs(SelShared<D>& S, int njob, int namb, const uint16_t* qg,
                                            int group, int n_q, int vt0, const float* kg, double theta) {
  auto score = [&](uint32_t pr) {
    const int v = vt0 + (int)(pr >> 16), b = (int)(pr & 0xFFFFu);
    return dot_exact_prefetched<D>(qg + ((size_t)(v / group) * n_q + (v % group)) * D, kg + (size_t)b * D);
  };
  if (njob + namb <= SEL_THREADS) {
    // one pair per thread: every score in one round, the ambiguous ones held in
    // a register across the barrier that completes the maxima
    const int e = fresh_tid();
    const bool has = e < njob + namb;
    const uint32_t pr = has ? (e < njob ? S.jobs[e] : S.amb[e - njob]) : 0u;
    const double r = has ? score(pr) : 0.0;
    if (has && e < njob) atomicMax(&S.mxkey[pr >> 16], dkey(r));
    __syncthreads();
    const int b = (int)(pr & 0xFFFFu);
    if (has && e >= njob && r - dval(S.mxkey[pr >> 16]) > theta) atomicOr(&S.flagw[b >> 5], 1u << (b & 31));
    return;
  }
  for (int e = fresh_tid(); e < njob; e += SEL_THREADS) {
    const uint32_t pr = S.jobs[e];
    atomicMax(&S.mxkey[pr >> 16], dkey(score(pr)));
  }
  __syncthreads();
  for (int e = fresh_tid(); e < namb; e += SEL_THREADS) {
    const uint32_t pr = S.amb[e];
    const int b = (int)(pr & 0xFFFFu);
    if (score(pr) - dval(S.mxkey[pr >> 16]) > theta) atomicOr(&S.flagw[b >> 5], 1u << (b & 31));
  }
}

// max(m, x[0..15])
__device__ __forceinline__ float slice_max(float m, const float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 16; i += 2) m = __builtin_fmaxf(m, __builtin_fmaxf(x[i], x[i + 1]));
  return m;
}

// OR of x over each half-wave: lane 31 returns the OR of lanes 0..31, lane 63 that
// of lanes 32..63 (prefix ORs within rows of 16 by row shifts, then row 0's and
// row 2's totals broadcast into rows 1 and 3)
__device__ __forceinline__ uint32_t or_half_waves(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  return x;
}

// The end of a selection: flagw holds the voted candidates of query block j
// (nc = j candidates, nw words). Adds the blocks kept by rule, then writes the
// ascending list with the diagonal j last, its count, and zeros to nb. Called by
// every thread of a SEL_THREADS workgroup after a barrier.
__device__ void finish_selection(uint32_t* flagw, uint32_t* wsum, int nb, int nc, int jj, int j,
                                 int n_qblk, int sink_blocks, int window_blocks,
                                 int dense_tail_blocks, int32_t* out, int32_t* cnt_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (nc + 31) >> 5;
  // kept by rule: sink blocks, a local window below the diagonal, and every
  // visible block for the call's last query blocks
  if (sink_blocks > 0 || window_blocks > 0 || dense_tail_blocks > 0) {
    const bool tail = jj > n_qblk - 1 - dense_tail_blocks;
    const int s_end = tail ? nc : min(sink_blocks, nc);
    const int w_beg = max(0, nc - window_blocks);
    for (int i = tid; i < nw; i += SEL_THREADS)
      flagw[i] |= range_bits(i * 32, 0, s_end) | range_bits(i * 32, w_beg, nc);
    __syncthreads();
  }
  // ascending compaction: thread t owns flag word t (nc <= 8191 -> at most 256 words)
  const uint32_t word = tid < nw ? flagw[tid] : 0u;
  const uint32_t cnt = __popc(word);
  uint32_t incl = cnt;  // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total_u = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const uint32_t c = wsum[w];
    before += w < wave ? c : 0u;
    total_u += c;
  }
  int pos = (int)(before + incl - cnt);
  for (uint32_t w = word; w != 0; w &= w - 1) out[pos++] = tid * 32 + __builtin_ctz(w);
  const int total = (int)total_u;
  if (tid == 0) {
    out[total] = j;  // the local diagonal block is always kept
    *cnt_out = total + 1;
  }
  for (int b = total + 1 + tid; b < nb; b += SEL_THREADS) out[b] = 0;
}

template <int D>
// 4 waves, one per SIMD, two workgroups per CU (two waves per SIMD: up to 256
// registers; the LDS holds a 64 KB candidate chunk per workgroup). Each wave
// scores 64 voters: two groups of 32, so every candidate fragment read from LDS
// feeds two MFMA chains.
__global__ void __launch_bounds__(SEL_THREADS) __attribute__((amdgpu_waves_per_eu(SEL_WPE, SEL_WPE))) select_kernel(
    const uint16_t* __restrict__ Q, int C, int q_start, int n_q, int n_kv,
    const float* __restrict__ Kp, int pool_ld, int nb, int block, double theta, float theta_f,
    float theta_slack,
    int exact_only, int n_qblk, int sink_blocks, int window_blocks, int dense_tail_blocks,
    int n_split, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt) {
  constexpr int NST = D / 16;                 // MFMA k-steps
  constexpr int CH = SelGeo<D>::CH;           // candidates per LDS chunk
  constexpr int UPR = D / 16;                 // 16-dim staging units per candidate row
  constexpr int SR = CH * UPR / SEL_THREADS;  // staging rounds per chunk
  __shared__ __attribute__((aligned(16))) SelShared<D> S;

  // heaviest query blocks first, KV heads interleaved; n_split workgroups share a
  // (KV head, query block), workgroup s taking voter tiles s, s + n_split, ...
  const int per = n_kv * n_split;
  const int jj = n_qblk - 1 - (int)blockIdx.x / per;
  const int g = (int)blockIdx.x % n_kv;
  const int sp = ((int)blockIdx.x % per) / n_kv;
  const int j = q_start / block + jj;
  const int group = n_q / n_kv;
  const int nc = j;  // candidates 0..j-1
  const int r0 = max(j * block, q_start) - q_start;
  const int r1 = min((j + 1) * block, q_start + C) - q_start;
  const int nv = (r1 - r0) * group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int nw = (nc + 31) >> 5;

  for (int i = tid; i < nw; i += SEL_THREADS) S.flagw[i] = 0;
  const float* kg = Kp + (size_t)g * pool_ld * D;
  const uint16_t* qg = Q + ((size_t)r0 * n_q + (size_t)g * group) * D;
  auto qptr = [&](int v) { return qg + ((size_t)(v / group) * n_q + (v % group)) * D; };

  if (nc > 0 && theta_f == -__builtin_inff()) {
    // alpha = 0: every fully visible block is kept
    for (int i = tid; i < nw; i += SEL_THREADS)
      S.flagw[i] = (i < (nc >> 5)) ? 0xFFFFFFFFu : ((1u << (nc & 31)) - 1u);
  } else if (nc > 0) {
    float mnorm = 0.f;  // max_b |kbar_b|_2 over the candidates (set in the first tile's pass 0)
    const bool resident = nc <= CH;   // every candidate fits in one chunk: stage once
    bool staged = false;              // the LDS chunk holds candidates 0 .. nc-1
    for (int vt0 = sp * SEL_VT; vt0 < nv; vt0 += n_split * SEL_VT) {
      __syncthreads();  // previous tile's readers of the shared state are done
      for (int i = fresh_tid(); i < SEL_VT; i += SEL_THREADS) { S.va[i] = 0; S.mxkey[i] = 0; }
      if (tid == 0) { S.amb_cnt = 0; S.job_cnt = 0; S.pcnt[0] = 0; S.pcnt[1] = 0; S.overflow = exact_only; }

      // B operands: q of the wave's SEL_NG groups of 32 voters (voter = lane % 32),
      // held for the whole tile; voter index in the tile vl = SEL_VW wave + 32 gi + col.
      // Loaded as bf16, converted to fp16 in place once the candidates are staged
      // (the norms |q| are formed at the end of pass 0, where the error bound needs them)
      u32x4 qf[SEL_NG][NST];
      bool vok[SEL_NG];
      auto load_q = [&]() {
        // lane-derived values formed afresh here, not held through the passes
        const int t = fresh_tid();
        const int wv = t >> 6, cl = t & 31, hf = (t >> 5) & 1;
#pragma unroll
        for (int gi = 0; gi < SEL_NG; ++gi) {
          const int vl = wv * SEL_VW + gi * 32 + cl;
          vok[gi] = vt0 + vl < nv;
          const uint16_t* qp = vok[gi] ? qptr(vt0 + vl) : Q;
#pragma unroll
          for (int st = 0; st < NST; ++st) {
            // loaded unconditionally (a missing voter reads row 0) and zeroed by a
            // select: no branch, so the loads queue without forcing waits
            u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 16 * st + 8 * hf);
            if (!vok[gi]) raw = u32x4{0u, 0u, 0u, 0u};
            qf[gi][st] = raw;
          }
        }
      };
      auto q_to_f16 = [&]() {
#pragma unroll
        for (int gi = 0; gi < SEL_NG; ++gi)
#pragma unroll
          for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int w = 0; w < 4; ++w)
              qf[gi][st][w] = pack_f16x2(__uint_as_float(qf[gi][st][w] << 16),
                                         __uint_as_float(qf[gi][st][w] & 0xFFFF0000u));
      };

      // per voter: running max over this lane's candidates (pass 0); then the
      // thresholds yes-above tY, ambiguous-from tA and near-max-from tN (pass 1)
      float m1[SEL_NG], tY[SEL_NG], tA[SEL_NG], tN[SEL_NG];
#pragma unroll
      for (int gi = 0; gi < SEL_NG; ++gi) {
        m1[gi] = -__builtin_inff();
        tY[gi] = tA[gi] = tN[gi] = 0.f;
      }
      float mloc = 0.f;
      uint32_t nbase = 0;   // entries in this wave's part of the near list (wave-uniform)
      const bool first_tile = vt0 == sp * SEL_VT;   // this workgroup's first voter tile
      // Stage candidates c0 .. min(c0 + CH, nc) - 1 as fp16, in SR rounds of one
      // 16-dim unit per thread (unit u: candidate row u / UPR, dims 16 (u % UPR)
      // onwards), the loads of the next round in flight while a round converts.
      // Every round is issued (units past the last candidate read zeros through
      // the buffer range and write nothing), so the waits are the same on every
      // path. Rows past the last candidate are left as they are: the tiles mask them.
      // WithQ: the voter tile's q loads are issued behind the last round's, so
      // the conversions do not wait for them.
      auto stage = [&](int c0, bool norms, auto with_q) {
        constexpr bool WithQ = decltype(with_q)::value;
        const int t = fresh_tid();   // recomputed here, not held through the passes
        const uint32_t range = (uint32_t)(nc * D * 4);
        auto issue = [&](int r, float4 (&f)[4]) {
          const int u = r * SEL_THREADS + t;
          const uint32_t voff = (uint32_t)(((c0 + u / UPR) * D + (u % UPR) * 16) * 4);
#pragma unroll
          for (int c = 0; c < 4; ++c) f[c] = __builtin_bit_cast(float4, buffer_load16(kg, range, voff + 16 * c));
        };
        auto convert = [&](int r, const float4 (&f)[4]) {
          const int u = r * SEL_THREADS + t;
          const int row = u / UPR, part = u % UPR;
          const bool live = c0 + row < nc;
          float ss = 0.f;
          if (live) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const float x[8] = {f[2 * c].x, f[2 * c].y, f[2 * c].z, f[2 * c].w,
                                  f[2 * c + 1].x, f[2 * c + 1].y, f[2 * c + 1].z, f[2 * c + 1].w};
              u32x4 h;
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                h[w] = pack_f16x2(x[2 * w], x[2 * w + 1]);
                ss = __builtin_fmaf(x[2 * w], x[2 * w], ss);
                ss = __builtin_fmaf(x[2 * w + 1], x[2 * w + 1], ss);
              }
              *reinterpret_cast<u32x4*>(&S.k.kh[sel_pos<D>(row, part * 2 + c)]) = h;
            }
          }
          if (norms) {   // the UPR units of a row sit in consecutive lanes
#pragma unroll
            for (int off = 1; off < UPR; off <<= 1) ss += __shfl_xor(ss, off);
            if (live) mloc = fmaxf(mloc, __builtin_sqrtf(ss));
          }
        };
        static_assert(SR == 2 || SR == 4, "staging is written for two or four rounds");
        float4 fa[4], fb[4];
        issue(0, fa);
        issue(1, fb);
        if constexpr (SR == 4) {
          convert(0, fa);
          issue(2, fa);
          convert(1, fb);
          issue(3, fb);
        }
        if constexpr (WithQ) load_q();
        convert(SR - 2, fa);
        convert(SR - 1, fb);
        staged = resident;
        lds_barrier();
      };
      // filtered scores of the staged chunk's slice t (its candidates 32 t ..
      // 32 t + 31) against the wave's voters
      auto slice_scores = [&](int t, f32x16 (&acc)[SEL_NG], int col, int half) {
#pragma unroll
        for (int gi = 0; gi < SEL_NG; ++gi) acc[gi] = f32x16{};
        const int arow = 32 * t + col;
        // candidate fragments read KA steps ahead of their MFMA (a few in flight
        // rather than all of them: registers)
        constexpr int KA = 3;
        auto kread = [&](int st) {
          return *reinterpret_cast<const f16x8*>(&S.k.kh[sel_pos<D>(arow, 2 * st + half)]);
        };
        f16x8 kf[KA];
#pragma unroll
        for (int st = 0; st < KA; ++st) kf[st] = kread(st);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const f16x8 ak = kf[st % KA];
          if (st + KA < NST) kf[st % KA] = kread(st + KA);
#pragma unroll
          for (int gi = 0; gi < SEL_NG; ++gi)
            acc[gi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, __builtin_bit_cast(f16x8, qf[gi][st]), acc[gi], 0, 0, 0);
        }
      };
      if (!(resident && staged)) stage(0, first_tile, std::true_type{});
      else load_q();
      q_to_f16();
      for (int pass = 0; pass < 2; ++pass) {
        for (int c0 = 0; c0 < nc; c0 += CH) {
          if ((pass > 0 || c0 > 0) && !(resident && staged)) {
            __syncthreads();  // readers of the previous chunk are done
            stage(c0, pass == 0 && first_tile, std::false_type{});
          }
          const int nch = min(CH, nc - c0);
#pragma unroll 1
          for (int t = 0; t < (nch + 31) / 32; ++t) {
            const int cb = c0 + 32 * t;
            f32x16 acc[SEL_NG];
            slice_scores(t, acc, col, half);
            // element i of acc[gi]: candidate cb + 4 half + 8(i/4) + i%4 against voter
            // SEL_VW wave + 32 gi + col
            const int cbase = cb + 4 * half;
            // RG: the tile runs past the last candidate (the final tile only)
            auto tile = [&](auto rg) {
              constexpr bool RG = decltype(rg)::value;
              if (pass == 0) {   // running max
#pragma unroll
                for (int gi = 0; gi < SEL_NG; ++gi) {
                  float x[16];
#pragma unroll
                  for (int i = 0; i < 16; ++i)
                    x[i] = (!RG || cbase + 8 * (i >> 2) + (i & 3) < nc) ? acc[gi][i] : -__builtin_inff();
                  m1[gi] = slice_max(m1[gi], x);
                }
                return;
              }
              // vote bits: bit 8(i/4) + i%4 of a lane's mask set when its voter clears
              // tY on element i (either group); then the OR over the 32 voters of each
              // half-wave gives the slice's vote word (the second half's candidates
              // sit 4 positions up)
              uint32_t ymask = 0;
              float dmin[SEL_NG], smax[SEL_NG];
#pragma unroll
              for (int gi = 0; gi < SEL_NG; ++gi) {
                dmin[gi] = __builtin_inff();
                smax[gi] = -__builtin_inff();
              }
              // threshold centre and the trigger band, formed here (from tA and tY) rather
              // than held through the loops
              float ctr[SEL_NG], band[SEL_NG];
#pragma unroll
              for (int gi = 0; gi < SEL_NG; ++gi) {
                float ya = tY[gi], aa = tA[gi];
                asm volatile("" : "+v"(ya), "+v"(aa));
                ctr[gi] = 0.5f * ya + 0.5f * aa;   // inf for a missing voter: |a - inf| = inf
                band[gi] = (ya - aa) + 0x1p-20f * __builtin_fabsf(ctr[gi]);
              }
#pragma unroll
              for (int gi = 0; gi < SEL_NG; ++gi)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                  // the four bits of elements 4 q4 .. 4 q4 + 3 as a nibble (small
                  // constants), then moved into place: no registers held for
                  // per-bit constants
                  uint32_t nib = 0;
#pragma unroll
                  for (int r = 0; r < 4; ++r) {
                    const float a = (!RG || cbase + 8 * q4 + r < nc) ? acc[gi][4 * q4 + r] : -__builtin_inff();
                    nib |= (uint32_t)(a > tY[gi]) << r;
                    dmin[gi] = fminf(dmin[gi], __builtin_fabsf(a - ctr[gi]));
                    smax[gi] = __builtin_fmaxf(smax[gi], a);
                  }
                  asm volatile("" : "+v"(nib));
                  ymask |= nib << (8 * q4);
                }
#pragma unroll
              for (int gi = 0; gi < SEL_NG; ++gi) {
                const int vl = wave * SEL_VW + gi * 32 + col;
                // ambiguous pairs lie within w of the threshold; dmin <= band is a
                // conservative trigger for them (band covers w and the roundings of
                // tA, tY and ctr), re-tested exactly below
                const bool near_th = dmin[gi] <= band[gi];
                if (__builtin_amdgcn_ballot_w64(near_th)) {
                  // the lane's ambiguous elements as a mask (bit i: element i), built
                  // from the top so that each step is a shift and an add; then listed
                  // one per lane per round, lowest first (the scores are dead by then)
                  uint32_t am = 0;
                  if (near_th) {
#pragma unroll
                    for (int i = 15; i >= 0; --i) {
                      const int c = cbase + 8 * (i >> 2) + (i & 3);
                      const bool hit = (!RG || c < nc) & (acc[gi][i] >= tA[gi]) & !(acc[gi][i] > tY[gi]);
                      am = 2u * am + (hit ? 1u : 0u);
                    }
                  }
                  while (__builtin_amdgcn_ballot_w64(am != 0u)) {
                    if (am != 0u) {
                      const int i = __builtin_ctz(am);
                      am &= am - 1u;
                      const int c = cbase + 8 * (i >> 2) + (i & 3);
                      const uint32_t k = atomicAdd(&S.amb_cnt, 1u);
                      if (k < SEL_AMB_CAP) S.amb[k] = ((uint32_t)vl << 16) | (uint32_t)c;
                      S.va[vl] = 1;
                    }
                  }
                }
                // near-max pairs (within 2E of the voter's filtered max), listed in
                // the wave's own part of the near list at a wave-uniform position
                // (no atomics: the wave's count stays in a scalar register)
                const bool near_max = smax[gi] >= tN[gi];
                if (__builtin_amdgcn_ballot_w64(near_max)) {
                  // as the mask of ambiguous elements above, then one per lane per round
                  uint32_t nm = 0;
                  if (near_max) {
#pragma unroll
                    for (int i = 15; i >= 0; --i) {
                      const int c = cbase + 8 * (i >> 2) + (i & 3);
                      const bool hit = (!RG || c < nc) & (acc[gi][i] >= tN[gi]);
                      nm = 2u * nm + (hit ? 1u : 0u);
                    }
                  }
                  for (;;) {
                    const bool has = nm != 0u;
                    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
                    if (!m) break;
                    if (has) {
                      const int i = __builtin_ctz(nm);
                      nm &= nm - 1u;
                      const int c = cbase + 8 * (i >> 2) + (i & 3);
                      const uint32_t pos = nbase + __builtin_amdgcn_mbcnt_hi(
                          (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                      if (pos < (uint32_t)SEL_NEAR_W)
                        S.nearl[wave * SEL_NEAR_W + pos] = ((uint32_t)vl << 16) | (uint32_t)c;
                    }
                    nbase += (uint32_t)__builtin_popcountll(m);
                  }
                }
              }
              const uint32_t r = or_half_waves(ymask);
              const uint32_t word = __builtin_amdgcn_readlane(r, 31) | (__builtin_amdgcn_readlane(r, 63) << 4);
              if (word != 0 && lane == 0) atomicOr(&S.flagw[cb >> 5], word);
            };
            if (cb + 32 > nc) tile(std::true_type{});
            else tile(std::false_type{});
          }
        }
        if (pass == 0) {
          if (first_tile) {
            float m = mloc;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            if (lane == 0) S.red[fresh_tid() >> 6] = m;   // (the slot's address formed here)
            __syncthreads();
            mnorm = S.red[0];
#pragma unroll
            for (int w = 1; w < SEL_WAVES; ++w) mnorm = fmaxf(mnorm, S.red[w]);
          }
          bool bad = false;
#pragma unroll
          for (int gi = 0; gi < SEL_NG; ++gi) {
            float ss = 0.f;
#pragma unroll
            for (int st = 0; st < NST; ++st) {
              const u32x4 raw = qf[gi][st];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const f32x2 ab = __builtin_convertvector(__builtin_bit_cast(f16x2, raw[w]), f32x2);
                ss = __builtin_fmaf(ab[0], ab[0], ss);
                ss = __builtin_fmaf(ab[1], ab[1], ss);
              }
            }
            const float qn = __builtin_sqrtf(ss + partner32(ss));
            const float M = fmaxf(m1[gi], partner32(m1[gi]));
            const float nm = qn * mnorm;
            bad = bad || (vok[gi] && !(qn <= SEL_MAG && mnorm <= SEL_MAG));
            const float e2 = 2.f * (SEL_ERR * nm + SEL_ABS * (qn + mnorm + 1.f));
            tN[gi] = M - e2;
            tY[gi] = M + (theta_f + (e2 + theta_slack));
            tA[gi] = M + (theta_f - (e2 + theta_slack));
            if (!vok[gi]) tN[gi] = tY[gi] = tA[gi] = __builtin_inff();  // no voter: nothing passes any test
          }
          if (__ballot(bad) && lane == 0) S.overflow = 1u;
          __syncthreads();
          if (S.overflow) break;  // uniform: redo this voter tile exactly
        }
      }
      // the voters' pass-1 thresholds, kept for pass 2
      if (((fresh_tid() >> 5) & 1) == 0) {
#pragma unroll
        for (int gi = 0; gi < SEL_NG; ++gi)
          S.thr[(fresh_tid() >> 6) * SEL_VW + gi * 32 + (fresh_tid() & 31)] = make_float2(tA[gi], tY[gi]);
      }
      if (lane == 0) {
        S.ncnt[fresh_tid() >> 6] = nbase;   // (the slot's address formed here)
        if (nbase > (uint32_t)SEL_NEAR_W) S.overflow = 1u;
      }
      __syncthreads();
      const uint32_t namb = S.amb_cnt;   // counted past the list's capacity
      const bool go = !S.overflow && namb > 0;
      const bool redo = namb > (uint32_t)SEL_AMB_CAP;   // the list overflowed: pass 2
      __syncthreads();  // every thread has read the flags before they change again
      if (go) {
        // pairs whose exact score may be the max of a voter with ambiguous pairs:
        // its near-max pairs
        for (int e = fresh_tid(); e < SEL_WAVES * SEL_NEAR_W; e += SEL_THREADS) {
          const int w = e / SEL_NEAR_W;
          if (e - w * SEL_NEAR_W >= (int)S.ncnt[w]) continue;
          const uint32_t pr = S.nearl[e];
          if (!S.va[pr >> 16]) continue;
          const uint32_t k = atomicAdd(&S.job_cnt, 1u);
          if (k < SEL_JOB_CAP) S.jobs[k] = pr;
          else S.overflow = 1u;
        }
        __syncthreads();
        if (!S.overflow)
          exact_pairs<D>(S, (int)S.job_cnt, redo ? 0 : (int)namb, qg, group, n_q, vt0, kg, theta);
      }
      __syncthreads();
      if (redo && !S.overflow) {
        // Pass 2, after an overflow of the ambiguous list: the same filtered scores
        // against the same thresholds give the same ambiguous pairs again; they are
        // listed and decided against the exact maxima found above, SEL_P2G slices
        // at a time. A group whose list overflows again decides every pair of its
        // candidates for the voters with ambiguous pairs (the rest of those voters'
        // pairs agree with the filter's decision).
        // (the voters' q and thresholds are loaded afresh for each group, so that
        // nothing of theirs is held through the exact evaluations)
        int grp = 0;
        for (int c0 = 0; c0 < nc; c0 += CH) {
          if (!resident) {
            __syncthreads();  // readers of the previous chunk are done
            stage(c0, false, std::false_type{});
          }
          const int nsl = (min(CH, nc - c0) + 31) / 32;
#pragma unroll 1
          for (int t0 = 0; t0 < nsl; t0 += SEL_P2G, ++grp) {
            const int t1 = min(t0 + SEL_P2G, nsl);
            load_q();
            q_to_f16();
            float tA2[SEL_NG], tY2[SEL_NG];
#pragma unroll
            for (int gi = 0; gi < SEL_NG; ++gi) {
              const int vl = (fresh_tid() >> 6) * SEL_VW + gi * 32 + (fresh_tid() & 31);
              const float2 th = S.thr[vl];
              tA2[gi] = S.va[vl] ? th.x : __builtin_inff();   // other voters list nothing
              tY2[gi] = th.y;
            }
#pragma unroll 1
            for (int t = t0; t < t1; ++t) {
              // lane values formed afresh (nothing lane-derived is held through the
              // exact evaluations between groups)
              const int ft = fresh_tid();
              const int fcol = ft & 31, fhalf = (ft >> 5) & 1;
              f32x16 acc[SEL_NG];
              slice_scores(t, acc, fcol, fhalf);
              const int cbase = c0 + 32 * t + 4 * fhalf;
#pragma unroll
              for (int gi = 0; gi < SEL_NG; ++gi) {
                const int vl = (ft >> 6) * SEL_VW + gi * 32 + fcol;
                uint32_t am = 0;
#pragma unroll
                for (int i = 15; i >= 0; --i) {
                  const int c = cbase + 8 * (i >> 2) + (i & 3);
                  const bool hit = (c < nc) & (acc[gi][i] >= tA2[gi]) & !(acc[gi][i] > tY2[gi]);
                  am = 2u * am + (hit ? 1u : 0u);
                }
                while (__builtin_amdgcn_ballot_w64(am != 0u)) {
                  if (am != 0u) {
                    const int i = __builtin_ctz(am);
                    am &= am - 1u;
                    const int c = cbase + 8 * (i >> 2) + (i & 3);
                    const uint32_t k = atomicAdd(&S.pcnt[grp & 1], 1u);
                    if (k < SEL_AMB_CAP) S.amb[k] = ((uint32_t)vl << 16) | (uint32_t)c;
                  }
                }
              }
            }
            __syncthreads();  // the group's list is complete
            const uint32_t n = S.pcnt[grp & 1];
            // the other count was last read before this barrier: cleared for the next group
            if (tid == 0) S.pcnt[(grp + 1) & 1] = 0;
            if (n <= (uint32_t)SEL_AMB_CAP) {
              exact_pairs<D>(S, 0, (int)n, qg, group, n_q, vt0, kg, theta);
            } else {
              const int cg0 = c0 + 32 * t0, w = min(c0 + 32 * t1, nc) - cg0;
              for (int e = fresh_tid(); e < SEL_VT * w; e += SEL_THREADS) {
                const int vl = e / w, c = cg0 + e % w;
                if (!S.va[vl]) continue;
                if (dot_exact_prefetched<D>(qptr(vt0 + vl), kg + (size_t)c * D) - dval(S.mxkey[vl]) > theta)
                  atomicOr(&S.flagw[c >> 5], 1u << (c & 31));
              }
            }
            __syncthreads();  // the list is read before the next group writes it
          }
        }
      }
      if (S.overflow) {
        // exact fp64 for every pair of this voter tile; one wave per voter
        // (lane values formed here, so that no lane address is held from the start)
        const int nvt = min(SEL_VT, nv - vt0);
        for (int u = fresh_tid() >> 6; u < nvt; u += SEL_WAVES) {
          const uint16_t* qp = qptr(vt0 + u);
          double m = -__builtin_inf();
#pragma unroll 1
          for (int b = fresh_tid() & 63; b < nc; b += 64) m = fmax(m, dot_exact<D>(qp, kg + (size_t)b * D));
          m = wave_max(m);
#pragma unroll 1
          for (int b = fresh_tid() & 63; b < nc; b += 64)
            if (dot_exact<D>(qp, kg + (size_t)b * D) - m > theta) atomicOr(&S.flagw[b >> 5], 1u << (b & 31));
        }
      }
      if (tid == 0) {   // the tile's path (S.overflow is final here: set before the last barrier)
        atomicAdd(&g_sel_paths[0], 1ull);
        const int path = S.overflow ? 3 : (redo ? 2 : (go ? 1 : -1));
        if (path > 0) atomicAdd(&g_sel_paths[path], 1ull);
      }
    }
  }
  __syncthreads();
  int32_t* out = sel_idx + ((size_t)g * n_qblk + jj) * nb;
  if (n_split > 1) {
    // partial votes: this workgroup's flag words go to words [sp nw, (sp + 1) nw)
    // of the row, where select_merge_kernel ORs them (n_split nw <= nb by the launch)
    for (int i = tid; i < nw; i += SEL_THREADS) out[sp * nw + i] = (int32_t)S.flagw[i];
    return;
  }
  finish_selection(S.flagw, S.wsum, nb, nc, jj, j, n_qblk, sink_blocks, window_blocks,
                   dense_tail_blocks, out, sel_cnt + (size_t)g * n_qblk + jj);
}

// One workgroup per (KV head, query block) after a split select_kernel: OR the
// n_split partial flag rows left at the front of the row, then finish as above.
__global__ void __launch_bounds__(SEL_THREADS) select_merge_kernel(
    int q_start, int n_kv, int nb, int block, int n_qblk, int sink_blocks, int window_blocks,
    int dense_tail_blocks, int n_split, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt) {
  __shared__ uint32_t flagw[SEL_MAX_NB / 32];
  __shared__ uint32_t wsum[SEL_WAVES];
  const int jj = (int)blockIdx.x / n_kv;
  const int g = (int)blockIdx.x % n_kv;
  const int j = q_start / block + jj;
  const int nc = j, nw = (nc + 31) >> 5;
  int32_t* out = sel_idx + ((size_t)g * n_qblk + jj) * nb;
  for (int i = threadIdx.x; i < nw; i += SEL_THREADS) {
    uint32_t w = 0;
    for (int s = 0; s < n_split; ++s) w |= (uint32_t)out[s * nw + i];
    flagw[i] = w;
  }
  __syncthreads();   // every partial word is read before the row is rewritten
  finish_selection(flagw, wsum, nb, nc, jj, j, n_qblk, sink_blocks, window_blocks, dense_tail_blocks,
                   out, sel_cnt + (size_t)g * n_qblk + jj);
}

hipError_t select_path_counts(int64_t* out, bool reset) {
  unsigned long long h[4] = {0, 0, 0, 0};
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(h, HIP_SYMBOL(g_sel_paths), sizeof(h), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  for (int i = 0; i < 4; ++i) out[i] = (int64_t)h[i];
  if (reset) {
    const unsigned long long z[4] = {0, 0, 0, 0};
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_sel_paths), z, sizeof(z), 0, hipMemcpyHostToDevice);
  }
  return e;
}

hipError_t launch_select(const uint16_t* Q, int C, int q_start, int n_q, int n_kv, int d,
                         const float* K_pool, int pool_ld, int T, int block, double theta,
                         int sink_blocks, int window_blocks, int dense_tail_blocks,
                         int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream) {
  const int nb = (T + block - 1) / block;
  const int j0 = q_start / block;
  const int j1 = (q_start + C - 1) / block;
  const int n_qblk = j1 - j0 + 1;
  // the filter's bound needs theta in fp32 range; larger |theta| is decided exactly
  const bool inf_theta = std::isinf(theta) && theta < 0;
  const int exact_only = (!inf_theta && !(std::fabs(theta) <= 1e30)) ? 1 : 0;
  const float theta_f = inf_theta ? -HUGE_VALF : (exact_only ? 0.f : (float)theta);
  const float theta_slack = inf_theta || exact_only ? 0.f : (float)std::ldexp(std::fabs(theta), -22);
  // Two select workgroups fit on a CU. When the (KV head, query block) pairs
  // are fewer than that, their voter tiles are spread over n_split
  // workgroups, as far as the tiles go and as the partial flag rows fit at the
  // front of a selection row (n_split nw <= nb).
  const int vt_max = (std::min(block, C) * (n_q / n_kv) + SEL_VT - 1) / SEL_VT;
  const int pairs = n_qblk * n_kv;
  const int nw_max = (nb - 1 + 31) / 32;
  int n_split = 1;
  if (theta_f != -HUGE_VALF) {
    const int want = (2 * device_cus() + pairs - 1) / pairs;
    n_split = std::max(1, std::min(std::min(want, vt_max), nw_max > 0 ? nb / nw_max : 1));
  }
  dim3 grid(pairs * n_split);
  if (d == 128)
    hipLaunchKernelGGL(select_kernel<128>, grid, dim3(SEL_THREADS), 0, stream, Q, C, q_start, n_q,
                       n_kv, K_pool, pool_ld, nb, block, theta, theta_f, theta_slack, exact_only, n_qblk,
                       sink_blocks, window_blocks, dense_tail_blocks, n_split, sel_idx, sel_cnt);
  else
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(SEL_THREADS), 0, stream, Q, C, q_start, n_q,
                       n_kv, K_pool, pool_ld, nb, block, theta, theta_f, theta_slack, exact_only, n_qblk,
                       sink_blocks, window_blocks, dense_tail_blocks, n_split, sel_idx, sel_cnt);
  if (n_split > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_merge_kernel, dim3(pairs), dim3(SEL_THREADS), 0, stream, q_start, n_kv, nb,
                       block, n_qblk, sink_blocks, window_blocks, dense_tail_blocks, n_split, sel_idx,
                       sel_cnt);
  }
  return hipGetLastError();
}

}  // namespace pa
