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
// select_blocks: one workgroup of 8 waves per (KV head g, query block j), or
// several sharing its voter tiles when the pairs are too few to fill the chip
// (their votes are merged by select_merge_kernel; see launch_select).
//
// Voters are the (row, query head) pairs of block j in this chunk; candidates
// are the blocks b < j. The result must equal the fixed-order fp64 rule
//   vote(i, b)  <=>  fl64(r_ib - M_i) > theta,  M_i = max_b r_ib,
// for every voter, bit for bit. Evaluating every r_ib in fp64 costs 2 d flops
// per pair on the fp64 vector units; instead the kernel
//
//  1. filters on the bf16 matrix cores: kbar = hi + lo with hi = bf16(kbar),
//     lo = bf16(kbar - hi) (round-to-nearest-even; kbar - hi is exact), and
//     r'_ib = q_i.hi_b + q_i.lo_b accumulated in fp32 by v_mfma_f32_32x32x16_bf16
//     (q is bf16, so every product is exact). With A = sum_d |q_d||kbar_d|
//     <= |q|_2 |kbar|_2 (Cauchy-Schwarz):
//        |kbar - hi - lo| <= 2^-16 |kbar|            (two roundings of 2^-8)
//        fp32 accumulation of 2d+1 terms in any order, each step rounding by
//        at most 2^-23 (also covers truncating adders): <= gamma_257 (1+2^-7) A
//        the fp64 reference itself: <= 128 * 2^-53 A
//     so |r' - r64| <= 4.6e-5 A. The kernel takes E = 1e-4 max|q| max|kbar|
//     over the wave's voters and the candidates (over twice the bound, which
//     also absorbs the fp32 norms and comparisons) plus 1e-30 per unit for
//     flushed denormals. Then |(r' - M') - (r - M)| <= 2E, so a pair whose
//     filtered gap lies more than 2E (+ 2^-22 |theta|) from theta is decided;
//  2. lists the other pairs as ambiguous. The exact argmax of voter i is the
//     filter's argmax unless another candidate came within 2E of the filtered
//     max; such voters are flagged and their near-max pairs listed;
//  3. re-evaluates the listed pairs in fp64 in the reference order: M_i
//     exactly (the filter's argmax, or the max over a flagged voter's near-max
//     pairs),
//     then each ambiguous pair against theta. Each exact dot product is done
//     by a wave: one coalesced load of the two rows, the exact fp64 products
//     staged in LDS, one lane summing them in order (4 pairs per wave at a
//     time).
// If a list overflows, or magnitudes leave the range where the bound holds
// (|q|, |kbar| or their product above 1e30), the voter tile is redone exactly
// in fp64 for all pairs. alpha = 0 (theta = -inf) keeps every visible block.
// Votes are ORed into a per-block bit mask in LDS, compacted in ascending
// order, and the diagonal block appended.
//
// MFMA orientation: A = kbar (32 candidates x 16 dims, LDS), B = Q^T (16 dims x
// 32 voters, registers). Accumulator element i of lane l is candidate
// 8(i/4) + 4(l/32) + i%4 against voter l%32, so a voter's max, near-max count
// and argmax live in lanes l and l^32; "some voter votes for candidate c" is one
// ballot per accumulator element, consumed on the scalar unit.
// ---------------------------------------------------------------------------
constexpr int SEL_WAVES = 8;
constexpr int SEL_THREADS = SEL_WAVES * 64;
constexpr int SEL_VT = SEL_WAVES * 32;   // voters per tile: 32 per wave
constexpr int SEL_CH = 64;               // candidates staged per chunk
constexpr int SEL_MAX_NB = 8192;
constexpr int SEL_AMB_CAP = 2048;        // ambiguous pairs per voter tile
constexpr int SEL_JOB_CAP = 2048;        // exact max evaluations per voter tile
constexpr int SEL_NEAR_CAP = 1024;       // near-max pairs of flagged voters per voter tile
constexpr int SEL_JOBS = 4;              // exact dot products per wave at a time
constexpr float SEL_ERR = 1.0e-4f;
constexpr float SEL_ABS = 1.0e-30f;
constexpr float SEL_MAG = 1.0e30f;

__device__ __forceinline__ int sel_swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

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

template <int D>
struct SelShared {
  union {
    struct {
      uint16_t khi[SEL_CH * D];   // bf16 hi parts, row-major [candidate][d], 16-byte chunks swizzled
      uint16_t klo[SEL_CH * D];   // bf16 lo parts, same layout
    } k;
    double prod[SEL_WAVES][SEL_JOBS][D];   // exact products of the re-evaluated pairs
  } u;
  unsigned long long mxkey[SEL_VT];        // exact max (as dkey) of voters with ambiguous pairs
  uint32_t amb[SEL_AMB_CAP];               // (voter << 16) | block
  uint32_t jobs[SEL_JOB_CAP];              // pairs whose exact score enters a max
  uint32_t nearl[SEL_NEAR_CAP];            // near-max pairs of flagged voters: (voter << 16) | block
  uint32_t flagw[SEL_MAX_NB / 32];
  uint32_t wsum[SEL_WAVES];
  uint16_t argb[SEL_VT];                   // the filter's argmax per voter
  uint8_t va[SEL_VT];                      // voter has ambiguous pairs
  uint8_t multi[SEL_VT];                   // several candidates came within 2E of the max
  float red[SEL_WAVES];
  uint32_t amb_cnt, job_cnt, near_cnt;
  uint32_t overflow;
};

// Exact fp64 scores of the listed (voter, block) pairs, SEL_JOBS pairs per wave
// at a time. MODE 0: raise the voter's exact max; MODE 1: vote if the pair clears
// theta against that max.
template <int D, int MODE>
__device__ __forceinline__ void exact_pairs(SelShared<D>& S, const uint32_t* list, int n,
                                            const uint16_t* qg, int group, int n_q, int vt0,
                                            const float* kg, double theta, int wave, int lane) {
  for (int base = wave * SEL_JOBS; base < n; base += SEL_WAVES * SEL_JOBS) {
#pragma unroll
    for (int k = 0; k < SEL_JOBS; ++k) {
      if (base + k >= n) break;  // wave-uniform
      const uint32_t job = list[base + k];
      const int v = vt0 + (int)(job >> 16), b = (int)(job & 0xFFFFu);
      const uint16_t* qp = qg + ((size_t)(v / group) * n_q + (v % group)) * D;
      const float* kb = kg + (size_t)b * D;
      double* pr = S.u.prod[wave][k];
      if (D == 128) {
        const uint32_t qq = reinterpret_cast<const uint32_t*>(qp)[lane];
        const float2 kk = reinterpret_cast<const float2*>(kb)[lane];
        pr[2 * lane] = (double)__uint_as_float(qq << 16) * (double)kk.x;
        pr[2 * lane + 1] = (double)__uint_as_float(qq & 0xFFFF0000u) * (double)kk.y;
      } else {
        pr[lane] = (double)bf16_to_f32(qp[lane]) * (double)kb[lane];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < SEL_JOBS && base + lane < n) {
      const double* pr = S.u.prod[wave][lane];
      double acc = 0.0;
#pragma unroll 8
      for (int d = 0; d < D; ++d) acc = acc + pr[d];   // increasing d, as the reference sums
      const uint32_t job = list[base + lane];
      const int vl = (int)(job >> 16), b = (int)(job & 0xFFFFu);
      if (MODE == 0) atomicMax(&S.mxkey[vl], dkey(acc));
      else if (acc - dval(S.mxkey[vl]) > theta) atomicOr(&S.flagw[b >> 5], 1u << (b & 31));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
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
// Four waves per SIMD (at most 128 registers): two workgroups share a CU, so one
// workgroup's staging and barriers overlap the other's scoring.
__global__ void __launch_bounds__(SEL_THREADS) __attribute__((amdgpu_waves_per_eu(4))) select_kernel(
    const uint16_t* __restrict__ Q, int C, int q_start, int n_q, int n_kv,
    const float* __restrict__ Kp, int pool_ld, int nb, int block, double theta, float theta_f,
    float theta_slack,
    int exact_only, int n_qblk, int sink_blocks, int window_blocks, int dense_tail_blocks,
    int n_split, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt) {
  constexpr int NST = D / 16;   // MFMA k-steps
  constexpr int TPR = SEL_THREADS / SEL_CH;   // staging threads per candidate row
  constexpr int DPT = D / TPR;                // staged dims per thread
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
    for (int vt0 = sp * SEL_VT; vt0 < nv; vt0 += n_split * SEL_VT) {
      __syncthreads();  // previous tile's readers of the shared state are done
      for (int i = tid; i < SEL_VT; i += SEL_THREADS) { S.va[i] = 0; S.mxkey[i] = 0; }
      if (tid == 0) { S.amb_cnt = 0; S.job_cnt = 0; S.near_cnt = 0; S.overflow = exact_only; }

      // B operand: q of the wave's 32 voters (voter = lane % 32), held for the whole tile
      const int vl = wave * 32 + col;  // voter within the tile
      const bool vok = vt0 + vl < nv;
      bf16x8 qf[NST];
      float qn;
      {
        const uint16_t* qp = vok ? qptr(vt0 + vl) : Q;
        float ss = 0.f;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          u32x4 raw = {0u, 0u, 0u, 0u};
          if (vok) raw = *reinterpret_cast<const u32x4*>(qp + 16 * st + 8 * half);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float a = __uint_as_float(raw[w] << 16), b = __uint_as_float(raw[w] & 0xFFFF0000u);
            ss = __builtin_fmaf(a, a, ss);
            ss = __builtin_fmaf(b, b, ss);
          }
          qf[st] = __builtin_bit_cast(bf16x8, raw);
        }
        qn = __builtin_sqrtf(ss + partner32(ss));
      }

      // the voter's running max and second max over this lane's candidates
      float m1 = -__builtin_inff(), m2 = -__builtin_inff();
      float M = 0.f, tY = 0.f, tA = 0.f;  // the voter's max; yes above tY; ambiguous from tA
      float tN = 0.f;                     // near-max from tN (recorded for flagged voters)
      int nidx = -1;                      // this lane's candidate equal to the max, if any
      bool multi = false;
      float mloc = 0.f;
      const bool first_tile = vt0 == sp * SEL_VT;   // this workgroup's first voter tile
      for (int pass = 0; pass < 2; ++pass) {
        for (int c0 = 0; c0 < nc; c0 += SEL_CH) {
          __syncthreads();  // readers of the previous chunk are done
          {  // stage candidates c0 .. c0+63 as bf16 hi/lo
            const int row = tid / TPR, part = tid % TPR;
            const int b = c0 + row;
            float x[DPT];
            if (b < nc) {
              const float4* src = reinterpret_cast<const float4*>(kg + (size_t)b * D + part * DPT);
#pragma unroll
              for (int e = 0; e < DPT / 4; ++e) {
                const float4 f = src[e];
                x[4 * e] = f.x; x[4 * e + 1] = f.y; x[4 * e + 2] = f.z; x[4 * e + 3] = f.w;
              }
            } else {
#pragma unroll
              for (int e = 0; e < DPT; ++e) x[e] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < DPT / 8; ++c) {
              u32x4 h, l;
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const float a = x[8 * c + 2 * w], bb = x[8 * c + 2 * w + 1];
                const uint32_t hp = pack_bf16x2(a, bb);
                h[w] = hp;
                l[w] = pack_bf16x2(a - __uint_as_float(hp << 16), bb - __uint_as_float(hp & 0xFFFF0000u));
              }
              const int off = row * D + (((part * (DPT / 8) + c) ^ sel_swz(row)) * 8);
              *reinterpret_cast<u32x4*>(&S.u.k.khi[off]) = h;
              *reinterpret_cast<u32x4*>(&S.u.k.klo[off]) = l;
            }
            if (pass == 0 && first_tile) {
              float ss = 0.f;
#pragma unroll
              for (int e = 0; e < DPT; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
#pragma unroll
              for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off);
              if (b < nc) mloc = fmaxf(mloc, __builtin_sqrtf(ss));
            }
          }
          __syncthreads();
#pragma unroll 1
          for (int t = 0; t < SEL_CH / 32; ++t) {
            const int cb = c0 + 32 * t;
            if (cb >= nc) break;
            f32x16 acc = {};
            const int arow = 32 * t + col;
#pragma unroll
            for (int st = 0; st < NST; ++st) {
              const int off = arow * D + (((2 * st + half) ^ sel_swz(arow)) * 8);
              const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&S.u.k.khi[off]);
              const bf16x8 al = *reinterpret_cast<const bf16x8*>(&S.u.k.klo[off]);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[st], acc, 0, 0, 0);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[st], acc, 0, 0, 0);
            }
            // element i: candidate cb + 4 half + 8(i/4) + i%4, voter col
            const int cbase = cb + 4 * half;
            // RG: the tile runs past the last candidate (the final tile only)
            auto tile = [&](auto rg) {
              constexpr bool RG = decltype(rg)::value;
              if (pass == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                  const float x = (!RG || cbase + 8 * (i >> 2) + (i & 3) < nc) ? acc[i] : -__builtin_inff();
                  m2 = __builtin_amdgcn_fmed3f(m1, x, m2);
                  m1 = fmaxf(m1, x);
                }
                return;
              }
              // one ballot per comparison: yes masks become the candidates' vote
              // bits, (>= tA) & !(> tY) marks ambiguous pairs
              uint32_t word = 0;
              uint64_t rare_m = 0;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int c = cbase + 8 * (i >> 2) + (i & 3);
                const float a = acc[i];
                bool yv = a > tY, av = a >= tA, ev = a == M;
                if (RG) {
                  const bool ok = c < nc;
                  yv = yv && ok;
                  av = av && ok;
                  ev = ev && ok;
                }
                const uint64_t ym = __builtin_amdgcn_ballot_w64(yv);
                const uint64_t am = __builtin_amdgcn_ballot_w64(av);
                rare_m |= am & ~ym;
                word |= ones_if_nonzero((uint32_t)ym) & (1u << (8 * (i >> 2) + (i & 3)));
                word |= ones_if_nonzero((uint32_t)(ym >> 32)) & (1u << (8 * (i >> 2) + 4 + (i & 3)));
                nidx = ev ? c : nidx;
              }
              if (rare_m != 0) {
                if ((rare_m >> lane) & 1) {
#pragma unroll
                  for (int i = 0; i < 16; ++i) {
                    const int c = cbase + 8 * (i >> 2) + (i & 3);
                    if ((!RG || c < nc) & (acc[i] >= tA) & !(acc[i] > tY)) {
                      const uint32_t k = atomicAdd(&S.amb_cnt, 1u);
                      if (k < SEL_AMB_CAP) S.amb[k] = ((uint32_t)vl << 16) | (uint32_t)c;
                      else S.overflow = 1u;
                      S.va[vl] = 1;
                    }
                  }
                }
              }
              if (__builtin_amdgcn_ballot_w64(multi)) {
                if (multi) {   // the exact max of a flagged voter is among these
#pragma unroll
                  for (int i = 0; i < 16; ++i) {
                    const int c = cbase + 8 * (i >> 2) + (i & 3);
                    if ((!RG || c < nc) & (acc[i] >= tN)) {
                      const uint32_t k = atomicAdd(&S.near_cnt, 1u);
                      if (k < SEL_NEAR_CAP) S.nearl[k] = ((uint32_t)vl << 16) | (uint32_t)c;
                      else S.overflow = 1u;
                    }
                  }
                }
              }
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
            if (lane == 0) S.red[wave] = m;
            __syncthreads();
            mnorm = S.red[0];
#pragma unroll
            for (int w = 1; w < SEL_WAVES; ++w) mnorm = fmaxf(mnorm, S.red[w]);
          }
          const float p1 = partner32(m1), p2 = partner32(m2);
          M = fmaxf(m1, p1);
          const float second = fmaxf(fmaxf(m2, p2), fminf(m1, p1));
          const float nm = qn * mnorm;
          const bool bad = vok && !(qn <= SEL_MAG && mnorm <= SEL_MAG && nm <= SEL_MAG);
          const float e2 = 2.f * (SEL_ERR * nm + SEL_ABS * (qn + mnorm + 1.f));
          tN = M - e2;
          multi = vok && second >= tN;  // another candidate may hold the exact max
          tY = M + (theta_f + (e2 + theta_slack));
          tA = M + (theta_f - (e2 + theta_slack));
          if (!vok) M = tY = tA = __builtin_inff();  // no voter: nothing passes any test
          if (__ballot(bad) && lane == 0) S.overflow = 1u;
          __syncthreads();
          if (S.overflow) break;  // uniform: redo this voter tile exactly
        }
      }
      {  // the filter's argmax, and whether another candidate came within 2E of it
        const int pidx = __float_as_int(partner32(__int_as_float(nidx)));
        if (half == 0 && vok) {
          S.argb[vl] = (uint16_t)(nidx >= 0 ? nidx : max(pidx, 0));
          S.multi[vl] = multi;
        }
      }
      __syncthreads();
      const bool go = !S.overflow && S.amb_cnt > 0;
      __syncthreads();  // every thread has read the flags before they change again
      if (go) {
        // pairs whose exact score may be the max of a voter with ambiguous pairs:
        // its argmax, or its recorded near-max pairs when several came within 2E
        for (int v = tid; v < SEL_VT; v += SEL_THREADS) {
          if (!S.va[v] || S.multi[v]) continue;
          const uint32_t k = atomicAdd(&S.job_cnt, 1u);
          if (k < SEL_JOB_CAP) S.jobs[k] = ((uint32_t)v << 16) | S.argb[v];
          else S.overflow = 1u;
        }
        const int nn = (int)min(S.near_cnt, (uint32_t)SEL_NEAR_CAP);
        for (int e = tid; e < nn; e += SEL_THREADS) {
          const uint32_t pr = S.nearl[e];
          if (!S.va[pr >> 16]) continue;
          const uint32_t k = atomicAdd(&S.job_cnt, 1u);
          if (k < SEL_JOB_CAP) S.jobs[k] = pr;
          else S.overflow = 1u;
        }
        __syncthreads();
        if (!S.overflow) {
          exact_pairs<D, 0>(S, S.jobs, (int)S.job_cnt, qg, group, n_q, vt0, kg, theta, wave, lane);
          __syncthreads();
          exact_pairs<D, 1>(S, S.amb, (int)S.amb_cnt, qg, group, n_q, vt0, kg, theta, wave, lane);
        }
      }
      __syncthreads();
      if (S.overflow) {
        // exact fp64 for every pair of this voter tile; one wave per voter
        const int nvt = min(SEL_VT, nv - vt0);
        for (int u = wave; u < nvt; u += SEL_WAVES) {
          const uint16_t* qp = qptr(vt0 + u);
          double m = -__builtin_inf();
#pragma unroll 1
          for (int b = lane; b < nc; b += 64) m = fmax(m, dot_exact<D>(qp, kg + (size_t)b * D));
          m = wave_max(m);
#pragma unroll 1
          for (int b = lane; b < nc; b += 64)
            if (dot_exact<D>(qp, kg + (size_t)b * D) - m > theta) atomicOr(&S.flagw[b >> 5], 1u << (b & 31));
        }
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
  // fill fewer slots than that (a 4,096-row chunk: 32 query blocks), their voter
  // tiles are spread over n_split workgroups, as far as the tiles go and as the
  // partial flag rows fit at the front of a selection row (n_split nw <= nb).
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
