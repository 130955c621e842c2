// Mask-tile classification and split-key combination for dense prefill attention.
#include "common.h"
#include <algorithm>

namespace pa {

// ---------------------------------------------------------------------------
// mask_classify: one workgroup per strip of 64 rows x 256 keys of the fp16 mask
// (four flag tiles of 64 rows x 64 keys along the keys). Per tile:
// ZERO     every entry is +-0      -> the attention kernel never reads the tile
// DROPPED  every entry <= -30000   -> the attention kernel skips the tile
// MIXED    anything else           -> the attention kernel reads the tile
// A dropped entry omits its key ("ANE Prefill Research", What worked, item 2),
// so a fully dropped tile contributes nothing and needs no arithmetic at all.
// Thread t reads 8 keys (16 bytes) at strip column 8 (t % 32) of rows
// t / 32 + 8 i, i < 8, so 32 lanes cover a 512-byte row segment. An interior
// strip issues all eight 16-byte loads before any test; strips at the right or
// bottom edge test key by key below T and C. (Same-process timing on the 32K
// chunks: 30.7 us per launch with one 64 x 64 tile per workgroup, 27.1 us with
// these strips, 29.5 us with strips of eight tiles.)
// A tile's verdict is the OR over waves of one ballot per property, restricted
// to the 16 lanes of the wave that read the tile.
// grid = (ceil(T/256), ceil(C/64)), block = 256; flags row stride n_ktile.
// ---------------------------------------------------------------------------
constexpr int CLS_TILES = 4;   // flag tiles per strip

__device__ __forceinline__ void classify8(u32x4 v, bool& all_zero, bool& all_drop) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint16_t lo = v[w] & 0xFFFF, hi = v[w] >> 16;
    all_zero &= ((lo & 0x7FFF) == 0) && ((hi & 0x7FFF) == 0);
    all_drop &= f16_dropped(lo) && f16_dropped(hi);
  }
}

template <bool VEC>
__global__ void __launch_bounds__(256) mask_classify_kernel(const uint16_t* __restrict__ mask,
                                                            int64_t ld, int C, int T, int n_ktile,
                                                            uint8_t* __restrict__ flags) {
  __shared__ uint64_t wz[4], wd[4];
  const int sx = blockIdx.x, qt = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int LPR = 8 * CLS_TILES;          // lanes per row segment
  constexpr int RPP = 256 / LPR;               // rows per pass
  constexpr int PASSES = FLAG_ROWS / RPP;
  const int c0 = sx * (CLS_TILES * FLAG_KEYS) + (tid % LPR) * 8;
  const int r0 = qt * FLAG_ROWS + tid / LPR;
  bool all_zero = true, all_drop = true;
  if (VEC && (sx + 1) * CLS_TILES * FLAG_KEYS <= T && (qt + 1) * FLAG_ROWS <= C) {
    u32x4 v[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i)
      v[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(mask + (size_t)(r0 + RPP * i) * ld + c0));
#pragma unroll
    for (int i = 0; i < PASSES; ++i) classify8(v[i], all_zero, all_drop);
  } else {
    for (int i = 0; i < PASSES; ++i) {
      const int r = r0 + RPP * i;
      if (r >= C) break;
      const uint16_t* p = mask + (size_t)r * ld + c0;
      if (VEC && c0 + 8 <= T) {
        classify8(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)), all_zero, all_drop);
      } else {
        for (int e = 0; e < 8; ++e) {
          if (c0 + e >= T) break;
          const uint16_t h = p[e];
          all_zero &= (h & 0x7FFF) == 0;
          all_drop &= f16_dropped(h);
        }
      }
    }
  }
  // tile t is read by lanes 8t .. 8t+7 of every LPR-lane group of every wave
  const uint64_t nz = __ballot(!all_zero), nd = __ballot(!all_drop);
  if (lane == 0) { wz[wave] = nz; wd[wave] = nd; }
  __syncthreads();
  if (tid < CLS_TILES) {
    const int kt = sx * CLS_TILES + tid;
    uint64_t sel = 0;
#pragma unroll
    for (int k = 0; k < 64 / LPR; ++k) sel |= 0xFFull << (8 * tid + LPR * k);
    const uint64_t z = (wz[0] | wz[1] | wz[2] | wz[3]) & sel;
    const uint64_t d = (wd[0] | wd[1] | wd[2] | wd[3]) & sel;
    if (kt < n_ktile) flags[(size_t)qt * n_ktile + kt] = d == 0 ? TILE_DROPPED : (z == 0 ? TILE_ZERO : TILE_MIXED);
  }
}

// ---------------------------------------------------------------------------
// fold_keep_mask: an indexer's compacted selection into the additive mask
// ("ANE Prefill Research", What worked, item 2). One workgroup per query row:
// the row's columns 0..T-1 are first set to -30000 (16-byte stores where the
// row is aligned), then, after a barrier, the kept keys are zeroed: every key of
// each listed `width`-key block and the `recent` keys ending at the row's own
// position p, both clipped to t <= p. Listed blocks outside [0, ceil(T/width))
// are ignored; at most keep_ld entries of a row are read.
// grid = C, block = 256.
// ---------------------------------------------------------------------------
constexpr uint16_t F16_M30000 = 0xF753;   // -30000 in fp16

template <bool VEC>
__global__ void __launch_bounds__(256) fold_keep_kernel(const int32_t* __restrict__ keep_idx,
                                                        int64_t keep_ld,
                                                        const int32_t* __restrict__ keep_cnt,
                                                        int q_start, int T, int width, int recent,
                                                        uint16_t* __restrict__ mask, int64_t mask_ld) {
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  uint16_t* row = mask + (size_t)i * mask_ld;
  if (VEC) {
    const uint32_t d2 = (uint32_t)F16_M30000 | ((uint32_t)F16_M30000 << 16);
    const u32x4 v = {d2, d2, d2, d2};
    const int n8 = T / 8;
    for (int c = tid; c < n8; c += 256) *reinterpret_cast<u32x4*>(row + 8 * c) = v;
    for (int t = 8 * n8 + tid; t < T; t += 256) row[t] = F16_M30000;
  } else {
    for (int t = tid; t < T; t += 256) row[t] = F16_M30000;
  }
  __syncthreads();
  const int p = q_start + i;
  const int last = min(p, T - 1);            // no key past the row's own position
  const int nblk = (T + width - 1) / width;
  const int cnt = (int)min((int64_t)max(keep_cnt[i], 0), keep_ld);
  const int32_t* ki = keep_idx + (size_t)i * keep_ld;
  for (int e = tid; e < cnt; e += 256) {
    const int c = ki[e];
    if (c < 0 || c >= nblk) continue;
    const int t1 = min(c * width + width - 1, last);
    for (int t = c * width; t <= t1; ++t) row[t] = 0;
  }
  for (int t = max(0, p - recent + 1) + tid; t <= last; t += 256) row[t] = 0;
}

hipError_t launch_fold_keep(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C,
                            int q_start, int T, int width, int recent, uint16_t* mask, int64_t mask_ld,
                            hipStream_t stream) {
  const bool vec = (mask_ld % 8) == 0 && (reinterpret_cast<uintptr_t>(mask) % 16) == 0;
  if (vec)
    hipLaunchKernelGGL(fold_keep_kernel<true>, dim3(C), dim3(256), 0, stream, keep_idx, keep_ld,
                       keep_cnt, q_start, T, width, recent, mask, mask_ld);
  else
    hipLaunchKernelGGL(fold_keep_kernel<false>, dim3(C), dim3(256), 0, stream, keep_idx, keep_ld,
                       keep_cnt, q_start, T, width, recent, mask, mask_ld);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fold_keep_bits: the same fold as bits (bit t % 32 of word t / 32 of a row set
// when key t is kept), for prefill_attn_dense_bits. One workgroup per query row;
// the row is built in LDS in segments of FOLD_SEG_WORDS words (cleared, then the
// kept ranges ORed in word by word, then copied out), so any T is taken.
// Bits of keys at or past T in the last word stay clear; words past the row's
// ceil(T/32) are untouched. grid = C, block = 256.
// ---------------------------------------------------------------------------
constexpr int FOLD_SEG_WORDS = 8192;   // 32 KB of LDS: 262,144 keys per segment

// OR the keys [a, b] (segment-relative, a <= b) into the segment's words
__device__ __forceinline__ void or_key_range(uint32_t* seg, int a, int b) {
  for (int w = a >> 5; w <= (b >> 5); ++w) {
    const int lo = max(a - 32 * w, 0), hi = min(b - 32 * w, 31);
    const uint32_t upto = hi == 31 ? 0xFFFFFFFFu : ((1u << (hi + 1)) - 1u);
    atomicOr(&seg[w], upto & ~((1u << lo) - 1u));
  }
}

__global__ void __launch_bounds__(256) fold_keep_bits_kernel(const int32_t* __restrict__ keep_idx,
                                                             int64_t keep_ld,
                                                             const int32_t* __restrict__ keep_cnt,
                                                             int q_start, int T, int width, int recent,
                                                             uint32_t* __restrict__ bits, int64_t bits_ld) {
  __shared__ uint32_t seg[FOLD_SEG_WORDS];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  uint32_t* row = bits + (size_t)i * bits_ld;
  const int p = q_start + i;
  const int last = min(p, T - 1);            // no key past the row's own position
  const int64_t nblk = ((int64_t)T + width - 1) / width;
  const int cnt = (int)min((int64_t)max(keep_cnt[i], 0), keep_ld);
  const int32_t* ki = keep_idx + (size_t)i * keep_ld;
  const int r_lo = max(0, p - recent + 1);   // the recent keys: r_lo .. last (none when recent == 0)
  const int nwords = (T + 31) / 32;
  for (int w0 = 0; w0 < nwords; w0 += FOLD_SEG_WORDS) {
    const int nw = min(FOLD_SEG_WORDS, nwords - w0);
    const int t_lo = 32 * w0, t_hi = min(T - 1, 32 * (w0 + nw) - 1);   // the segment's keys
    for (int w = tid; w < nw; w += 256) seg[w] = 0u;
    __syncthreads();
    for (int e = tid; e < cnt; e += 256) {
      const int c = ki[e];
      if (c < 0 || c >= nblk) continue;
      const int64_t k0 = (int64_t)c * width;
      const int a = (int)max(k0, (int64_t)t_lo);
      const int b = (int)min(min(k0 + width - 1, (int64_t)last), (int64_t)t_hi);
      if (a <= b) or_key_range(seg, a - t_lo, b - t_lo);
    }
    if (recent > 0) {
      // the recent range, one word per thread
      const int a = max(r_lo, t_lo), b = min(last, t_hi);
      if (a <= b)
        for (int w = (a - t_lo) / 32 + tid; w <= (b - t_lo) / 32; w += 256)
          or_key_range(seg, max(a - t_lo, 32 * w), min(b - t_lo, 32 * w + 31));
    }
    __syncthreads();
    for (int w = tid; w < nw; w += 256) row[w0 + w] = seg[w];
    __syncthreads();   // the segment is read out before it is cleared again
  }
}

hipError_t launch_fold_keep_bits(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C,
                                 int q_start, int T, int width, int recent, uint32_t* bits, int64_t bits_ld,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(fold_keep_bits_kernel, dim3(C), dim3(256), 0, stream, keep_idx, keep_ld, keep_cnt, q_start,
                     T, width, recent, bits, bits_ld);
  return hipGetLastError();
}

// mask_classify for a bit-packed mask: one workgroup per tile of 64 rows x 64 keys
// (64 rows x 2 words, one word per thread of the first 128); only the bits of
// keys below T count.
__global__ void __launch_bounds__(256) mask_classify_bits_kernel(const uint32_t* __restrict__ bits,
                                                                 int64_t ld, int C, int T,
                                                                 uint8_t* __restrict__ flags) {
  const int kt = blockIdx.x, qt = blockIdx.y;
  bool all_keep = true, all_drop = true;
  {
    const int p = threadIdx.x;
    const int r = qt * FLAG_ROWS + (p >> 1);
    const int wi = kt * (FLAG_KEYS / 32) + (p & 1);
    const int nvalid = min(max(T - 32 * wi, 0), 32);
    if (p < 2 * FLAG_ROWS && r < C && nvalid > 0) {
      const uint32_t vmask = nvalid == 32 ? ~0u : ((1u << nvalid) - 1u);
      const uint32_t w = bits[(size_t)r * ld + wi] & vmask;
      all_keep &= w == vmask;
      all_drop &= w == 0u;
    }
  }
  const int z = __syncthreads_and(all_keep);
  const int dr = __syncthreads_and(all_drop);
  if (threadIdx.x == 0)
    flags[(size_t)qt * gridDim.x + kt] = dr ? TILE_DROPPED : (z ? TILE_ZERO : TILE_MIXED);
}

hipError_t launch_mask_classify_bits(const uint32_t* bits, int64_t bits_ld, int C, int T,
                                     uint8_t* flags, hipStream_t stream) {
  const dim3 grid((T + FLAG_KEYS - 1) / FLAG_KEYS, (C + FLAG_ROWS - 1) / FLAG_ROWS);
  hipLaunchKernelGGL(mask_classify_bits_kernel, grid, dim3(256), 0, stream, bits, bits_ld, C, T, flags);
  return hipGetLastError();
}

hipError_t launch_mask_classify(const uint16_t* mask, int64_t mask_ld, int C, int T,
                                uint8_t* flags, hipStream_t stream) {
  const int n_ktile = (T + FLAG_KEYS - 1) / FLAG_KEYS;
  dim3 grid((n_ktile + CLS_TILES - 1) / CLS_TILES, (C + FLAG_ROWS - 1) / FLAG_ROWS);
  const bool vec = (mask_ld % 8) == 0 && (reinterpret_cast<uintptr_t>(mask) % 16) == 0;
  if (vec)
    hipLaunchKernelGGL(mask_classify_kernel<true>, grid, dim3(256), 0, stream, mask, mask_ld, C, T,
                       n_ktile, flags);
  else
    hipLaunchKernelGGL(mask_classify_kernel<false>, grid, dim3(256), 0, stream, mask, mask_ld, C, T,
                       n_ktile, flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// attn_combine: merge the partial (m, l, O) of the key-range splits of each
// (row, head). m is in log2 units and is the reference each split used for its
// weights: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max m_s over
// splits with l_s > 0. A row with no visible key in any split outputs zeros.
// part_o [splits][rows*heads][d], part_ml [splits][rows*heads][2].
// One thread per 4 output columns; block = 256.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) attn_combine_kernel(int rows, int d, int splits,
                                                           const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           float* __restrict__ O) {
  const int per_row = d / 4;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid / per_row;
  if (row >= rows) return;
  const int c = (gid % per_row) * 4;
  float M = -__builtin_inff();
  for (int s = 0; s < splits; ++s) {
    const float* ml = part_ml + ((size_t)s * rows + row) * 2;
    if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < splits; ++s) {
      const float* ml = part_ml + ((size_t)s * rows + row) * 2;
      if (!(ml[1] > 0.f)) continue;
      const float w = exp2f(ml[0] - M);
      L += w * ml[1];
      const float4 o = *reinterpret_cast<const float4*>(part_o + ((size_t)s * rows + row) * d + c);
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(O + (size_t)row * d + c) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

hipError_t launch_attn_combine(int C, int n_q, int d, int splits, const float* part_o,
                               const float* part_ml, float* O, hipStream_t stream) {
  const int rows = C * n_q;
  const long threads = (long)rows * (d / 4);
  const int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(blocks), dim3(256), 0, stream, rows, d, splits,
                     part_o, part_ml, O);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Value staging (see StagePlan): the PV products of the attention kernels run
// on fp16 MFMAs, so the softmax weights are rounded to fp16 (11 significant
// bits) rather than bf16 (8). Values are converted once per call, times a
// power of two 2^-k (k may be negative) chosen from max |V| so that the scaled
// maximum lies in [2^14, 2^15): bf16 -> fp16 is then exact for every value
// within 2^-28 of the maximum, and smaller ones lose at most 2^-25 absolutely in
// scaled units, 2^-39 of the maximum. The attention kernels multiply their
// outputs by 2^k.
//   stage_range_kernel: STAGE_PARTS workgroups, partial max of the bf16
//     magnitude bits (monotone in |v|) over a grid-strided share of V.
//   stage_convert_kernel: each workgroup reduces the partials to k, converts
//     its share; workgroup 0 writes scales = {2^-k, 2^k}.
// ---------------------------------------------------------------------------
constexpr int STAGE_THREADS = 256;
constexpr int STAGE_CONVERT_WG = 1024;

__device__ __forceinline__ uint32_t mag_max8(u32x4 v, uint32_t m) {
#pragma unroll
  for (int w = 0; w < 4; ++w) m = max(m, max(v[w] & 0x7FFFu, (v[w] >> 16) & 0x7FFFu));
  return m;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t m, uint32_t* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < STAGE_THREADS / 64; ++w) m = max(m, red[w]);
  return m;
}

__global__ void __launch_bounds__(STAGE_THREADS) stage_range_kernel(const u32x4* __restrict__ V, size_t n8,
                                                                     uint32_t* __restrict__ part) {
  __shared__ uint32_t red[STAGE_THREADS / 64];
  const size_t stride = (size_t)gridDim.x * STAGE_THREADS;
  size_t c = (size_t)blockIdx.x * STAGE_THREADS + threadIdx.x;
  uint32_t m = 0;
  for (; c + 3 * stride < n8; c += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = V[c + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) m = mag_max8(v[u], m);
  }
  for (; c < n8; c += stride) m = mag_max8(V[c], m);
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

__global__ void __launch_bounds__(STAGE_THREADS) stage_convert_kernel(const u32x4* __restrict__ V, size_t n8,
                                                                       const uint32_t* __restrict__ part,
                                                                       u32x4* __restrict__ V16,
                                                                       float* __restrict__ scales) {
  __shared__ uint32_t red[STAGE_THREADS / 64];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < STAGE_PARTS; i += STAGE_THREADS) m = max(m, part[i]);
  m = block_max_u32(m, red);
  // bf16 exponent field e of max |v| (max in [2^(e-127), 2^(e-126))): k = e - 141
  // puts the scaled max in [2^14, 2^15); clamped so both factors stay normal fp32
  // (an all-zero V takes the lower clamp, non-finite values the upper)
  const int e = (int)(m >> 7);
  const int k = min(max(e - 141, -100), 114);
  const float dn = __builtin_ldexpf(1.0f, -k);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    scales[0] = dn;
    scales[1] = __builtin_ldexpf(1.0f, k);
  }
  const size_t stride = (size_t)gridDim.x * STAGE_THREADS;
  for (size_t c = (size_t)blockIdx.x * STAGE_THREADS + threadIdx.x; c < n8; c += stride) {
    const u32x4 v = V[c];
    u32x4 h;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      h[w] = pack_f16x2(__uint_as_float(v[w] << 16) * dn, __uint_as_float(v[w] & 0xFFFF0000u) * dn);
    V16[c] = h;
  }
}

// Pooled operands of the block-sparse kernel, once per call: rows 0 .. nb-1 of
// K_pool and V_pool ([n_kv][pool_ld][d] fp32) rounded to nearest even, keys to
// bf16 and values times the staged values' factor to fp16, written token-major
// ([nb][n_kv][d]) like K and V, so that the attention kernel loads 64 pooled rows
// at a time straight into LDS as it does key and value tiles.
__global__ void __launch_bounds__(STAGE_THREADS) stage_pooled_kernel(const float* __restrict__ Kp,
                                                                      const float* __restrict__ Vp, int pool_ld,
                                                                      int nb, int n_kv, int d,
                                                                      const float* __restrict__ scales,
                                                                      u32x4* __restrict__ Kp16,
                                                                      u32x4* __restrict__ Vp16) {
  const float dn = scales[0];
  const int cpr = d / 8;   // 8-dim chunks per row
  const size_t n8 = (size_t)nb * n_kv * cpr;
  const size_t stride = (size_t)gridDim.x * STAGE_THREADS;
  for (size_t c = (size_t)blockIdx.x * STAGE_THREADS + threadIdx.x; c < n8; c += stride) {
    const size_t row = c / cpr;   // b * n_kv + g
    const int cc = (int)(c % cpr);
    const int b = (int)(row / n_kv), g = (int)(row % n_kv);
    const size_t src = ((size_t)g * pool_ld + b) * d + (size_t)cc * 8;
    const float4 k0 = *reinterpret_cast<const float4*>(Kp + src);
    const float4 k1 = *reinterpret_cast<const float4*>(Kp + src + 4);
    const float4 v0 = *reinterpret_cast<const float4*>(Vp + src);
    const float4 v1 = *reinterpret_cast<const float4*>(Vp + src + 4);
    Kp16[c] = u32x4{pack_bf16x2(k0.x, k0.y), pack_bf16x2(k0.z, k0.w), pack_bf16x2(k1.x, k1.y),
                    pack_bf16x2(k1.z, k1.w)};
    Vp16[c] = u32x4{pack_f16x2(v0.x * dn, v0.y * dn), pack_f16x2(v0.z * dn, v0.w * dn),
                    pack_f16x2(v1.x * dn, v1.y * dn), pack_f16x2(v1.z * dn, v1.w * dn)};
  }
}

static size_t align256_s(size_t x) { return (x + 255) & ~(size_t)255; }

StagePlan plan_stage(int T, int n_kv, int d, int pool_rows) {
  StagePlan p{};
  p.v16_off = 0;
  p.part_off = align256_s((size_t)T * n_kv * d * 2);
  p.scales_off = p.part_off + align256_s(STAGE_PARTS * sizeof(uint32_t));
  p.kp16_off = p.scales_off + 256;
  p.vp16_off = p.kp16_off + align256_s((size_t)pool_rows * n_kv * d * 2);
  p.bytes = p.vp16_off + align256_s((size_t)pool_rows * n_kv * d * 2);
  return p;
}

hipError_t launch_stage_pooled(const float* K_pool, const float* V_pool, int pool_ld, int nb, int n_kv, int d,
                               void* stage, const StagePlan& plan, hipStream_t stream) {
  uint8_t* base = static_cast<uint8_t*>(stage);
  const size_t n8 = (size_t)nb * n_kv * d / 8;
  const int wgs = (int)std::min<size_t>((n8 + STAGE_THREADS - 1) / STAGE_THREADS, STAGE_CONVERT_WG);
  hipLaunchKernelGGL(stage_pooled_kernel, dim3(std::max(wgs, 1)), dim3(STAGE_THREADS), 0, stream, K_pool, V_pool,
                     pool_ld, nb, n_kv, d, reinterpret_cast<const float*>(base + plan.scales_off),
                     reinterpret_cast<u32x4*>(base + plan.kp16_off), reinterpret_cast<u32x4*>(base + plan.vp16_off));
  return hipGetLastError();
}

hipError_t launch_stage_values(const uint16_t* V, int T, int n_kv, int d, void* stage, hipStream_t stream) {
  const StagePlan p = plan_stage(T, n_kv, d);
  uint8_t* base = static_cast<uint8_t*>(stage);
  const size_t n8 = (size_t)T * n_kv * d / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(V);
  uint32_t* part = reinterpret_cast<uint32_t*>(base + p.part_off);
  hipLaunchKernelGGL(stage_range_kernel, dim3(STAGE_PARTS), dim3(STAGE_THREADS), 0, stream, src, n8, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stage_convert_kernel, dim3(STAGE_CONVERT_WG), dim3(STAGE_THREADS), 0, stream, src, n8, part,
                     reinterpret_cast<u32x4*>(base + p.v16_off), reinterpret_cast<float*>(base + p.scales_off));
  return hipGetLastError();
}

}  // namespace pa
