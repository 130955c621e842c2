// Attention over a folded sparse-indexer selection by gathering the kept keys
// ("ANE Prefill Research", What worked, item 2: the indexer's compacted
// selection, keepIndices / keepCounts, names per query row the blocks of keys the
// row keeps; and "What would re-open it": score only the kept keys instead of
// masking the whole history). The result is the dense attention under the mask
// that fold_keep_mask builds from the same lists; here no mask is formed and the
// cost grows with the kept keys per row, not with the history.
//
// gfx950 mapping. One wave per (query row, KV head); the row's kept keys are
// the same for every query head of the group (one mask for all heads), and the
// rows of a chunk keep unrelated key sets, so there is no key tile for the
// matrix cores to share: the products run on the VALU in fp32.
//   * The row's listed blocks are deduplicated through a bitmap in the wave's
//     LDS slice (atomic OR), then compacted in ascending block order into a list
//     there; the `recent` keys ending at the row's position follow, skipping those
//     that a listed block already covers.
//   * Keys are taken 64 at a time (one per lane): the lane's score is its own
//     dot product over the row of K (fp32, dims in increasing order); then an
//     online softmax over the wave (running max, weights exp2 in fp32); then the
//     lanes switch to dims for P V: for each kept key of the 64, its weight and
//     key index are read out of the lane that holds them and every lane adds the
//     weight times its dims of the key's V row.
//   * Query heads of the group are done one after the other (the K and V rows of
//     the row's keys come from cache the second time).
#include <algorithm>
#include <cmath>

#include "common.h"

namespace pa {

constexpr int GATHER_MAX_WAVES = 4;

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// this wave's LDS operations have completed and are visible to all its lanes
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vector-memory and export counts untouched
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ void __launch_bounds__(64 * GATHER_MAX_WAVES) gather_attn_kernel(
    const uint16_t* __restrict__ Q, int C, int q_start, int n_q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int T, int n_kv, const int32_t* __restrict__ keep_idx,
    int64_t keep_ld, const int32_t* __restrict__ keep_cnt, int width, int recent, int words_cap,
    int list_cap, float scale_log2, float* __restrict__ O) {
  constexpr int DPL = D / 64;   // dims per lane in the P V product
  extern __shared__ uint32_t gsm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int task = (int)blockIdx.x * ((int)blockDim.x >> 6) + wave;
  if (task >= C * n_kv) return;   // waves are independent: no workgroup barrier below
  const int i = task / n_kv, g = task % n_kv;
  const int group = n_q / n_kv;
  uint32_t* bm = gsm + (size_t)wave * (words_cap + list_cap);
  int32_t* list = reinterpret_cast<int32_t*>(bm + words_cap);

  const int p = q_start + i;                  // the row's position; keys t <= p are its past
  const int nbv = p / width + 1;              // blocks holding keys <= p
  const int nw = (nbv + 31) >> 5;

  // 1) listed blocks, deduplicated: bitmap, then ascending list
  for (int w = lane; w < nw; w += 64) bm[w] = 0u;
  wave_lds_sync();
  const int cnt = (int)min((int64_t)max(keep_cnt[i], 0), keep_ld);
  const int32_t* kl = keep_idx + (size_t)i * (size_t)keep_ld;
  for (int e = lane; e < cnt; e += 64) {
    const int b = kl[e];
    if (b >= 0 && b < nbv) atomicOr(&bm[b >> 5], 1u << (b & 31));
  }
  wave_lds_sync();
  int nlist = 0;
  for (int w0 = 0; w0 < nw; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t word = w < nw ? bm[w] : 0u;
    const int c = __popc(word);
    int incl = c;   // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int pos = nlist + incl - c;
    for (uint32_t x = word; x != 0u; x &= x - 1u) list[pos++] = w * 32 + __builtin_ctz(x);
    nlist += __shfl(incl, 63);
  }
  wave_lds_sync();

  // 2) the row's keys: the listed blocks' keys up to p, then the recent keys not
  // in a listed block
  const int nl = nlist * width;
  const int rlo = max(0, p - recent + 1);
  const int nrec = recent > 0 ? p - rlo + 1 : 0;
  const int ns = nl + nrec;
  auto key_of = [&](int s, bool& ok) {
    int key;
    if (s < nl) {
      const int blk = list[s / width];
      key = blk * width + s % width;
      ok = key <= p;
    } else {
      key = rlo + (s - nl);
      ok = s < ns && !((bm[key / width >> 5] >> ((key / width) & 31)) & 1u);
    }
    return ok ? key : 0;
  };

  const size_t krow = (size_t)n_kv * D;   // elements between consecutive keys
  const uint16_t* kg = K + (size_t)g * D;
  const uint16_t* vg = V + (size_t)g * D;
  for (int hh = 0; hh < group; ++hh) {
    const int head = g * group + hh;
    // q as fp32 pairs held by every lane (the same row for all lanes)
    const uint16_t* qp = Q + ((size_t)i * n_q + head) * D;
    float q[D];
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 r = *reinterpret_cast<const u32x4*>(qp + 8 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        q[8 * c + 2 * w] = __uint_as_float(r[w] << 16);
        q[8 * c + 2 * w + 1] = __uint_as_float(r[w] & 0xFFFF0000u);
      }
    }
    float m = -__builtin_inff(), lsum = 0.f;
    float o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      bool ok = false;
      const int key = key_of(s0 + lane, ok);
      float sc = -__builtin_inff();
      if (ok) {
        const uint16_t* kp = kg + (size_t)key * krow;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
          const u32x4 r = *reinterpret_cast<const u32x4*>(kp + 8 * c);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc = __builtin_fmaf(q[8 * c + 2 * w], __uint_as_float(r[w] << 16), acc);
            acc = __builtin_fmaf(q[8 * c + 2 * w + 1], __uint_as_float(r[w] & 0xFFFF0000u), acc);
          }
        }
        sc = acc * scale_log2;
      }
      const float cm = wave_max_f(sc);
      if (cm == -__builtin_inff()) continue;   // no key of this slice is the row's
      const float m_new = fmaxf(m, cm);
      const float alpha = m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] *= alpha;
      lsum *= alpha;
      m = m_new;
      const float pw = ok ? __builtin_amdgcn_exp2f(sc - m) : 0.f;
      lsum += pw;
      // P V: lanes over dims (lane l: dims l*DPL .. l*DPL + DPL-1), the slice's
      // keys eight at a time with their V loads issued together (a key that is
      // not the row's has weight 0 and reads row 0)
      const int kq = ok ? key : 0;
#pragma unroll 1
      for (int k0 = 0; k0 < 64; k0 += 8) {
        uint32_t r[8];
        float pk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kk = __builtin_amdgcn_readlane(kq, k0 + u);
          pk[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pw), k0 + u));
          const uint16_t* vp = vg + (size_t)kk * krow + lane * DPL;
          r[u] = DPL == 2 ? *reinterpret_cast<const uint32_t*>(vp) : (uint32_t)vp[0];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (DPL == 2) {
            o[0] = __builtin_fmaf(pk[u], __uint_as_float(r[u] << 16), o[0]);
            o[DPL - 1] = __builtin_fmaf(pk[u], __uint_as_float(r[u] & 0xFFFF0000u), o[DPL - 1]);
          } else {
            o[0] = __builtin_fmaf(pk[u], __uint_as_float(r[u] << 16), o[0]);
          }
        }
      }
    }
    const float l = wave_sum_f(lsum);
    const float inv = l > 0.f ? 1.f / l : 0.f;   // a row with no kept key outputs zeros
    float* op = O + ((size_t)i * n_q + head) * D + lane * DPL;
    if (DPL == 2) {
      *reinterpret_cast<float2*>(op) = make_float2(o[0] * inv, o[DPL - 1] * inv);
    } else {
      op[0] = o[0] * inv;
    }
  }
}

GatherPlan plan_gather(int T, int64_t keep_ld, int width) {
  GatherPlan pl{};
  const int nb = (T - 1) / width + 1;
  pl.words_cap = (nb + 31) / 32;
  pl.list_cap = (int)std::max<int64_t>(1, std::min<int64_t>(keep_ld, nb));
  const size_t per_wave = (size_t)(pl.words_cap + pl.list_cap) * 4;
  const size_t lds_max = 160 * 1024;
  pl.waves = (int)std::min<size_t>(GATHER_MAX_WAVES, lds_max / per_wave);
  pl.lds_bytes = per_wave * (size_t)std::max(pl.waves, 1);
  return pl;
}

hipError_t launch_gather_attn(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                              const uint16_t* V, int T, int n_kv, int d, const int32_t* keep_idx,
                              int64_t keep_ld, const int32_t* keep_cnt, int width, int recent,
                              float scale, float* O, const GatherPlan& pl, hipStream_t stream) {
  const int tasks = C * n_kv;
  dim3 grid((tasks + pl.waves - 1) / pl.waves), block(64 * pl.waves);
  const float scale_log2 = scale * 1.4426950408889634f;
  if (d == 128) {
    hipFuncSetAttribute((const void*)gather_attn_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)pl.lds_bytes);
    hipLaunchKernelGGL(gather_attn_kernel<128>, grid, block, pl.lds_bytes, stream, Q, C, q_start, n_q, K,
                       V, T, n_kv, keep_idx, keep_ld, keep_cnt, width, recent, pl.words_cap, pl.list_cap,
                       scale_log2, O);
  } else {
    hipFuncSetAttribute((const void*)gather_attn_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)pl.lds_bytes);
    hipLaunchKernelGGL(gather_attn_kernel<64>, grid, block, pl.lds_bytes, stream, Q, C, q_start, n_q, K,
                       V, T, n_kv, keep_idx, keep_ld, keep_cnt, width, recent, pl.words_cap, pl.list_cap,
                       scale_log2, O);
  }
  return hipGetLastError();
}

}  // namespace pa
