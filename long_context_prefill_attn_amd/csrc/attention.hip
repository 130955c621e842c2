// Tiled prefill attention for gfx950 (MI355X): dense chunked attention under an
// additive mask, and block-sparse attention with a pooled correction.
//
// Method: FlashAttention-style tiling with an online softmax ("Flash attention
// on ANE: fast long-context prefill", section "Flash attention: the core
// insight"): for each tile of queries, walk tiles of keys, keep a running max
// and sum per query row, and accumulate weighted values; the score matrix is
// never written out. The mask is added to the scaled scores before the softmax
// and an entry <= -30000 omits its key ("ANE Prefill Research", How the ANE
// prefill path works; What worked, item 2).
//
// gfx950 mapping (one workgroup = 4 waves = 128 query rows of one query head):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = a 32-key slice of the K tile
//     (LDS), B = Q^T held in registers for the whole kernel. The accumulator
//     puts query n = lane%32 in every lane, so each lane owns the softmax state
//     of one query row; the row's other 16 keys of a 32-key slice sit in lane
//     l^32 and one v_permlane32_swap completes each row reduction.
//   * O^T = V^T P^T on the same MFMA: A = V^T from LDS (V is transposed while
//     it is staged), B = P^T straight from the S^T accumulators (packed to
//     bf16), so P never leaves registers and O^T lands with the row's head_dim
//     values in the lane that owns the row's softmax state.
//   * K/V tiles of 64 keys are double-buffered in LDS; the next tile's global
//     loads are in flight while the current tile is computed.
//   * Softmax in exp2 units with log2(e) folded into the scale. The running max
//     is raised only when it grows by more than 2^8 (all weights stay <= 256),
//     so the O rescale is rare; results are exact up to rounding either way.
//   * Workgroup ids are remapped so that the workgroups of one query head run
//     on one XCD (shared L2 for that KV head), longest query tiles first.
#include <algorithm>

#include "common.h"

namespace pa {

constexpr int BM = 128;         // query rows per workgroup
constexpr int BN = 64;          // keys per inner step
constexpr int NT = 256;         // threads per workgroup (4 waves)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float SLACK = 8.0f;   // lazy-rescale threshold in log2 units

enum { MODE_PLAIN = 0, MODE_GMASK = 1, MODE_CAUSAL = 2, MODE_POOLED = 3 };

template <int D>
struct Geo {
  static constexpr int KP = D + 8;               // K row pitch in halves (16-byte pad)
  static constexpr int VP = BN + 4;              // V^T row pitch in halves (8-byte pad)
  static constexpr int KH = BN * KP;             // halves of one K tile
  static constexpr int VH = D * VP;              // halves of one V^T tile
  static constexpr int STAGE = KH + VH;
  static constexpr size_t LDS_BYTES = 2 * STAGE * sizeof(uint16_t);
  static constexpr int KCH = BN * D / 8 / NT;    // 16-byte K chunks per thread
  static constexpr int VUNITS = 2 * D;           // (4 keys x 8 dims) V units per tile
};

// ---------------------------------------------------------------------------
// global -> register -> LDS staging of a 64-key K/V tile of KV head g
// ---------------------------------------------------------------------------
template <int D>
struct KVRegs {
  u32x4 k[Geo<D>::KCH];
  u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_kv(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                        int T, int n_kv, int g, int kbase, KVRegs<D>& r) {
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;  // 16-byte chunks per key row
#pragma unroll
  for (int i = 0; i < Geo<D>::KCH; ++i) {
    const int c = tid + NT * i;
    const int t = kbase + c / CPR;
    r.k[i] = (t < T) ? *reinterpret_cast<const u32x4*>(K + ((size_t)t * n_kv + g) * D + (c % CPR) * 8)
                     : u32x4{0, 0, 0, 0};
  }
  if (tid < Geo<D>::VUNITS) {
    const int kg = tid % 16, col = tid / 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = kbase + 4 * kg + q;
      r.v[q] = (t < T) ? *reinterpret_cast<const u32x4*>(V + ((size_t)t * n_kv + g) * D + col * 8)
                       : u32x4{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_kv(uint16_t* ks, uint16_t* vts, const KVRegs<D>& r) {
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < Geo<D>::KCH; ++i) {
    const int c = tid + NT * i;
    *reinterpret_cast<u32x4*>(ks + (c / CPR) * Geo<D>::KP + (c % CPR) * 8) = r.k[i];
  }
  if (tid < Geo<D>::VUNITS) {
    const int kg = tid % 16, col = tid / 16;
    // transpose 4 keys x 8 dims -> 8 dims x 4 keys
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a0 = r.v[0][w], a1 = r.v[1][w], a2 = r.v[2][w], a3 = r.v[3][w];
      const u32x2 even = {(a0 & 0xFFFFu) | (a1 << 16), (a2 & 0xFFFFu) | (a3 << 16)};
      const u32x2 odd = {(a0 >> 16) | (a1 & 0xFFFF0000u), (a2 >> 16) | (a3 & 0xFFFF0000u)};
      const int d0 = col * 8 + 2 * w;
      *reinterpret_cast<u32x2*>(vts + d0 * Geo<D>::VP + 4 * kg) = even;
      *reinterpret_cast<u32x2*>(vts + (d0 + 1) * Geo<D>::VP + 4 * kg) = odd;
    }
  }
}

// ---------------------------------------------------------------------------
// one 64-key step for the wave's 32 query rows
// ---------------------------------------------------------------------------
struct StepCtx {
  float scale_log2;
  int kvalid;                        // keys of the step inside [0, T)
  const uint16_t* __restrict__ mrow; // MODE_GMASK: mask row of this lane's query (may be null)
  int key0;                          // absolute key (or pooled block) index of the step's first key
  int qpos;                          // MODE_CAUSAL: absolute position of this lane's query
  const uint32_t* selbits;           // MODE_POOLED: selected-block bitmap (LDS)
  int jlimit;                        // MODE_POOLED: pooled rows exist only for blocks < jlimit
  float pool_bias;                   // MODE_POOLED: log2(block)
};

template <int D>
__device__ __forceinline__ f32x16 qk_slice(const uint16_t* __restrict__ kp, const bf16x8 (&qf)[D / 16]) {
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + 16 * st);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s, 0, 0, 0);
  }
  return s;
}

template <int D, int MODE>
__device__ __forceinline__ void attn_step(const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vts,
                                          const uint16_t* __restrict__ ks2,
                                          const uint16_t* __restrict__ vts2,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32], float& m,
                                          float& l, const StepCtx& cx) {
  const int lane = __lane_id();
  const int n = lane & 31, h = lane >> 5;
  constexpr int KP = Geo<D>::KP, VP = Geo<D>::VP;

  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int off = (kb * 32 + n) * KP + 8 * h;
    s[kb] = qk_slice<D>(ks + off, qf);
    if (MODE == MODE_POOLED) {
      const f32x16 s2 = qk_slice<D>(ks2 + off, qf);
      s[kb] += s2;
    }
  }

  // scale, mask, row max. Element i of slice kb holds key kb*32 + 8*(i/4) + 4*h + i%4.
  float x[2][16];
  float mx = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      float v = s[kb][i] * cx.scale_log2;
      if (MODE == MODE_GMASK) {
        uint16_t mv = 0;
        if (cx.mrow != nullptr && kk < cx.kvalid) mv = cx.mrow[cx.key0 + kk];
        v = f16_dropped(mv) ? -__builtin_inff() : __builtin_fmaf((float)__builtin_bit_cast(_Float16, mv), LOG2E, v);
      } else if (MODE == MODE_CAUSAL) {
        if (cx.key0 + kk > cx.qpos) v = -__builtin_inff();
      } else if (MODE == MODE_POOLED) {
        const int b = cx.key0 + kk;
        const bool live = b < cx.jlimit && !((cx.selbits[b >> 5] >> (b & 31)) & 1u);
        v = live ? v + cx.pool_bias : -__builtin_inff();
      }
      if (kk >= cx.kvalid) v = -__builtin_inff();
      x[kb][i] = v;
      mx = fmaxf(mx, v);
    }
  }
  mx = fmaxf(mx, partner32(mx));
  const float m_new = fmaxf(m, mx);
  if (__any(m_new > m + SLACK)) {
    const float alpha = (m_new == -__builtin_inff()) ? 1.f : exp2f(m - m_new);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
    l *= alpha;
    m = m_new;
  }
  const float mu = (m == -__builtin_inff()) ? 0.f : m;

  // P = 2^(x - m), packed to bf16 in MFMA B-operand order
  u32x4 P[2][2];
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(x[kb][8 * c + 2 * w] - mu);
        const float p1 = __builtin_amdgcn_exp2f(x[kb][8 * c + 2 * w + 1] - mu);
        psum += p0 + p1;
        P[kb][c][w] = pack_bf16x2(p0, p1);
      }
    }
  }
  l += psum;

  // O^T += V^T P^T. Slot 8h+i' of MFMA c holds key 16c + 8*(i'/4) + 4h + i'%4.
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    const int voff = (nb * 32 + n) * VP + 4 * h;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ko = voff + kb * 32 + 16 * c;
        const bf16x8 b = __builtin_bit_cast(bf16x8, P[kb][c]);
        {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vts + ko);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vts + ko + 8);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), b, o[nb], 0, 0, 0);
        }
        if (MODE == MODE_POOLED) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vts2 + ko);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vts2 + ko + 8);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
          o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), b, o[nb], 0, 0, 0);
        }
      }
    }
  }
}

// load this wave's 32 query rows as the B operand: lane holds Q[row n][dims 16st+8h .. +7]
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* __restrict__ Q, int n_q, int head, int qrow,
                                       bool valid, bf16x8 (&qf)[D / 16]) {
  const int h = __lane_id() >> 5;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    u32x4 v = {0, 0, 0, 0};
    if (valid) v = *reinterpret_cast<const u32x4*>(Q + ((size_t)qrow * n_q + head) * D + 16 * st + 8 * h);
    qf[st] = __builtin_bit_cast(bf16x8, v);
  }
}

// write O (normalised) or the split partials for this wave's 32 rows
template <int D>
__device__ __forceinline__ void store_rows(float* __restrict__ dst, const f32x16 (&o)[D / 32], float scale) {
  const int h = __lane_id() >> 5;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = nb * 32 + 8 * r + 4 * h;
      *reinterpret_cast<float4*>(dst + d) =
          make_float4(o[nb][4 * r] * scale, o[nb][4 * r + 1] * scale, o[nb][4 * r + 2] * scale,
                      o[nb][4 * r + 3] * scale);
    }
  }
}

__device__ __forceinline__ int remap_xcd(int bid, int nblk) {
  // dispatch sends consecutive workgroup ids to consecutive XCDs (round robin over 8);
  // give each XCD a contiguous range of logical ids instead
  if ((nblk & 7) == 0) return (bid & 7) * (nblk >> 3) + (bid >> 3);
  return bid;
}

// ---------------------------------------------------------------------------
// dense chunked prefill attention
// ---------------------------------------------------------------------------
template <int D, bool SPLIT>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
attn_dense_kernel(const uint16_t* __restrict__ Q, int C, int n_q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, int T, int n_kv, const uint16_t* __restrict__ mask,
                  int64_t mask_ld, float scale_log2, float* __restrict__ O,
                  const uint8_t* __restrict__ flags, int n_qt, int n_ktile, int splits,
                  float* __restrict__ part_o, float* __restrict__ part_ml) {
  extern __shared__ uint16_t lds[];
  __shared__ int s_lo, s_hi;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, n = lane & 31;

  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  const int per_head = n_qt * splits;
  const int head = bid / per_head;
  const int rem = bid % per_head;
  const int qt = n_qt - 1 - rem / splits;
  const int split = rem % splits;
  const int g = head / (n_q / n_kv);
  const uint8_t* frow = flags + (size_t)qt * n_ktile;

  // key range of this query tile: first..last tile that is not fully dropped
  if (tid == 0) { s_lo = n_ktile; s_hi = 0; }
  __syncthreads();
  for (int t = tid; t < n_ktile; t += NT) {
    if (frow[t] != TILE_DROPPED) { atomicMin(&s_lo, t); atomicMax(&s_hi, t + 1); }
  }
  __syncthreads();
  const int n_steps = (T + BN - 1) / BN;
  const int st_lo = s_lo * (FLAG_TILE / BN);
  const int st_hi = min(s_hi * (FLAG_TILE / BN), n_steps);
  const int len = max(st_hi - st_lo, 0);
  const int a = st_lo + (int)((long)len * split / splits);
  const int b = st_lo + (int)((long)len * (split + 1) / splits);

  const int qrow = qt * BM + wave * 32 + n;
  const bool qvalid = qrow < C;
  bf16x8 qf[D / 16];
  load_q<D>(Q, n_q, head, qrow, qvalid, qf);

  f32x16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;

  StepCtx cx;
  cx.scale_log2 = scale_log2;
  cx.mrow = qvalid ? mask + (size_t)qrow * mask_ld : nullptr;
  cx.qpos = 0; cx.selbits = nullptr; cx.jlimit = 0; cx.pool_bias = 0.f;

  auto next_live = [&](int s) {
    while (s < b && frow[s / (FLAG_TILE / BN)] == TILE_DROPPED) ++s;
    return s;
  };

  KVRegs<D> regs;
  int s = next_live(a);
  if (s < b) {
    load_kv<D>(K, V, T, n_kv, g, s * BN, regs);
    store_kv<D>(lds, lds + Geo<D>::KH, regs);
  }
  __syncthreads();
  int cur = 0;
  while (s < b) {
    const int nx = next_live(s + 1);
    if (nx < b) load_kv<D>(K, V, T, n_kv, g, nx * BN, regs);
    const uint16_t* ks = lds + cur * Geo<D>::STAGE;
    const uint16_t* vts = ks + Geo<D>::KH;
    cx.key0 = s * BN;
    cx.kvalid = min(BN, T - s * BN);
    if (frow[s / (FLAG_TILE / BN)] == TILE_MIXED)
      attn_step<D, MODE_GMASK>(ks, vts, nullptr, nullptr, qf, o, m, l, cx);
    else
      attn_step<D, MODE_PLAIN>(ks, vts, nullptr, nullptr, qf, o, m, l, cx);
    if (nx < b) {
      uint16_t* kn = lds + (cur ^ 1) * Geo<D>::STAGE;
      store_kv<D>(kn, kn + Geo<D>::KH, regs);
    }
    __syncthreads();
    cur ^= 1;
    s = nx;
  }

  const float lt = l + partner32(l);
  if (!qvalid) return;
  const size_t row = (size_t)qrow * n_q + head;
  if (SPLIT) {
    const size_t rows = (size_t)C * n_q;
    store_rows<D>(part_o + ((size_t)split * rows + row) * D, o, 1.f);
    if (lane < 32) {
      float2* ml = reinterpret_cast<float2*>(part_ml + ((size_t)split * rows + row) * 2);
      *ml = make_float2(m == -__builtin_inff() ? 0.f : m, lt);
    }
  } else {
    store_rows<D>(O + row * D, o, lt > 0.f ? 1.f / lt : 0.f);
  }
}

// ---------------------------------------------------------------------------
// block-sparse prefill attention: one workgroup per (query block of 128
// positions, query head). Exact steps over the selected key blocks (the
// diagonal block causally), then the pooled rows of the unselected visible
// blocks with multiplicity `block` ("Porting FlashPrefill V2 to Apple
// silicon", Compute the peaks, summarize the rest). Pooled keys/values are fp32;
// they enter the bf16 MFMA as hi + lo bf16 pairs (about 16 significant bits).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void split_hi_lo(float f, uint16_t& hi, uint16_t& lo) {
  const uint32_t hb = pack_bf16x2(f, 0.f) & 0xFFFFu;
  const float rest = f - __uint_as_float(hb << 16);
  hi = (uint16_t)hb;
  lo = (uint16_t)(pack_bf16x2(rest, 0.f) & 0xFFFFu);
}

template <int D>
__device__ __forceinline__ void stage_pooled(const float* __restrict__ Kp, const float* __restrict__ Vp,
                                             int nb, int g, int pbase, int jlimit, uint16_t* khi,
                                             uint16_t* klo, uint16_t* vhi, uint16_t* vlo) {
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;
  const float* kg = Kp + (size_t)g * nb * D;
  const float* vg = Vp + (size_t)g * nb * D;
#pragma unroll
  for (int i = 0; i < Geo<D>::KCH; ++i) {
    const int c = tid + NT * i;
    const int key = c / CPR, col = (c % CPR) * 8;
    const int bb = pbase + key;
    uint16_t hv[8], lv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = (bb < jlimit) ? kg[(size_t)bb * D + col + e] : 0.f;
      split_hi_lo<D>(f, hv[e], lv[e]);
    }
    u32x4 H, L;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      H[w] = hv[2 * w] | ((uint32_t)hv[2 * w + 1] << 16);
      L[w] = lv[2 * w] | ((uint32_t)lv[2 * w + 1] << 16);
    }
    *reinterpret_cast<u32x4*>(khi + key * Geo<D>::KP + col) = H;
    *reinterpret_cast<u32x4*>(klo + key * Geo<D>::KP + col) = L;
  }
  if (tid < Geo<D>::VUNITS) {
    const int kg4 = tid % 16, col = (tid / 16) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t hv[4], lv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int bb = pbase + 4 * kg4 + q;
        const float f = (bb < jlimit) ? vg[(size_t)bb * D + col + e] : 0.f;
        split_hi_lo<D>(f, hv[q], lv[q]);
      }
      const u32x2 H = {hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16)};
      const u32x2 L = {lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16)};
      *reinterpret_cast<u32x2*>(vhi + (col + e) * Geo<D>::VP + 4 * kg4) = H;
      *reinterpret_cast<u32x2*>(vlo + (col + e) * Geo<D>::VP + 4 * kg4) = L;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
attn_blocksparse_kernel(const uint16_t* __restrict__ Q, int C, int q_start, int n_q,
                        const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, int T,
                        int n_kv, const float* __restrict__ Kp, const float* __restrict__ Vp,
                        int nb, int n_qblk, const int32_t* __restrict__ sel_idx,
                        const int32_t* __restrict__ sel_cnt, float scale_log2, float* __restrict__ O) {
  extern __shared__ uint16_t lds[];
  __shared__ uint32_t selbits[256];  // up to 8192 blocks
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, n = lane & 31;
  constexpr int BLK = 128;

  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  const int head = bid / n_qblk;
  const int jj = n_qblk - 1 - bid % n_qblk;
  const int j = q_start / BLK + jj;
  const int g = head / (n_q / n_kv);
  const int32_t* sl = sel_idx + ((size_t)g * n_qblk + jj) * nb;
  const int cnt = sel_cnt[(size_t)g * n_qblk + jj];

  const int nwords = (nb + 31) / 32;
  for (int w = tid; w < nwords; w += NT) selbits[w] = 0;
  __syncthreads();
  for (int e = tid; e < cnt; e += NT) {
    const int bb = sl[e];
    atomicOr(&selbits[bb >> 5], 1u << (bb & 31));
  }

  const int qpos = j * BLK + wave * 32 + n;
  const bool qvalid = qpos >= q_start && qpos < q_start + C;
  const int qrow = qpos - q_start;
  bf16x8 qf[D / 16];
  load_q<D>(Q, n_q, head, qrow, qvalid, qf);

  f32x16 o[D / 32];
#pragma unroll
  for (int q = 0; q < D / 32; ++q) o[q] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;

  StepCtx cx;
  cx.scale_log2 = scale_log2;
  cx.mrow = nullptr;
  cx.qpos = qpos;
  cx.selbits = selbits;
  cx.jlimit = j;
  cx.pool_bias = __builtin_log2f((float)BLK);

  // exact steps: two 64-key steps per selected block
  const int n_ex = 2 * cnt;
  KVRegs<D> regs;
  if (n_ex > 0) {
    load_kv<D>(K, V, T, n_kv, g, sl[0] * BLK, regs);
    store_kv<D>(lds, lds + Geo<D>::KH, regs);
  }
  __syncthreads();
  int cur = 0;
  for (int e = 0; e < n_ex; ++e) {
    const int kbase = sl[e >> 1] * BLK + (e & 1) * BN;
    if (e + 1 < n_ex) load_kv<D>(K, V, T, n_kv, g, sl[(e + 1) >> 1] * BLK + ((e + 1) & 1) * BN, regs);
    const uint16_t* ks = lds + cur * Geo<D>::STAGE;
    const uint16_t* vts = ks + Geo<D>::KH;
    cx.key0 = kbase;
    cx.kvalid = min(BN, T - kbase);
    if (kbase >= j * BLK)
      attn_step<D, MODE_CAUSAL>(ks, vts, nullptr, nullptr, qf, o, m, l, cx);
    else
      attn_step<D, MODE_PLAIN>(ks, vts, nullptr, nullptr, qf, o, m, l, cx);
    if (e + 1 < n_ex) {
      uint16_t* kn = lds + (cur ^ 1) * Geo<D>::STAGE;
      store_kv<D>(kn, kn + Geo<D>::KH, regs);
    }
    __syncthreads();
    cur ^= 1;
  }

  // pooled rows of the unselected visible blocks b < j, 64 per step
  uint16_t* khi = lds;
  uint16_t* vhi = lds + Geo<D>::KH;
  uint16_t* klo = lds + Geo<D>::STAGE;
  uint16_t* vlo = klo + Geo<D>::KH;
  for (int pbase = 0; pbase < j; pbase += BN) {
    stage_pooled<D>(Kp, Vp, nb, g, pbase, j, khi, klo, vhi, vlo);
    __syncthreads();
    cx.key0 = pbase;
    cx.kvalid = min(BN, j - pbase);
    attn_step<D, MODE_POOLED>(khi, vhi, klo, vlo, qf, o, m, l, cx);
    __syncthreads();
  }

  const float lt = l + partner32(l);
  if (!qvalid) return;
  store_rows<D>(O + ((size_t)qrow * n_q + head) * D, o, lt > 0.f ? 1.f / lt : 0.f);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int num_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DensePlan plan_dense(int C, int T, int n_q, int n_kv, int d) {
  (void)n_kv;
  DensePlan p{};
  p.n_qt = (C + BM - 1) / BM;
  p.n_ktile = (T + FLAG_TILE - 1) / FLAG_TILE;
  const long wgs = (long)p.n_qt * n_q;
  const int target = 2 * num_cus();             // two resident workgroups per CU
  const int n_steps = (T + BN - 1) / BN;
  int splits = 1;
  if (wgs < target) splits = (int)((target + wgs - 1) / wgs);
  splits = std::max(1, std::min(splits, n_steps / 4));  // at least 4 steps (256 keys) per split
  splits = std::min(splits, 32);
  p.splits = splits;
  p.flags_bytes = align256((size_t)p.n_qt * p.n_ktile);
  if (splits > 1) {
    p.part_o_bytes = align256((size_t)splits * C * n_q * d * sizeof(float));
    p.part_ml_bytes = align256((size_t)splits * C * n_q * 2 * sizeof(float));
  }
  p.total_bytes = p.flags_bytes + p.part_o_bytes + p.part_ml_bytes;
  return p;
}

template <int D>
static hipError_t dense_impl(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V,
                             int T, int n_kv, const uint16_t* mask, int64_t mask_ld, float scale,
                             float* O, const DensePlan& p, const uint8_t* flags, float* part_o,
                             float* part_ml, hipStream_t stream) {
  const float sl2 = scale * LOG2E;
  const int grid = p.n_qt * n_q * p.splits;
  const size_t lds = Geo<D>::LDS_BYTES;
  if (p.splits > 1) {
    hipFuncSetAttribute((const void*)attn_dense_kernel<D, true>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((attn_dense_kernel<D, true>), dim3(grid), dim3(NT), lds, stream, Q, C, n_q, K, V,
                       T, n_kv, mask, mask_ld, sl2, O, flags, p.n_qt, p.n_ktile, p.splits, part_o,
                       part_ml);
  } else {
    hipFuncSetAttribute((const void*)attn_dense_kernel<D, false>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((attn_dense_kernel<D, false>), dim3(grid), dim3(NT), lds, stream, Q, C, n_q, K,
                       V, T, n_kv, mask, mask_ld, sl2, O, flags, p.n_qt, p.n_ktile, 1, part_o,
                       part_ml);
  }
  return hipGetLastError();
}

hipError_t launch_attn_dense(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V,
                             int T, int n_kv, int d, const uint16_t* mask, int64_t mask_ld,
                             float scale, float* O, const DensePlan& plan, const uint8_t* flags,
                             float* part_o, float* part_ml, hipStream_t stream) {
  if (d == 128)
    return dense_impl<128>(Q, C, n_q, K, V, T, n_kv, mask, mask_ld, scale, O, plan, flags, part_o,
                           part_ml, stream);
  return dense_impl<64>(Q, C, n_q, K, V, T, n_kv, mask, mask_ld, scale, O, plan, flags, part_o,
                        part_ml, stream);
}

template <int D>
static hipError_t blocksparse_impl(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                                   const uint16_t* V, int T, int n_kv, const float* Kp,
                                   const float* Vp, int block, const int32_t* sel_idx,
                                   const int32_t* sel_cnt, float scale, float* O, hipStream_t stream) {
  const int nb = (T + block - 1) / block;
  const int n_qblk = (q_start + C - 1) / block - q_start / block + 1;
  const size_t lds = Geo<D>::LDS_BYTES;
  hipFuncSetAttribute((const void*)attn_blocksparse_kernel<D>,
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(attn_blocksparse_kernel<D>, dim3(n_qblk * n_q), dim3(NT), lds, stream, Q, C,
                     q_start, n_q, K, V, T, n_kv, Kp, Vp, nb, n_qblk, sel_idx, sel_cnt,
                     scale * LOG2E, O);
  return hipGetLastError();
}

hipError_t launch_attn_blocksparse(const uint16_t* Q, int C, int q_start, int n_q,
                                   const uint16_t* K, const uint16_t* V, int T, int n_kv, int d,
                                   const float* K_pool, const float* V_pool, int block,
                                   const int32_t* sel_idx, const int32_t* sel_cnt, float scale,
                                   float* O, hipStream_t stream) {
  if (d == 128)
    return blocksparse_impl<128>(Q, C, q_start, n_q, K, V, T, n_kv, K_pool, V_pool, block, sel_idx,
                                 sel_cnt, scale, O, stream);
  return blocksparse_impl<64>(Q, C, q_start, n_q, K, V, T, n_kv, K_pool, V_pool, block, sel_idx,
                              sel_cnt, scale, O, stream);
}

}  // namespace pa
