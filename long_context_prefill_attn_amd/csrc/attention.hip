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
// gfx950 mapping. A workgroup is 8 waves; each wave owns 32 query rows of one
// query head. The waves of a workgroup cover Hg query heads of one KV group
// (grouped-query attention) x 256/Hg rows, so every K/V tile staged in LDS
// feeds 8 waves' MFMAs.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = a 32-key slice of the K tile
//     (LDS), B = Q^T held in registers for the whole kernel. The accumulator
//     puts query n = lane%32 in every lane, so each lane owns the softmax state
//     of one query row; the row's other 16 keys of a 32-key slice sit in lane
//     l^32 and one v_permlane32_swap completes each row reduction.
//   * O^T = V^T P^T on the same MFMA: A = V^T read from the row-major V tile
//     with ds_read_b64_tr_b16, B = P^T straight from the S^T accumulators
//     (packed to bf16), so P never leaves registers and O^T lands with the row's
//     head_dim values in the lane that owns the row's softmax state.
//   * K/V tiles of 64 keys go HBM -> LDS directly (buffer loads with the LDS
//     bit) into 4-deep K and V rings, issued one step-pair ahead of use (one
//     workgroup barrier per pair of steps).
//     One loop iteration alternates the QK^T MFMAs of the next step with the PV
//     MFMAs of the previous one and forms the current step's weights between
//     them, so the softmax VALU work is spread evenly over all MFMAs.
//   * Softmax in exp2 units with log2(e) folded into the scale. The running max
//     starts at the first tile's max and is raised only when a row's weights
//     for a tile sum past 2^12, so the O rescale is rare and no per-tile max is
//     taken; results are exact up to rounding either way. (Masked steps take
//     their max and raise it when it grows by more than 2^8.)
//   * Workgroup ids are remapped so that the workgroups of one KV head run on
//     one XCD (shared L2 for that head's K/V), longest query tiles first.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace pa {

constexpr int BN = 64;          // keys per inner step
constexpr int NW = 8;           // waves per workgroup
constexpr int NT = 64 * NW;     // threads per workgroup
constexpr int KRK = 4;          // K ring depth (tiles)
constexpr int KRV = 4;          // V ring depth (tiles)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float SLACK = 8.0f;   // lazy-rescale threshold in log2 units

#define LDS_AS __attribute__((address_space(3)))
typedef short v4i16 __attribute__((ext_vector_type(4)));

enum { MODE_PLAIN = 0, MODE_GMASK = 1, MODE_BSEL = 2, MODE_POOLED = 3, MODE_CAUSAL_K = 4, MODE_GBITS = 5 };
// how the dense kernel reads its mask: fp16 (8-byte loads when aligned) or bit-packed
enum { MASK_F16 = 0, MASK_F16_VEC = 1, MASK_BITS = 2 };

// LDS tiles: a tile of 64 keys x D is D/64 half-tiles, each [64 keys][64 dims]
// with rows of 128 bytes and no padding; dims 64h .. 64h+63 live in half-tile h.
// Within a half-tile, the 16-byte chunk c of row r sits at chunk position
// c ^ kswz(r) in K tiles and c ^ vswz(r) in V tiles. gfx950's LDS serves 256 bytes
// per clock from 64 banks, so a read is conflict-free when each 256-byte group of
// lanes touches 16 distinct 16-byte bank groups:
//   * a K-operand read (ds_read_b128): lanes 0..15 take rows n .. n+15 at one
//     chunk; kswz gives the 8 even and the 8 odd rows 8 distinct positions
//     (two rows share a 256-byte bank line);
//   * a transposed V read (ds_read_b64_tr_b16): 32 lanes take 4 rows x 4 chunks;
//     vswz moves the 4 rows into distinct 4-chunk groups, and repeats every 8
//     rows so that the read 8 rows further on keeps the same lane offsets.
// Splitting the rows in halves keeps the swizzle inside the low 3 bits of the
// chunk index, so dims 64.. of a row sit a fixed HT halves after dims 0..
// (immediate offsets instead of per-lane registers).
template <int D>
struct Geo {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int NH = D / 64;              // half-tiles per tile
  static constexpr int HT = BN * 64;             // halves of one half-tile
  static constexpr int TILE = BN * D;            // halves of one K or V tile
  static constexpr int RING = (KRK + KRV) * TILE;  // K ring then V ring (halves)
  static constexpr size_t LDS_BYTES = RING * sizeof(uint16_t);
  static constexpr int RPI = 8;                  // half-rows written by one wave-wide 16-byte load
  static constexpr int NIW = NH;                 // such loads per wave per tile
  static constexpr int KCH = BN * D / 8 / NT;    // 16-byte chunks per thread per tile
};
constexpr int RS = 64;   // halves between consecutive rows of a half-tile

// The lane id, opaque to the optimiser: what is derived from it after the long
// step loop is recomputed there instead of being held in registers through it.
__device__ __forceinline__ int fresh_lane_id() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}

__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int vswz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// halves offset of chunk c (16 bytes, dims 8c .. 8c+7) of row r inside a K (V false)
// or V (V true) tile
template <int D, bool V>
__device__ __forceinline__ int tile_pos(int r, int c) {
  return (c >> 3) * Geo<D>::HT + r * RS + (((c & 7) ^ (V ? vswz(r) : kswz(r))) * 8);
}

static_assert(FLAG_KEYS == BN, "one mask-flag tile per key step");

// The workgroup's flag row in LDS: two bits per 64-key step, 16 steps per word.
__device__ __forceinline__ int step_flag(const uint32_t* frow, int st) {
  return (int)((frow[st >> 4] >> (2 * (st & 15))) & 3u);
}

// One wave-wide 16-byte-per-lane buffer load into LDS. (Kept outside the
// templates: hipcc's host pass drops kernel stubs when the buffer-resource type
// appears inside templated device code.)
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t range, LDS_AS void* dst,
                                                  uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, range, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// Direct HBM -> LDS loads of 64-key tiles of K or V for KV head g, through a
// buffer resource per tile whose range ends at row T: rows past T read as zeros
// (their scores are masked). Load j of a tile writes 8 half-rows (1 KB) of half-tile
// j / 8; lane l lands at byte 16*l, so each lane fetches the global chunk that
// belongs at that swizzled position (K and V tiles swizzle differently, hence two
// offset sets). Each of the 8 waves issues NIW such loads per tile.
template <int D>
struct TileLoader {
  const uint16_t* kptr;   // K + g*D
  const uint16_t* vptr;   // V + g*D
  size_t row_elems;       // elements between consecutive tokens (n_kv * D)
  uint32_t row_bytes;     // the same in bytes
  uint32_t range;         // whole-tensor range (bytes readable from kptr / vptr, rows 0..T-1)
  int T;
  bool rebase;            // K/V too large for 32-bit offsets: one buffer resource per tile
  uint32_t koff[Geo<D>::NIW];   // per-lane byte offsets inside a K tile
  uint32_t voff[Geo<D>::NIW];   // and inside a V tile

  __device__ __forceinline__ void init(const uint16_t* K, const uint16_t* V, int T_, int n_kv, int g) {
    constexpr int RPI = Geo<D>::RPI, NIW = Geo<D>::NIW;
    row_elems = (size_t)n_kv * D;
    row_bytes = (uint32_t)n_kv * D * 2;
    T = T_;
    // T * row_bytes >= 2^31, in 32-bit scalar arithmetic
    rebase = ((__umulhi((uint32_t)T_, row_bytes) | (((uint32_t)T_ * row_bytes) >> 31)) != 0);
    range = rebase ? 0u : (uint32_t)T_ * row_bytes - (uint32_t)g * D * 2;
    kptr = K + (size_t)g * D;
    vptr = V + (size_t)g * D;
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
    const int r_in = lane / 8, pc = lane % 8;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int j = wave * NIW + i;
      const int row = (j % 8) * RPI + r_in;
      const uint32_t rb = (uint32_t)row * row_bytes + (uint32_t)(j / 8) * 128;
      koff[i] = rb + (uint32_t)((pc ^ kswz(row)) * 16);
      voff[i] = rb + (uint32_t)((pc ^ vswz(row)) * 16);
    }
  }

  // Up to 2 GiB the buffer resource covers the whole tensor and the tile's row
  // offset joins the per-lane offset. Beyond that the resource starts at the
  // tile's first row (64-bit address) and its range ends with this head's slice
  // of the tile's last valid row. Either way rows at or past T read as zeros.
  __device__ __forceinline__ void issue(bool is_v, int kbase, uint16_t* tile) const {
    constexpr int NIW = Geo<D>::NIW;
    const int wave = threadIdx.x >> 6;
    const uint16_t* base = is_v ? vptr : kptr;
    uint32_t rng = range, toff = (uint32_t)kbase * row_bytes;
    if (rebase) {
      base += (size_t)kbase * row_elems;
      const int rows = min(T - kbase, BN);
      rng = rows > 0 ? (uint32_t)(rows - 1) * row_bytes + D * 2 : 0u;
      toff = 0;
    }
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      LDS_AS void* dst = (LDS_AS void*)(tile + (wave * NIW + i) * 512);
      buffer_load_lds16(base, rng, dst, (is_v ? voff[i] : koff[i]) + toff, 0);
    }
  }
};

// Workgroup barrier without a memory fence. Inside the pipelined loop the only
// cross-wave data are the LDS-DMA tiles, whose arrival each wave has already
// awaited with wait_vm, and every LDS read of an earlier tile has returned
// (its value was consumed); a fenced barrier would also drain the tiles that
// are deliberately still in flight.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Per-lane LDS offsets (in halves) of the MFMA operands inside a tile.
template <int D>
struct LaneOffs {
  // Dims 64.. sit in the second half-tile, a fixed HT halves on: four K and
  // two V base offsets serve every slice, the rest being immediate offsets.
  int k[4];   // K slice rows n, dims 16*st + 8*h .. +7 for st < 4
  int v[2];   // transposed V read for output blocks 0 and 1 (see attn_step)
  __device__ __forceinline__ int kofs(int st) const { return k[st & 3] + (st >> 2) * Geo<D>::HT; }
  __device__ __forceinline__ int vofs(int nb) const { return v[nb & 1] + (nb >> 1) * Geo<D>::HT; }
};

template <int D>
__device__ __forceinline__ LaneOffs<D> lane_offsets() {
  LaneOffs<D> o;
  const int lane = fresh_lane_id();
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int st = 0; st < 4; ++st) o.k[st] = n * RS + (((2 * st + h) ^ kswz(n)) * 8);
  const int blk = lane >> 4, s = lane & 15, r = s >> 2, q = s & 3;
  const int vrow = 4 * (blk >> 1) + r;   // row inside each 8-row group
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int chunk = nb * 4 + (blk & 1) * 2 + (q >> 1);
    o.v[nb] = vrow * RS + ((chunk ^ vswz(vrow)) * 8) + (q & 1) * 4;
  }
  return o;
}

// acc + lo + hi of a packed fp16 pair (v_dot2_f32_f16 against (1, 1), fp32
// accumulate): the row sum is taken over the same rounded weights that enter
// the PV product, so the normalised weights sum to one.
__device__ __forceinline__ float row_sum_add(uint32_t packed, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
}

// O^T += V^T P^T on the fp16 matrix cores: A = four V rows x 8 dims gathered by two
// transposed LDS reads, B = a fragment of packed fp16 weights
__device__ __forceinline__ f32x16 pv_mfma(v4i16 a0, v4i16 a1, const u32x4& p, f32x16 acc) {
  const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, p), acc, 0, 0, 0);
}

struct StepCtx {
  float scale_log2;
  int kvalid;                        // keys of the step inside [0, T)
  const uint16_t* __restrict__ mrow; // MODE_GMASK: mask row of this lane's query (may be null)
  const uint32_t* __restrict__ brow; // MODE_GBITS: bit-mask row of this lane's query (may be null)
  bool mask_vec;                     // MODE_GMASK: 8-byte aligned mask rows
  int key0;                          // absolute key (or pooled block) index of the step's first key
  int qpos;                          // MODE_CAUSAL_K, MODE_BSEL: absolute position of this lane's query
  const uint32_t* selrow;            // MODE_BSEL, MODE_POOLED: selected-block bitmap of the row's query block (LDS)
  int jrow;                          // MODE_BSEL, MODE_POOLED: the row's query block (-1: no row)
  int blog2;                         // MODE_BSEL: log2(block)
  float pool_bias;                   // MODE_POOLED: log2(block)
};

template <int D>
__device__ __forceinline__ f32x16 qk_slice(const uint16_t* __restrict__ kt, const LaneOffs<D>& lo,
                                           const bf16x8 (&qf)[D / 16], f32x16 s) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + lo.kofs(st));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s, 0, 0, 0);
  }
  return s;
}

// One 64-key step for the wave's 32 query rows.
//   S^T slice kb (keys kb*32 .. +31): element i of a lane holds key kb*32 + 8*(i/4) + 4*h + i%4.
//   P^T feeds the PV MFMA directly: slot 8h+i' of MFMA c holds key 16c + 8*(i'/4) + 4h + i'%4.
//   The matching V^T operand comes from two ds_read_b64_tr_b16 reads per MFMA: in each
//   16-lane block, lane 4r+q supplies the address of V[row base + r][d0 + 4q .. +3] and
//   receives V[row base + 0..3][d0 + lane%16].
template <int D, int MODE, bool TAIL>
__device__ __forceinline__ void attn_step(const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt,
                                          const LaneOffs<D>& lo,
                                          const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32], float& m,
                                          float& l, const StepCtx& cx) {
  const int lane = fresh_lane_id();
  const int h = lane >> 5;

  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = qk_slice<D>(kt + kb * 32 * RS, lo, qf, f32x16{});
  }
  // MODE_BSEL: the row's selection bits of the step's blocks, from block b0 (a
  // step spans at most four blocks, all in one word); MODE_POOLED: the bits of
  // the step's 64 pooled rows (blocks key0 .. key0 + 63)
  uint32_t sw0 = 0, sw1 = 0;
  int b0 = 0;
  if (MODE == MODE_BSEL) {
    b0 = cx.key0 >> cx.blog2;
    if (b0 < cx.jrow) sw0 = cx.selrow[b0 >> 5] >> (b0 & 31);
  } else if (MODE == MODE_POOLED) {
    if (cx.key0 < cx.jrow) sw0 = cx.selrow[cx.key0 >> 5];
    if (cx.key0 + 32 < cx.jrow) sw1 = cx.selrow[(cx.key0 >> 5) + 1];
  }

  float x[2][16];
  float mx = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    uint32_t mw = ~0u;   // MODE_GBITS: the row's keep bits for keys key0 + 32kb .. +31
    if (MODE == MODE_GBITS && cx.brow != nullptr && 32 * kb < cx.kvalid) mw = cx.brow[(cx.key0 >> 5) + kb];
    uint16_t mv[16];
    if (MODE == MODE_GMASK) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int kk = kb * 32 + 8 * i4 + 4 * h;
        if (!TAIL && cx.mask_vec) {
          u32x2 w = {0, 0};
          if (cx.mrow != nullptr) w = *reinterpret_cast<const u32x2*>(cx.mrow + cx.key0 + kk);
          mv[4 * i4 + 0] = w[0] & 0xFFFF; mv[4 * i4 + 1] = w[0] >> 16;
          mv[4 * i4 + 2] = w[1] & 0xFFFF; mv[4 * i4 + 3] = w[1] >> 16;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mv[4 * i4 + e] = (cx.mrow != nullptr && kk + e < cx.kvalid) ? cx.mrow[cx.key0 + kk + e] : 0;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      float v = s[kb][i] * cx.scale_log2;
      if (MODE == MODE_GMASK) {
        v = f16_dropped(mv[i]) ? -__builtin_inff()
                               : __builtin_fmaf((float)__builtin_bit_cast(_Float16, mv[i]), LOG2E, v);
      } else if (MODE == MODE_GBITS) {
        if (!((mw >> (kk - 32 * kb)) & 1u)) v = -__builtin_inff();
      } else if (MODE == MODE_BSEL) {
        // exact keys of a row: every key of a selected block below its own, and
        // the keys of its own block up to its position
        const int key = cx.key0 + kk, b = key >> cx.blog2;
        const bool vis = b < cx.jrow ? ((sw0 >> (b - b0)) & 1u) != 0 : (b == cx.jrow && key <= cx.qpos);
        if (!vis) v = -__builtin_inff();
      } else if (MODE == MODE_CAUSAL_K) {
        // causal by position, plus the per-key mask (cx.mrow, shared by all rows) if any
        const int key = cx.key0 + kk;
        if (key > cx.qpos) {
          v = -__builtin_inff();
        } else if (cx.mrow != nullptr && kk < cx.kvalid) {
          const uint16_t hv = cx.mrow[key];
          v = f16_dropped(hv) ? -__builtin_inff()
                              : __builtin_fmaf((float)__builtin_bit_cast(_Float16, hv), LOG2E, v);
        }
      } else if (MODE == MODE_POOLED) {
        // a pooled row stands for an unselected block below the row's own
        const int b = cx.key0 + kk;
        const bool live = b < cx.jrow && !(((kb == 0 ? sw0 : sw1) >> (kk & 31)) & 1u);
        v = live ? v + cx.pool_bias : -__builtin_inff();
      }
      if (TAIL && kk >= cx.kvalid) v = -__builtin_inff();
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
        P[kb][c][w] = pack_f16x2(p0, p1);
        psum = row_sum_add(P[kb][c][w], psum);
      }
    }
  }
  l += psum;

#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int off = lo.vofs(nb) + (kb * 32 + 16 * c) * RS;
        const v4i16 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(vt + off));
        const v4i16 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(vt + off + 8 * RS));
        o[nb] = pv_mfma(a0, a1, P[kb][c], o[nb]);
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void qk_tile(const uint16_t* __restrict__ kt, const LaneOffs<D>& lo,
                                        const bf16x8 (&qf)[D / 16], f32x16 (&s)[2]) {
  s[0] = qk_slice<D>(kt, lo, qf, f32x16{});
  s[1] = qk_slice<D>(kt + 32 * RS, lo, qf, f32x16{});
}

// The same scores with the K operands read straight from global memory (kg =
// the tile's first row of this KV head; rows row_elems apart): the rare rescale
// path, which may not rely on the tile still being in its ring slot.
template <int D>
__device__ __forceinline__ void qk_tile_global(const uint16_t* __restrict__ kg, size_t row_elems,
                                               const bf16x8 (&qf)[D / 16], f32x16 (&s)[2]) {
  const int lane = fresh_lane_id();
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const uint16_t* rp = kg + (size_t)(kb * 32 + n) * row_elems + 8 * h;
    f32x16 acc = {};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(rp + 16 * st);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], acc, 0, 0, 0);
    }
    s[kb] = acc;
  }
}

// Row max of a raw (unscaled) S tile pair, completed across the two half-waves.
__device__ __forceinline__ float row_max(const f32x16 (&s)[2]) {
  float mx = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, s[kb][i]);
  return __builtin_fmaxf(mx, partner32(mx));
}

// Keep bits of a step for masked pipelined steps. Element i of a lane's S^T
// slice kb holds key 32 kb + 8 (i / 4) + 4 h + i % 4 of the step, so once the
// slice's keep word (bit t: key 32 kb + t) is shifted down by 4 h, element i's
// bit is bit 8 (i / 4) + i % 4.
// keep_or_zero: p if element i's keep bit is set, else +0: the bit sign-extended
// to a 32-bit mask and ANDed with p's bits (two VALU instructions, no condition
// registers)
__device__ __forceinline__ float keep_or_zero(float p, uint32_t ws, int i) {
  const uint32_t msk = (uint32_t)__builtin_amdgcn_sbfe((int)ws, (uint32_t)(8 * (i >> 2) + (i & 3)), 1u);
  return __uint_as_float(__float_as_uint(p) & msk);
}

// The two keep words of a step shifted for this lane (see keep_or_zero).
__device__ __forceinline__ void shift_keep(const uint32_t (&w)[2], uint32_t (&ws)[2]) {
  const int h = fresh_lane_id() >> 5;
  ws[0] = w[0] >> (4 * h);
  ws[1] = w[1] >> (4 * h);
}

// Scores of dropped keys set to -inf in place (a bit-field insert per element:
// the keep bit sign-extended selects the score's bits or those of -inf).
__device__ __forceinline__ void drop_masked(f32x16 (&s)[2], const uint32_t (&ws)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t msk = (uint32_t)__builtin_amdgcn_sbfe((int)ws[kb], (uint32_t)(8 * (i >> 2) + (i & 3)), 1u);
      s[kb][i] = __uint_as_float((__float_as_uint(s[kb][i]) & msk) | (0xFF800000u & ~msk));
    }
}

// P = 2^(S*scale_log2 - m) packed to fp16 in PV-operand order; l += sum of the packed values
__device__ __forceinline__ void exp_pack(const f32x16 (&s)[2], float m, float scale_log2, u32x4 (&P)[2][2],
                                         float& l) {
  const float nmu = (m == -__builtin_inff()) ? 0.f : -m;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e = 8 * c + 2 * w;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], scale_log2, nmu));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e + 1], scale_log2, nmu));
        P[kb][c][w] = pack_f16x2(p0, p1);
        l = row_sum_add(P[kb][c][w], l);
      }
    }
  }
}

// Lazy rescaling in the pipelined loop: a tile's weights are formed against the
// running max m as it stands; m is raised (and O, l rescaled) only when a row's
// weights for the tile sum to more than this, so every weight stays <= 2^12.
constexpr float PSUM_LIMIT = 4096.0f;

// One pipeline iteration for step i: the QK^T MFMAs of step i+1 alternate with
// the PV MFMAs of step i-1 (whose weights were formed in the previous
// iteration), and each MFMA pair carries one packed pair of step i's weights
// (fma, exp2, pack, row-sum). The VALU work is thereby spread evenly over all
// MFMAs of the iteration. K fragments are read KA MFMAs ahead, V fragments VA
// ahead; sched_barrier fences keep the compiler from regrouping the work.
//   S^T accumulator kb (keys 32kb .. +31) takes its MFMAs in slots kb*NS/2 ..;
//   PV slot k uses weight fragment f = k / (D/32) (keys 16f .. +15) and output
//   block nb = k % (D/32), so fragment f is dead after its D/32 MFMAs.
// Returns the row's sum of step i's packed weights.
template <int D, bool PV, bool MASKED = false>
__device__ __forceinline__ float pipe_step(const uint16_t* __restrict__ kt_next, const uint16_t* __restrict__ vt_prev,
                                           const LaneOffs<D>& lo, const bf16x8 (&qf)[D / 16],
                                           const f32x16 (&sc)[2], f32x16 (&sn)[2], const u32x4 (&pp)[2][2],
                                           u32x4 (&pc)[2][2], f32x16 (&o)[D / 32], float m, float scale_log2,
                                           const uint32_t (&mw)[2] = {0u, 0u}) {
  constexpr int NS = D / 8;             // QK^T MFMAs = PV MFMAs per step
  constexpr int HS = NS / 2;            // QK^T MFMAs per S^T accumulator
  constexpr int NB = D / 32;            // output blocks
  constexpr int KA = 3;                 // K fragments in flight
  constexpr int VA = 2;                 // V fragment pairs in flight
  const float nmu = (m == -__builtin_inff()) ? 0.f : -m;
  uint32_t ws[2] = {0u, 0u};   // MASKED: step i's keep words, shifted for this lane
  if (MASKED) shift_keep(mw, ws);

  auto kread = [&](int k) {
    return *reinterpret_cast<const bf16x8*>(kt_next + (k / HS) * 32 * RS + lo.kofs(k % HS));
  };
  auto vread = [&](int k, v4i16 (&dst)[2]) {
    const int f = k / NB, nb = k % NB;
    const int off = lo.vofs(nb) + ((f >> 1) * 32 + 16 * (f & 1)) * RS;
    dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(vt_prev + off));
    dst[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(vt_prev + off + 8 * RS));
  };
  bf16x8 kf[KA];
#pragma unroll
  for (int k = 0; k < KA; ++k) kf[k] = kread(k);
  v4i16 vf[VA + 1][2];
  if (PV) {
#pragma unroll
    for (int k = 0; k < VA; ++k) vread(k, vf[k]);
  }
  float psum = 0.f;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    // the operand reads and the two MFMAs at raised wave priority, the weights
    // of step i at the normal one: of the SIMD's two waves, the one about to
    // feed the matrix core issues first, the other's VALU work fills in behind
    __builtin_amdgcn_s_setprio(1);
    const bf16x8 a = kf[k % KA];
    if (k + KA < NS) kf[k % KA] = kread(k + KA);
    if (PV && k + VA < NS) vread(k + VA, vf[(k + VA) % (VA + 1)]);
    sn[k / HS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k % HS], k % HS == 0 ? f32x16{} : sn[k / HS], 0, 0, 0);
    if (PV) {
      const int f = k / NB;
      const v4i16 (&v)[2] = vf[k % (VA + 1)];
      o[k % NB] = pv_mfma(v[0], v[1], pp[f >> 1][f & 1], o[k % NB]);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int pi = k * 16 / NS; pi < (k + 1) * 16 / NS; ++pi) {
      const int kb = pi >> 3, c = (pi >> 2) & 1, w = pi & 3, e = 8 * c + 2 * w;
      float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][e], scale_log2, nmu));
      float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][e + 1], scale_log2, nmu));
      if (MASKED) {
        p0 = keep_or_zero(p0, ws[kb], e);
        p1 = keep_or_zero(p1, ws[kb], e + 1);
      }
      pc[kb][c][w] = pack_f16x2(p0, p1);
      psum = row_sum_add(pc[kb][c][w], psum);
    }
    // (weights' VALU work may move across slots; memory and MFMA order stay fenced)
    __builtin_amdgcn_sched_barrier(0x2);
  }
  return psum;
}

// The PV MFMAs of one step on their own (the pipeline's last step).
template <int D>
__device__ __forceinline__ void pv_only(const uint16_t* __restrict__ vt, const LaneOffs<D>& lo,
                                        const u32x4 (&P)[2][2], f32x16 (&o)[D / 32]) {
  constexpr int NS = D / 8, NB = D / 32;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int f = k / NB, nb = k % NB;
    const int off = lo.vofs(nb) + ((f >> 1) * 32 + 16 * (f & 1)) * RS;
    const v4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(vt + off));
    const v4i16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(vt + off + 8 * RS));
    o[nb] = pv_mfma(v0, v1, P[f >> 1][f & 1], o[nb]);
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined loop over "plain" 64-key steps (every key visible, no mask
// to read). Iteration i runs S = K Q^T of step i+1 and O += V P of step i-1 on
// the MFMA pipe while step i's weights are formed on the VALU. Iterations go in
// pairs (i even, i+1) with one workgroup barrier per pair; K tile j and V tile j
// sit in slot j % 4 of their rings:
//   top of pair i: wait for every load issued so far (K[i+1], K[i+2], V[i-1],
//   V[i] were issued one pair earlier), barrier, then issue K[i+3], K[i+4] into
//   the slots of K[i-1], K[i] and V[i+1], V[i+2] into those of V[i-3], V[i-2]:
//   all were last read in the previous pair. A rescale (rare) recomputes step
//   i's scores from K in global memory.
// Steps are visited in any order the source yields; the online softmax does not
// depend on the order. Loads past the last step re-read the first tile.
// Src: int first(); int next(int st); int kbase(int st); a state < 0 ends the walk.
// ---------------------------------------------------------------------------
// Keep bits for the pipelined loop: NoMask (every key of a step kept), or
// BitsMask, the bit-packed keep row of the lane's query (bit t of word w: key
// 32 w + t; no row: every key dropped).
struct NoMask {
  static constexpr bool kOn = false;
  __device__ __forceinline__ void load(int, uint32_t (&w)[2]) const { w[0] = w[1] = 0u; }
};
struct BitsMask {
  static constexpr bool kOn = true;
  const uint32_t* __restrict__ row;
  __device__ __forceinline__ void load(int st, uint32_t (&w)[2]) const {
    w[0] = w[1] = 0u;
    if (row != nullptr && st >= 0) {
      w[0] = row[2 * st];
      w[1] = row[2 * st + 1];
    }
  }
};

template <int D, class Src, class Msk = NoMask>
__device__ __forceinline__ void plain_steps(const TileLoader<D>& tl, uint16_t* lds, Src& src,
                                            const LaneOffs<D>& lo, const bf16x8 (&qf)[D / 16],
                                            f32x16 (&o)[D / 32], float& m, float& l, float scale_log2,
                                            const Msk& msk = Msk{}) {
  static_assert(KRK == 4 && KRV == 4, "ring slots are step % 4");
  constexpr int TL = Geo<D>::TILE, NIW = Geo<D>::NIW;
  constexpr bool MASKED = Msk::kOn;
  uint16_t* kring = lds;
  uint16_t* vring = lds + KRK * TL;
  const int s0 = src.first();
  if (s0 < 0) return;
  const int kfb = src.kbase(s0);
  auto kb = [&](int st) { return st >= 0 ? src.kbase(st) : kfb; };
  int t0 = s0;                           // step i
  int t1 = src.next(s0);                 // step i+1
  int t2 = t1 >= 0 ? src.next(t1) : -1;  // step i+2
  int t3 = -1, t4 = -1;
  // MASKED: keep words of the pair's two steps (mcur) and of the next pair's
  // (mnxt, loaded at the top of the pair ahead of its tile loads, so that no
  // wait for them holds up a tile)
  uint32_t mcur[2][2], mnxt[2][2];
  if (MASKED) {
    msk.load(t0, mcur[0]);
    msk.load(t1, mcur[1]);
  }
  tl.issue(false, kfb, kring);              // K[0]
  tl.issue(false, kb(t1), kring + TL);      // K[1]
  tl.issue(true, kfb, vring);               // V[0]
  tl.issue(false, kb(t2), kring + 2 * TL);  // K[2]
  wait_vm<3 * NIW>();   // K[0] landed
  bare_barrier();
  int tail_slot = 0;      // V slot of the last step
  bool tail_a = false;    // the last step's weights are in pa (else pb)
  // top of pair i, kc = i % 4 (0 or 2)
  auto top = [&](auto kcc) {
    const int kc = kcc;
    wait_vm<0>();
    bare_barrier();
    t3 = t2 >= 0 ? src.next(t2) : -1;
    t4 = t3 >= 0 ? src.next(t3) : -1;
    if (MASKED) {
      msk.load(t2, mnxt[0]);
      msk.load(t3, mnxt[1]);
    }
    tl.issue(false, kb(t3), kring + ((kc + 3) & 3) * TL);
    tl.issue(false, kb(t4), kring + kc * TL);
    tl.issue(true, kb(t1), vring + ((kc + 1) & 3) * TL);
    tl.issue(true, kb(t2), vring + ((kc + 2) & 3) * TL);
  };
  // iteration i, kc = i % 4; ti = step i, tn = the step after it (< 0: step i is the last)
  auto iter = [&](auto pvc, auto kcc, const f32x16 (&sc)[2], f32x16 (&sn)[2], const u32x4 (&pp)[2][2],
                  u32x4 (&pc)[2][2], auto pc_is_a, int ti, int tn) -> bool {
    constexpr bool HAS_PV = decltype(pvc)::value;
    const int kc = kcc;
    const uint32_t (&mw)[2] = mcur[decltype(pc_is_a)::value ? 0 : 1];   // MASKED: step i's keep words
    // MASKED: a row with no max yet (every key so far dropped) that keeps a key
    // here takes the rescale path, so that its max is the tile's max from then on
    const bool first_kept = MASKED && m == -__builtin_inff() && (mw[0] | mw[1]) != 0u;
    float psum = pipe_step<D, HAS_PV, MASKED>(kring + ((kc + 1) & 3) * TL, vring + ((kc + 3) & 3) * TL, lo, qf,
                                              sc, sn, pp, pc, o, m, scale_log2, mw);
    if (__builtin_expect(__any(psum > PSUM_LIMIT || first_kept), 0)) {
      // a row's weights outgrew the bound: raise m to the tile's max, rescale
      // what has been accumulated, and form the tile's weights again from
      // scores recomputed out of K[i] (read from global memory: its ring slot
      // may already be refilled, and sc's registers are reused inside pipe_step)
      f32x16 sr[2];
      qk_tile_global<D>(tl.kptr + (size_t)kb(ti) * tl.row_elems, tl.row_elems, qf, sr);
      if (MASKED) {
        uint32_t ws[2];
        shift_keep(mw, ws);
        drop_masked(sr, ws);
      }
      const float m_new = __builtin_fmaxf(m, row_max(sr) * scale_log2);
      const float alpha = (m == -__builtin_inff()) ? 1.f : exp2f(m - m_new);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
      l *= alpha;
      m = m_new;
      psum = 0.f;
      exp_pack(sr, m, scale_log2, pc, psum);
    }
    l += psum;
    if (tn < 0) {   // step i was the last
      tail_slot = kc;
      tail_a = decltype(pc_is_a)::value;
      return false;
    }
    return true;
  };
  auto advance = [&]() {
    t0 = t2;
    t1 = t3;
    t2 = t4;
    if (MASKED) {
      mcur[0][0] = mnxt[0][0]; mcur[0][1] = mnxt[0][1];
      mcur[1][0] = mnxt[1][0]; mcur[1][1] = mnxt[1][1];
    }
    return true;
  };
  using PV0 = std::integral_constant<bool, false>;
  using PV1 = std::integral_constant<bool, true>;
  using A = std::integral_constant<bool, true>;
  using B = std::integral_constant<bool, false>;
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  f32x16 sa[2], sb[2];
  u32x4 pa[2][2], pb[2][2];
  qk_tile<D>(kring, lo, qf, sa);
  {
    if (MASKED) {   // (the first step's weights are formed from these scores: -inf gives 0)
      uint32_t ws[2];
      shift_keep(mcur[0], ws);
      drop_masked(sa, ws);
    }
    const float m_new = __builtin_fmaxf(m, row_max(sa) * scale_log2);
    const float alpha = (m == -__builtin_inff()) ? 1.f : exp2f(m - m_new);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
    l *= alpha;
    m = m_new;
  }
  // even i: S[i] in sa, weights into pa; odd i: S[i] in sb, weights into pb.
  if constexpr (D == 128) {
    // four iterations (two pairs) per pass cover the ring slots and both
    // buffers; the slots are compile-time constants folded into LDS offsets
    top(C0{});
    if (iter(PV0{}, C0{}, sa, sb, pb, pa, A{}, t0, t1) && iter(PV1{}, C1{}, sb, sa, pa, pb, B{}, t1, t2) &&
        advance()) {
      while ((top(C2{}), true) && iter(PV1{}, C2{}, sa, sb, pb, pa, A{}, t0, t1) &&
             iter(PV1{}, C3{}, sb, sa, pa, pb, B{}, t1, t2) && advance() && (top(C0{}), true) &&
             iter(PV1{}, C0{}, sa, sb, pb, pa, A{}, t0, t1) && iter(PV1{}, C1{}, sb, sa, pa, pb, B{}, t1, t2) &&
             advance()) {
      }
    }
  } else {
    // one pair per pass with run-time ring slots (constant slots spill here)
    int kc = 0;
    top(kc);
    if (iter(PV0{}, kc, sa, sb, pb, pa, A{}, t0, t1) && iter(PV1{}, kc + 1, sb, sa, pa, pb, B{}, t1, t2) &&
        advance()) {
      for (;;) {
        kc ^= 2;
        asm volatile("" : "+s"(kc));   // keep the slot a run-time value
        top(kc);
        if (!(iter(PV1{}, kc, sa, sb, pb, pa, A{}, t0, t1) && iter(PV1{}, kc + 1, sb, sa, pa, pb, B{}, t1, t2) &&
              advance()))
          break;
      }
    }
  }
  // the last step's PV, once its V tile has landed
  wait_vm<0>();
  bare_barrier();
  const uint16_t* vt = vring + tail_slot * TL;
  if (tail_a)
    pv_only<D>(vt, lo, pa, o);
  else
    pv_only<D>(vt, lo, pb, o);
  __syncthreads();   // LDS free for whatever follows
}

// Plain-step sources (see plain_steps).
// Dense: steps [a, b) whose flag tile is ZERO (any: ZERO or MIXED, for the
// pipelined loop over bit-packed keep masks) and whose 64 keys all lie below T.
// The walk keeps a 64-step window of plain bits in scalar registers, filled by one
// wave-wide ballot over the LDS flag row; finding the next step is scalar bit
// arithmetic, so an iteration never waits on an LDS read for it (the walk only
// moves forward, and every lane of the wave is active in the step loop).
struct DenseSrc {
  int a, b, T;
  const uint32_t* frow;
  int wbase;        // first step of the window
  uint64_t wmask;   // bit k: step wbase + k is taken
  bool any = false;
  __device__ void fill(int base) {
    const int sl = base + fresh_lane_id();
    const int f = sl < b ? step_flag(frow, sl) : TILE_DROPPED;
    const bool p = (f == TILE_ZERO || (any && f == TILE_MIXED)) && (sl + 1) * BN <= T;
    wbase = base;
    wmask = __ballot(p);
  }
  __device__ int scan(int st) {
    while (st < b) {
      if (st < wbase || st >= wbase + 64) fill(st);
      const uint64_t bits = wmask >> (st - wbase);
      if (bits != 0) return st + __builtin_ctzll(bits);   // set bits lie below b
      st = wbase + 64;
    }
    return -1;
  }
  __device__ int first() { return scan(a); }
  __device__ int next(int st) { return scan(st + 1); }
  __device__ int kbase(int st) const { return st * BN; }
};

// The steps that are neither plain nor skipped (flag MIXED, or a ragged last
// step) in [a, b): found 64 steps at a time by a wave-wide ballot over the LDS
// flag row (every wave forms the same mask, so the barriers inside stay
// uniform), their K and V tiles double buffered in the first two ring slots
// (the next such step's tiles load while this one computes). run(st, kt, vt)
// computes step st from the K and V tiles kt, vt. mixed_piped: the MIXED steps
// whose keys all lie below T were taken by the masked pipelined pass.
template <int D, class Run>
__device__ __forceinline__ void special_steps(const TileLoader<D>& tl, uint16_t* lds, const uint32_t* frow,
                                              int a, int b, int T, Run&& run, bool mixed_piped = false) {
  constexpr int TL = Geo<D>::TILE, NIW = Geo<D>::NIW;
  const int lane = fresh_lane_id();
  auto next_special = [&](int st) -> int {
    for (int base = st; base < b; base += 64) {
      const int sl = base + lane;
      const int fl = sl < b ? step_flag(frow, sl) : TILE_DROPPED;
      const bool piped = (fl == TILE_ZERO || (mixed_piped && fl == TILE_MIXED)) && (sl + 1) * BN <= T;
      const uint64_t hit = __ballot(!(fl == TILE_DROPPED || piped));
      if (hit != 0) return base + __builtin_ctzll(hit);
    }
    return b;
  };
  int st = next_special(a), buf = 0;
  if (st < b) {
    tl.issue(false, st * BN, lds);
    tl.issue(true, st * BN, lds + KRK * TL);
  }
  while (st < b) {
    const int nx = next_special(st + 1);
    if (nx < b) {
      tl.issue(false, nx * BN, lds + (buf ^ 1) * TL);
      tl.issue(true, nx * BN, lds + (KRK + (buf ^ 1)) * TL);
      wait_vm<2 * NIW>();   // this step's tiles landed
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    run(st, lds + buf * TL, lds + (KRK + buf) * TL);
    __syncthreads();
    st = nx;
    buf ^= 1;
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
  const int h = fresh_lane_id() >> 5;
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
// Workgroup = (KV head g, head slice hs, query tile qt, key split). Its 8 waves
// cover query heads g*group + hs*Hg .. +Hg-1 and rows qt*R .. qt*R+R-1, R = 256/Hg.
// ---------------------------------------------------------------------------
template <int D, bool SPLIT, bool BITS>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
attn_dense_kernel(const uint16_t* __restrict__ Q, int C, int n_q, const uint16_t* __restrict__ K,
                  const uint16_t* __restrict__ V, const float* __restrict__ vscales, int T, int n_kv,
                  const uint16_t* __restrict__ mask,
                  int64_t mask_ld, float scale_log2, float* __restrict__ O,
                  const uint8_t* __restrict__ flags, int n_qt, int n_ktile, int splits,
                  float* __restrict__ part_o, float* __restrict__ part_ml, int mask_mode, int hg_log2,
                  int causal_q0) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ int s_lo, s_hi;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 31;
  const int Hg = 1 << hg_log2;
  const int R = 256 >> hg_log2;
  const int group = n_q / n_kv;
  const int n_hs = group >> hg_log2;

  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  const int per_unit = n_qt * splits;
  const int unit = bid / per_unit;
  const int g = unit / n_hs, hs = unit % n_hs;
  const int rem = bid % per_unit;
  const int qt = n_qt - 1 - rem / splits;
  const int split = rem % splits;
  const int wph = R / 32;   // waves per head
  const int head = g * group + hs * Hg + wave / wph;

  // the workgroup's rows' mask-tile flags (one per 64-key step), combined over
  // the (one or two) flag rows they span and copied to LDS after the rings, two
  // bits each (16 steps per word): walking the steps never waits on global memory
  uint32_t* frow = reinterpret_cast<uint32_t*>(lds + Geo<D>::RING);
  const int fr0 = (qt * R) / FLAG_ROWS;
  const int fr1 = (min(qt * R + R, C) - 1) / FLAG_ROWS;
  if (tid == 0) { s_lo = n_ktile; s_hi = 0; }
  for (int wd = tid; wd < (n_ktile + 15) / 16; wd += NT) frow[wd] = 0u;
  __syncthreads();
  for (int t = tid; t < n_ktile; t += NT) {
    uint8_t f;
    if (causal_q0 >= 0) {
      // causal by position: rows causal_q0 + [qt*R, min(qt*R + R, C)); flags (if any)
      // classify the per-key mask's 64-key tiles
      const int rmin = causal_q0 + qt * R, rmax = causal_q0 + min(qt * R + R, C) - 1;
      const int k0 = t * FLAG_KEYS, k1 = k0 + FLAG_KEYS - 1;
      f = k0 > rmax ? TILE_DROPPED : (k1 <= rmin ? TILE_ZERO : TILE_MIXED);
      if (flags != nullptr) {
        const uint8_t kf = flags[t];
        f = (f == TILE_DROPPED || kf == TILE_DROPPED) ? TILE_DROPPED
            : (f == TILE_ZERO && kf == TILE_ZERO)      ? TILE_ZERO
                                                       : TILE_MIXED;
      }
    } else {
      f = flags[(size_t)fr0 * n_ktile + t];
      for (int fr = fr0 + 1; fr <= fr1; ++fr) {
        const uint8_t f2 = flags[(size_t)fr * n_ktile + t];
        f = (f == f2) ? f : TILE_MIXED;
      }
    }
    if (f != TILE_ZERO) atomicOr(&frow[t >> 4], (uint32_t)f << (2 * (t & 15)));
    if (f != TILE_DROPPED) { atomicMin(&s_lo, t); atomicMax(&s_hi, t + 1); }
  }
  __syncthreads();
  const int n_steps = (T + BN - 1) / BN;
  const int st_lo = s_lo;
  const int st_hi = min(s_hi, n_steps);
  const int len = max(st_hi - st_lo, 0);
  const int a = st_lo + (int)((long)len * split / splits);
  const int b = st_lo + (int)((long)len * (split + 1) / splits);

  const int qrow = qt * R + (wave % wph) * 32 + n;
  const bool qvalid = qrow < C;
  bf16x8 qf[D / 16];
  load_q<D>(Q, n_q, head, qrow, qvalid, qf);

  f32x16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;

  const LaneOffs<D> lo = lane_offsets<D>();
  TileLoader<D> tl;
  tl.init(K, V, T, n_kv, g);

  if constexpr (BITS) {
    // 1) bit-packed keep masks: every step whose 64 keys lie below T and are not
    // all dropped, pipelined, each key's weight kept or zeroed by its bit
    DenseSrc dsrc{a, b, T, frow, -64, 0, true};
    const BitsMask bm{qvalid ? reinterpret_cast<const uint32_t*>(mask) + (size_t)qrow * mask_ld : nullptr};
    plain_steps<D>(tl, lds, dsrc, lo, qf, o, m, l, scale_log2, bm);
  } else {
    // 1) plain steps: tiles flagged ZERO whose 64 keys all lie below T
    DenseSrc dsrc{a, b, T, frow, -64, 0};
    plain_steps<D>(tl, lds, dsrc, lo, qf, o, m, l, scale_log2);
  }

  // lane-derived values for what follows, formed afresh (see fresh_lane_id)
  const int lane2 = fresh_lane_id();
  const int qrow2 = qt * R + (wave % wph) * 32 + (lane2 & 31);
  const bool qvalid2 = qrow2 < C;
  const LaneOffs<D> lo2 = lane_offsets<D>();
  StepCtx cx;
  cx.scale_log2 = scale_log2;
  cx.brow = nullptr;
  if (causal_q0 >= 0) {
    cx.mrow = mask;   // the per-key mask (or null)
    cx.qpos = causal_q0 + qrow2;
  } else if (mask_mode == MASK_BITS) {
    cx.mrow = nullptr;
    cx.brow = qvalid2 ? reinterpret_cast<const uint32_t*>(mask) + (size_t)qrow2 * mask_ld : nullptr;
    cx.qpos = 0;
  } else {
    cx.mrow = qvalid2 ? mask + (size_t)qrow2 * mask_ld : nullptr;
    cx.qpos = 0;
  }
  cx.mask_vec = mask_mode == MASK_F16_VEC;
  cx.selrow = nullptr; cx.jrow = -1; cx.blog2 = 0; cx.pool_bias = 0.f;

  // 2) the remaining steps: mask tiles (MIXED; with keep bits only a ragged
  // one) and a ragged last step
  special_steps<D>(tl, lds, frow, a, b, T, [&](int st, const uint16_t* kt, const uint16_t* vt) {
    const int f = step_flag(frow, st);
    cx.key0 = st * BN;
    cx.kvalid = min(BN, T - st * BN);
    if constexpr (BITS) {
      if (f == TILE_MIXED)
        attn_step<D, MODE_GBITS, true>(kt, vt, lo2, qf, o, m, l, cx);
      else
        attn_step<D, MODE_PLAIN, true>(kt, vt, lo2, qf, o, m, l, cx);
    } else {
      if (f == TILE_MIXED && causal_q0 >= 0)
        attn_step<D, MODE_CAUSAL_K, true>(kt, vt, lo2, qf, o, m, l, cx);
      else if (f == TILE_MIXED && cx.kvalid == BN)   // a full step: 8-byte mask loads where aligned
        attn_step<D, MODE_GMASK, false>(kt, vt, lo2, qf, o, m, l, cx);
      else if (f == TILE_MIXED)
        attn_step<D, MODE_GMASK, true>(kt, vt, lo2, qf, o, m, l, cx);
      else
        attn_step<D, MODE_PLAIN, true>(kt, vt, lo2, qf, o, m, l, cx);
    }
  }, BITS);

  const float lt = l + partner32(l);
  if (!qvalid2) return;
  const float vup = vscales[1];   // the staged values were scaled by 1 / vup
  const size_t row = (size_t)qrow2 * n_q + head;
  if (SPLIT) {
    const size_t rows = (size_t)C * n_q;
    store_rows<D>(part_o + ((size_t)split * rows + row) * D, o, vup);
    if (lane2 < 32) {
      float2* ml = reinterpret_cast<float2*>(part_ml + ((size_t)split * rows + row) * 2);
      *ml = make_float2(m == -__builtin_inff() ? 0.f : m, lt);
    }
  } else {
    store_rows<D>(O + row * D, o, lt > 0.f ? vup / lt : 0.f);
  }
}

// ---------------------------------------------------------------------------
// block-sparse prefill attention ("Porting FlashPrefill V2 to Apple silicon",
// Compute the peaks, summarize the rest): one workgroup per (128 aligned query
// positions, pair of query heads of one KV group). With block size B, those
// positions lie in one query block (B >= 128) or span 128/B of them (B < 128).
// A row of query block j takes exact attention over every key of each selected
// block below j and the keys of block j up to its own position, and one pooled
// row (mean key, mean value) of multiplicity B for every unselected block below
// j. The selections enter as bitmaps in LDS (list entries outside [0, j) and
// duplicates are ignored), and each 64-key step is classified for the
// workgroup's rows as in the dense kernel: plain (every row takes all 64 keys
// exactly: the pipelined loop), skipped (no row takes any), or masked (a per-key
// test against the row's own selection and position). Then the pooled rows, 64
// per step: the pooled keys and values arrive staged once per call (bf16 keys,
// fp16 values with the staged values' factor, token-major like K and V) and go
// into LDS as tiles, the next tile's loads in flight while one is computed.
// With an odd number of query heads per KV head, the second half of the
// workgroup repeats the first head and does not store.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
attn_blocksparse_kernel(const uint16_t* __restrict__ Q, int C, int q_start, int n_q,
                        const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                        const float* __restrict__ vscales, int T, int n_kv,
                        const uint16_t* __restrict__ Kp16, const uint16_t* __restrict__ Vp16, int nb,
                        int blog2, int n_qblk, int n_wrb, const int32_t* __restrict__ sel_idx,
                        const int32_t* __restrict__ sel_cnt, float scale_log2, float* __restrict__ O) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, n = lane & 31;
  const int group = n_q / n_kv;
  const int hpw = (group % 2 == 0) ? 2 : 1;   // query heads per workgroup

  // workgroup ids, after the XCD remap, run KV head by KV head, longest row
  // blocks first, with the head pairs of one (KV head, row block) adjacent: they
  // share the selections, so the second reads the first's K/V tiles from L2
  const int bid = remap_xcd(blockIdx.x, gridDim.x);
  const int hpk = group / hpw;                  // workgroups per (KV head, row block)
  const int g = bid / (n_wrb * hpk);
  const int rr = bid % (n_wrb * hpk);
  const int wrb = n_wrb - 1 - rr / hpk;
  const int hp = g * hpk + rr % hpk;            // head pair (or single head)
  const int head = hp * hpw + (hpw == 2 ? (wave >> 2) : 0);
  const bool storer = hpw == 2 || wave < 4;

  // this workgroup's rows: positions [r_lo, r_hi) of the aligned block of 128
  const int P0 = (q_start / 128 + wrb) * 128;
  const int r_lo = max(P0, q_start), r_hi = min(P0 + 128, q_start + C);
  const int j_lo = r_lo >> blog2, j_hi = (r_hi - 1) >> blog2;
  const int nq = j_hi - j_lo + 1;               // query blocks among the rows (<= 8)
  const int jj0 = j_lo - (q_start >> blog2);    // their index in the selection arrays
  const int sw = (j_hi + 31) >> 5;              // bitmap words per query block (blocks < j_hi)
  const int n_steps = (r_hi + BN - 1) / BN;     // keys at or past r_hi are in every row's future

  // LDS after the rings: the step flag row (2 bits per step), then the bitmaps
  uint32_t* frow = reinterpret_cast<uint32_t*>(lds + Geo<D>::RING);
  const int fwords = (n_steps + 15) / 16;
  uint32_t* selw = frow + fwords;
  for (int i = tid; i < fwords + nq * sw; i += NT) frow[i] = 0u;
  __syncthreads();
  for (int qi = 0; qi < nq; ++qi) {
    const size_t srow = (size_t)g * n_qblk + jj0 + qi;
    const int cnt = min(max(sel_cnt[srow], 0), nb);
    const int jq = j_lo + qi;
    const int32_t* sl = sel_idx + srow * nb;
    for (int e = tid; e < cnt; e += NT) {
      const int b = sl[e];
      if (b >= 0 && b < jq) atomicOr(&selw[qi * sw + (b >> 5)], 1u << (b & 31));
    }
  }
  __syncthreads();
  // step flags over the workgroup's rows: ZERO = every row takes all 64 keys
  // exactly, DROPPED = no row takes any key exactly, MIXED = otherwise
  for (int st = tid; st < n_steps; st += NT) {
    const int k0 = st * BN;
    const int bA = k0 >> blog2, bZ = (k0 + BN - 1) >> blog2;
    bool all = true, any = false;
    for (int qi = 0; qi < nq; ++qi) {
      const int jq = j_lo + qi;
      const int plo = max(jq << blog2, r_lo), phi = min((jq + 1) << blog2, r_hi) - 1;  // its rows here
      for (int b = bA; b <= bZ; ++b) {
        bool a_ = false, y_ = false;   // every row of jq takes all the step's keys of b / some row takes some
        if (b < jq) {
          a_ = y_ = ((selw[qi * sw + (b >> 5)] >> (b & 31)) & 1u) != 0;
        } else if (b == jq) {
          const int t0 = max(k0, b << blog2), t1 = min(k0 + BN, (b + 1) << blog2) - 1;
          a_ = t1 <= plo;
          y_ = t0 <= phi;
        }
        all = all && a_;
        any = any || y_;
      }
    }
    const uint32_t f = all ? TILE_ZERO : (any ? TILE_MIXED : TILE_DROPPED);
    if (f != TILE_ZERO) atomicOr(&frow[st >> 4], f << (2 * (st & 15)));
  }

  const int qpos = P0 + (wave & 3) * 32 + n;
  const bool qvalid = qpos >= r_lo && qpos < r_hi;
  bf16x8 qf[D / 16];
  load_q<D>(Q, n_q, head, qpos - q_start, qvalid, qf);

  f32x16 o[D / 32];
#pragma unroll
  for (int q = 0; q < D / 32; ++q) o[q] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;

  const LaneOffs<D> lo = lane_offsets<D>();
  TileLoader<D> tl;
  tl.init(K, V, T, n_kv, g);
  __syncthreads();

  // 1) plain steps: the pipelined loop
  DenseSrc dsrc{0, n_steps, T, frow, -64, 0};
  plain_steps<D>(tl, lds, dsrc, lo, qf, o, m, l, scale_log2);

  // lane-derived values for what follows, formed afresh (see fresh_lane_id)
  const int qpos2 = P0 + (wave & 3) * 32 + (fresh_lane_id() & 31);
  const bool qvalid2 = qpos2 >= r_lo && qpos2 < r_hi;
  const int jrow = qvalid2 ? (qpos2 >> blog2) : -1;
  const LaneOffs<D> lo2 = lane_offsets<D>();
  StepCtx cx;
  cx.scale_log2 = scale_log2;
  cx.mrow = nullptr;
  cx.brow = nullptr;
  cx.mask_vec = false;
  cx.qpos = qpos2;
  cx.jrow = jrow;
  cx.selrow = selw + (qvalid2 ? (jrow - j_lo) * sw : 0);
  cx.blog2 = blog2;
  cx.pool_bias = (float)blog2;

  // 2) masked steps: the diagonal blocks and partly selected steps. With blocks
  // of 64 keys or more a wave's 32 rows lie in one query block, and a step inside
  // that block is causal by position alone for the wave: it is skipped when every
  // key lies past the wave's rows, taken unmasked when every key lies at or
  // before them, and masked by position otherwise (the same weights as the
  // per-key test, with less work per key).
  int own = -1, qlo = 0, qhi = 0;   // the wave's query block (-1: none or several), its positions
  {
    const bool mixed_blocks = __any(qvalid2 && jrow != __builtin_amdgcn_readfirstlane(jrow));
    const uint64_t vb = __ballot(qvalid2);
    if (blog2 >= 6 && vb != 0 && !mixed_blocks) {
      // positions are consecutive over the lanes of a half-wave: the valid rows
      // run from the lowest valid lane's position to the highest's
      const int lo_lane = __builtin_ctzll(vb), hi_lane = 63 - __builtin_clzll(vb);
      qlo = __shfl(qpos2, lo_lane);
      qhi = __shfl(qpos2, hi_lane);
      own = __shfl(jrow, lo_lane);
    }
  }
  special_steps<D>(tl, lds, frow, 0, n_steps, T, [&](int st, const uint16_t* kt, const uint16_t* vt) {
    cx.key0 = st * BN;
    cx.kvalid = min(BN, T - st * BN);
    if (own >= 0 && (cx.key0 >> blog2) == own) {
      if (cx.key0 > qhi) return;   // every key lies past every row of the wave
      if (cx.key0 + BN - 1 <= qlo && cx.kvalid == BN) {
        attn_step<D, MODE_PLAIN, false>(kt, vt, lo2, qf, o, m, l, cx);
      } else {
        attn_step<D, MODE_CAUSAL_K, true>(kt, vt, lo2, qf, o, m, l, cx);
      }
      return;
    }
    attn_step<D, MODE_BSEL, true>(kt, vt, lo2, qf, o, m, l, cx);
  });

  // 3) pooled rows of blocks 0 .. j_hi - 1, 64 per step, in ring slots 0 and 1
  // alternately (one barrier per step: tile p has landed for every wave and tile
  // p-1's readers are done before tile p+1 is issued into its slot); each row
  // keeps those of its unselected blocks below its own. Rows at or past j_hi read
  // as zeros.
  const int n_pool = (j_hi + BN - 1) / BN;
  if (n_pool > 0) {
    constexpr int TL = Geo<D>::TILE;
    TileLoader<D> tp;
    tp.init(Kp16, Vp16, j_hi, n_kv, g);
    __syncthreads();   // every wave is done with the rings
    tp.issue(false, 0, lds);
    tp.issue(true, 0, lds + KRK * TL);
    for (int p = 0; p < n_pool; ++p) {
      wait_vm<0>();
      bare_barrier();
      if (p + 1 < n_pool) {
        tp.issue(false, (p + 1) * BN, lds + ((p + 1) & 1) * TL);
        tp.issue(true, (p + 1) * BN, lds + (KRK + ((p + 1) & 1)) * TL);
      }
      cx.key0 = p * BN;
      cx.kvalid = BN;
      attn_step<D, MODE_POOLED, false>(lds + (p & 1) * TL, lds + (KRK + (p & 1)) * TL, lo2, qf, o, m, l, cx);
    }
  }

  const float lt = l + partner32(l);
  if (!qvalid2 || !storer) return;
  store_rows<D>(O + ((size_t)(qpos2 - q_start) * n_q + head) * D, o, lt > 0.f ? vscales[1] / lt : 0.f);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int device_cus() {
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

// log2 of the query heads one workgroup packs: the largest power of two (<= 8)
// that divides the group size n_q / n_kv
static int hg_log2_for(int n_q, int n_kv) {
  const int group = n_q / n_kv;
  int lg = 0;
  while (lg < 3 && group % (2 << lg) == 0) ++lg;
  return lg;
}

DensePlan plan_dense(int C, int T, int n_q, int n_kv, int d) {
  (void)d;
  DensePlan p{};
  p.hg_log2 = hg_log2_for(n_q, n_kv);
  const int R = 256 >> p.hg_log2;
  p.n_qt = (C + R - 1) / R;
  p.n_ktile = (T + FLAG_KEYS - 1) / FLAG_KEYS;
  p.n_qft = (C + FLAG_ROWS - 1) / FLAG_ROWS;
  const long wgs = (long)p.n_qt * (n_q >> p.hg_log2);
  // split the key range only to reach one resident workgroup per CU: splitting
  // further shortens the longest causal tile but adds a combine pass, and was
  // slower on 1,024- and 4,096-row chunks over 1-5K keys
  const int target = device_cus();
  const int n_steps = (T + BN - 1) / BN;
  int splits = 1;
  if (wgs < target) splits = (int)((target + wgs - 1) / wgs);
  splits = std::max(1, std::min(splits, n_steps / 4));  // at least 4 steps (256 keys) per split
  splits = std::min(splits, 32);
  p.splits = splits;
  p.flags_bytes = align256((size_t)p.n_qft * p.n_ktile);
  if (splits > 1) {
    p.part_o_bytes = align256((size_t)splits * C * n_q * d * sizeof(float));
    p.part_ml_bytes = align256((size_t)splits * C * n_q * 2 * sizeof(float));
  }
  p.stage_off = p.flags_bytes + p.part_o_bytes + p.part_ml_bytes;
  p.stage = plan_stage(T, n_kv, d);
  p.total_bytes = p.stage_off + p.stage.bytes;
  return p;
}

template <int D>
static hipError_t dense_impl(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V,
                             const float* vscales, int T, int n_kv, const uint16_t* mask, int64_t mask_ld,
                             float scale,
                             float* O, const DensePlan& p, const uint8_t* flags, float* part_o,
                             float* part_ml, int causal_q0, hipStream_t stream, bool mask_bits) {
  const float sl2 = scale * LOG2E;
  const int grid = p.n_qt * (n_q >> p.hg_log2) * p.splits;
  const size_t lds = Geo<D>::LDS_BYTES + (size_t)((p.n_ktile + 63) / 64) * 16;   // rings + 2-bit flag row
  const bool vec = (mask_ld % 4 == 0) && (reinterpret_cast<uintptr_t>(mask) % 8 == 0);
  const int mask_mode = mask_bits ? MASK_BITS : vec ? MASK_F16_VEC : MASK_F16;
  if (mask_bits && causal_q0 >= 0) return hipErrorInvalidValue;   // keep bits come without a causal rule
  auto launch = [&](auto kern, int splits) {
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), lds, stream, Q, C, n_q, K, V, vscales, T, n_kv, mask,
                       mask_ld, sl2, O, flags, p.n_qt, p.n_ktile, splits, part_o, part_ml, mask_mode, p.hg_log2,
                       causal_q0);
  };
  if (p.splits > 1 && mask_bits) launch(attn_dense_kernel<D, true, true>, p.splits);
  else if (p.splits > 1) launch(attn_dense_kernel<D, true, false>, p.splits);
  else if (mask_bits) launch(attn_dense_kernel<D, false, true>, 1);
  else launch(attn_dense_kernel<D, false, false>, 1);
  return hipGetLastError();
}

hipError_t launch_attn_dense(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V16,
                             const float* vscales, int T, int n_kv, int d, const uint16_t* mask,
                             int64_t mask_ld, float scale, float* O, const DensePlan& plan,
                             const uint8_t* flags, float* part_o, float* part_ml, int causal_q0,
                             hipStream_t stream, bool mask_bits) {
  if (d == 128)
    return dense_impl<128>(Q, C, n_q, K, V16, vscales, T, n_kv, mask, mask_ld, scale, O, plan, flags,
                           part_o, part_ml, causal_q0, stream, mask_bits);
  return dense_impl<64>(Q, C, n_q, K, V16, vscales, T, n_kv, mask, mask_ld, scale, O, plan, flags, part_o,
                        part_ml, causal_q0, stream, mask_bits);
}

template <int D>
static hipError_t blocksparse_impl(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                                   const uint16_t* V, const float* vscales, int T, int n_kv, const uint16_t* Kp16,
                                   const uint16_t* Vp16, int block, const int32_t* sel_idx,
                                   const int32_t* sel_cnt, float scale, float* O, hipStream_t stream) {
  const int nb = (T + block - 1) / block;
  const int blog2 = __builtin_ctz((unsigned)block);
  const int n_qblk = (q_start + C - 1) / block - q_start / block + 1;
  const int n_wrb = (q_start + C - 1) / 128 - q_start / 128 + 1;   // aligned blocks of 128 rows
  const int hpw = ((n_q / n_kv) % 2 == 0) ? 2 : 1;
  // LDS: the rings, the step flag row of the longest key range and the bitmaps
  const int max_steps = (q_start + C + BN - 1) / BN;
  const int max_nq = block >= 128 ? 1 : 128 / block;
  const size_t lds = Geo<D>::LDS_BYTES + (size_t)((max_steps + 15) / 16) * 4 +
                     (size_t)max_nq * ((nb + 31) / 32) * 4;
  hipFuncSetAttribute((const void*)attn_blocksparse_kernel<D>,
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(attn_blocksparse_kernel<D>, dim3(n_wrb * (n_q / hpw)), dim3(NT), lds, stream, Q, C,
                     q_start, n_q, K, V, vscales, T, n_kv, Kp16, Vp16, nb, blog2, n_qblk, n_wrb, sel_idx,
                     sel_cnt, scale * LOG2E, O);
  return hipGetLastError();
}

hipError_t launch_attn_blocksparse(const uint16_t* Q, int C, int q_start, int n_q,
                                   const uint16_t* K, const uint16_t* V16, const float* vscales,
                                   int T, int n_kv, int d,
                                   const uint16_t* Kp16, const uint16_t* Vp16, int block,
                                   const int32_t* sel_idx, const int32_t* sel_cnt, float scale,
                                   float* O, hipStream_t stream) {
  if (d == 128)
    return blocksparse_impl<128>(Q, C, q_start, n_q, K, V16, vscales, T, n_kv, Kp16, Vp16, block, sel_idx,
                                 sel_cnt, scale, O, stream);
  return blocksparse_impl<64>(Q, C, q_start, n_q, K, V16, vscales, T, n_kv, Kp16, Vp16, block, sel_idx, sel_cnt,
                              scale, O, stream);
}

}  // namespace pa
