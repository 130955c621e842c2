// Shared device helpers and host-side launch declarations for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// tile classification of the additive mask: one flag per tile of 64 rows x 64
// keys (64 keys = one step of the attention kernels' key loop; 64 rows = the
// rows of a dense workgroup when it packs four query heads)
enum : uint8_t { TILE_ZERO = 0, TILE_DROPPED = 1, TILE_MIXED = 2 };
constexpr int FLAG_ROWS = 64;
constexpr int FLAG_KEYS = 64;

// fp16 bit pattern of -30000; an entry is "dropped" when its value is <= -30000
constexpr uint16_t F16_DROP_MAG = 0x7753;

__device__ __forceinline__ bool f16_dropped(uint16_t h) {
  const uint16_t mag = h & 0x7FFF;
  return (h & 0x8000) && mag >= F16_DROP_MAG && mag <= 0x7C00;  // excludes NaN
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Swap values between lane l and lane l^32 of a wave64 and return the partner's value.
__device__ __forceinline__ float partner32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // r[0]: lanes 0..31 keep their own value, lanes 32..63 receive lanes 0..31;
  // r[1]: lanes 0..31 receive lanes 32..63, lanes 32..63 keep their own value.
  const bool low = (__lane_id() < 32);
  return __uint_as_float(low ? r[1] : r[0]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  f16x2 h = __builtin_convertvector(f, f16x2);   // v_cvt_pk_f16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace pa

// ---------------------------------------------------------------------------
// host-side launchers (defined next to their kernels); all enqueue on `stream`
// ---------------------------------------------------------------------------
namespace pa {

struct KernelTimer;  // opaque; see api.cpp

// compute units of the current device (256 if the query fails); read once
int device_cus();

hipError_t launch_pool(const uint16_t* K, const uint16_t* V, int T, int n_kv, int d, int block,
                       int b_first, float* K_pool, float* V_pool, int pool_ld, hipStream_t stream);

// The selection path counters since the last reset (waits for the device).
hipError_t select_path_counts(int64_t* out, bool reset);
hipError_t launch_select(const uint16_t* Q, int C, int q_start, int n_q, int n_kv, int d,
                         const float* K_pool, int pool_ld, int T, int block, double theta,
                         int sink_blocks, int window_blocks, int dense_tail_blocks,
                         int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream);

hipError_t launch_mask_classify(const uint16_t* mask, int64_t mask_ld, int C, int T,
                                uint8_t* flags, hipStream_t stream);

// Tile flags of a bit-packed mask: bit t % 32 of word t / 32 of a row set = key t kept.
hipError_t launch_fold_keep_bits(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C,
                                 int q_start, int T, int width, int recent, uint32_t* bits, int64_t bits_ld,
                                 hipStream_t stream);
hipError_t launch_mask_classify_bits(const uint32_t* bits, int64_t bits_ld, int C, int T,
                                     uint8_t* flags, hipStream_t stream);

hipError_t launch_fold_keep(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C,
                            int q_start, int T, int width, int recent, uint16_t* mask, int64_t mask_ld,
                            hipStream_t stream);

// Value staging: the attention kernels take V as fp16 (the PV product runs on
// fp16 MFMAs so the softmax weights keep 11 significant bits), scaled by a
// power of two 2^-k that maps max |V| into [2^14, 2^15). Two passes over V[0..T):
// partial maxima of |V| per workgroup, then every workgroup reduces the
// partials, converts its share of V and (workgroup 0) writes
// scales = {2^-k, 2^k} for the kernels that use the staged copy.
constexpr int STAGE_PARTS = 512;   // workgroups of the range pass
struct StagePlan {
  size_t v16_off, part_off, scales_off;   // byte offsets inside the stage region
  size_t kp16_off, vp16_off;              // pooled operands (pool_rows > 0)
  size_t bytes;
};
// pool_rows: rows of pooled operands to make room for (0: none)
StagePlan plan_stage(int T, int n_kv, int d, int pool_rows = 0);
hipError_t launch_stage_values(const uint16_t* V, int T, int n_kv, int d, void* stage, hipStream_t stream);
hipError_t launch_stage_pooled(const float* K_pool, const float* V_pool, int pool_ld, int nb, int n_kv, int d,
                               void* stage, const StagePlan& plan, hipStream_t stream);

struct DensePlan {
  int hg_log2;   // log2 of the query heads packed into one workgroup
  int n_qt;      // query tiles of 256 >> hg_log2 rows
  int n_qft;     // rows of mask-flag tiles (64 query rows each)
  int n_ktile;   // flag tiles along the keys (64 keys each)
  int splits;    // key-range splits per (query tile, head slice)
  size_t flags_bytes, part_o_bytes, part_ml_bytes, stage_off, total_bytes;
  StagePlan stage;
};
DensePlan plan_dense(int C, int T, int n_q, int n_kv, int d);

// mask: fp16 [C][mask_ld] (mask_bits false) or, with mask_bits true, uint32 words
// [C][mask_ld] of a bit-packed mask (the pointer is reinterpreted).
// V16: the staged fp16 values, vscales: {2^-k, 2^k} (see launch_stage_values)
hipError_t launch_attn_dense(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V16,
                             const float* vscales, int T, int n_kv, int d, const uint16_t* mask,
                             int64_t mask_ld, float scale, float* O, const DensePlan& plan,
                             const uint8_t* flags, float* part_o, float* part_ml, int causal_q0,
                             hipStream_t stream, bool mask_bits = false);

hipError_t launch_attn_combine(int C, int n_q, int d, int splits, const float* part_o,
                               const float* part_ml, float* O, hipStream_t stream);

// Gather attention over a folded sparse-indexer selection (gather.hip): LDS per
// wave holds the row's listed-block bitmap (words_cap words) and its compacted
// block list (list_cap entries); `waves` waves per workgroup fit in 160 KB.
struct GatherPlan {
  int words_cap, list_cap, waves;
  size_t lds_bytes;
};
GatherPlan plan_gather(int T, int64_t keep_ld, int width);
hipError_t launch_gather_attn(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                              const uint16_t* V, int T, int n_kv, int d, const int32_t* keep_idx,
                              int64_t keep_ld, const int32_t* keep_cnt, int width, int recent,
                              float scale, float* O, const GatherPlan& plan, hipStream_t stream);

hipError_t launch_attn_blocksparse(const uint16_t* Q, int C, int q_start, int n_q,
                                   const uint16_t* K, const uint16_t* V16, const float* vscales,
                                   int T, int n_kv, int d,
                                   const uint16_t* Kp16, const uint16_t* Vp16, int block,
                                   const int32_t* sel_idx, const int32_t* sel_cnt,
                                   float scale, float* O, hipStream_t stream);


}  // namespace pa
