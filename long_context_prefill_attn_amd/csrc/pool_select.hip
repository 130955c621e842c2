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
#include "common.h"

namespace pa {

// ---------------------------------------------------------------------------
// build_pooled_index: one lane owns 8 adjacent columns (of the n_kv*d columns
// of a token row) of one key block, and walks the block's tokens in order.
// A wave reads 64 x 16 contiguous bytes per token: coalesced, HBM-bound.
// grid = (ceil(cols8 / 64), n_blocks, 2 [K, V]), block = 64.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) pool_kernel(const uint16_t* __restrict__ K,
                                                  const uint16_t* __restrict__ V, int T,
                                                  int cols8, int d, int block, int nb,
                                                  float* __restrict__ Kp, float* __restrict__ Vp) {
  const int c8 = blockIdx.x * 64 + threadIdx.x;
  if (c8 >= cols8) return;
  const int b = blockIdx.y;
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
  float4* dst = reinterpret_cast<float4*>(P + ((size_t)g * nb + b) * d + dd);
  dst[0] = make_float4(out[0], out[1], out[2], out[3]);
  dst[1] = make_float4(out[4], out[5], out[6], out[7]);
}

hipError_t launch_pool(const uint16_t* K, const uint16_t* V, int T, int n_kv, int d, int block,
                       float* K_pool, float* V_pool, hipStream_t stream) {
  const int cols8 = n_kv * d / 8;
  const int nb = (T + block - 1) / block;
  dim3 grid((cols8 + 63) / 64, nb, 2);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(64), 0, stream, K, V, T, cols8, d, block, nb, K_pool,
                     V_pool);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// select_blocks: one workgroup per (KV head g, query block j).
//
// Voters are the (row, query head) pairs of block j in this chunk. For each
// tile of VT voters the workgroup computes r[v][b] for all candidates b < j
// (thread <-> candidate block, voter queries broadcast from LDS in fp64),
// keeps r in LDS, reduces each voter's max, and ORs the votes into a per-block
// flag. The flags are then compacted in ascending order and the diagonal
// block appended.
// ---------------------------------------------------------------------------
constexpr int SEL_THREADS = 256;
constexpr int SEL_R_BUDGET = 4096;  // doubles of r kept in LDS per voter tile

template <int D>
__global__ void __launch_bounds__(SEL_THREADS) select_kernel(
    const uint16_t* __restrict__ Q, int C, int q_start, int n_q, int n_kv,
    const float* __restrict__ Kp, int nb, int block, double theta, int vt_max,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt) {
  extern __shared__ __attribute__((aligned(16))) double smem[];
  const int g = blockIdx.y;
  const int jj = blockIdx.x;
  const int j0 = q_start / block;
  const int j = j0 + jj;
  const int group = n_q / n_kv;
  const int nc = j;  // candidates 0..j-1
  const int r0 = max(j * block, q_start) - q_start;
  const int r1 = min((j + 1) * block, q_start + C) - q_start;
  const int nv = (r1 - r0) * group;
  const int tid = threadIdx.x;

  double* q_s = smem;                              // [vt_max][D]
  double* r_s = q_s + (size_t)vt_max * D;          // [vt_max][nc]
  int* flag_s = reinterpret_cast<int*>(r_s + (size_t)vt_max * max(nc, 1));  // [nb]
  __shared__ int cnt_s[SEL_THREADS + 1];

  for (int b = tid; b < nb; b += SEL_THREADS) flag_s[b] = 0;

  const float* kg = Kp + (size_t)g * nb * D;
  if (nc > 0) {
    for (int v0 = 0; v0 < nv; v0 += vt_max) {
      const int vt = min(vt_max, nv - v0);
      __syncthreads();  // previous tile's r_s / q_s readers are done
      for (int e = tid; e < vt * D; e += SEL_THREADS) {
        const int v = e / D, dd = e % D;
        const int voter = v0 + v;
        const int row = r0 + voter / group;
        const int h = g * group + voter % group;
        q_s[v * D + dd] = (double)bf16_to_f32(Q[((size_t)row * n_q + h) * D + dd]);
      }
      __syncthreads();
      for (int b = tid; b < nc; b += SEL_THREADS) {
        const float* kb = kg + (size_t)b * D;
        for (int vs = 0; vs < vt; vs += 8) {
          const int nvs = min(8, vt - vs);
          double acc[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) acc[u] = 0.0;
#pragma unroll 1
          for (int ds = 0; ds < D; ds += 32) {
            double kr[32];
#pragma unroll
            for (int e = 0; e < 32; e += 4) {
              const float4 f = *reinterpret_cast<const float4*>(kb + ds + e);
              kr[e] = f.x; kr[e + 1] = f.y; kr[e + 2] = f.z; kr[e + 3] = f.w;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              if (u < nvs) {
                const double* qv = q_s + (vs + u) * D + ds;
#pragma unroll
                for (int e = 0; e < 32; ++e) acc[u] = __builtin_fma(qv[e], kr[e], acc[u]);
              }
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (u < nvs) r_s[(size_t)(vs + u) * nc + b] = acc[u];
        }
      }
      __syncthreads();
      // per voter: max over candidates, then votes (one wave per voter)
      const int wave = tid / 64, lane = tid % 64;
      for (int v = wave; v < vt; v += SEL_THREADS / 64) {
        const double* rv = r_s + (size_t)v * nc;
        double mx = -__builtin_inf();
        for (int b = lane; b < nc; b += 64) mx = fmax(mx, rv[b]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
        for (int b = lane; b < nc; b += 64)
          if (rv[b] - mx > theta) flag_s[b] = 1;
      }
    }
  }
  __syncthreads();
  // ascending compaction of flags[0..nc) via per-thread contiguous chunks
  const int per = (nc + SEL_THREADS - 1) / SEL_THREADS;
  const int c0 = min(tid * per, nc), c1 = min(c0 + per, nc);
  int mine = 0;
  for (int b = c0; b < c1; ++b) mine += flag_s[b];
  cnt_s[tid] = mine;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < SEL_THREADS; ++t) {
      const int c = cnt_s[t];
      cnt_s[t] = run;
      run += c;
    }
    cnt_s[SEL_THREADS] = run;
  }
  __syncthreads();
  int32_t* out = sel_idx + ((size_t)g * gridDim.x + jj) * nb;
  int pos = cnt_s[tid];
  for (int b = c0; b < c1; ++b)
    if (flag_s[b]) out[pos++] = b;
  const int total = cnt_s[SEL_THREADS];
  if (tid == 0) {
    out[total] = j;  // the local diagonal block is always kept
    sel_cnt[(size_t)g * gridDim.x + jj] = total + 1;
  }
  for (int b = total + 1 + tid; b < nb; b += SEL_THREADS) out[b] = 0;
}

hipError_t launch_select(const uint16_t* Q, int C, int q_start, int n_q, int n_kv, int d,
                         const float* K_pool, int T, int block, double theta,
                         int32_t* sel_idx, int32_t* sel_cnt, hipStream_t stream) {
  const int nb = (T + block - 1) / block;
  const int j0 = q_start / block;
  const int j1 = (q_start + C - 1) / block;
  const int n_qblk = j1 - j0 + 1;
  const int nc_max = max(j1, 1);
  int vt = SEL_R_BUDGET / nc_max;
  vt = max(1, min(vt, 32));
  const size_t lds = (size_t)vt * d * 8 + (size_t)vt * nc_max * 8 + (size_t)nb * 4;
  dim3 grid(n_qblk, n_kv);
  if (d == 128) {
    hipFuncSetAttribute((const void*)select_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)lds);
    hipLaunchKernelGGL(select_kernel<128>, grid, dim3(SEL_THREADS), lds, stream, Q, C, q_start, n_q,
                       n_kv, K_pool, nb, block, theta, vt, sel_idx, sel_cnt);
  } else {
    hipFuncSetAttribute((const void*)select_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)lds);
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(SEL_THREADS), lds, stream, Q, C, q_start, n_q,
                       n_kv, K_pool, nb, block, theta, vt, sel_idx, sel_cnt);
  }
  return hipGetLastError();
}

}  // namespace pa
