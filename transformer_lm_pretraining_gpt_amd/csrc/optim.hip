// AdamW update, parameter initialisation and the bf16 weight copy (all HBM-bound, flat over N).
//
// AdamW keeps two moments per parameter ("Pré-treinar um LLM", paragraph on memory: weight,
// gradient, m and v in fp32) and is the optimiser of the pretraining objective (same page,
// opening paragraph). Per element, with the bias corrections bc1 = 1 / (1 - b1^t) and
// bc2 = 1 / (1 - b2^t) computed on the host in double precision:
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   p = p - lr * ( m bc1 / (sqrt(v bc2) + eps) + wd p ),  wd applied to 2-D tensors only.
// One pass reads p, g, m, v (16 B) and writes p, m, v (12 B) plus the bf16 copy (2 B) that the
// matrix products read (the half-precision weights of the ZeRO accounting, same page).
//
// Initialisation draws N(0, std^2) with Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011) as a counter-based generator: element i takes
// output word i%4 of block i/4, keyed by the seed, through the Box-Muller transform.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int THREADS = 256;

// The decay runs that meet one launch's range, by value (kernel arguments are read with scalar
// loads, so the per-element lookup is a few compares against uniform values).
constexpr int ADAM_RUNS = 16;
struct AdamRuns {
  int64_t begin[ADAM_RUNS];  // begin[0] <= first element of the launch
  uint32_t decay;            // bit j: run j is decayed
  int n;
};

__global__ __launch_bounds__(THREADS) void adamw_kernel(int64_t begin, int64_t n4,
                                                        float* __restrict__ p,
                                                        const float* __restrict__ g,
                                                        float* __restrict__ m,
                                                        float* __restrict__ v,
                                                        bf16* __restrict__ shadow, AdamRuns runs,
                                                        float lr, float b1, float b2, float eps,
                                                        float wd, float bc1, float bc2) {
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * THREADS) {
    const int64_t e = begin + 4 * i;
    // run holding element e (its four elements share it: run boundaries are multiples of 4)
    uint32_t dec = runs.decay & 1u;
#pragma unroll
    for (int j = 1; j < ADAM_RUNS; ++j)
      if (j < runs.n && e >= runs.begin[j]) dec = (runs.decay >> j) & 1u;
    const float wdi = dec ? wd : 0.0f;
    f32x4 pv = *reinterpret_cast<const f32x4*>(p + e);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(g + e);
    f32x4 mv = *reinterpret_cast<const f32x4*>(m + e);
    f32x4 vv = *reinterpret_cast<const f32x4*>(v + e);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      mv[k] = b1 * mv[k] + (1.0f - b1) * gv[k];
      vv[k] = b2 * vv[k] + (1.0f - b2) * gv[k] * gv[k];
      const float upd = (mv[k] * bc1) / (sqrtf(vv[k] * bc2) + eps);
      pv[k] = pv[k] - lr * (upd + wdi * pv[k]);
    }
    *reinterpret_cast<f32x4*>(p + e) = pv;
    *reinterpret_cast<f32x4*>(m + e) = mv;
    *reinterpret_cast<f32x4*>(v + e) = vv;
    if (shadow) st8(shadow + e, u32x2{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])});
  }
}

DEV void mulhilo(uint32_t a, uint32_t b, uint32_t& hi, uint32_t& lo) {
  const uint64_t r = (uint64_t)a * b;
  hi = (uint32_t)(r >> 32);
  lo = (uint32_t)r;
}

DEV u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(0xD2511F53u, c[0], hi0, lo0);
    mulhilo(0xCD9E8D57u, c[2], hi1, lo1);
    c = u32x4{hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// uniform in (0, 1]
DEV float u01(uint32_t x) { return ((float)(x >> 8) + 1.0f) * (1.0f / 16777216.0f); }

__global__ __launch_bounds__(THREADS) void init_normal_kernel(int64_t begin, int64_t count,
                                                              float* __restrict__ p,
                                                              uint64_t seed, float stdv) {
  const int64_t n4 = (count + 3) / 4;
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * THREADS) {
    const int64_t gi = begin + 4 * i;  // global element index drives the counter
    const int64_t blk = gi >> 2;
    const u32x4 r = philox4x32_10(u32x4{(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u},
                                  (uint32_t)seed, (uint32_t)(seed >> 32));
    float z[4];
    for (int pr = 0; pr < 2; ++pr) {
      const float u1 = u01(r[2 * pr]), u2 = u01(r[2 * pr + 1]);
      const float rad = sqrtf(-2.0f * logf(u1));
      const float ang = 6.283185307179586f * u2;
      z[2 * pr] = rad * cosf(ang);
      z[2 * pr + 1] = rad * sinf(ang);
    }
    // begin may not be a multiple of 4: element gi + k uses word (gi + k) % 4 of its own block
    for (int k = 0; k < 4; ++k) {
      const int64_t j = 4 * i + k;
      if (j >= count) break;
      const int64_t ge = begin + j;
      float val;
      if ((ge >> 2) == blk) {
        val = z[ge & 3];
      } else {
        const u32x4 r2 = philox4x32_10(u32x4{(uint32_t)(ge >> 2), (uint32_t)(ge >> 34), 0u, 0u},
                                       (uint32_t)seed, (uint32_t)(seed >> 32));
        const int w = (int)(ge & 3), pr = w >> 1;
        const float u1 = u01(r2[2 * pr]), u2 = u01(r2[2 * pr + 1]);
        const float rad = sqrtf(-2.0f * logf(u1));
        const float ang = 6.283185307179586f * u2;
        val = (w & 1) ? rad * sinf(ang) : rad * cosf(ang);
      }
      p[j] = stdv * val;
    }
  }
}

__global__ __launch_bounds__(THREADS) void fill_kernel(int64_t count, float* __restrict__ p,
                                                       float value) {
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * THREADS)
    p[i] = value;
}

__global__ __launch_bounds__(THREADS) void cast_bf16_kernel(int64_t count,
                                                            const float* __restrict__ src,
                                                            bf16* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * THREADS)
    dst[i] = (bf16)src[i];
}

unsigned grid_for(int64_t work) {
  const int64_t g = (work + THREADS - 1) / THREADS;
  return (unsigned)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

// Global-norm gradient clipping: ||g|| over the whole flat gradient, then g *= max / (||g|| +
// 1e-6) when that factor is below 1. Block b of the first pass sums the squares of a fixed strided
// set of float4s (fp32 per lane, then a fixed-order tree); the second pass adds the block sums in
// double in a fixed order, so the norm does not depend on scheduling.
__global__ __launch_bounds__(THREADS) void sumsq_partial_kernel(int64_t n4, const float* __restrict__ g,
                                                                float* __restrict__ part) {
  __shared__ float sh[THREADS / 64];
  float s = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * THREADS) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(g + 4 * i);
    s = fmaf(v[0], v[0], s);
    s = fmaf(v[1], v[1], s);
    s = fmaf(v[2], v[2], s);
    s = fmaf(v[3], v[3], s);
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = sh[0];
    for (int w = 1; w < THREADS / 64; ++w) t += sh[w];
    part[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(64) void clip_coef_kernel(int nparts, const float* __restrict__ part,
                                                       float max_norm, float* __restrict__ out,
                                                       float* __restrict__ user_norm) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int i = 0; i < nparts; ++i) s += (double)part[i];
  const float norm = (float)sqrt(s);
  const float coef = max_norm / (norm + 1e-6f);
  out[0] = norm;
  out[1] = coef < 1.0f ? coef : 1.0f;
  if (user_norm) user_norm[0] = norm;
}

__global__ __launch_bounds__(THREADS) void scale_by_kernel(int64_t n4, float* __restrict__ g,
                                                           const float* __restrict__ coef) {
  const float c = *coef;
  if (c >= 1.0f) return;
  for (int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * THREADS) {
    f32x4 v = *reinterpret_cast<const f32x4*>(g + 4 * i);
    *reinterpret_cast<f32x4*>(g + 4 * i) = v * c;
  }
}

}  // namespace

hipError_t launch_clip_grad_norm(int64_t n, float* g, float max_norm, float* scratch,
                                 float* user_norm, hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(sumsq_partial_kernel, dim3(CLIP_PARTS), dim3(THREADS), 0, s, n4, g, scratch);
  hipLaunchKernelGGL(clip_coef_kernel, dim3(1), dim3(64), 0, s, CLIP_PARTS, scratch, max_norm,
                     scratch + CLIP_PARTS, user_norm);
  hipLaunchKernelGGL(scale_by_kernel, dim3(grid_for(n4)), dim3(THREADS), 0, s, n4, g,
                     scratch + CLIP_PARTS + 1);
  return hipGetLastError();
}

hipError_t launch_adamw(int64_t begin, int64_t n, float* p, const float* g, float* m, float* v,
                        void* shadow, const AdamSeg* segs, int nseg, float lr, float b1, float b2,
                        float eps, float wd, float bc1, float bc2, hipStream_t s) {
  if (n % 4 || begin % 4 || nseg < 1 || segs[0].begin != 0) return hipErrorInvalidValue;
  const int64_t end = begin + n;
  // run holding `begin`, then one launch per ADAM_RUNS runs
  int r = 0;
  while (r + 1 < nseg && segs[r + 1].begin <= begin) ++r;
  for (int64_t lo = begin; lo < end;) {
    AdamRuns runs{};
    int64_t hi = end;
    for (int j = 0; r + j < nseg; ++j) {
      const int64_t b = segs[r + j].begin;
      if (j > 0 && b >= end) break;
      if (j == ADAM_RUNS) {
        hi = b;
        break;
      }
      if (b % 4) return hipErrorInvalidValue;
      runs.begin[j] = b;
      runs.decay |= (segs[r + j].decay ? 1u : 0u) << j;
      runs.n = j + 1;
    }
    const int64_t n4 = (hi - lo) / 4;
    hipLaunchKernelGGL(adamw_kernel, dim3(grid_for(n4)), dim3(THREADS), 0, s, lo, n4, p, g, m, v,
                       static_cast<bf16*>(shadow), runs, lr, b1, b2, eps, wd, bc1, bc2);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    r += runs.n;  // the next launch starts at the run that begins at hi
    lo = hi;
  }
  return hipSuccess;
}

hipError_t launch_init_normal(int64_t begin, int64_t count, float* p, uint64_t seed, float stdv,
                              hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(init_normal_kernel, dim3(grid_for((count + 3) / 4)), dim3(THREADS), 0, s,
                     begin, count, p, seed, stdv);
  return hipGetLastError();
}

hipError_t launch_fill(int64_t count, float* p, float value, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(count)), dim3(THREADS), 0, s, count, p, value);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(int64_t count, const float* src, void* dst, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for(count)), dim3(THREADS), 0, s, count, src,
                     static_cast<bf16*>(dst));
  return hipGetLastError();
}
