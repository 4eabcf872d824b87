// LayerNorm forward / backward and deterministic column reductions (bias and LN-parameter
// gradients). HBM-bound; one wave per row, fp32 statistics.
//
// LayerNorm of the pre-LN GPT-2 block (the block the nanoGPT-style code of "Criei GPT-2 do zero
// com uma RTX 4090", section "Ambiente", builds): mean, biased variance, eps = 1e-5,
//   y = (x - mean) * rstd * g + b,  rstd = 1 / sqrt(var + eps).
// Backward, with xhat = (x - mean) * rstd and dxh = dy * g:
//   dx = rstd * (dxh - mean(dxh) - xhat * mean(dxh * xhat)),  dg = sum_rows dy * xhat,
//   db = sum_rows dy.
// Column sums never use atomics: each block writes its partial row, a second kernel adds the
// partials in a fixed order, so results are bitwise reproducible.
#include <type_traits>

#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int MAXV = 8;  // float4 vectors per lane: d <= 2048
constexpr float LN_EPS = 1e-5f;

template <typename T>
DEV f32x4 load4(const T* src) {
  if constexpr (sizeof(T) == 4) {
    return *reinterpret_cast<const f32x4*>(src);
  } else {
    const u32x2 u = ld8(src);
    return f32x4{bf16lo(u[0]), bf16hi(u[0]), bf16lo(u[1]), bf16hi(u[1])};
  }
}

template <typename T>
DEV void store4(T* dst, const float (&v)[4]) {
  if constexpr (sizeof(T) == 2)
    st8(dst, u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])});
  else
    st16(dst, u32x4{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                    __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])});
}

template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_fwd_kernel(int M, int d, const float* __restrict__ x,
                                                     const float* __restrict__ g,
                                                     const float* __restrict__ b,
                                                     T* __restrict__ y, float* __restrict__ mean,
                                                     float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nv = d >> 2;
  const float* xr = x + (int64_t)row * d;
  f32x4 xv[NV];
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = lane + 64 * k;
    xv[k] = v < nv ? *reinterpret_cast<const f32x4*>(xr + 4 * v) : f32x4{0, 0, 0, 0};
    s += (xv[k][0] + xv[k][1]) + (xv[k][2] + xv[k][3]);
  }
  const float mu = wave_sum(s) / (float)d;
  float s2 = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = lane + 64 * k;
    if (v < nv) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = xv[k][e] - mu;
        s2 += c * c;
      }
    }
  }
  const float var = wave_sum(s2) / (float)d;
  const float r = 1.0f / sqrtf(var + LN_EPS);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = lane + 64 * k;
    if (v < nv) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(g + 4 * v);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(b + 4 * v);
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (xv[k][e] - mu) * r * gv[e] + bv[e];
      store4<T>(y + (int64_t)row * d + 4 * v, o);
    }
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = r;
  }
}

// One block = 4 waves over rows [blk*rpb, blk*rpb + rpb); wave w takes rows w, w+4, ...
template <typename T, int NV>
__global__ __launch_bounds__(256) void ln_bwd_kernel(
    int M, int d, const T* __restrict__ dy, const float* __restrict__ x,
    const float* __restrict__ mean, const float* __restrict__ rstd, const float* __restrict__ g,
    float* __restrict__ dres, int has_dres, T* __restrict__ dres_t, float* __restrict__ part,
    int rpb) {
  extern __shared__ float red[];  // [4][d]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nv = d >> 2;
  f32x4 pg[NV], pb[NV], pr[NV], gv[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    pg[k] = pb[k] = pr[k] = f32x4{0, 0, 0, 0};
    const int v = lane + 64 * k;
    gv[k] = v < nv ? *reinterpret_cast<const f32x4*>(g + 4 * v) : f32x4{0, 0, 0, 0};
  }
  const int r0 = blockIdx.x * rpb, r1 = min(M, r0 + rpb);
  for (int row = r0 + wave; row < r1; row += 4) {
    const float mu = mean[row], rs = rstd[row];
    const int64_t base = (int64_t)row * d;
    f32x4 xh[NV], dyv[NV], dr[NV];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = lane + 64 * k;
      if (v < nv) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(x + base + 4 * v);
        dyv[k] = load4<T>(dy + base + 4 * v);
        // the incoming residual gradient is loaded with the row, ahead of the reductions
        dr[k] = has_dres ? *reinterpret_cast<const f32x4*>(dres + base + 4 * v) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[k][e] = (xv[e] - mu) * rs;
          const float dxh = dyv[k][e] * gv[k][e];
          s1 += dxh;
          s2 += dxh * xh[k][e];
        }
      }
    }
    s1 = wave_sum(s1) / (float)d;
    s2 = wave_sum(s2) / (float)d;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = lane + 64 * k;
      if (v < nv) {
        f32x4 nw = dr[k];
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dxh = dyv[k][e] * gv[k][e];
          nw[e] += rs * (dxh - s1 - xh[k][e] * s2);
          o[e] = nw[e];
          pg[k][e] += dyv[k][e] * xh[k][e];
          pb[k][e] += dyv[k][e];
          pr[k][e] += nw[e];
        }
        *reinterpret_cast<f32x4*>(dres + base + 4 * v) = nw;
        store4<T>(dres_t + base + 4 * v, o);
      }
    }
  }
  // combine the 4 waves in a fixed order, one partial kind at a time
  float* out = part + (int64_t)blockIdx.x * 3 * d;
#pragma unroll
  for (int kind = 0; kind < 3; ++kind) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = lane + 64 * k;
      if (v < nv)
        *reinterpret_cast<f32x4*>(red + wave * d + 4 * v) =
            kind == 0 ? pg[k] : (kind == 1 ? pb[k] : pr[k]);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < d; j += 256)
      out[kind * d + j] = ((red[j] + red[d + j]) + red[2 * d + j]) + red[3 * d + j];
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(int M, int N,
                                                             const T* __restrict__ src,
                                                             int64_t ld, float* __restrict__ part,
                                                             int rpb) {
  constexpr int VE = 16 / (int)sizeof(T);
  const int nvec = N / VE;
  const int r0 = blockIdx.x * rpb, r1 = min(M, r0 + rpb);
  for (int cv = threadIdx.x; cv < nvec; cv += 256) {
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.0f;
    for (int row = r0; row < r1; ++row) {
      float f[VE];
      Vec<T>::unpack(ld16(src + (int64_t)row * ld + cv * VE), f);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] += f[e];
    }
    float* out = part + (int64_t)blockIdx.x * N + cv * VE;
#pragma unroll
    for (int e = 0; e < VE; ++e) out[e] = acc[e];
  }
}

// Sum of nparts partial rows per column. One block = 16 waves over 64 columns; wave w adds the
// partials w, w+16, w+32, ... (four independent accumulators), then the 16 wave sums are added
// in wave order. Columns [0, n) go to up to three outputs of `seg` columns each.
struct ColOut {
  float* out[3];
};
constexpr int RED_WAVES = 16;

DEV void colsum_reduce_block(const float* __restrict__ part, int nparts, int64_t stride, int n,
                             int seg, float* const (&outs)[3], int accumulate, int chunk) {
  __shared__ float sh[RED_WAVES][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = chunk * 64 + lane;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  if (j < n) {
    int p = wave;
    for (; p + 3 * RED_WAVES < nparts; p += 4 * RED_WAVES) {
      a0 += part[(int64_t)p * stride + j];
      a1 += part[(int64_t)(p + RED_WAVES) * stride + j];
      a2 += part[(int64_t)(p + 2 * RED_WAVES) * stride + j];
      a3 += part[(int64_t)(p + 3 * RED_WAVES) * stride + j];
    }
    for (; p < nparts; p += RED_WAVES) a0 += part[(int64_t)p * stride + j];
  }
  sh[wave][lane] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (wave == 0 && j < n) {
    float s = 0.0f;
    for (int w = 0; w < RED_WAVES; ++w) s += sh[w][lane];
    float* o = outs[j / seg];
    if (o) {
      const int c = j % seg;
      o[c] = accumulate ? o[c] + s : s;
    }
  }
}

__global__ __launch_bounds__(64 * RED_WAVES) void colsum_reduce_kernel(
    const float* __restrict__ part, int nparts, int64_t stride, int n, int seg, ColOut outs,
    int accumulate) {
  colsum_reduce_block(part, nparts, stride, n, seg, outs.out, accumulate, blockIdx.x);
}

// The batch: block b finds the last task whose first block is <= b (tasks are few).
__global__ __launch_bounds__(64 * RED_WAVES) void colsum_reduce_batch_kernel(
    const ColTask* __restrict__ tasks, int ntasks, int accumulate) {
  const int blk = blockIdx.x;
  int t = 0;
  while (t + 1 < ntasks && tasks[t + 1].block0 <= blk) ++t;
  const ColTask& tk = tasks[t];
  float* const outs[3] = {tk.out[0], tk.out[1], tk.out[2]};
  colsum_reduce_block(tk.part, tk.nparts, tk.stride, tk.n, tk.seg, outs, accumulate, blk - tk.block0);
}

}  // namespace

namespace {
// Calls f(std::integral_constant<int, NV>) with NV = float4 vectors per lane for rows of d floats
// (1 .. MAXV), so that the per-lane arrays are sized for the actual width.
template <typename F>
hipError_t with_nv(int d, F&& f) {
  switch ((d / 4 + 63) / 64) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_ln_fwd(bool is_bf16, int M, int d, const float* x, const float* g,
                         const float* b, void* y, float* mean, float* rstd, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (d % 4 || d > 4 * 64 * MAXV) return hipErrorInvalidValue;
  dim3 grid((M + 3) / 4);
  return with_nv(d, [&](auto nv) {
    constexpr int NV = decltype(nv)::value;
    if (is_bf16)
      hipLaunchKernelGGL((ln_fwd_kernel<bf16, NV>), grid, dim3(256), 0, s, M, d, x, g, b,
                         static_cast<bf16*>(y), mean, rstd);
    else
      hipLaunchKernelGGL((ln_fwd_kernel<float, NV>), grid, dim3(256), 0, s, M, d, x, g, b,
                         static_cast<float*>(y), mean, rstd);
    return hipGetLastError();
  });
}

int ln_bwd_blocks(int M, int rows_per_block) { return (M + rows_per_block - 1) / rows_per_block; }

hipError_t launch_ln_bwd(bool is_bf16, int M, int d, const void* dy, const float* x,
                         const float* mean, const float* rstd, const float* g, float* dres,
                         int has_dres, void* dres_t, float* part, int rows_per_block,
                         hipStream_t s, hipEvent_t done) {
  if (M == 0) return hipSuccess;
  if (d % 4 || d > 4 * 64 * MAXV) return hipErrorInvalidValue;
  dim3 grid(ln_bwd_blocks(M, rows_per_block));
  const size_t lds = 4 * (size_t)d * sizeof(float);
  return with_nv(d, [&](auto nv) {
    constexpr int NV = decltype(nv)::value;
    // `done`, when given, is recorded by the launch itself (no marker packet of its own)
    if (is_bf16)
      hipExtLaunchKernelGGL((ln_bwd_kernel<bf16, NV>), grid, dim3(256), lds, s, nullptr, done, 0,
                            M, d, static_cast<const bf16*>(dy), x, mean, rstd, g, dres, has_dres,
                            static_cast<bf16*>(dres_t), part, rows_per_block);
    else
      hipExtLaunchKernelGGL((ln_bwd_kernel<float, NV>), grid, dim3(256), lds, s, nullptr, done, 0,
                            M, d, static_cast<const float*>(dy), x, mean, rstd, g, dres, has_dres,
                            static_cast<float*>(dres_t), part, rows_per_block);
    return hipGetLastError();
  });
}

hipError_t launch_colsum_partial(bool src_bf16, int M, int N, const void* src, int64_t ld,
                                 float* part, int rows_per_block, hipStream_t s) {
  if (M == 0) return hipSuccess;
  dim3 grid((M + rows_per_block - 1) / rows_per_block);
  if (src_bf16)
    hipLaunchKernelGGL(colsum_partial_kernel<bf16>, grid, dim3(256), 0, s, M, N,
                       static_cast<const bf16*>(src), ld, part, rows_per_block);
  else
    hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, s, M, N,
                       static_cast<const float*>(src), ld, part, rows_per_block);
  return hipGetLastError();
}

hipError_t launch_colsum_reduce_batch(const ColTask* d_tasks, int ntasks, int nblocks,
                                      int accumulate, hipStream_t s) {
  if (ntasks == 0 || nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_reduce_batch_kernel, dim3(nblocks), dim3(64 * RED_WAVES), 0, s, d_tasks,
                     ntasks, accumulate);
  return hipGetLastError();
}

hipError_t launch_colsum_reduce(const float* part, int nparts, int64_t stride, int n, float* out,
                                int accumulate, hipStream_t s) {
  return launch_colsum_reduce3(part, nparts, stride, n, out, nullptr, nullptr, accumulate, s);
}

hipError_t launch_colsum_reduce3(const float* part, int nparts, int64_t stride, int seg,
                                 float* out0, float* out1, float* out2, int accumulate,
                                 hipStream_t s) {
  if (seg == 0) return hipSuccess;
  const int nseg = out2 ? 3 : (out1 ? 2 : 1);
  const int n = nseg * seg;
  ColOut outs{{out0, out1, out2}};
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((n + 63) / 64), dim3(64 * RED_WAVES), 0, s, part,
                     nparts, stride, n, seg, outs, accumulate);
  return hipGetLastError();
}
