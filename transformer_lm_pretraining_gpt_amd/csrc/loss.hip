// Fused softmax cross-entropy over the padded vocabulary (HBM-bound).
//
// The loss is the cross-entropy of the next token ("Pré-treinar um LLM", opening paragraph on the
// objective). Logits have vocab_padded columns (50257 padded to 50304, "Criei GPT-2 do zero com
// uma RTX 4090", section "Configuração do treinamento"); the padded columns are masked out: they
// take no part in the log-sum-exp and receive zero gradient.
//
// One block of 1024 threads per row reads the row once into registers (16-byte vectors), forms the max, the sum
// of exponentials and the log-sum-exp, writes the per-row loss lse - z[y], and overwrites the row
// in place with softmax(z) - onehot(y) (zeros in the padded columns). The mean's 1/n and the
// backward's grad_scale are applied later, as the alpha of the LM-head gradient products, so no
// probability matrix is ever written besides this in-place gradient.
//
// Positions whose target is -1 are not trained (loss 0, gradient row 0) and the loss is the mean
// over the others: the instruction-tuning run trains only the assistant's answer and its end
// marker, the prompt being only read ("Criei GPT-2 do zero com uma RTX 4090", section on SFT, list
// item on training only the answer). Its chat markers reuse the spare ids of the padded vocabulary
// (same list), which a configuration with vocab = vocab_padded makes real columns.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int THREADS = 1024;
constexpr int MAXV = 8;   // 16-byte vectors per thread held in registers
constexpr float LOG2E = 1.4426950408889634f;

DEV float block_reduce(float v, float* sh, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float r = sh[0];
  for (int w = 1; w < THREADS / 64; ++w) r = is_max ? fmaxf(r, sh[w]) : r + sh[w];
  return r;
}

// Elements j0 + e >= V of a loaded vector set to -inf (padded vocabulary columns), so that they
// drop out of the max and every exponential without a test per element.
template <typename T>
DEV u32x4 mask_tail(u32x4 r, int j0, int V) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (j0 + 2 * w >= V) r[w] = (r[w] & 0xffff0000u) | 0xff80u;
      if (j0 + 2 * w + 1 >= V) r[w] = (r[w] & 0x0000ffffu) | 0xff800000u;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (j0 + w >= V) r[w] = 0xff800000u;
  }
  return r;
}

// The row through a buffer resource: one per-lane offset register and a scalar offset per
// vector, instead of a 64-bit address per vector (the vectors lie 16 KB apart, beyond the reach of
// an instruction's immediate offset); those address registers made the kernel spill.
DEV __amdgpu_buffer_rsrc_t row_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
DEV u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
typedef __attribute__((ext_vector_type(4))) unsigned int uint4v;
DEV void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4v, v), r, voff, soff, 0);
}

// Hide the packed registers from the optimizer between passes: unpacking again is cheap, while
// keeping every unpacked float alive across passes would cost the occupancy this kernel needs.
DEV void opaque(u32x4 (&reg)[MAXV]) {
#pragma unroll
  for (int k = 0; k < MAXV; ++k) asm volatile("" : "+v"(reg[k]));
}

template <typename T>
__global__ __launch_bounds__(THREADS, 8) void xent_kernel(int V, int Vp, T* __restrict__ logits,
                                                          const int32_t* __restrict__ targets,
                                                          float* __restrict__ row_loss,
                                                          int* __restrict__ err) {
  constexpr int VE = 16 / (int)sizeof(T);
  __shared__ float sh[THREADS / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  T* z = logits + (int64_t)row * Vp;
  const int nvec = Vp / VE;
  const int nfull = V / VE;  // vectors with no padded column
  int y = targets[row];
  if (y == TARGET_IGNORE) {
    // a position that is not trained: no loss, a zero gradient row, the logits are not read
    if (tid == 0) row_loss[row] = 0.0f;
    for (int v = tid; v < nvec; v += THREADS) st16(z + v * VE, u32x4{0, 0, 0, 0});
    return;
  }
  if (y < 0 || y >= V) {
    if (tid == 0) atomicOr(err, ERR_TARGET_RANGE);
    y = 0;  // keep the reads in bounds; the flagged result is not used
  }
  const auto rz = row_rsrc(z, (uint32_t)Vp * sizeof(T));
  const uint32_t voff = 16u * tid;
  u32x4 reg[MAXV];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int v = tid + k * THREADS;
    if (v < nvec) {
      reg[k] = buf_ld16(rz, voff, 16u * THREADS * k);
      if (v >= nfull) reg[k] = mask_tail<T>(reg[k], v * VE, V);
      float f[VE];
      Vec<T>::unpack(reg[k], f);
#pragma unroll
      for (int e = 0; e < VE; ++e) mx = fmaxf(mx, f[e]);
    }
  }
  opaque(reg);
  mx = block_reduce(mx, sh, true);
  const float mx2 = mx * LOG2E;
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int v = tid + k * THREADS;
    if (v < nvec) {
      float f[VE];
      Vec<T>::unpack(reg[k], f);
#pragma unroll
      for (int e = 0; e < VE; ++e) sum += fast_exp2(fmaf(f[e], LOG2E, -mx2));
    }
  }
  opaque(reg);
  sum = block_reduce(sum, sh, false);
  const float lse = mx + logf(sum);
  const float lse2 = lse * LOG2E;
  if (tid == 0) row_loss[row] = lse - to_f32(z[y]);
  __syncthreads();  // z[y] is read before any thread overwrites the row
  // softmax(z) - onehot(y); padded columns give exp2(-inf) = 0
  const int vy = y / VE, ey = y % VE;
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int v = tid + k * THREADS;
    if (v < nvec) {
      float f[VE];
      Vec<T>::unpack(reg[k], f);
#pragma unroll
      for (int e = 0; e < VE; ++e) f[e] = fast_exp2(fmaf(f[e], LOG2E, -lse2));
      if (v == vy) {
#pragma unroll
        for (int e = 0; e < VE; ++e)
          if (e == ey) f[e] -= 1.0f;
      }
      buf_st16(rz, voff, 16u * THREADS * k, Vec<T>::pack(f));
    }
  }
}

// Mean over the trained positions (ignored rows hold loss 0), and the matching gradient scale.
// One block of 1024 threads (it sits between the forward and the backward, so its latency counts):
// each thread adds a strided set of rows, then the 16 wave sums are added in wave order.
constexpr int MEAN_THREADS = 1024;
__global__ __launch_bounds__(MEAN_THREADS) void loss_mean_kernel(
    int M, const float* __restrict__ rows, const int32_t* __restrict__ targets,
    float* __restrict__ out, float* __restrict__ out_user) {
  constexpr int NW = MEAN_THREADS / 64;
  __shared__ float sh[NW];
  __shared__ int shn[NW];
  float s = 0.0f;
  int n = 0;
#pragma unroll 4
  for (int i = threadIdx.x; i < M; i += MEAN_THREADS) {
    s += rows[i];
    n += targets[i] != TARGET_IGNORE;
  }
  s = wave_sum(s);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
  if ((threadIdx.x & 63) == 0) {
    sh[threadIdx.x >> 6] = s;
    shn[threadIdx.x >> 6] = n;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.0f;
    int cnt = 0;
    for (int w = 0; w < NW; ++w) {
      tot += sh[w];
      cnt += shn[w];
    }
    const float mean = cnt > 0 ? tot / (float)cnt : 0.0f;
    out[0] = mean;
    out[1] = cnt > 0 ? 1.0f / (float)cnt : 0.0f;
    if (out_user) out_user[0] = mean;
  }
}

}  // namespace

hipError_t launch_xent(bool is_bf16, int M, int V, int Vp, void* logits, const int32_t* targets,
                       float* row_loss, int* err, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int ve = is_bf16 ? 8 : 4;
  if (Vp % ve || Vp / ve > MAXV * THREADS) return hipErrorInvalidValue;
  if (is_bf16)
    hipLaunchKernelGGL(xent_kernel<bf16>, dim3(M), dim3(THREADS), 0, s, V, Vp,
                       static_cast<bf16*>(logits), targets, row_loss, err);
  else
    hipLaunchKernelGGL(xent_kernel<float>, dim3(M), dim3(THREADS), 0, s, V, Vp,
                       static_cast<float*>(logits), targets, row_loss, err);
  return hipGetLastError();
}

hipError_t launch_loss_mean(int M, const float* row_loss, const int32_t* targets, float* loss_out,
                            float* loss_user, hipStream_t s) {
  hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(MEAN_THREADS), 0, s, M, row_loss, targets,
                     loss_out, loss_user);
  return hipGetLastError();
}
