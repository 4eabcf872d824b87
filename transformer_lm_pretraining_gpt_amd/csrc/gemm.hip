// Tiled MFMA matrix product for gfx950, C = op(A) op(B) with fused epilogues.
//
// Every linear layer of the step is one of these products: the forward x W + b, the input
// gradient dY W^T and the weight gradient X^T dY ("Pré-treinar um LLM", paragraph deriving 6ND:
// forward and both backward products are matmuls of the forward's size). The tied LM head is the
// same kernel with the (Vp, d) embedding as the B operand.
//
// Design:
//  * 256 threads = 4 waves in a 2 x 2 arrangement; block tile BM x BN, wave tile BM/2 x BN/2 made
//    of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16, or 4 x v_mfma_f32_32x32x2f32 for fp32).
//  * K advances in 128-byte slabs (64 bf16 or 32 fp32). Each operand tile lives in LDS as rows of
//    128 bytes, k contiguous, with the 16-byte chunk index XOR-swizzled by (row + row/8) mod 8 so
//    that both the fills and the MFMA fragment reads are free of bank conflicts.
//  * Two LDS stages: the global loads of slab k+1 are issued before the MFMAs of slab k and land
//    in registers; they are written to the other stage after the MFMAs; one barrier per slab.
//  * Operands whose k is the strided dimension (the weight in x W, and both operands of X^T dY)
//    are loaded along their contiguous dimension and transposed in registers on the way to LDS,
//    so every MFMA reads k-contiguous 16-byte fragments.
//  * Blocks are renumbered so that consecutive tiles share an XCD (8 XCDs, own L2 each) and
//    walk the output in groups of 8 row-tiles for L2 reuse of A and B.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int ROWB = 128;  // bytes of one k-slab row in LDS
constexpr int THREADS = 256;

DEV int swz(int row) { return (row + (row >> 3)) & 7; }
DEV int lds_off(int row, int chunk) { return row * ROWB + ((chunk ^ swz(row)) << 4); }

DEV float gelu_tanh(float u) {
  const float c = 0.7978845608028654f, a = 0.044715f;
  return 0.5f * u * (1.0f + tanhf(c * (u + a * u * u * u)));
}
DEV float gelu_tanh_grad(float u) {
  const float c = 0.7978845608028654f, a = 0.044715f;
  float t = tanhf(c * (u + a * u * u * u));
  return 0.5f * (1.0f + t) + 0.5f * u * (1.0f - t * t) * c * (1.0f + 3.0f * a * u * u);
}

// Global -> register -> LDS movement of one operand tile of R rows x one k-slab.
// KMAJOR: stored [r][k] (ld = row pitch in elements); else stored [k][r].
template <typename T, int R, bool KMAJOR>
struct TileLoader {
  static constexpr int VE = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int KT = ROWB / (int)sizeof(T);  // k elements per slab
  static constexpr int NLD = R / 32;                // 16-byte loads per thread per slab
  u32x4 reg[NLD];

  // r0: first row of the tile; k0: first k of the slab; k_end: exclusive bound of k.
  DEV void load(const T* __restrict__ base, int64_t ld, int r0, int r_total, int k0, int k_end,
                int tid) {
    if constexpr (KMAJOR) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        int c = tid + i * THREADS;
        int row = c >> 3, kc = c & 7;
        int r = r0 + row, k = k0 + kc * VE;
        if (r < r_total && k < k_end)
          reg[i] = ld16(base + (int64_t)r * ld + k);
        else
          reg[i] = u32x4{0, 0, 0, 0};
      }
    } else {
      // sub-block of NLD k-rows x VE r-values; 256 sub-blocks cover the slab exactly
      constexpr int RB = R / VE;
      int rb = tid % RB, kb = tid / RB;
      int r = r0 + rb * VE;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        int k = k0 + kb * NLD + j;
        if (r < r_total && k < k_end)
          reg[j] = ld16(base + (int64_t)k * ld + r);
        else
          reg[j] = u32x4{0, 0, 0, 0};
      }
    }
  }

  DEV void store(char* lds, int tid) const {
    if constexpr (KMAJOR) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        int c = tid + i * THREADS;
        int row = c >> 3, kc = c & 7;
        st16(lds + lds_off(row, kc), reg[i]);
      }
    } else {
      constexpr int RB = R / VE;
      int rb = tid % RB, kb = tid / RB;
      const int kbyte = kb * NLD * (int)sizeof(T);  // byte offset of this sub-block's k-range
      if constexpr (sizeof(T) == 2) {
        // bf16: out row e holds element e of each of the NLD loaded vectors
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          int row = rb * VE + e;
          const int w = e >> 1;
          const bool hi = e & 1;
          uint32_t q[NLD / 2];
#pragma unroll
          for (int j = 0; j < NLD / 2; ++j) {
            uint32_t a = reg[2 * j][w], b = reg[2 * j + 1][w];
            q[j] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
          }
          char* dst = lds + row * ROWB + (((kbyte >> 4) ^ swz(row)) << 4) + (kbyte & 15);
          if constexpr (NLD == 8)
            st16(dst, u32x4{q[0], q[1], q[2], q[3]});
          else
            st8(dst, u32x2{q[0], q[1]});
        }
      } else {
        // fp32: out row e holds element e of each loaded vector (NLD = 4 or 8 values)
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          int row = rb * VE + e;
#pragma unroll
          for (int h = 0; h < NLD / 4; ++h) {
            u32x4 q{reg[4 * h][e], reg[4 * h + 1][e], reg[4 * h + 2][e], reg[4 * h + 3][e]};
            int kb2 = kbyte + h * 16;
            st16(lds + row * ROWB + (((kb2 >> 4) ^ swz(row)) << 4), q);
          }
        }
      }
    }
  }
};

// Write one wave's MB x NB 32x32 accumulator tiles; row0/col0: the wave tile's origin.
template <typename T, int EPI, int MB, int NB>
DEV void epilogue(const f32x16 (&acc)[MB][NB], const GemmParams& p, int row0, int col0, int h,
                  int l32) {
  float* cf = static_cast<float*>(p.C);
  if (EPI == EPI_F32) cf += (int64_t)blockIdx.z * p.c_split_stride;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int col = col0 + j * 32 + l32;
    const bool col_ok = col < p.N;
    const float bias = (p.bias && col_ok) ? p.bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + mfma_row(r, h);
        if (!col_ok || row >= p.M) continue;
        const int64_t o = (int64_t)row * p.ldc + col;
        const float a = acc[i][j][r];
        if constexpr (EPI == EPI_STORE) {
          static_cast<T*>(p.C)[o] = from_f32<T>(p.alpha * a + bias);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
          const float u = a + bias;
          static_cast<T*>(p.C)[o] = from_f32<T>(u);
          static_cast<T*>(p.C2)[o] = from_f32<T>(gelu_tanh(u));
        } else if constexpr (EPI == EPI_BIAS_RESID) {
          cf[o] = p.resid[o] + a + bias;
        } else if constexpr (EPI == EPI_GELU_BWD) {
          const float u = to_f32(static_cast<const T*>(p.aux)[o]);
          static_cast<T*>(p.C)[o] = from_f32<T>(a * gelu_tanh_grad(u));
        } else {
          const float prev = p.beta != 0.0f ? p.beta * cf[o] : 0.0f;
          cf[o] = p.alpha * a + prev;
        }
      }
    }
  }
}

template <typename T, int AK, int BKM, int BM, int BN, int TAG>
__global__ __launch_bounds__(THREADS) void gemm_kernel(GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int KT = ROWB / (int)sizeof(T);
  constexpr int STAGE = (BM + BN) * ROWB;  // one stage: A tile then B tile
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;

  // XCD-aware renumbering, then grouped tile order
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GROUP = 8;
  const int in_group = GROUP * tiles_n;
  const int g = bid / in_group;
  const int first_m = g * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % in_group) % gsize;
  const int tn = (bid % in_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int k_begin = blockIdx.z * p.k_split;
  const int k_end = min(p.K, k_begin + p.k_split);
  const int nk = (k_end - k_begin + KT - 1) / KT;

  const T* A = static_cast<const T*>(p.A);
  const T* B = static_cast<const T*>(p.B);
  TileLoader<T, BM, AK == 1> la;
  TileLoader<T, BN, BKM == 1> lb;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;

  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, k_begin, k_end, tid);
    lb.load(B, p.ldb, n0, p.N, k_begin, k_end, tid);
    la.store(smem, tid);
    lb.store(smem + BM * ROWB, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int kn = k_begin + (kt + 1) * KT;
      la.load(A, p.lda, m0, p.M, kn, k_end, tid);
      lb.load(B, p.ldb, n0, p.N, kn, k_end, tid);
    }
    const char* sa = smem + cur * STAGE;
    const char* sb = sa + BM * ROWB;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 fa[MB], fb[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(sa + lds_off(wm0 + i * 32 + l32, 2 * s + h));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(sb + lds_off(wn0 + j * 32 + l32, 2 * s + h));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) Mfma<T>::mma(acc[i][j], fa[i], fb[j]);
    }
    if (more) {
      la.store(smem + (cur ^ 1) * STAGE, tid);
      lb.store(smem + (cur ^ 1) * STAGE + BM * ROWB, tid);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  const int row0 = m0 + wm0, col0 = n0 + wn0;
  switch (p.epi) {
    case EPI_STORE: epilogue<T, EPI_STORE, MB, NB>(acc, p, row0, col0, h, l32); break;
    case EPI_BIAS_GELU: epilogue<T, EPI_BIAS_GELU, MB, NB>(acc, p, row0, col0, h, l32); break;
    case EPI_BIAS_RESID: epilogue<T, EPI_BIAS_RESID, MB, NB>(acc, p, row0, col0, h, l32); break;
    case EPI_GELU_BWD: epilogue<T, EPI_GELU_BWD, MB, NB>(acc, p, row0, col0, h, l32); break;
    default: epilogue<T, EPI_F32, MB, NB>(acc, p, row0, col0, h, l32); break;
  }
}

__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t stride,
                                     int M, int N, float* __restrict__ C, int64_t ldc, float alpha,
                                     float beta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int row = (int)(idx / N), col = (int)(idx % N);
  const int64_t src = (int64_t)row * ldc + col;
  float s = 0.0f;
  for (int z = 0; z < splits; ++z) s += part[z * stride + src];
  const float prev = beta != 0.0f ? beta * C[src] : 0.0f;
  C[src] = alpha * s + prev;
}

template <typename T, int AK, int BKM, int BM, int BN>
hipError_t launch_t(int splits, int tag, const GemmParams& p, hipStream_t s) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  dim3 grid(tiles, 1, splits), block(THREADS);
  // tag 1: a separately named copy of the LM-head product, so profilers report it on its own
  if constexpr (sizeof(T) == 2 && AK == 1 && BKM == 1 && BM == 256 && BN == 256) {
    if (tag == 1) {
      hipLaunchKernelGGL((gemm_kernel<T, AK, BKM, BM, BN, 1>), grid, block, 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<T, AK, BKM, BM, BN, 0>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename T, int BM, int BN>
hipError_t launch_layout(int a_kmajor, int b_kmajor, int splits, int tag, const GemmParams& p,
                         hipStream_t s) {
  if (a_kmajor && !b_kmajor) return launch_t<T, 1, 0, BM, BN>(splits, tag, p, s);
  if (a_kmajor && b_kmajor) return launch_t<T, 1, 1, BM, BN>(splits, tag, p, s);
  if (!a_kmajor && !b_kmajor) return launch_t<T, 0, 0, BM, BN>(splits, tag, p, s);
  return launch_t<T, 0, 1, BM, BN>(splits, tag, p, s);
}

template <typename T>
hipError_t launch_type(int a_kmajor, int b_kmajor, int tile, int splits, int tag,
                       const GemmParams& p, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    // fp32 runs the small configurations only
    return launch_layout<T, 128, 128>(a_kmajor, b_kmajor, splits, tag, p, s);
  } else {
    switch (tile) {
      case TILE_256: return launch_layout<T, 256, 256>(a_kmajor, b_kmajor, splits, tag, p, s);
      case TILE_256x128: return launch_layout<T, 256, 128>(a_kmajor, b_kmajor, splits, tag, p, s);
      default: return launch_layout<T, 128, 128>(a_kmajor, b_kmajor, splits, tag, p, s);
    }
  }
}

}  // namespace

int gemm_k_tile(bool is_bf16) { return is_bf16 ? ROWB / 2 : ROWB / 4; }

hipError_t launch_gemm(bool is_bf16, int a_kmajor, int b_kmajor, int tile, int splits, int tag,
                       const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  return is_bf16 ? launch_type<bf16>(a_kmajor, b_kmajor, tile, splits, tag, p, s)
                 : launch_type<float>(a_kmajor, b_kmajor, tile, splits, tag, p, s);
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t split_stride, int M, int N,
                                float* C, int64_t ldc, float alpha, float beta, hipStream_t s) {
  const int64_t n = (int64_t)M * N;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     part, splits, split_stride, M, N, C, ldc, alpha, beta);
  return hipGetLastError();
}
