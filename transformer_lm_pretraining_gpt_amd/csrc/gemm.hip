// Tiled MFMA matrix product for gfx950, C = op(A) op(B) with fused epilogues.
//
// Every linear layer of the step is one of these products: the forward x W + b, the input
// gradient dY W^T and the weight gradient X^T dY ("Pré-treinar um LLM", paragraph deriving 6ND:
// forward and both backward products are matmuls of the forward's size). The tied LM head is the
// same kernel with the (Vp, d) embedding as the B operand.
//
// Two kernels share the block shape: 256 threads = 4 waves in a 2 x 2 arrangement, block tile
// BM x BN, wave tile BM/2 x BN/2 made of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16, or
// 4 x v_mfma_f32_32x32x2f32 for fp32), and the same fused epilogues.
//  * gemm_kernel (fp32, and bf16 when K is not a multiple of 64): 128-byte slabs loaded through
//    registers, transposed in registers where k is the strided dimension, written to one of two
//    XOR-swizzled LDS stages; one barrier per slab.
//  * gemm_dma_kernel (bf16, K a multiple of 64): persistent blocks, loads straight from memory
//    into three LDS stages, spread through the MFMAs, and an epilogue that overlaps the next
//    tile's first loads; details at its definition below.
// Both walk output tiles in groups of row-tiles column by column for L2 reuse, with each of the
// 8 XCDs (own L2 each) working on its own contiguous part of that order.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace {

constexpr int ROWB = 128;  // bytes of one k-slab row in LDS
constexpr int THREADS = 256;

// 16-byte chunk swizzle of a 128-byte LDS row: chosen by measurement (bank-conflict counter) to
// make the 32-row fragment reads of the MFMA loop conflict-free on gfx950
DEV int swz(int row) { return (row >> 1) & 7; }
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

// The same two functions for the bf16 direct-to-LDS epilogues, where they run on every element
// of a product with no MFMA work to hide them: with z = c (u + a u^3), (1 + tanh z) / 2 = s =
// 1 / (1 + e^(-2z)), so gelu(u) = u s and gelu'(u) = s + 2 u s (1 - s) c (1 + 3 a u^2); one
// v_exp_f32 and one v_rcp_f32 per element instead of tanhf (measured: the bias + GELU product
// 28 % faster, the GELU-backward one 16 %). Large |u| saturate to s = 0 or 1 (exp2 overflowing
// to +inf gives rcp = 0). Error: a few fp32 ulps of s (absolute ~1e-7 in s (1 - s)).
constexpr float GELU_E1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2c log2(e)
constexpr float GELU_E3 = GELU_E1 * 0.044715f;
DEV float gelu_sigmoid(float u, float u2) {  // s = 1 / (1 + 2^(-2z log2 e))
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(u * fmaf(GELU_E3, u2, GELU_E1)));
}
DEV float gelu_fast(float u) { return u * gelu_sigmoid(u, u * u); }
DEV float gelu_grad_fast(float u) {
  const float u2 = u * u;
  const float s = gelu_sigmoid(u, u2);
  constexpr float c2 = 2.0f * 0.7978845608028654f, c6 = c2 * 3.0f * 0.044715f;
  return fmaf(u * (s - s * s), fmaf(c6, u2, c2), s);
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
  if (p.alpha_scale) p.alpha *= *p.alpha_scale;
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

// ------------------------------------------------------------------------------------------
// bf16 product with direct global->LDS loads (buffer_load_dwordx4 ... lds), for K a multiple of 64.
//
// (Load primitives and tile layouts: lds_dma.h.)

// Epilogue through LDS, eight rows of the wave tile at a time: register group q (r = 4q..4q+3) of
// every 32x32 accumulator holds rows 8q + 4h + e (h = lane / 32); those rows go to the wave's
// LDS buffer in MFMA layout and come back in row layout, so that each lane applies the epilogue
// to 4 consecutive columns and writes them with one vector store. The pitch is 8 floats more
// than the row so that the two lane halves hit disjoint banks.
template <int NB>
constexpr int epi_pitch() { return NB * 32 + 8; }
template <int NB>
constexpr int epi_wave_bytes() { return 8 * epi_pitch<NB>() * 4; }

// bf16-output epilogue (plain store with alpha and bias, or bias + GELU with both outputs) for
// 64-column wave tiles. The arithmetic runs in the MFMA register layout (a lane's column is fixed
// within an accumulator tile, so its bias is one value), the results are converted to bf16 there
// and written as 16-bit values into the wave's 4 KB LDS buffer, 32 rows at a time; each lane then
// reads one 16-byte chunk of a row and stores it. Rows are 128 bytes with chunk c at
// c ^ 4((row/4) mod 2): the two lane halves write rows four apart into opposite halves of the row,
// and the 16-lane groups of the b128 reads cover all banks. With NT the stores are nontemporal:
// for an output far larger than the caches (the logits), written once and read by a later
// kernel, this keeps the operand panels of the following tiles in L2 (measured: 7% faster).
DEV int epi16_swz(int row) { return ((row >> 2) & 1) << 2; }
DEV int epi16_off(int row, int col) {  // byte offset of element (row, col) of a 32 x 64 tile
  return row * 128 + (((col >> 3) ^ epi16_swz(row)) << 4) + (col & 7) * 2;
}

template <int EPI, int MB, int NB, bool NT>
DEV void epilogue_bf16(const f32x16 (&acc)[MB][NB], const GemmParams& p, char* buf, int row0,
                       int col0, int lane) {
  static_assert(NB == 2, "64-column wave tiles");
  const int h = lane >> 5, l32 = lane & 31;
  float bias[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int col = col0 + j * 32 + l32;
    bias[j] = (p.bias && col < p.N) ? p.bias[col] : 0.0f;
  }
  constexpr int NOUT = EPI == EPI_BIAS_GELU ? 2 : 1;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int out = 0; out < NOUT; ++out) {
      // 32 rows x 64 columns of this output into LDS
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float x0, x1;
          if constexpr (EPI == EPI_STORE) {
            x0 = p.alpha * acc[i][j][r] + bias[j];
            x1 = p.alpha * acc[i][j][r + 1] + bias[j];
          } else {
            x0 = acc[i][j][r] + bias[j];
            x1 = acc[i][j][r + 1] + bias[j];
            if (out == 1) {
              x0 = gelu_fast(x0);
              x1 = gelu_fast(x1);
            }
          }
          const uint32_t pk = pack_bf16(x0, x1);
          const int rr = mfma_row(r, h), col = j * 32 + l32;  // rows rr and rr + 1
          *reinterpret_cast<uint16_t*>(buf + epi16_off(rr, col)) = (uint16_t)pk;
          *reinterpret_cast<uint16_t*>(buf + epi16_off(rr + 1, col)) = (uint16_t)(pk >> 16);
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      asm volatile("" ::: "memory");
      bf16* dst = static_cast<bf16*>(out == 0 ? p.C : p.C2);
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int rl = pass * 8 + lane / 8, pos = lane % 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(buf + rl * 128 + pos * 16);
        const int row = row0 + i * 32 + rl;
        const int col = col0 + ((pos ^ epi16_swz(rl)) << 3);
        if (row < p.M && col < p.N) {
          u32x4* q = reinterpret_cast<u32x4*>(dst + (int64_t)row * p.ldc + col);
          if constexpr (NT) __builtin_nontemporal_store(v, q);
          else *q = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
    }
  }
}

// bf16 store (alpha, bias) for 96-column wave tiles: as epilogue_bf16, in 16-row halves of each
// 32-row block (16 x 96 bf16 fit the wave's LDS block). Rows are 208 bytes apart (192 + 16), so
// the two lane halves, which write rows four apart, fall on disjoint banks; each lane then reads
// 16-byte row chunks (three passes over the 12 chunks of 16 rows) and stores them.
constexpr int EPI96_PITCH = 208;
template <int MB, int NB>
DEV void epilogue_bf16_96(const f32x16 (&acc)[MB][NB], const GemmParams& p, char* buf, int row0,
                          int col0, int lane) {
  static_assert(NB == 3, "96-column wave tiles");
  static_assert(16 * EPI96_PITCH <= 4096, "the wave's LDS block");
  const int h = lane >> 5, l32 = lane & 31;
  float bias[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int col = col0 + j * 32 + l32;
    bias[j] = (p.bias && col < p.N) ? p.bias[col] : 0.0f;
  }
  bf16* dst = static_cast<bf16*>(p.C);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 8 * half; r < 8 * half + 8; r += 2) {
          const float x0 = p.alpha * acc[i][j][r] + bias[j];
          const float x1 = p.alpha * acc[i][j][r + 1] + bias[j];
          const uint32_t pk = pack_bf16(x0, x1);
          const int rr = mfma_row(r, h) - 16 * half, col = j * 32 + l32;  // rows rr and rr + 1
          *reinterpret_cast<uint16_t*>(buf + rr * EPI96_PITCH + col * 2) = (uint16_t)pk;
          *reinterpret_cast<uint16_t*>(buf + (rr + 1) * EPI96_PITCH + col * 2) = (uint16_t)(pk >> 16);
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        const int idx = pass * 64 + lane;
        const int rl = idx / 12, ch = idx % 12;
        const u32x4 v = *reinterpret_cast<const u32x4*>(buf + rl * EPI96_PITCH + ch * 16);
        const int row = row0 + i * 32 + 16 * half + rl, col = col0 + ch * 8;
        if (row < p.M && col < p.N) *reinterpret_cast<u32x4*>(dst + (int64_t)row * p.ldc + col) = v;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
    }
  }
}

// Bias + residual, fp32 out, for 96-column wave tiles: 8 rows at a time go through the wave's
// fp32 LDS block and come back as 8 x 24 float4, three full passes of the 64 lanes. The residual
// float4s of the 8 rows are requested before the block's stores (one memory round trip per 8
// rows, not one per pass) and each lane's three bias float4s are read once.
template <int MB, int NB>
DEV void epilogue_resid_96(const f32x16 (&acc)[MB][NB], const GemmParams& p, float* buf,
                           int row0, int col0, int lane) {
  static_assert(NB == 3, "96-column wave tiles");
  constexpr int PITCH = epi_pitch<NB>();
  const int h = lane >> 5, l32 = lane & 31;
  float* cf = static_cast<float*>(p.C);
  int rl[3], c4[3];
  f32x4 bias[3];
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int idx = pass * 64 + lane;
    rl[pass] = idx / 24;
    c4[pass] = idx % 24;
    const int col = col0 + 4 * c4[pass];
    bias[pass] = (p.bias && col < p.N) ? *reinterpret_cast<const f32x4*>(p.bias + col)
                                       : f32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 rs[3];
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        const int row = row0 + i * 32 + 8 * q + rl[pass], col = col0 + 4 * c4[pass];
        rs[pass] = (row < p.M && col < p.N)
                       ? *reinterpret_cast<const f32x4*>(p.resid + (int64_t)row * p.ldc + col)
                       : f32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) buf[(4 * h + e) * PITCH + j * 32 + l32] = acc[i][j][4 * q + e];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(buf + rl[pass] * PITCH + 4 * c4[pass]);
        const int row = row0 + i * 32 + 8 * q + rl[pass], col = col0 + 4 * c4[pass];
        if (row < p.M && col < p.N)
          *reinterpret_cast<f32x4*>(cf + (int64_t)row * p.ldc + col) = rs[pass] + v + bias[pass];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
    }
  }
}

// GELU-backward epilogue for 64-column wave tiles: out = acc * GELU'(u), bf16, with u the saved
// pre-activation (bf16, laid out like the output). Each 32-row block goes through the wave's LDS
// block: the lanes load u one 16-byte row chunk each, the arithmetic runs in the MFMA register
// layout on u read back from LDS, the bf16 results overwrite u in place and leave as 16-byte row
// chunks. The column sums of the rounded results (the fc-bias gradient, summed from the same
// bf16 values the weight-gradient products read) are taken from those row chunks: one partial
// row per wave tile.
template <int MB, int NB>
DEV void epilogue_gelu_bwd_bf16(const f32x16 (&acc)[MB][NB], const GemmParams& p, char* buf,
                                int row0, int col0, int lane) {
  static_assert(NB == 2, "64-column wave tiles");
  const int h = lane >> 5, l32 = lane & 31;
  const int rq = lane / 8, pos = lane % 8;  // row (within 8) and 16-byte chunk of the row passes
  // the rows of a lane's passes share one swizzle, so its chunk holds the same 8 columns in each
  const int chunk = pos ^ epi16_swz(rq);
  const int col8 = col0 + chunk * 8;
  const bf16* aux = static_cast<const bf16*>(p.aux);
  bf16* dst = static_cast<bf16*>(p.C);
  float cs[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    u32x4 un[4];
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int row = row0 + i * 32 + pass * 8 + rq, col = col0 + pos * 8;
      un[pass] = (row < p.M && col < p.N) ? ld16(aux + (int64_t)row * p.ldc + col)
                                          : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass)
      *reinterpret_cast<u32x4*>(buf + epi16_off(pass * 8 + rq, pos * 8)) = un[pass];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this block's u is in LDS
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int rr = mfma_row(r, h), col = j * 32 + l32;  // rows rr and rr + 1
        uint16_t* a = reinterpret_cast<uint16_t*>(buf + epi16_off(rr, col));
        uint16_t* b = reinterpret_cast<uint16_t*>(buf + epi16_off(rr + 1, col));
        const float x0 = acc[i][j][r] * gelu_grad_fast(bf16lo(*a));
        const float x1 = acc[i][j][r + 1] * gelu_grad_fast(bf16lo(*b));
        const uint32_t pk = pack_bf16(x0, x1);
        *a = (uint16_t)pk;
        *b = (uint16_t)(pk >> 16);
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int rl = pass * 8 + rq;
      const u32x4 v = *reinterpret_cast<const u32x4*>(buf + rl * 128 + pos * 16);
      const int row = row0 + i * 32 + rl;
      if (row < p.M && col8 < p.N) {
        *reinterpret_cast<u32x4*>(dst + (int64_t)row * p.ldc + col8) = v;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          cs[2 * w] += bf16lo(v[w]);
          cs[2 * w + 1] += bf16hi(v[w]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
  }
  if (p.colsum) {
    // lanes holding the same chunk: rq 0..3 at pos = chunk, rq 4..7 at pos = chunk ^ 4; add them
    // in a fixed order, then lanes 0..7 write the wave's partial row
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cs[e] += __shfl_xor(cs[e], 8, 64);
      cs[e] += __shfl_xor(cs[e], 16, 64);
      cs[e] += __shfl_xor(cs[e], 36, 64);
    }
    if (rq == 0 && col8 < p.N) {
      float* prow = p.colsum + (int64_t)(row0 / (MB * 32)) * p.N + col8;
      *reinterpret_cast<f32x4*>(prow) = f32x4{cs[0], cs[1], cs[2], cs[3]};
      *reinterpret_cast<f32x4*>(prow + 4) = f32x4{cs[4], cs[5], cs[6], cs[7]};
    }
  }
}

template <int EPI, int MB, int NB>
DEV void epilogue_rows(const f32x16 (&acc)[MB][NB], const GemmParams& p, float* buf, int row0,
                       int col0, int lane, int z) {
  constexpr int WN = NB * 32;
  constexpr int PITCH = epi_pitch<NB>();
  constexpr int V4 = WN / 4;     // float4 per row
  constexpr int RPP = 64 / V4;   // rows per pass (lanes from RPP * V4 on idle when V4 is 24)
  static_assert(8 % RPP == 0, "whole passes over the 8 rows");
  const int h = lane >> 5, l32 = lane & 31;
  float* cf = static_cast<float*>(p.C);
  if (EPI == EPI_F32) cf += (int64_t)z * p.c_split_stride;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) buf[(4 * h + e) * PITCH + j * 32 + l32] = acc[i][j][4 * q + e];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pass = 0; pass < 8 / RPP; ++pass) {
        if (RPP * V4 < 64 && lane >= RPP * V4) continue;
        const int rl = pass * RPP + lane / V4;
        const int c4 = lane % V4;
        const int row = row0 + i * 32 + 8 * q + rl;
        const int col = col0 + c4 * 4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(buf + rl * PITCH + c4 * 4);
        if (row < p.M && col < p.N) {
          const int64_t o = (int64_t)row * p.ldc + col;
          f32x4 bias = p.bias ? *reinterpret_cast<const f32x4*>(p.bias + col) : f32x4{0, 0, 0, 0};
          float out[4];
          if constexpr (EPI == EPI_STORE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = p.alpha * v[e] + bias[e];
            st8(static_cast<bf16*>(p.C) + o, u32x2{pack_bf16(out[0], out[1]), pack_bf16(out[2], out[3])});
          } else if constexpr (EPI == EPI_BIAS_GELU) {
            float gl[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              out[e] = v[e] + bias[e];
              gl[e] = gelu_fast(out[e]);
            }
            st8(static_cast<bf16*>(p.C) + o, u32x2{pack_bf16(out[0], out[1]), pack_bf16(out[2], out[3])});
            st8(static_cast<bf16*>(p.C2) + o, u32x2{pack_bf16(gl[0], gl[1]), pack_bf16(gl[2], gl[3])});
          } else if constexpr (EPI == EPI_BIAS_RESID) {
            const f32x4 rs = *reinterpret_cast<const f32x4*>(p.resid + o);
            *reinterpret_cast<f32x4*>(cf + o) = rs + v + bias;
          } else if constexpr (EPI == EPI_GELU_BWD) {
            const u32x2 u = ld8(static_cast<const bf16*>(p.aux) + o);
            const float uf[4] = {bf16lo(u[0]), bf16hi(u[0]), bf16lo(u[1]), bf16hi(u[1])};
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = v[e] * gelu_grad_fast(uf[e]);
            st8(static_cast<bf16*>(p.C) + o, u32x2{pack_bf16(out[0], out[1]), pack_bf16(out[2], out[3])});
          } else {
            f32x4 prev = f32x4{0, 0, 0, 0};
            if (p.beta != 0.0f) prev = p.beta * *reinterpret_cast<const f32x4*>(cf + o);
            *reinterpret_cast<f32x4*>(cf + o) = p.alpha * v + prev;
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
    }
  }
}

// MFMAs of one slab (KSTEPS k-steps of 16) on the stage (sa, sb). Fragments of k-step s+1 are
// read during k-step s; with ISSUE, the loads of a later slab into (dst_a, dst_b) are spread over
// the k-steps, PER_WAVE / KSTEPS per operand each.
template <bool ISSUE, class TA, class TB, int MB, int NB, int KSTEPS>
DEV void slab_mma(f32x16 (&acc)[MB][NB], const char* sa, const char* sb, int wm0, int wn0,
                  int lane, int wave, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                  const uint32_t (&offa)[TA::PER_WAVE], const uint32_t (&offb)[TB::PER_WAVE],
                  char* dst_a, char* dst_b) {
  constexpr int LA = TA::PER_WAVE / KSTEPS, LB = TB::PER_WAVE / KSTEPS;
  static_assert(LA * KSTEPS == TA::PER_WAVE && LB * KSTEPS == TB::PER_WAVE, "even load split");
  constexpr int NM = MB * NB;
  constexpr int ND = MB * TA::DS_PER_FRAG + NB * TB::DS_PER_FRAG;
  constexpr int NV = ISSUE ? LA + LB : 0;
  u32x4 fa[2][MB], fb[2][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i) fa[0][i] = TA::frag(sa, wm0 + i * 32, 0, lane);
#pragma unroll
  for (int j = 0; j < NB; ++j) fb[0][j] = TB::frag(sb, wn0 + j * 32, 0, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int cur = s & 1;
    if (s < KSTEPS - 1) {
#pragma unroll
      for (int i = 0; i < MB; ++i) fa[cur ^ 1][i] = TA::frag(sa, wm0 + i * 32, s + 1, lane);
#pragma unroll
      for (int j = 0; j < NB; ++j) fb[cur ^ 1][j] = TB::frag(sb, wn0 + j * 32, s + 1, lane);
    }
    if constexpr (ISSUE) {
#pragma unroll
      for (int t = 0; t < LA; ++t) TA::issue(ra, offa, s * LA + t, dst_a, wave);
#pragma unroll
      for (int t = 0; t < LB; ++t) TB::issue(rb, offb, s * LB + t, dst_b, wave);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) Mfma<bf16>::mma(acc[i][j], fa[cur][i], fb[cur][j]);
    if (s < KSTEPS - 1) interleave<NM, ND, NV>();
    else interleave<NM, 0, NV>();
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Fragments of k-step s of the stage (sa, sb) for this wave's tile.
template <class TA, class TB, int MB, int NB>
DEV void read_frags(u32x4 (&fa)[MB], u32x4 (&fb)[NB], const char* sa, const char* sb, int wm0,
                    int wn0, int s, int lane) {
#pragma unroll
  for (int i = 0; i < MB; ++i) fa[i] = TA::frag(sa, wm0 + i * 32, s, lane);
#pragma unroll
  for (int j = 0; j < NB; ++j) fb[j] = TB::frag(sb, wn0 + j * 32, s, lane);
}

// MFMAs of one slab with the fragments of its first k-step in (fa, fb) on entry. With NEXT the
// next slab's wait and barrier sit inside the last k-step, after half of its MFMAs have been
// issued, and the next slab's first fragments (returned in fa, fb) are read under the other half,
// so no k-step waits for a fragment read right after a barrier. With ISSUE all loads of a later
// slab go out during the first k-step (the wait for the next slab counts them as issued).
template <bool ISSUE, bool NEXT, class TA, class TB, int MB, int NB, int KSTEPS, int LW, int NWAIT>
DEV void slab_mma_next(f32x16 (&acc)[MB][NB], u32x4 (&fa)[MB], u32x4 (&fb)[NB], const char* sa,
                const char* sb, const char* na, const char* nb, int wait_after, int wm0, int wn0,
                int lane, int wave, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                const uint32_t (&offa)[TA::PER_WAVE], const uint32_t (&offb)[TB::PER_WAVE],
                char* dst_a, char* dst_b) {
  static_assert(KSTEPS == 2, "two k-steps per slab");
  constexpr int NM = MB * NB;
  constexpr int ND = MB * TA::DS_PER_FRAG + NB * TB::DS_PER_FRAG;
  constexpr int NV = ISSUE ? TA::PER_WAVE + TB::PER_WAVE : 0;
  static_assert(MB % 2 == 0, "split of the last k-step");
  constexpr int NPRE = MB / 2;  // MFMA rows of the last k-step issued before the barrier
  {
    u32x4 ga[MB], gb[NB];
    read_frags<TA, TB, MB, NB>(ga, gb, sa, sb, wm0, wn0, 1, lane);
    if constexpr (ISSUE) {
#pragma unroll
      for (int t = 0; t < TA::PER_WAVE; ++t) TA::issue(ra, offa, t, dst_a, wave);
#pragma unroll
      for (int t = 0; t < TB::PER_WAVE; ++t) TB::issue(rb, offb, t, dst_b, wave);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) Mfma<bf16>::mma(acc[i][j], fa[i], fb[j]);
    interleave<NM, ND, NV>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[i] = ga[i];
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[j] = gb[j];
  }
  if constexpr (NEXT) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) Mfma<bf16>::mma(acc[i][j], fa[i], fb[j]);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's reads of the current stage are done (a later slab's loads may overwrite it
    // once every wave is past the barrier) and the next slab has landed
    wait_slabs_lgkm0<LW, NWAIT>(wait_after);
    wave_barrier_all();
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ga[MB], gb[NB];
    read_frags<TA, TB, MB, NB>(ga, gb, na, nb, wm0, wn0, 0, lane);
#pragma unroll
    for (int i = NPRE; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) Mfma<bf16>::mma(acc[i][j], fa[i], fb[j]);
    interleave<(MB - NPRE) * NB, ND, 0>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[i] = ga[i];
#pragma unroll
    for (int j = 0; j < NB; ++j) fb[j] = gb[j];
  } else {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) Mfma<bf16>::mma(acc[i][j], fa[i], fb[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Persistent tiles: the grid holds at most as many blocks as fit on the chip at once, and each
// block walks a strided sequence of output tiles (see the XCD partition below). Slabs go to stage
// (slab count so far) mod NSTAGE across tiles, so when a tile's k loop ends the stage of its last
// slab is free while the next tile's first NSTAGE-1 slabs go to the others: those loads are issued
// first and stream in while the finished tile is written out through the free stage.
template <int AK, int BKM, int BM, int BN, int RB, int NSTAGE, int MINB, int TAG, int NW = 4>
__global__ __launch_bounds__(64 * NW, MINB) void gemm_dma_kernel(GemmParams p) {
  // a device-side scale of alpha, read before any of the pipeline's loads is in flight
  if (p.alpha_scale)
    p.alpha *= __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, *p.alpha_scale)));
  // NW waves in a 2 x NW/2 grid over the block tile
  constexpr int WGN = NW / 2;
  constexpr int WM = BM / 2, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int KT = RB / 2;
  constexpr int KSTEPS = RB / 32;
  constexpr int STAGE = (BM + BN) * RB;
  using TA = DmaTile<BM, AK == 1, RB, NW>;
  using TB = DmaTile<BN, BKM == 1, RB, NW>;
  constexpr int LW = TA::PER_WAVE + TB::PER_WAVE;  // loads per wave per slab
  static_assert(NW * epi_wave_bytes<NB>() <= STAGE, "epilogue buffer must fit one stage");
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to M0

  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int nblk = tiles_m * tiles_n;
  // Work items are (K split, output tile) pairs, split-major: item = z * nblk + tile. Block b runs
  // on XCD b mod 8; when the grid is a multiple of 8, XCD x owns the contiguous run of items
  // [x * per_xcd, (x + 1) * per_xcd) and its G/8 blocks stride through it, so the blocks that
  // run together on one XCD share the K range of a split and the operand panels of neighbouring
  // tiles, and each XCD's L2 serves those panels to all of them.
  const int nitems = nblk * p.splits;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  int w, w_end, stride;
  if ((G & 7) == 0) {
    const int per_xcd = (nitems + 7) >> 3;
    w = (b & 7) * per_xcd + (b >> 3);
    w_end = min(nitems, ((b & 7) + 1) * per_xcd);
    stride = G >> 3;
  } else {
    w = b;
    w_end = nitems;
    stride = G;
  }
  if (w >= w_end) return;
  // Tile order within a split: GROUP row-tiles walked column by column; for weight gradients
  // (both operands read k-row by k-row) with few column tiles, column tiles fastest instead, so
  // the tiles that share a row panel of A (the largest operand there, e.g. the LM head's logit
  // gradient) run side by side and read it once through L2.
  const bool n_fast = AK == 0 && tiles_n <= 8;
  const int GROUP = tiles_m <= 8 ? tiles_m : (tiles_m + 7) / 8;
  const int in_group = GROUP * tiles_n;

  const bf16* A = static_cast<const bf16*>(p.A);
  const bf16* B = static_cast<const bf16*>(p.B);
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;

  // output tile, first k and slab count of work item `item`, and its split z
  auto item_of = [&](int item, int& m0, int& n0, int& kb, int& nk, int& z) {
    z = item / nblk;
    const int t = item - z * nblk;
    if (n_fast) {
      m0 = (t / tiles_n) * BM;
      n0 = (t % tiles_n) * BN;
    } else {
      const int g = t / in_group;
      const int first_m = g * GROUP;
      const int gsize = min(tiles_m - first_m, GROUP);
      m0 = (first_m + (t % in_group) % gsize) * BM;
      n0 = ((t % in_group) / gsize) * BN;
    }
    kb = z * p.k_split;
    nk = (min(p.K, kb + p.k_split) - kb) / KT;
  };
  uint32_t offa[TA::PER_WAVE], offb[TB::PER_WAVE];  // this wave's load offsets for the tile
  // whole slab `ks` of the item at (m0, n0) with first k kb into stage `st`
  auto issue = [&](int m0, int n0, int kb, int ks, int st) {
    char* dst = smem + st * STAGE;
    const __amdgpu_buffer_rsrc_t ra = TA::slab(A, p.lda, m0, kb + ks * KT);
    const __amdgpu_buffer_rsrc_t rb = TB::slab(B, p.ldb, n0, kb + ks * KT);
#pragma unroll
    for (int i = 0; i < TA::PER_WAVE; ++i) TA::issue(ra, offa, i, dst, wave);
#pragma unroll
    for (int i = 0; i < TB::PER_WAVE; ++i) TB::issue(rb, offb, i, dst + BM * RB, wave);
  };

  int m0, n0, kb, nk, z;
  item_of(w, m0, n0, kb, nk, z);
  TA::offsets(offa, p.lda, m0, p.M, wave, lane);
  TB::offsets(offb, p.ldb, n0, p.N, wave, lane);
  int base = 0;  // stage of this tile's slab 0
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < nk) issue(m0, n0, kb, s, s);

  while (true) {
    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

    // slabs of this tile issued after slab kt: min(NSTAGE - 2, nk - 1 - kt); loads complete in
    // issue order, so waiting until at most that many slabs' loads are pending (stores of the
    // previous tile's epilogue only add to the count) means slab kt has landed. Slabs that still
    // have a later slab to load (kt < nk - NSTAGE + 1) spread its loads over their MFMAs; the last
    // NSTAGE - 1 slabs run in a loop of their own with no loads, so each loop has one body.
    const int nmain = max(nk - (NSTAGE - 1), 0);
    if constexpr (AK == 1) {
      // the next slab's wait and barrier inside each slab's last k-step (slab_mma_next)
      u32x4 fa[MB], fb[NB];
      {
        wait_slabs_lgkm0<LW, NSTAGE - 2>(min(NSTAGE - 2, nk - 1));
        wave_barrier_all();
        const char* s0 = smem + base * STAGE;
        read_frags<TA, TB, MB, NB>(fa, fb, s0, s0 + BM * RB, wm0, wn0, 0, lane);
      }
      for (int kt = 0; kt < nmain; ++kt) {
        const char* sa = smem + ((base + kt) % NSTAGE) * STAGE;
        const char* na = smem + ((base + kt + 1) % NSTAGE) * STAGE;
        const int nxt = kt + NSTAGE - 1;
        char* dst = smem + ((base + nxt) % NSTAGE) * STAGE;
        slab_mma_next<true, true, TA, TB, MB, NB, KSTEPS, LW, NSTAGE - 2>(
            acc, fa, fb, sa, sa + BM * RB, na, na + BM * RB, NSTAGE - 2, wm0, wn0, lane, wave,
            TA::slab(A, p.lda, m0, kb + nxt * KT), TB::slab(B, p.ldb, n0, kb + nxt * KT),
            offa, offb, dst, dst + BM * RB);
      }
      const __amdgpu_buffer_rsrc_t unused = buffer_at(A);  // no loads left for this tile
      for (int kt = nmain; kt < nk - 1; ++kt) {
        const char* sa = smem + ((base + kt) % NSTAGE) * STAGE;
        const char* na = smem + ((base + kt + 1) % NSTAGE) * STAGE;
        slab_mma_next<false, true, TA, TB, MB, NB, KSTEPS, LW, NSTAGE - 2>(
            acc, fa, fb, sa, sa + BM * RB, na, na + BM * RB, nk - 2 - kt, wm0, wn0, lane, wave,
            unused, unused, offa, offb, nullptr, nullptr);
      }
      if (nk > 0) {
        const char* sa = smem + ((base + nk - 1) % NSTAGE) * STAGE;
        slab_mma_next<false, false, TA, TB, MB, NB, KSTEPS, LW, NSTAGE - 2>(
            acc, fa, fb, sa, sa + BM * RB, sa, sa + BM * RB, 0, wm0, wn0, lane, wave, unused,
            unused, offa, offb, nullptr, nullptr);
      }
    } else {
      for (int kt = 0; kt < nmain; ++kt) {
        wait_slabs<LW, NSTAGE - 2>(NSTAGE - 2);
        wave_barrier_all();
        const char* sa = smem + ((base + kt) % NSTAGE) * STAGE;
        const int nxt = kt + NSTAGE - 1;
        char* dst = smem + ((base + nxt) % NSTAGE) * STAGE;
        slab_mma<true, TA, TB, MB, NB, KSTEPS>(
            acc, sa, sa + BM * RB, wm0, wn0, lane, wave, TA::slab(A, p.lda, m0, kb + nxt * KT),
            TB::slab(B, p.ldb, n0, kb + nxt * KT), offa, offb, dst, dst + BM * RB);
      }
      for (int kt = nmain; kt < nk; ++kt) {
        wait_slabs<LW, NSTAGE - 2>(nk - 1 - kt);
        wave_barrier_all();
        const char* sa = smem + ((base + kt) % NSTAGE) * STAGE;
        const __amdgpu_buffer_rsrc_t unused = buffer_at(A);  // no loads left for this tile
        slab_mma<false, TA, TB, MB, NB, KSTEPS>(acc, sa, sa + BM * RB, wm0, wn0, lane, wave, unused,
                                                unused, offa, offb, nullptr, nullptr);
      }
    }

    // every wave is done reading this tile's stages; the last one becomes the epilogue buffer
    wave_barrier_all();
    const int last = (base + nk + NSTAGE - 1) % NSTAGE;
    const int nbase = (base + nk) % NSTAGE;
    const int wnext = w + stride;
    int m1 = 0, n1 = 0, kb1 = 0, nk1 = 0, z1 = 0;
    if (wnext < w_end) {
      item_of(wnext, m1, n1, kb1, nk1, z1);
      TA::offsets(offa, p.lda, m1, p.M, wave, lane);
      TB::offsets(offb, p.ldb, n1, p.N, wave, lane);
#pragma unroll
      for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nk1) issue(m1, n1, kb1, s, (nbase + s) % NSTAGE);
    }
    float* buf = reinterpret_cast<float*>(smem + last * STAGE + wave * epi_wave_bytes<NB>());
    const int row0 = m0 + wm0, col0 = n0 + wn0;
    char* buf16 = smem + last * STAGE + wave * 4096;
    static_assert(NW * 4096 <= STAGE, "bf16 epilogue buffers must fit one stage");
    switch (p.epi) {
      case EPI_STORE:
        if constexpr (NB == 2) epilogue_bf16<EPI_STORE, MB, NB, TAG == 1>(acc, p, buf16, row0, col0, lane);
        else if constexpr (NB == 3) epilogue_bf16_96<MB, NB>(acc, p, buf16, row0, col0, lane);
        else epilogue_rows<EPI_STORE, MB, NB>(acc, p, buf, row0, col0, lane, z);
        break;
      case EPI_BIAS_GELU:
        if constexpr (NB == 2) epilogue_bf16<EPI_BIAS_GELU, MB, NB, false>(acc, p, buf16, row0, col0, lane);
        else epilogue_rows<EPI_BIAS_GELU, MB, NB>(acc, p, buf, row0, col0, lane, z);
        break;
      case EPI_BIAS_RESID:
        if constexpr (NB == 3) epilogue_resid_96<MB, NB>(acc, p, buf, row0, col0, lane);
        else epilogue_rows<EPI_BIAS_RESID, MB, NB>(acc, p, buf, row0, col0, lane, z);
        break;
      case EPI_GELU_BWD:
        if constexpr (NB == 2) epilogue_gelu_bwd_bf16<MB, NB>(acc, p, buf16, row0, col0, lane);
        else epilogue_rows<EPI_GELU_BWD, MB, NB>(acc, p, buf, row0, col0, lane, z);
        break;
      default: epilogue_rows<EPI_F32, MB, NB>(acc, p, buf, row0, col0, lane, z); break;
    }
    if (wnext >= w_end) break;
    w = wnext;
    m0 = m1;
    n0 = n1;
    kb = kb1;
    nk = nk1;
    z = z1;
    base = nbase;
  }
}

// C = alpha * (sum of the K-split partials, in split order) + beta * C. The order is fixed, so the
// result does not depend on scheduling.
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

// The same with four columns per thread (N, ldc and stride multiples of 4, 16-byte aligned).
__global__ void splitk_reduce4_kernel(const float* __restrict__ part, int splits, int64_t stride,
                                      int M, int N, float* __restrict__ C, int64_t ldc,
                                      float alpha, float beta) {
  const int nv = N / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * nv) return;
  const int row = (int)(idx / nv), c4 = (int)(idx % nv);
  const int64_t src = (int64_t)row * ldc + 4 * c4;
  f32x4 s = f32x4{0, 0, 0, 0};
  int z = 0;
  for (; z + 4 <= splits; z += 4) {  // four loads in flight, still added in split order
    const f32x4 a = *reinterpret_cast<const f32x4*>(part + (int64_t)z * stride + src);
    const f32x4 b = *reinterpret_cast<const f32x4*>(part + (int64_t)(z + 1) * stride + src);
    const f32x4 c = *reinterpret_cast<const f32x4*>(part + (int64_t)(z + 2) * stride + src);
    const f32x4 d = *reinterpret_cast<const f32x4*>(part + (int64_t)(z + 3) * stride + src);
    s = (((s + a) + b) + c) + d;
  }
  for (; z < splits; ++z) s += *reinterpret_cast<const f32x4*>(part + (int64_t)z * stride + src);
  f32x4* out = reinterpret_cast<f32x4*>(C + src);
  const f32x4 prev = beta != 0.0f ? beta * *out : f32x4{0, 0, 0, 0};
  *out = alpha * s + prev;
}

// Split-K partials (dense (M, N) per split) summed in split order, scaled by alpha times
// *alpha_scale (when given) and rounded to bf16 into C; four columns per thread.
__global__ void splitk_reduce_bf16_kernel(const float* __restrict__ part, int splits,
                                          int64_t stride, int M, int N, bf16* __restrict__ C,
                                          int64_t ldc, float alpha,
                                          const float* __restrict__ alpha_scale) {
  const int nv = N / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * nv) return;
  const int row = (int)(idx / nv), c4 = (int)(idx % nv);
  const int64_t src = (int64_t)row * N + 4 * c4;
  f32x4 s = f32x4{0, 0, 0, 0};
  int z = 0;
  for (; z + 4 <= splits; z += 4) {  // four loads in flight, still added in split order
    const f32x4 a = *reinterpret_cast<const f32x4*>(part + (int64_t)z * stride + src);
    const f32x4 b = *reinterpret_cast<const f32x4*>(part + (int64_t)(z + 1) * stride + src);
    const f32x4 c = *reinterpret_cast<const f32x4*>(part + (int64_t)(z + 2) * stride + src);
    const f32x4 d = *reinterpret_cast<const f32x4*>(part + (int64_t)(z + 3) * stride + src);
    s = (((s + a) + b) + c) + d;
  }
  for (; z < splits; ++z) s += *reinterpret_cast<const f32x4*>(part + (int64_t)z * stride + src);
  const float a = alpha_scale ? alpha * *alpha_scale : alpha;
  const f32x4 v = a * s;
  st8(C + (int64_t)row * ldc + 4 * c4, u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])});
}

// Blocks of `kernel` (nt threads each) resident at once on the current device.
template <typename K>
int resident_blocks(K kernel, int nt) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, 0) != hipSuccess)
    return 256;
  return std::max(1, cus * std::max(per_cu, 1));
}

// One block per resident slot at most, over the tiles x splits work items; rounded up to a multiple
// of 8 blocks (blocks past the items exit at once) so that every XCD gets its own run of items.
template <void (*KERNEL)(GemmParams), int NT = THREADS>
hipError_t launch_persistent(int tiles, int splits, const GemmParams& p, hipStream_t s) {
  static const int resident = resident_blocks(KERNEL, NT);  // one value per kernel
  const int items = tiles * splits;
  int g = std::min(items, resident);
  if (g > 8 && resident % 8 == 0) g = std::min(resident, (g + 7) / 8 * 8);
  GemmParams q = p;
  q.splits = splits;
  hipLaunchKernelGGL(KERNEL, dim3(g), dim3(NT), 0, s, q);
  return hipGetLastError();
}

// Tile configurations of the direct-to-LDS kernel, all with 64-byte slabs (32 k) and three
// stages: 256x256 with 8 waves (wave tiles 128 x 64, two waves per SIMD, 96 KB LDS, one block per
// CU), 128x384 with 8 waves (wave tiles 64 x 96), 256x128 with 4 waves (wave tiles 128 x 64,
// 72 KB, two blocks per CU) and 128x128 with 4 waves (48 KB, up to three blocks per CU). Two waves
// per SIMD let one wave's barriers and epilogue overlap the other's MFMAs; the large tile issues
// the fewest loads per MFMA. Chosen by measurement over the GPT-2 shapes against deeper or
// shallower pipelines and 128-byte slabs in two stages; 256x128 and 128x256 tiles lose to the
// 8-wave tiles wherever those fill the chip, and beat 128x128 on the input-gradient products
// that the 8-wave tiles do not fill. Tag 1 (the LM-head
// forward, an instantiation of its own so that timings and profiles can single it out) writes
// its output with nontemporal stores.
template <int AK, int BKM, int BM, int BN>
hipError_t launch_dma(int splits, int tag, const GemmParams& p, hipStream_t s) {
  constexpr int RB = 64;
  constexpr int STAGE = (BM + BN) * RB;
  constexpr int NSTAGE = 3;
  constexpr int NW = BM + BN >= 512 ? 8 : 4;
  constexpr int MINB = NW == 8 ? 1 : 2;
  static_assert(NSTAGE * STAGE * MINB <= 160 * 1024, "LDS");
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if constexpr (AK == 1 && BKM == 1 && BM == 256) {
    if (tag == 1)
      return launch_persistent<gemm_dma_kernel<AK, BKM, BM, BN, RB, NSTAGE, MINB, 1, NW>, 64 * NW>(
          tiles, splits, p, s);
  }
  return launch_persistent<gemm_dma_kernel<AK, BKM, BM, BN, RB, NSTAGE, MINB, 0, NW>, 64 * NW>(
      tiles, splits, p, s);
}

template <typename T, int AK, int BKM, int BM, int BN>
hipError_t launch_t(int splits, int tag, const GemmParams& p, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // direct-to-LDS pipeline when every slab is a whole 64-wide k-slab, rows fit the tiles and
    // 256 rows of either operand span less than 2 GiB (32-bit buffer offsets within a slab)
    if (p.K % 64 == 0 && (splits == 1 || p.k_split % 64 == 0) && p.M >= (AK ? 1 : 8) &&
        p.N >= (BKM ? 1 : 8) && p.lda < (1 << 22) && p.ldb < (1 << 22))
      return launch_dma<AK, BKM, BM, BN>(splits, tag, p, s);
  }
  if constexpr (BM != 128 || BN != 128) {
    // the register-staged kernel runs 128x128 tiles only
    return launch_t<T, AK, BKM, 128, 128>(splits, tag, p, s);
  } else {
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    dim3 grid(tiles, 1, splits), block(THREADS);
    hipLaunchKernelGGL((gemm_kernel<T, AK, BKM, BM, BN, 0>), grid, block, 0, s, p);
    return hipGetLastError();
  }
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
      case TILE_128x384:
        // k-major A only (its loads all go out in the first k-step), and not with the column sums
        // of the GELU-backward epilogue
        if (a_kmajor && !p.colsum) {
          if (b_kmajor) return launch_t<T, 1, 1, 128, 384>(splits, tag, p, s);
          return launch_t<T, 1, 0, 128, 384>(splits, tag, p, s);
        }
        return launch_layout<T, 256, 256>(a_kmajor, b_kmajor, splits, tag, p, s);
      case TILE_256: return launch_layout<T, 256, 256>(a_kmajor, b_kmajor, splits, tag, p, s);
      case TILE_256x128: return launch_layout<T, 256, 128>(a_kmajor, b_kmajor, splits, tag, p, s);
      default: return launch_layout<T, 128, 128>(a_kmajor, b_kmajor, splits, tag, p, s);
    }
  }
}

}  // namespace

int gemm_k_tile(bool is_bf16) { return is_bf16 ? ROWB / 2 : ROWB / 4; }

int gemm_pick_tile(int M, int N) {
  const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  // Both large tiles run one 8-wave block per CU, a round of tiles per 256 CUs. Where N is a
  // multiple of 384, or 256 x 256 tiles fill the chip anyway, the 128 x 384 tile (3/4 of the work
  // of a 256 x 256 one; a partly filled last column of tiles counted whole) is taken when its
  // rounds cost at least 10 % less: a partly filled last round of 256 x 256 tiles leaves CUs idle
  // (an output of 192 tiles, the QKV product's 2.25 rounds at GPT-2 124M, or 1.19 rounds at 1.5B,
  // N = 4800, where 128 x 384 tiles were 10 % faster).
  if (N % 384 == 0 || t256 >= 192) {
    const int64_t t384 = (int64_t)((M + 127) / 128) * ((N + 383) / 384);
    const int64_t c256 = 4 * ((t256 + 255) / 256), c384 = 3 * ((t384 + 255) / 256);
    if (c384 < c256 && 10 * (c256 - c384) >= c256) return TILE_128x384;
  }
  return t256 >= 192 ? TILE_256 : TILE_128;
}

int gemm_pick_tile_epi(int M, int N, int a_kmajor, int b_kmajor, int epi, bool colsum) {
  const int t = gemm_pick_tile(M, N);
  // Products with both operands k-major and a plain bf16 output (the input gradients) whose
  // 256x256 tiles would not fill the chip take 256x128 tiles at two blocks per CU instead of
  // 128x128 ones: at GPT-2 350M and 1.5B (N = 1024 and 1600) 6-14 % faster standalone. The
  // forward products of those shapes (fp32 residual epilogue, weights read transposed) are
  // faster on 128x128 tiles.
  if (t == TILE_128 && a_kmajor && b_kmajor && epi == EPI_STORE && !colsum) return TILE_256x128;
  return t;
}

hipError_t launch_gemm(bool is_bf16, int a_kmajor, int b_kmajor, int tile, int splits, int tag,
                       const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  return is_bf16 ? launch_type<bf16>(a_kmajor, b_kmajor, tile, splits, tag, p, s)
                 : launch_type<float>(a_kmajor, b_kmajor, tile, splits, tag, p, s);
}

hipError_t launch_splitk_reduce_bf16(const float* part, int splits, int64_t split_stride, int M,
                                     int N, void* C, int64_t ldc, float alpha,
                                     const float* alpha_scale, hipStream_t s) {
  if (N % 4 || ldc % 4 || split_stride % 4) return hipErrorInvalidValue;
  const int64_t n4 = (int64_t)M * (N / 4);
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     part, splits, split_stride, M, N, static_cast<bf16*>(C), ldc, alpha,
                     alpha_scale);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t split_stride, int M, int N,
                                float* C, int64_t ldc, float alpha, float beta, hipStream_t s) {
  const int64_t n = (int64_t)M * N;
  if (n == 0) return hipSuccess;
  const bool vec = N % 4 == 0 && ldc % 4 == 0 && split_stride % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(part) % 16 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0;
  if (vec) {
    const int64_t n4 = n / 4;
    hipLaunchKernelGGL(splitk_reduce4_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       part, splits, split_stride, M, N, C, ldc, alpha, beta);
  } else {
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       part, splits, split_stride, M, N, C, ldc, alpha, beta);
  }
  return hipGetLastError();
}
