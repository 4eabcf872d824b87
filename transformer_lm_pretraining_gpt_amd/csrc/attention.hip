// Causal multi-head attention, forward and backward, tiled with online softmax (gfx950 MFMA).
//
// Per (batch, head): O = softmax(Q K^T / sqrt(hd), keys j <= query i) V. This is the O(T^2) term
// that Kaplan's Eq. (2.2) adds to the 2N forward cost ("Pré-treinar um LLM", paragraph on the
// attention term). No T x T matrix ever reaches memory: scores live in MFMA accumulators.
//
// Orientation. The forward computes S^T = K Q^T: the 32x32 MFMA result puts one query per lane
// (column) and 16 keys per lane in registers, so the softmax row statistics of a query are a
// per-lane reduction plus one exchange with the other lane half, and the probabilities are
// already laid out as the B operand of O^T = V^T P^T (no trip through LDS). V^T is staged
// transposed in LDS so its fragments line up with the probabilities' key order.
//
// Backward (deterministic, no atomics): kernel 1 owns a block of keys and accumulates dK, dV
// over all later queries (S = Q K^T orientation: one key per lane); kernel 2 owns a block of
// queries and accumulates dQ over all earlier keys (S^T orientation). Both recompute P from the
// saved row log-sum-exp, and use D_i = sum_d dO_id O_id, computed by a small kernel first:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = dS K / sqrt(hd),  dK = dS^T Q / sqrt(hd).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lds_dma.h"

namespace {

constexpr int THREADS = 256;
constexpr int BKV = 64;  // keys (or queries) per LDS stage
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <typename T, int HD>
struct AttnGeom {
  static constexpr int VE = 16 / (int)sizeof(T);             // elements per 16-byte vector
  static constexpr int ROWBYTES = HD * (int)sizeof(T);        // one head row
  static constexpr int CPR = ROWBYTES / 16;                   // 16-byte chunks per head row
  static constexpr int NS = ROWBYTES / 32;                    // MFMA k-steps over head_dim
  static constexpr int RP = ROWBYTES + 16;                    // padded LDS pitch, row layout
  static constexpr int TP = BKV * (int)sizeof(T) + (sizeof(T) == 2 ? 8 : 16);  // transposed
  static constexpr int DB = HD / 32 > 0 ? HD / 32 : 1;        // 32-row blocks of head_dim
  static_assert(HD % 32 == 0 || HD == 16, "head_dim");
};

// Stage rows [row0, row0+64) of a head (one 16-byte chunk per thread step) into row layout.
template <typename T, int HD>
DEV void stage_rows(char* lds, const T* base, int64_t ld, int row0, int nrows, int tid) {
  using G = AttnGeom<T, HD>;
  for (int c = tid; c < BKV * G::CPR; c += THREADS) {
    const int r = c / G::CPR, ch = c % G::CPR;
    u32x4 v{0, 0, 0, 0};
    if (row0 + r < nrows) v = ld16(base + (int64_t)(row0 + r) * ld + ch * G::VE);
    st16(lds + r * G::RP + ch * 16, v);
  }
}

// Stage rows [row0, row0+64) of a head transposed: lds[d][r] (r contiguous). A task is 4 rows x
// one 16-byte vector of d-values.
template <typename T, int HD>
DEV void stage_transposed(char* lds, const T* base, int64_t ld, int row0, int nrows, int tid) {
  using G = AttnGeom<T, HD>;
  constexpr int TASKS = (BKV / 4) * G::CPR;
  for (int t = tid; t < TASKS; t += THREADS) {
    const int rq = t / G::CPR, ch = t % G::CPR;
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = row0 + rq * 4 + j;
      v[j] = r < nrows ? ld16(base + (int64_t)r * ld + ch * G::VE) : u32x4{0, 0, 0, 0};
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t q0, q1;
        if (e & 1) {
          q0 = (v[0][w] >> 16) | (v[1][w] & 0xffff0000u);
          q1 = (v[2][w] >> 16) | (v[3][w] & 0xffff0000u);
        } else {
          q0 = (v[0][w] & 0xffffu) | (v[1][w] << 16);
          q1 = (v[2][w] & 0xffffu) | (v[3][w] << 16);
        }
        st8(lds + (ch * 8 + e) * G::TP + rq * 8, u32x2{q0, q1});
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        st16(lds + (ch * 4 + e) * G::TP + rq * 16, u32x4{v[0][e], v[1][e], v[2][e], v[3][e]});
    }
  }
}

// Load this lane's head row (row `row`, zero if out of range) as NS B-operand fragments.
template <typename T, int HD, int NS = AttnGeom<T, HD>::NS>
DEV void load_row_frags(u32x4 (&f)[NS], const T* base, int64_t ld, int row, int nrows, int h) {
  using G = AttnGeom<T, HD>;
#pragma unroll
  for (int s = 0; s < G::NS; ++s)
    f[s] = row < nrows ? ld16(base + (int64_t)row * ld + (2 * s + h) * G::VE) : u32x4{0, 0, 0, 0};
}

// acc (32 x 32) += rows [r0, r0+32) of a row-layout LDS tile (A operand) times fragments f.
template <typename T, int HD, int NS = AttnGeom<T, HD>::NS>
DEV void mma_rows(f32x16& acc, const char* lds, int r0, const u32x4 (&f)[NS], int h, int l32) {
  using G = AttnGeom<T, HD>;
#pragma unroll
  for (int s = 0; s < G::NS; ++s) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(lds + (r0 + l32) * G::RP + (2 * s + h) * 16);
    Mfma<T>::mma(acc, a, f[s]);
  }
}

// out[db] (HD x 32) += Xt[d][c0 .. c0+32) (transposed LDS tile, A operand) times the 32x32
// probability-like matrix p held in MFMA result layout (B operand: lane column, 16 rows).
template <typename T, int HD, int DB = AttnGeom<T, HD>::DB>
DEV void mma_transposed(f32x16 (&out)[DB], const char* ldst, int c0, const float (&p)[16], int h,
                        int l32) {
  using G = AttnGeom<T, HD>;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 b{pack_bf16(p[8 * u], p[8 * u + 1]), pack_bf16(p[8 * u + 2], p[8 * u + 3]),
              pack_bf16(p[8 * u + 4], p[8 * u + 5]), pack_bf16(p[8 * u + 6], p[8 * u + 7])};
      const int ca = c0 + 16 * u + 4 * h;  // slots 8u..8u+3 -> columns ca..ca+3; +8 for the rest
#pragma unroll
      for (int db = 0; db < HD / 32; ++db) {
        const char* row = ldst + (db * 32 + l32) * G::TP;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(row + ca * 2);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(row + (ca + 8) * 2);
        Mfma<T>::mma(out[db], u32x4{lo[0], lo[1], hi[0], hi[1]}, b);
      }
      if constexpr (HD == 16) {
        // 16 rows of head_dim: lanes 16..31 of the A operand read zero rows
        const char* row = ldst + (l32 & 15) * G::TP;
        u32x4 a{0, 0, 0, 0};
        if (l32 < 16) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row + ca * 2);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + (ca + 8) * 2);
          a = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        Mfma<T>::mma(out[0], a, b);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 b{__builtin_bit_cast(uint32_t, p[4 * u]), __builtin_bit_cast(uint32_t, p[4 * u + 1]),
                    __builtin_bit_cast(uint32_t, p[4 * u + 2]),
                    __builtin_bit_cast(uint32_t, p[4 * u + 3])};
      const int ca = c0 + 8 * u + 4 * h;
#pragma unroll
      for (int db = 0; db < HD / 32; ++db) {
        const char* row = ldst + (db * 32 + l32) * G::TP;
        Mfma<T>::mma(out[db], *reinterpret_cast<const u32x4*>(row + ca * 4), b);
      }
      if constexpr (HD == 16) {
        u32x4 a{0, 0, 0, 0};
        if (l32 < 16) a = *reinterpret_cast<const u32x4*>(ldst + l32 * G::TP + ca * 4);
        Mfma<T>::mma(out[0], a, b);
      }
    }
  }
}

// Store a (HD x 32) result held transposed in MFMA layout (lane = column `row`, registers = d)
// into row `row` of a head slice: dst + row * ld + d.
template <typename T, int HD, int DB = AttnGeom<T, HD>::DB>
DEV void store_head_row(const f32x16 (&acc)[DB], T* dst, int64_t ld, int row, int nrows,
                        float scale, int h, int l32) {
  if (row >= nrows) return;
  T* out = dst + (int64_t)row * ld;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + h * 4;  // rows mfma_row(4g .. 4g+3, h)
      if (HD == 16 && d >= 16) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * g + e] * scale;
      if constexpr (sizeof(T) == 2)
        st8(out + d, u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])});
      else
        st16(out + d, u32x4{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                            __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])});
    }
  }
}

// ----------------------------------------------------------------------------------- forward
template <typename T, int HD>
__global__ __launch_bounds__(THREADS) void attn_fwd_kernel(const T* __restrict__ qkv,
                                                           T* __restrict__ out,
                                                           float* __restrict__ lse, int T_,
                                                           int H) {
  using G = AttnGeom<T, HD>;
  __shared__ __attribute__((aligned(16))) char ks[BKV * G::RP];
  __shared__ __attribute__((aligned(16))) char vt[HD * G::TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nqb = (T_ + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.y;  // heaviest query blocks dispatched first
  const int bh = blockIdx.x, b = bh / H, hh = bh % H;
  const int dm = H * HD;
  const int64_t ld = 3 * (int64_t)dm;
  const T* Q = qkv + (int64_t)b * T_ * ld + hh * HD;
  const T* K = Q + dm;
  const T* V = Q + 2 * dm;

  const int q0 = qb * 128;
  const int qw = q0 + wave * 32;  // this wave's first query
  const int qi = qw + l32;        // this lane's query
  u32x4 qf[G::NS];
  load_row_frags<T, HD>(qf, Q, ld, qi, T_, h);

  f32x16 o[G::DB];
#pragma unroll
  for (int i = 0; i < G::DB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float c = LOG2E / sqrtf((float)HD);

  const int kv_end = min(T_, q0 + 128);
  for (int kv0 = 0; kv0 < kv_end; kv0 += BKV) {
    __syncthreads();
    stage_rows<T, HD>(ks, K, ld, kv0, T_, tid);
    stage_transposed<T, HD>(vt, V, ld, kv0, T_, tid);
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const int j0 = kv0 + jb * 32;
      if (j0 > qw + 31 || j0 >= T_) continue;  // fully masked for this wave
      f32x16 s = f32x16{};
      mma_rows<T, HD>(s, ks, jb * 32, qf, h, l32);
      float p[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + mfma_row(r, h);
        p[r] = (j > qi || j >= T_) ? -INFINITY : s[r] * c;
        mloc = fmaxf(mloc, p[r]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - m_new);
      float lsum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(p[r] - m_new);
        lsum += p[r];
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < G::DB; ++i) o[i] *= alpha;
      mma_transposed<T, HD>(o, vt, jb * 32, p, h, l32);
    }
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  store_head_row<T, HD>(o, out + (int64_t)b * T_ * dm + hh * HD, dm, qi, T_, 1.0f / l_tot, h, l32);
  if (h == 0 && qi < T_) lse[(int64_t)bh * T_ + qi] = (m_run + log2f(l_tot)) * LN2;
}

// ------------------------------------------------------- forward, bf16 with head_dim 64
// Path for bf16 heads of 64 when T is a multiple of 64. K and V tiles of 64 keys go straight
// from memory into a two-stage LDS ring; the K tile is read as K-major A fragments of S^T =
// K Q^T, and the V tile, stored as it is ([key][d] rows), is read transposed with
// ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T, in the key order that the probability
// registers already have. A block owns 128 queries, wave w the 32-query group w: a wave needs
// about 110 registers and a block 32 KB of LDS, so four blocks (four waves per SIMD) share a CU.
// Two groups per wave (256 queries per block, groups w and 7 - w) with a three-stage ring ran
// three waves per SIMD and was 12-14 % slower at T = 1024 and 8192. Only the diagonal tile of a
// group is masked, and the running output is rescaled only when some lane's maximum grew
// (alpha = 1 otherwise, so skipping it changes nothing).
constexpr int F64_Q = 128;        // queries per block
constexpr int F64_NST = 2;        // LDS stages
constexpr int F64_STAGE = 16384;  // K tile (8 KB) then V tile (8 KB)

// A operand V^T[d0 + l%32][keys key0 + 4h + 0..3, key0 + 8 + 4h + 0..3] (h = l / 32) from a V
// tile of [key][d] rows: the keys of probability registers p[8u .. 8u+7] of an S^T accumulator
// (rows mfma_row(r, h)) for key0 = 32 js + 16 u.
DEV u32x4 vt_frag(const char* vtile, int d0, int key0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = d0 + (g & 1) * 16 + 4 * (j & 3);
  const int chunk = r >> 3, within = (r & 7) * 2;
  u32x2 out[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int krow = key0 + 4 * (g >> 1) + 8 * t + (j >> 2);
    const char* a = vtile + krow * 128 + ((chunk ^ tr_swz<64>(krow)) << 4) + within;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
    out[t] = __builtin_bit_cast(u32x2, v);
  }
  return u32x4{out[0][0], out[0][1], out[1][0], out[1][1]};
}

__global__ __launch_bounds__(THREADS, 3) void attn_fwd64_kernel(const bf16* __restrict__ qkv,
                                                                bf16* __restrict__ out,
                                                                float* __restrict__ lse, int T_,
                                                                int H) {
  using TK = DmaTile<64, true, 128>;   // keys x d, K-major
  using TV = DmaTile<64, false, 128>;  // [key][d] rows, read transposed
  constexpr int LW = TK::PER_WAVE + TV::PER_WAVE;
  __shared__ __attribute__((aligned(1024))) char smem[F64_NST * F64_STAGE];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (T_ + F64_Q - 1) / F64_Q;
  const int qb = nqb - 1 - (int)blockIdx.y;  // heaviest query blocks dispatched first
  const int bh = blockIdx.x, b = bh / H, hh = bh % H;
  const int dm = H * 64;
  const int64_t ld = 3 * (int64_t)dm;
  const bf16* Q = qkv + (int64_t)b * T_ * ld + hh * 64;
  const bf16* K = Q + dm;
  const bf16* V = Q + 2 * dm;
  const int q0 = qb * F64_Q;
  const int ntiles = min(T_, q0 + F64_Q) / 64;

  const int qg = q0 + 32 * wave;  // this wave's first query
  const int qi = qg + l32;        // this lane's query
  u32x4 qf[4];
  load_row_frags<bf16, 64>(qf, Q, ld, qi, T_, h);
  f32x16 o[2];
  o[0] = o[1] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float c = LOG2E / 8.0f;  // log2(e) / sqrt(64)

  uint32_t offk[TK::PER_WAVE], offv[TV::PER_WAVE];
  TK::offsets(offk, ld, 0, 64, wave, lane);
  TV::offsets(offv, ld, 0, 64, wave, lane);
  auto issue = [&](int kt) {
    char* st = smem + (kt % F64_NST) * F64_STAGE;
    const __amdgpu_buffer_rsrc_t rk = TK::slab(K, ld, kt * 64, 0);
    const __amdgpu_buffer_rsrc_t rv = TV::slab(V, ld, 0, kt * 64);
#pragma unroll
    for (int i = 0; i < TK::PER_WAVE; ++i) TK::issue(rk, offk, i, st, wave);
#pragma unroll
    for (int i = 0; i < TV::PER_WAVE; ++i) TV::issue(rv, offv, i, st + 8192, wave);
  };
#pragma unroll
  for (int s = 0; s < F64_NST - 1; ++s)
    if (s < ntiles) issue(s);

  // the tile loop is unrolled over the two stages so that each stage's LDS offset is a
  // compile-time constant (folded into the LDS instructions' offsets)
  auto tile = [&](auto stc, int kt) {
    constexpr int ST = decltype(stc)::value;
    wait_slabs<LW, F64_NST - 2>(min(F64_NST - 2, ntiles - 1 - kt));
    wave_barrier_all();
    if (kt + F64_NST - 1 < ntiles) issue(kt + F64_NST - 1);
    const char* ktile = smem + ST * F64_STAGE;
    const char* vtile = ktile + 8192;
    const int key0 = kt * 64;
    if (key0 > qg + 31 || qg >= T_) return;  // every key of the tile is after the group
    // the group in three steps: S^T, then the online softmax (P^T packed to bf16), then
    // O^T += V^T P^T
    auto scores = [&](f32x16 (&sacc)[2]) {
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        sacc[js] = f32x16{};
#pragma unroll
        for (int s = 0; s < 4; ++s) Mfma<bf16>::mma(sacc[js], TK::frag(ktile, js * 32, s, lane), qf[s]);
      }
    };
    auto softmax = [&](bool diag, f32x16 (&sacc)[2], u32x4 (&pb)[2][2]) {
      float mloc = -INFINITY;
      if (diag) {
#pragma unroll
        for (int js = 0; js < 2; ++js)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = key0 + js * 32 + mfma_row(r, h);
            if (j > qi) sacc[js][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int js = 0; js < 2; ++js)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[js][r]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64)) * c;
      // The running maximum moves only when some row's maximum grew by more than 2^8: below
      // that, exp2 of the scores minus the older maximum stays below 256 (no overflow; bf16
      // keeps its relative precision), and the normalisation by the row sum is unchanged.
      if (__builtin_amdgcn_ballot_w64(mloc > m_run + 8.0f) != 0) {
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = fast_exp2(m_run - m_new);
        o[0] *= alpha;
        o[1] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run;
      float lsum = 0.0f;
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(fmaf(sacc[js][r], c, -m_use));
          lsum += p[r];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
          pb[js][u] = u32x4{pack_bf16(p[8 * u], p[8 * u + 1]), pack_bf16(p[8 * u + 2], p[8 * u + 3]),
                            pack_bf16(p[8 * u + 4], p[8 * u + 5]), pack_bf16(p[8 * u + 6], p[8 * u + 7])};
      }
      l_run += lsum;
    };
    auto pv = [&](const u32x4 (&pb)[2][2]) {
#pragma unroll
      for (int js = 0; js < 2; ++js)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < 2; ++db)
            Mfma<bf16>::mma(o[db], vt_frag(vtile, db * 32, js * 32 + 16 * u, lane), pb[js][u]);
    };
    f32x16 sacc[2];
    u32x4 pb[2][2];
    scores(sacc);
    softmax(key0 + 63 > qg, sacc, pb);
    pv(pb);
  };
  for (int kt0 = 0; kt0 < ntiles; kt0 += 2) {
    tile(std::integral_constant<int, 0>{}, kt0);
    if (kt0 + 1 < ntiles) tile(std::integral_constant<int, 1>{}, kt0 + 1);
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  store_head_row<bf16, 64>(o, out + (int64_t)b * T_ * dm + hh * 64, dm, qi, T_, 1.0f / l_tot, h, l32);
  if (h == 0 && qi < T_) lse[(int64_t)bh * T_ + qi] = (m_run + log2f(l_tot)) * LN2;
}

// --------------------------------------------------------------------- backward: D = rowsum
template <typename T, int HD>
__global__ void attn_dsum_kernel(const T* __restrict__ out, const T* __restrict__ dout,
                                 float* __restrict__ dsum, int T_, int H, int rows) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int LPH = HD / VE;  // lanes per head
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int dm = H * HD;
  const int b = row / T_, t = row % T_;
  for (int v0 = 0; v0 < dm / VE; v0 += 64) {
    const int v = v0 + lane;
    float s = 0.0f;
    if (v < dm / VE) {
      float a[VE], g[VE];
      Vec<T>::unpack(ld16(out + (int64_t)row * dm + v * VE), a);
      Vec<T>::unpack(ld16(dout + (int64_t)row * dm + v * VE), g);
#pragma unroll
      for (int e = 0; e < VE; ++e) s += a[e] * g[e];
    }
#pragma unroll
    for (int o = 1; o < LPH; o <<= 1) s += __shfl_xor(s, o, 64);
    if (v < dm / VE && (v % LPH) == 0) {
      const int hh = v / LPH;
      dsum[((int64_t)b * H + hh) * T_ + t] = s;
    }
  }
}

// ------------------------------------------------------------------- backward: dK and dV
template <typename T, int HD>
__global__ __launch_bounds__(THREADS) void attn_bwd_dkdv_kernel(
    const T* __restrict__ qkv, const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dsum, T* __restrict__ dqkv, int T_, int H) {
  using G = AttnGeom<T, HD>;
  __shared__ __attribute__((aligned(16))) char qs[BKV * G::RP];
  __shared__ __attribute__((aligned(16))) char dos[BKV * G::RP];
  __shared__ __attribute__((aligned(16))) char qt[HD * G::TP];
  __shared__ __attribute__((aligned(16))) char dot[HD * G::TP];
  __shared__ float lse_s[BKV], d_s[BKV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nkb = (T_ + 127) / 128;
  const int kb = (int)blockIdx.y;  // key blocks near the start (most queries) go first
  const int bh = blockIdx.x, b = bh / H, hh = bh % H;
  const int dm = H * HD;
  const int64_t ld = 3 * (int64_t)dm;
  const T* Q = qkv + (int64_t)b * T_ * ld + hh * HD;
  const T* K = Q + dm;
  const T* V = Q + 2 * dm;
  const T* dO = dout + (int64_t)b * T_ * dm + hh * HD;
  const float* lse_bh = lse + (int64_t)bh * T_;
  const float* d_bh = dsum + (int64_t)bh * T_;
  (void)nkb;

  const int k0 = kb * 128;
  const int kw = k0 + wave * 32;
  const int kj = kw + l32;  // this lane's key
  u32x4 kf[G::NS], vf[G::NS];
  load_row_frags<T, HD>(kf, K, ld, kj, T_, h);
  load_row_frags<T, HD>(vf, V, ld, kj, T_, h);
  f32x16 dv[G::DB], dk[G::DB];
#pragma unroll
  for (int i = 0; i < G::DB; ++i) dv[i] = dk[i] = f32x16{};
  const float c = LOG2E / sqrtf((float)HD);

  for (int i0 = (k0 / BKV) * BKV; i0 < T_; i0 += BKV) {
    __syncthreads();
    stage_rows<T, HD>(qs, Q, ld, i0, T_, tid);
    stage_rows<T, HD>(dos, dO, dm, i0, T_, tid);
    stage_transposed<T, HD>(qt, Q, ld, i0, T_, tid);
    stage_transposed<T, HD>(dot, dO, dm, i0, T_, tid);
    if (tid < BKV) {
      const int i = i0 + tid;
      lse_s[tid] = i < T_ ? lse_bh[i] * LOG2E : 0.0f;
      d_s[tid] = i < T_ ? d_bh[i] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int iq = i0 + ib * 32;
      if (iq + 31 < kw || iq >= T_) continue;  // all queries before this wave's keys
      f32x16 s = f32x16{}, dp = f32x16{};
      mma_rows<T, HD>(s, qs, ib * 32, kf, h, l32);
      mma_rows<T, HD>(dp, dos, ib * 32, vf, h, l32);
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int il = ib * 32 + g * 8 + h * 4;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(lse_s + il);
        const f32x4 dd = *reinterpret_cast<const f32x4*>(d_s + il);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const int i = i0 + il + e;
          const float pr = (i < kj || i >= T_) ? 0.0f : fast_exp2(s[r] * c - lv[e]);
          p[r] = pr;
          ds[r] = pr * (dp[r] - dd[e]);
        }
      }
      mma_transposed<T, HD>(dv, dot, ib * 32, p, h, l32);
      mma_transposed<T, HD>(dk, qt, ib * 32, ds, h, l32);
    }
  }
  T* dK = dqkv + (int64_t)b * T_ * ld + dm + hh * HD;
  store_head_row<T, HD>(dk, dK, ld, kj, T_, 1.0f / sqrtf((float)HD), h, l32);
  store_head_row<T, HD>(dv, dK + dm, ld, kj, T_, 1.0f, h, l32);
}

// ----------------------------------------------------------------------- backward: dQ
template <typename T, int HD>
__global__ __launch_bounds__(THREADS) void attn_bwd_dq_kernel(
    const T* __restrict__ qkv, const T* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dsum, T* __restrict__ dqkv, int T_, int H) {
  using G = AttnGeom<T, HD>;
  __shared__ __attribute__((aligned(16))) char ks[BKV * G::RP];
  __shared__ __attribute__((aligned(16))) char vs[BKV * G::RP];
  __shared__ __attribute__((aligned(16))) char kt[HD * G::TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nqb = (T_ + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.y;
  const int bh = blockIdx.x, b = bh / H, hh = bh % H;
  const int dm = H * HD;
  const int64_t ld = 3 * (int64_t)dm;
  const T* Q = qkv + (int64_t)b * T_ * ld + hh * HD;
  const T* K = Q + dm;
  const T* V = Q + 2 * dm;
  const T* dO = dout + (int64_t)b * T_ * dm + hh * HD;

  const int q0 = qb * 128;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  u32x4 qf[G::NS], df[G::NS];
  load_row_frags<T, HD>(qf, Q, ld, qi, T_, h);
  load_row_frags<T, HD>(df, dO, dm, qi, T_, h);
  const float lse_i = qi < T_ ? lse[(int64_t)bh * T_ + qi] * LOG2E : 0.0f;
  const float d_i = qi < T_ ? dsum[(int64_t)bh * T_ + qi] : 0.0f;
  f32x16 dq[G::DB];
#pragma unroll
  for (int i = 0; i < G::DB; ++i) dq[i] = f32x16{};
  const float c = LOG2E / sqrtf((float)HD);

  const int kv_end = min(T_, q0 + 128);
  for (int kv0 = 0; kv0 < kv_end; kv0 += BKV) {
    __syncthreads();
    stage_rows<T, HD>(ks, K, ld, kv0, T_, tid);
    stage_rows<T, HD>(vs, V, ld, kv0, T_, tid);
    stage_transposed<T, HD>(kt, K, ld, kv0, T_, tid);
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const int j0 = kv0 + jb * 32;
      if (j0 > qw + 31 || j0 >= T_) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
      mma_rows<T, HD>(s, ks, jb * 32, qf, h, l32);
      mma_rows<T, HD>(dp, vs, jb * 32, df, h, l32);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + mfma_row(r, h);
        const float pr = (j > qi || j >= T_) ? 0.0f : fast_exp2(s[r] * c - lse_i);
        ds[r] = pr * (dp[r] - d_i);
      }
      mma_transposed<T, HD>(dq, kt, jb * 32, ds, h, l32);
    }
  }
  store_head_row<T, HD>(dq, dqkv + (int64_t)b * T_ * ld + hh * HD, ld, qi, T_,
                        1.0f / sqrtf((float)HD), h, l32);
}

// ------------------------------------------------------ backward, bf16 with head_dim 64
// Head tiles of 64 rows x 64 bf16 ([row][d], 128-byte rows) in LDS, read both as K-major MFMA
// fragments (rows x d) and transposed (d x rows, ds_read_b64_tr_b16). Chunk c of row r sits at
// c ^ hswz(r): over 16 consecutive rows the b128 fragment reads cover every bank once, and the
// four rows x four chunks of a 32-lane transposed read do too (rows r and r+2 land in opposite
// halves of their 128-byte rows).
DEV int hswz(int r) { return ((r & 2) << 1) | ((r >> 2) & 3); }

struct HeadTile {
  static constexpr int PER_WAVE = 2;  // 1 KB wave-loads per tile per wave
  // per-lane byte offsets (from the tile's first row) of this wave's two loads
  DEV static void offsets(uint32_t (&off)[2], int64_t ld, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (wave * 2 + i) * 8 + lane / 8;
      off[i] = (uint32_t)(row * ld * 2 + (((lane % 8) ^ hswz(row)) << 4));
    }
  }
  DEV static void issue(__amdgpu_buffer_rsrc_t r, const uint32_t (&off)[2], char* dst, int wave) {
    lds_dma16(r, off[0], dst + (wave * 2) * 1024);
    lds_dma16(r, off[1], dst + (wave * 2 + 1) * 1024);
  }
  // A fragment: rows rw + l%32, d = 16 s + 8 h .. +7
  DEV static u32x4 frag(const char* st, int rw, int s, int lane) {
    const int row = rw + (lane & 31);
    return *reinterpret_cast<const u32x4*>(st + row * 128 + (((2 * s + (lane >> 5)) ^ hswz(row)) << 4));
  }
  // A fragment of the transpose: X^T[d0 + l%32][rows row0 + 4h + 0..3, row0 + 8 + 4h + 0..3], the
  // row order of registers p[8u .. 8u+7] of an MFMA result (rows mfma_row(r, h)), row0 = 32 b + 16 u
  DEV static u32x4 tfrag(const char* st, int d0, int row0, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const int r = d0 + (g & 1) * 16 + 4 * (j & 3);
    const int chunk = r >> 3, within = (r & 7) * 2;
    u32x2 out[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int krow = row0 + 4 * (g >> 1) + 8 * t + (j >> 2);
      const char* a = st + krow * 128 + ((chunk ^ hswz(krow)) << 4) + within;
      out[t] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a)));
    }
    return u32x4{out[0][0], out[0][1], out[1][0], out[1][1]};
  }
};

DEV u32x4 pack8(const float* p) {
  return u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
}

// dK and dV for 128 keys per block (32 per wave, one key per lane): S = Q K^T and dP = dO V^T
// with the key's K and V rows as register B operands, then dV^T += dO^T P and dK^T += Q^T dS from
// the transposed tiles. Query tiles of 64 stream through a three-stage LDS ring with their
// lse log2 e and -D values; dP's accumulators start from -D, so the MFMAs leave dP - D and
// dS = P (dP - D) takes one multiply per element.
constexpr int B64_KEYS = 128;
constexpr int B64_STAGE = 8192 + 8192 + 512;  // Q tile, dO tile, 64 lse log2 e and 64 -D

__global__ __launch_bounds__(THREADS, 2) void attn_bwd_dkdv64_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ dout, const float* __restrict__ lsd,
    bf16* __restrict__ dqkv, int T_, int H) {
  constexpr int NST = 3;
  constexpr int LW = 2 * HeadTile::PER_WAVE + 1;
  __shared__ __attribute__((aligned(1024))) char smem[NST * B64_STAGE];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x, b = bh / H, hh = bh % H;
  const int dm = H * 64;
  const int64_t ld = 3 * (int64_t)dm;
  const bf16* Q = qkv + (int64_t)b * T_ * ld + hh * 64;
  const bf16* K = Q + dm;
  const bf16* V = Q + 2 * dm;
  const bf16* dO = dout + (int64_t)b * T_ * dm + hh * 64;
  const float* lsd_bh = lsd + (int64_t)bh * T_;
  // lanes 0..3 load four lse log2 e each, lanes 4..7 four -D from the second half of the buffer
  const uint32_t lsd_off = lane < 4 ? 16u * lane : 4u * (uint32_t)gridDim.x * T_ + 16u * (lane - 4);
  const int k0 = blockIdx.y * B64_KEYS;  // key blocks near the start (most queries) go first
  const int kg = k0 + 32 * wave;         // this wave's first key
  const int kj = kg + l32;               // this lane's key
  u32x4 kf[4], vf[4];
  load_row_frags<bf16, 64>(kf, K, ld, kj, T_, h);
  load_row_frags<bf16, 64>(vf, V, ld, kj, T_, h);
  f32x16 dk[2], dv[2];
  dk[0] = dk[1] = dv[0] = dv[1] = f32x16{};
  const float c = LOG2E / 8.0f;

  const int qt0 = k0 / 64;               // first query tile with a query >= k0
  const int ntl = T_ / 64 - qt0;
  uint32_t offq[2], offo[2];
  HeadTile::offsets(offq, ld, wave, lane);
  HeadTile::offsets(offo, dm, wave, lane);
  auto issue = [&](int t) {
    char* st = smem + (t % NST) * B64_STAGE;
    const int q = (qt0 + t) * 64;
    HeadTile::issue(buffer_at(Q + (int64_t)q * ld), offq, st, wave);
    HeadTile::issue(buffer_at(dO + (int64_t)q * dm), offo, st + 8192, wave);
    // per wave 16 queries: their lse log2 e (64 bytes), then their -D (64 bytes)
    if (lane < 8) lds_dma16(buffer_at(lsd_bh + q + 16 * wave), lsd_off, st + 16384 + wave * 128);
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
    if (t < ntl) issue(t);

  // the tile loop is unrolled over the three stages so that each stage's LDS offset is a
  // compile-time constant (folded into the LDS instructions' offsets)
  auto tile = [&](auto stc, auto mc, int t) {
    constexpr int ST = decltype(stc)::value;
    constexpr bool MASKED = decltype(mc)::value;
    wait_slabs<LW, NST - 2>(min(NST - 2, ntl - 1 - t));
    wave_barrier_all();
    if (t + NST - 1 < ntl) issue(t + NST - 1);
    const char* qt = smem + ST * B64_STAGE;
    const char* dot = qt + 8192;
    const char* ls = qt + 16384;
    const int q = (qt0 + t) * 64;
    // rows mfma_row(4g .. 4g+3, h) of sub-tile ib: queries il .. il+3 of the tile, il = 32 ib + 8 g
    // + 4 h; their 16-query group holds lse log2 e at +0 and -D at +64
    auto lsd_at = [&](int ib, int g) { const int il = ib * 32 + g * 8 + h * 4; return ls + (il >> 4) * 128 + (il & 15) * 4; };
    // one 32-query sub-tile in three steps: S and dP, then P and dS, then dV and dK
    auto scores = [&](int ib, f32x16& sacc, f32x16& dpacc) {
      sacc = f32x16{};
      // dP starts from -D, so that the MFMAs leave dP - D
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 nd = *reinterpret_cast<const f32x4*>(lsd_at(ib, g) + 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) dpacc[4 * g + e] = nd[e];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Mfma<bf16>::mma(sacc, HeadTile::frag(qt, ib * 32, s, lane), kf[s]);
        Mfma<bf16>::mma(dpacc, HeadTile::frag(dot, ib * 32, s, lane), vf[s]);
      }
    };
    auto probs = [&](int ib, bool diag, const f32x16& sacc, const f32x16& dpacc, u32x4 (&pb)[2],
                     u32x4 (&dsb)[2]) {
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(lsd_at(ib, g));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          p[r] = fast_exp2(fmaf(sacc[r], c, -lv[e]));
          ds[r] = p[r] * dpacc[r];
        }
      }
      if (diag) {  // queries before the key: zero (a branch of its own, taken on diagonal tiles)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (q + ib * 32 + mfma_row(r, h) < kj) p[r] = ds[r] = 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pb[u] = pack8(p + 8 * u);
        dsb[u] = pack8(ds + 8 * u);
      }
    };
    auto accumulate = [&](int ib, const u32x4 (&pb)[2], const u32x4 (&dsb)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          Mfma<bf16>::mma(dv[db], HeadTile::tfrag(dot, db * 32, ib * 32 + 16 * u, lane), pb[u]);
          Mfma<bf16>::mma(dk[db], HeadTile::tfrag(qt, db * 32, ib * 32 + 16 * u, lane), dsb[u]);
        }
    };
    if constexpr (!MASKED) {
      // every query of the tile is after this wave's keys (no mask): both sub-tiles as one
      // straight-line block, so that one's MFMAs can overlap the other's exponentials
      f32x16 s0, d0, s1, d1;
      u32x4 pb0[2], ds0[2], pb1[2], ds1[2];
      scores(0, s0, d0);
      scores(1, s1, d1);
      probs(0, false, s0, d0, pb0, ds0);
      accumulate(0, pb0, ds0);
      probs(1, false, s1, d1, pb1, ds1);
      accumulate(1, pb1, ds1);
    } else {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int iq = q + ib * 32;
        if (iq + 31 < kg) continue;  // every query of the sub-tile is before this wave's keys
        const bool diag = iq < kg + 32;
        f32x16 sacc, dpacc;
        u32x4 pb[2], dsb[2];
        scores(ib, sacc, dpacc);
        probs(ib, diag, sacc, dpacc, pb, dsb);
        accumulate(ib, pb, dsb);
      }
    }
    };
  // The first two query tiles hold every wave's diagonal and take the masked form; from the
  // third on no query is before any of the block's keys, and the loop has the unmasked form only.
  // With both forms in the loop the compiler kept the dK/dV accumulators in other registers in
  // each and copied 64 registers per tile (about 3 % of the kernel's time).
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using MK = std::true_type;
  using NM = std::false_type;
  tile(I0{}, MK{}, 0);
  if (ntl > 1) tile(I1{}, MK{}, 1);
  for (int t0 = 2; t0 < ntl; t0 += 3) {
    tile(I2{}, NM{}, t0);
    if (t0 + 1 < ntl) tile(I0{}, NM{}, t0 + 1);
    if (t0 + 2 < ntl) tile(I1{}, NM{}, t0 + 2);
  }
  bf16* dK = dqkv + (int64_t)b * T_ * ld + dm + hh * 64;
  store_head_row<bf16, 64>(dk, dK, ld, kj, T_, 1.0f / 8.0f, h, l32);
  store_head_row<bf16, 64>(dv, dK + dm, ld, kj, T_, 1.0f, h, l32);
}

// dQ for 128 queries per block (wave w: the 32-query group w, one query per lane): S^T = K Q^T
// and dP^T = V dO^T with the query's Q and dO rows as register B operands, then dQ^T += K^T dS^T
// from the transposed K tile. Key tiles stream through a three-stage LDS ring. One group per wave
// keeps a wave at about 130 registers, so three blocks (48 KB of LDS each) share a CU; two groups
// per wave (256 queries per block) needed about 200 registers and ran two waves per SIMD, about 8 %
// slower over the whole attention backward at the GPT-2 124M shape. Each query's D = dO . O is
// computed here from its own rows and written, negated, beside lse log2 e for the dK/dV kernel
// (launched after this one).
constexpr int DQ64_Q = 128;  // queries per block

__global__ __launch_bounds__(THREADS, 3) void attn_bwd_dq64_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ out, const bf16* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ lsd, bf16* __restrict__ dqkv, int T_,
    int H) {
  constexpr int NST = 3;
  constexpr int LW = 2 * HeadTile::PER_WAVE;
  __shared__ __attribute__((aligned(1024))) char smem[NST * 16384];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (T_ + DQ64_Q - 1) / DQ64_Q;
  const int qb = nqb - 1 - (int)blockIdx.y;  // heaviest query blocks dispatched first
  const int bh = blockIdx.x, b = bh / H, hh = bh % H;
  const int dm = H * 64;
  const int64_t ld = 3 * (int64_t)dm;
  const bf16* Q = qkv + (int64_t)b * T_ * ld + hh * 64;
  const bf16* K = Q + dm;
  const bf16* V = Q + 2 * dm;
  const bf16* dO = dout + (int64_t)b * T_ * dm + hh * 64;
  const bf16* O = out + (int64_t)b * T_ * dm + hh * 64;
  const int q0 = qb * DQ64_Q;
  const int ntiles = min(T_, q0 + DQ64_Q) / 64;

  const int qg = q0 + 32 * wave;  // this wave's first query
  const int qi = qg + l32;        // this lane's query
  u32x4 qf[4], df[4];
  load_row_frags<bf16, 64>(qf, Q, ld, qi, T_, h);
  load_row_frags<bf16, 64>(df, dO, dm, qi, T_, h);
  float dsum;
  {
    // D = dO . O over the head's 64 columns: this lane holds 32 of them (half h), the lane 32
    // apart the other 32
    u32x4 of[4];
    load_row_frags<bf16, 64>(of, O, dm, qi, T_, h);
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float a[8], g[8];
      Vec<bf16>::unpack(of[s], a);
      Vec<bf16>::unpack(df[s], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf(a[e], g[e], part);
    }
    dsum = part + __shfl_xor(part, 32, 64);
  }
  const float lse2 = qi < T_ ? lse[(int64_t)bh * T_ + qi] * LOG2E : 0.0f;
  // lse log2 e and -D, which the dK/dV kernel streams with its query tiles (two arrays of
  // B H T floats)
  if (h == 0 && qi < T_) {
    lsd[(int64_t)bh * T_ + qi] = lse2;
    lsd[((int64_t)gridDim.x + bh) * T_ + qi] = -dsum;
  }
  f32x16 dq[2];
  dq[0] = dq[1] = f32x16{};
  const float c = LOG2E / 8.0f;

  uint32_t off[2];
  HeadTile::offsets(off, ld, wave, lane);
  auto issue = [&](int kt) {
    char* st = smem + (kt % NST) * 16384;
    HeadTile::issue(buffer_at(K + (int64_t)kt * 64 * ld), off, st, wave);
    HeadTile::issue(buffer_at(V + (int64_t)kt * 64 * ld), off, st + 8192, wave);
  };
#pragma unroll
  for (int t = 0; t < NST - 1; ++t)
    if (t < ntiles) issue(t);

  // the tile loop is unrolled over the three stages so that each stage's LDS offset is a
  // compile-time constant (folded into the LDS instructions' offsets)
  auto tile = [&](auto stc, int kt) {
    constexpr int ST = decltype(stc)::value;
    wait_slabs<LW, NST - 2>(min(NST - 2, ntiles - 1 - kt));
    wave_barrier_all();
    if (kt + NST - 1 < ntiles) issue(kt + NST - 1);
    const char* ktile = smem + ST * 16384;
    const char* vtile = ktile + 8192;
    const int key0 = kt * 64;
    if (key0 > qg + 31 || qg >= T_) return;  // every key of the tile is after the group
    // one 32-key sub-tile in three steps: S^T and dP^T, then dS^T, then dQ^T
    auto scores = [&](int js, f32x16& sacc, f32x16& dpacc) {
      sacc = f32x16{};
      dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Mfma<bf16>::mma(sacc, HeadTile::frag(ktile, js * 32, s, lane), qf[s]);
        Mfma<bf16>::mma(dpacc, HeadTile::frag(vtile, js * 32, s, lane), df[s]);
      }
    };
    auto dscores = [&](int js, bool diag, const f32x16& sacc, const f32x16& dpacc,
                       u32x4 (&dsb)[2]) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ds[r] = fast_exp2(fmaf(sacc[r], c, -lse2)) * (dpacc[r] - dsum);
      if (diag) {  // keys after the query: zero (a branch of its own, taken on diagonal tiles)
        const int j0 = key0 + js * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j0 + mfma_row(r, h) > qi) ds[r] = 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) dsb[u] = pack8(ds + 8 * u);
    };
    auto accumulate = [&](int js, const u32x4 (&dsb)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < 2; ++db)
          Mfma<bf16>::mma(dq[db], HeadTile::tfrag(ktile, db * 32, js * 32 + 16 * u, lane), dsb[u]);
    };
    // The two 32-key sub-tiles one after the other: keeping both sub-tiles' scores live (so one's
    // MFMAs overlap the other's exponentials) takes the wave to about 210 registers, two waves per
    // SIMD instead of three (or spills at three).
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      const int j0 = key0 + js * 32;
      if (j0 > qg + 31) continue;
      f32x16 sacc, dpacc;
      u32x4 dsb[2];
      scores(js, sacc, dpacc);
      dscores(js, j0 + 31 > qg, sacc, dpacc, dsb);
      accumulate(js, dsb);
    }
  };
  for (int kt0 = 0; kt0 < ntiles; kt0 += 3) {
    tile(std::integral_constant<int, 0>{}, kt0);
    if (kt0 + 1 < ntiles) tile(std::integral_constant<int, 1>{}, kt0 + 1);
    if (kt0 + 2 < ntiles) tile(std::integral_constant<int, 2>{}, kt0 + 2);
  }
  store_head_row<bf16, 64>(dq, dqkv + (int64_t)b * T_ * ld + hh * 64, ld, qi, T_, 1.0f / 8.0f, h,
                           l32);
}

// Grids are (batch * heads, blocks along the sequence) with the heaviest causal blocks at y = 0.
// Blocks are dispatched x fastest, so every block of the heaviest kind starts before any lighter
// one and the lighter ones fill the CUs that free up first (longest job first). The transposed
// order, whose heavy-to-light pattern repeated every few blocks, gave some CUs only heavy blocks
// and others only light ones: 27-29 % slower at the GPT-2 124M shape.
template <typename T, int HD>
hipError_t fwd_t(int B, int T_, int H, const void* qkv, void* out, float* lse, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && HD == 64) {
    if (T_ % 64 == 0) {
      dim3 grid(B * H, (T_ + F64_Q - 1) / F64_Q);
      hipLaunchKernelGGL(attn_fwd64_kernel, grid, dim3(THREADS), 0, s, static_cast<const bf16*>(qkv),
                         static_cast<bf16*>(out), lse, T_, H);
      return hipGetLastError();
    }
  }
  dim3 grid(B * H, (T_ + 127) / 128);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HD>), grid, dim3(THREADS), 0, s,
                     static_cast<const T*>(qkv), static_cast<T*>(out), lse, T_, H);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t bwd_t(int B, int T_, int H, const void* qkv, const void* out, const float* lse,
                 const void* dout, void* dqkv, float* dsum, hipStream_t s) {
  const int rows = B * T_;
  if constexpr (sizeof(T) == 2 && HD == 64) {
    if (T_ % 64 == 0) {
      // dQ first: it also writes the lse log2 e and -D values that dK/dV read
      hipLaunchKernelGGL(attn_bwd_dq64_kernel, dim3(B * H, (T_ + DQ64_Q - 1) / DQ64_Q), dim3(THREADS),
                         0, s, static_cast<const bf16*>(qkv), static_cast<const bf16*>(out),
                         static_cast<const bf16*>(dout), lse, dsum, static_cast<bf16*>(dqkv), T_,
                         H);
      hipLaunchKernelGGL(attn_bwd_dkdv64_kernel, dim3(B * H, (T_ + B64_KEYS - 1) / B64_KEYS),
                         dim3(THREADS), 0, s, static_cast<const bf16*>(qkv),
                         static_cast<const bf16*>(dout), dsum, static_cast<bf16*>(dqkv), T_, H);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_dsum_kernel<T, HD>), dim3((rows + 3) / 4), dim3(256), 0, s,
                     static_cast<const T*>(out), static_cast<const T*>(dout), dsum, T_, H, rows);
  dim3 grid(B * H, (T_ + 127) / 128);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HD>), grid, dim3(THREADS), 0, s,
                     static_cast<const T*>(qkv), static_cast<const T*>(dout), lse, dsum,
                     static_cast<T*>(dqkv), T_, H);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD>), grid, dim3(THREADS), 0, s,
                     static_cast<const T*>(qkv), static_cast<const T*>(dout), lse, dsum,
                     static_cast<T*>(dqkv), T_, H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(bool is_bf16, int B, int T, int H, int hd, const void* qkv, void* out,
                           float* lse, hipStream_t s) {
  if (B * T == 0) return hipSuccess;
  if (is_bf16) {
    if (hd == 64) return fwd_t<bf16, 64>(B, T, H, qkv, out, lse, s);
    if (hd == 32) return fwd_t<bf16, 32>(B, T, H, qkv, out, lse, s);
    if (hd == 16) return fwd_t<bf16, 16>(B, T, H, qkv, out, lse, s);
  } else {
    if (hd == 64) return fwd_t<float, 64>(B, T, H, qkv, out, lse, s);
    if (hd == 32) return fwd_t<float, 32>(B, T, H, qkv, out, lse, s);
    if (hd == 16) return fwd_t<float, 16>(B, T, H, qkv, out, lse, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd(bool is_bf16, int B, int T, int H, int hd, const void* qkv,
                           const void* out, const float* lse, const void* dout, void* dqkv,
                           float* dsum, hipStream_t s) {
  if (B * T == 0) return hipSuccess;
  if (is_bf16) {
    if (hd == 64) return bwd_t<bf16, 64>(B, T, H, qkv, out, lse, dout, dqkv, dsum, s);
    if (hd == 32) return bwd_t<bf16, 32>(B, T, H, qkv, out, lse, dout, dqkv, dsum, s);
    if (hd == 16) return bwd_t<bf16, 16>(B, T, H, qkv, out, lse, dout, dqkv, dsum, s);
  } else {
    if (hd == 64) return bwd_t<float, 64>(B, T, H, qkv, out, lse, dout, dqkv, dsum, s);
    if (hd == 32) return bwd_t<float, 32>(B, T, H, qkv, out, lse, dout, dqkv, dsum, s);
    if (hd == 16) return bwd_t<float, 16>(B, T, H, qkv, out, lse, dout, dqkv, dsum, s);
  }
  return hipErrorInvalidValue;
}
