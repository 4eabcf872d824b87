// Token + position embedding: gather forward and deterministic scatter-add backward.
//
// h0[b, t] = wte[x[b, t]] + wpe[t]. The token matrix is the tied embedding / LM head of GPT-2
// (built the nanoGPT way, "Criei GPT-2 do zero com uma RTX 4090", section "Ambiente"), so its
// gradient is the LM head's dW plus the scatter of dh0 rows by token id:
//   dwte[v] += sum over positions p with x_p = v of dh0[p],   dwpe[t] = sum over b of dh0[b, t].
// Determinism without float atomics: the positions are cut into sort chunks of 16384; each sort
// chunk's (token, position) pairs are sorted by one workgroup (stable LSD radix sort in LDS, all
// sort chunks in one launch); each sorted list is cut into fixed chunks of 64 entries; a token
// whose run lies inside one chunk is summed and added by that chunk alone, and a run that crosses
// chunk borders is summed from per-chunk partials, in chunk order, by the chunk where it starts.
// The sort chunks add into the token gradient one after another, in position order. Every sum
// therefore has one fixed order.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int SORT_THREADS = 1024;
constexpr int SORT_EPT = 16;  // elements per thread
constexpr int SORT_CHUNK = SORT_THREADS * SORT_EPT;  // positions per sort chunk (16-bit in a key)
constexpr int CHUNK = 64;

__global__ __launch_bounds__(256) void embed_fwd_kernel(int M, int T, int d, int V,
                                                        const int32_t* __restrict__ tokens,
                                                        const float* __restrict__ wte,
                                                        const float* __restrict__ wpe,
                                                        float* __restrict__ h0,
                                                        int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  int tok = tokens[row];
  if (tok < 0 || tok >= V) {
    if (lane == 0) atomicOr(err, ERR_TOKEN_RANGE);
    tok = 0;  // keep the reads in bounds; the flagged result is not used
  }
  const int t = row % T;
  const float* a = wte + (int64_t)tok * d;
  const float* b = wpe + (int64_t)t * d;
  float* o = h0 + (int64_t)row * d;
  for (int v = lane; v < d / 4; v += 64) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a + 4 * v);
    const f32x4 y = *reinterpret_cast<const f32x4*>(b + 4 * v);
    *reinterpret_cast<f32x4*>(o + 4 * v) = x + y;
  }
}

// Block c sorts the positions [c * SORT_CHUNK, min(M, (c + 1) * SORT_CHUNK)): stable sort of
// key = token << 16 | position within the sort chunk, by token (LSD, 4 bits per pass over bits
// 16..31). The initial order is by position, so the result is ascending in (token, position).
__global__ __launch_bounds__(SORT_THREADS) void token_sort_kernel(int M_all, int V,
                                                                   const int32_t* __restrict__ tokens,
                                                                   uint32_t* __restrict__ keys) {
  const int64_t base = (int64_t)blockIdx.x * SORT_CHUNK;
  const int M = (int)min<int64_t>(SORT_CHUNK, M_all - base);
  tokens += base;
  keys += base;
  __shared__ uint32_t cnt[16 * SORT_THREADS];  // digit-major counters, scanned in place
  __shared__ uint32_t buf[SORT_EPT * SORT_THREADS];
  __shared__ uint32_t wsum[SORT_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t k[SORT_EPT];
#pragma unroll
  for (int i = 0; i < SORT_EPT; ++i) {
    const int e = tid * SORT_EPT + i;
    int tok = e < M ? tokens[e] : 0;
    if (tok < 0 || tok >= V) tok = 0;  // flagged by the forward gather; keeps indices in bounds
    k[i] = e < M ? ((uint32_t)tok << 16) | (uint32_t)e : 0xffffffffu;
  }
  for (int shift = 16; shift < 32; shift += 4) {
    uint32_t c[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) c[g] = 0;
#pragma unroll
    for (int i = 0; i < SORT_EPT; ++i) {
      const uint32_t dg = (k[i] >> shift) & 15u;
#pragma unroll
      for (int g = 0; g < 16; ++g) c[g] += dg == (uint32_t)g;
    }
#pragma unroll
    for (int g = 0; g < 16; ++g) cnt[g * SORT_THREADS + tid] = c[g];
    __syncthreads();
    // exclusive scan of the 16*1024 counters in digit-major order: thread t owns 16 consecutive
    uint32_t own[16], tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      own[i] = cnt[tid * 16 + i];
      tot += own[i];
    }
    uint32_t incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    uint32_t run = before + incl - tot;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      cnt[tid * 16 + i] = run;
      run += own[i];
    }
    __syncthreads();
    uint32_t off[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) off[g] = cnt[g * SORT_THREADS + tid];
#pragma unroll
    for (int i = 0; i < SORT_EPT; ++i) {
      const uint32_t dg = (k[i] >> shift) & 15u;
      uint32_t pos = 0;
#pragma unroll
      for (int g = 0; g < 16; ++g)
        if (dg == (uint32_t)g) pos = off[g]++;
      buf[pos] = k[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SORT_EPT; ++i) k[i] = buf[tid * SORT_EPT + i];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < SORT_EPT; ++i) {
    const int e = tid * SORT_EPT + i;
    if (e < M) keys[e] = k[i];
  }
}

DEV int tok_of(uint32_t key) { return (int)(key >> 16); }

// Chunk c covers sorted entries [c*64, min(M, c*64+64)). Per chunk and column vector: walk the
// runs; add a run that is wholly inside to dwte; keep the partial of a run that crosses a border:
// slot 0 = the chunk's first run when it began in an earlier chunk, slot 1 = the chunk's last run
// when it began in this chunk and continues into the next.
__global__ __launch_bounds__(256) void embed_seg_kernel(int M, int d,
                                                        const uint32_t* __restrict__ keys,
                                                        const float* __restrict__ dh0,
                                                        float* __restrict__ dwte,
                                                        float* __restrict__ part) {
  constexpr int AHEAD = 8;  // rows loaded before any is added: one memory wait per 8 entries
  const int c = blockIdx.x;
  const int e0 = c * CHUNK, e1 = min(M, e0 + CHUNK);
  const int tok_prev = e0 > 0 ? tok_of(keys[e0 - 1]) : -1;
  const int tok_next = e1 < M ? tok_of(keys[e1]) : -1;
  const int nv = d / 4;
  for (int cv = threadIdx.x; cv < nv; cv += 256) {
    f32x4 acc{0, 0, 0, 0};
    int cur = tok_of(keys[e0]);
    int start = e0;
    // dwte's row of the current run, loaded with the run's first entry: no other flush of this
    // kernel writes it (a token's entries are one run, added by one chunk; runs that cross a
    // chunk border go to the partial slots), so the value is still current at the flush
    f32x4 wcur = *reinterpret_cast<const f32x4*>(dwte + (int64_t)cur * d + 4 * cv);
    // the run `cur` that began at `start` ends before entry e
    auto flush = [&](int e) {
      const bool before = start == e0 && cur == tok_prev;
      const bool after = e == e1 && cur == tok_next;
      if (before)
        *reinterpret_cast<f32x4*>(part + ((int64_t)c * 2 + 0) * d + 4 * cv) = acc;
      else if (after)
        *reinterpret_cast<f32x4*>(part + ((int64_t)c * 2 + 1) * d + 4 * cv) = acc;
      else
        *reinterpret_cast<f32x4*>(dwte + (int64_t)cur * d + 4 * cv) = wcur + acc;
    };
    for (int eb = e0; eb < e1; eb += AHEAD) {
      f32x4 row[AHEAD], wrow[AHEAD];
      int tk[AHEAD];
#pragma unroll
      for (int j = 0; j < AHEAD; ++j) {
        const int e = eb + j;
        if (e < e1) {
          const uint32_t key = keys[e];
          tk[j] = tok_of(key);
          row[j] = *reinterpret_cast<const f32x4*>(dh0 + (int64_t)(key & 0xffffu) * d + 4 * cv);
          wrow[j] = *reinterpret_cast<const f32x4*>(dwte + (int64_t)tk[j] * d + 4 * cv);
        }
      }
#pragma unroll
      for (int j = 0; j < AHEAD; ++j) {
        const int e = eb + j;
        if (e >= e1) break;
        if (tk[j] != cur) {
          flush(e);
          acc = f32x4{0, 0, 0, 0};
          cur = tk[j];
          start = e;
          wcur = wrow[j];
        }
        acc += row[j];
      }
    }
    flush(e1);
  }
}

// For each chunk whose last run begins inside it and continues: sum that run's pieces in chunk
// order and add the total to dwte.
__global__ __launch_bounds__(256) void embed_fixup_kernel(int M, int d, int nchunks,
                                                          const uint32_t* __restrict__ keys,
                                                          float* __restrict__ dwte,
                                                          const float* __restrict__ part) {
  const int c = blockIdx.x;
  const int e0 = c * CHUNK, e1 = min(M, e0 + CHUNK);
  if (e1 >= M) return;
  const int tok = tok_of(keys[e1 - 1]);
  if (tok_of(keys[e1]) != tok) return;  // last run ends here
  const bool whole = tok_of(keys[e0]) == tok;
  if (whole && e0 > 0 && tok_of(keys[e0 - 1]) == tok) return;  // run began earlier: not the owner
  const int nv = d / 4;
  constexpr int AHEAD = 8;  // following chunks whose pieces are loaded before any is added
  for (int cv = threadIdx.x; cv < nv; cv += 256) {
    // the run began in this chunk and continues: the seg kernel kept its head in slot 1
    f32x4 acc = *reinterpret_cast<const f32x4*>(part + ((int64_t)c * 2 + 1) * d + 4 * cv);
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(dwte + (int64_t)tok * d + 4 * cv);
    bool open = true;
    for (int kb = c + 1; open && kb < nchunks; kb += AHEAD) {
      f32x4 piece[AHEAD];
#pragma unroll
      for (int j = 0; j < AHEAD; ++j)
        if (kb + j < nchunks)
          piece[j] = *reinterpret_cast<const f32x4*>(part + ((int64_t)(kb + j) * 2 + 0) * d + 4 * cv);
#pragma unroll
      for (int j = 0; j < AHEAD; ++j) {
        const int k = kb + j;
        if (!open || k >= nchunks) break;
        const int k0 = k * CHUNK, k1 = min(M, k0 + CHUNK);
        if (tok_of(keys[k0]) != tok) {
          open = false;
          break;
        }
        acc += piece[j];
        open = k1 < M && tok_of(keys[k1 - 1]) == tok && tok_of(keys[k1]) == tok;
      }
    }
    *reinterpret_cast<f32x4*>(dwte + (int64_t)tok * d + 4 * cv) = w0 + acc;
  }
}

__global__ __launch_bounds__(256) void embed_wpe_kernel(int B, int T, int d,
                                                        const float* __restrict__ dh0,
                                                        float* __restrict__ dwpe, int accumulate) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over T * d/4
  const int nv = d / 4;
  if (idx >= (int64_t)T * nv) return;
  const int t = (int)(idx / nv), cv = (int)(idx % nv);
  f32x4 s{0, 0, 0, 0};
#pragma unroll 8
  for (int b = 0; b < B; ++b)  // in b order; the unrolled loads are in flight together
    s += *reinterpret_cast<const f32x4*>(dh0 + ((int64_t)b * T + t) * d + 4 * cv);
  f32x4* w = reinterpret_cast<f32x4*>(dwpe + (int64_t)t * d + 4 * cv);
  *w = accumulate ? *w + s : s;
}

}  // namespace

hipError_t launch_embed_fwd(int B, int T, int d, int V, const int32_t* tokens, const float* wte,
                            const float* wpe, float* h0, int* err, hipStream_t s) {
  const int M = B * T;
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(embed_fwd_kernel, dim3((M + 3) / 4), dim3(256), 0, s, M, T, d, V, tokens,
                     wte, wpe, h0, err);
  return hipGetLastError();
}

hipError_t launch_token_sort(int M, int V, const int32_t* tokens, uint32_t* keys, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (V > 65536) return hipErrorInvalidValue;
  const int nsort = (M + SORT_CHUNK - 1) / SORT_CHUNK;
  hipLaunchKernelGGL(token_sort_kernel, dim3(nsort), dim3(SORT_THREADS), 0, s, M, V, tokens, keys);
  return hipGetLastError();
}

// 64-entry chunks of one sort chunk (the partial buffer is reused by every sort chunk)
int embed_bwd_chunks(int M) { return (std::min(M, SORT_CHUNK) + CHUNK - 1) / CHUNK; }

hipError_t launch_embed_bwd(int B, int T, int d, const uint32_t* keys, const float* dh0,
                            float* dwte, float* dwpe, int accumulate, float* seg_part,
                            hipStream_t s) {
  const int M = B * T;
  if (M == 0) return hipSuccess;
  // one sort chunk after another on the stream: each adds into dwte after the previous one
  for (int base = 0; base < M; base += SORT_CHUNK) {
    const int Mc = std::min(SORT_CHUNK, M - base);
    const int nch = (Mc + CHUNK - 1) / CHUNK;
    const uint32_t* kc = keys + base;
    const float* hc = dh0 + (int64_t)base * d;
    hipLaunchKernelGGL(embed_seg_kernel, dim3(nch), dim3(256), 0, s, Mc, d, kc, hc, dwte,
                       seg_part);
    hipLaunchKernelGGL(embed_fixup_kernel, dim3(nch), dim3(256), 0, s, Mc, d, nch, kc, dwte,
                       seg_part);
  }
  const int64_t n = (int64_t)T * (d / 4);
  hipLaunchKernelGGL(embed_wpe_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, B, T, d,
                     dh0, dwpe, accumulate);
  return hipGetLastError();
}
