// Host-side launch interface of the gfx950 kernels (one .hip file per kernel family).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// ------------------------------------------------------------------------------------ GEMM
enum GemmEpi {
  EPI_STORE = 0,      // C(T)   = alpha*acc + bias
  EPI_BIAS_GELU = 1,  // C(T)   = u = acc + bias;  C2(T) = gelu_tanh(u)
  EPI_BIAS_RESID = 2, // C(f32) = resid + acc + bias
  EPI_GELU_BWD = 3,   // C(T)   = acc * gelu_tanh'(aux)
  EPI_F32 = 4         // C(f32) = alpha*acc + beta*C   (split z writes C + z*c_split_stride)
};

struct GemmParams {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int M, N, K;
  int k_split;  // K-range per grid.z slice (multiple of the k-tile); >= K when not split
  int epi;
  void* C;
  int64_t ldc;
  int64_t c_split_stride;
  void* C2;
  const float* bias;
  const float* resid;
  const void* aux;
  float alpha, beta;
  // when set, alpha is multiplied by this device scalar (read once per block): the loss scale
  // 1 / (number of trained positions) that only the device knows
  const float* alpha_scale;
  // EPI_GELU_BWD on the direct-to-LDS path with 64-column wave tiles only: when set, column sums
  // of the bf16 output over each 128-row block of a wave tile go to colsum[(row / 128) * N + col]
  float* colsum;
  // number of K splits of the direct-to-LDS kernel's work items (set by the launcher)
  int splits;
};

enum GemmTile { TILE_128 = 0, TILE_256 = 1, TILE_128x384 = 2, TILE_256x128 = 3 };

// Launch C = op(A) op(B) with the given operand layouts (1 = k contiguous). is_bf16 selects the
// element type of A, B, C(T), C2, aux. splits > 1 requires epi == EPI_F32.
hipError_t launch_gemm(bool is_bf16, int a_kmajor, int b_kmajor, int tile, int splits, int tag,
                       const GemmParams& p, hipStream_t s);
int gemm_k_tile(bool is_bf16);
// Measured tile choice for a bf16 product with an M x N output.
int gemm_pick_tile(int M, int N);
// the tile for a bf16 product with the given layouts and epilogue (colsum: fused column sums)
int gemm_pick_tile_epi(int M, int N, int a_kmajor, int b_kmajor, int epi, bool colsum);

// Sum split-K partials: C[m, n] = alpha * sum_z part[z][m, n] + beta * C[m, n] (fixed z order).
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t split_stride, int M, int N,
                                float* C, int64_t ldc, float alpha, float beta, hipStream_t s);
// The same into a bf16 C from dense (M, N) partials, scaled by alpha * *alpha_scale (when given):
// C[m, n] = bf16(alpha * sum_z part[z][m, n]). N, ldc and split_stride multiples of 4.
hipError_t launch_splitk_reduce_bf16(const float* part, int splits, int64_t split_stride, int M,
                                     int N, void* C, int64_t ldc, float alpha,
                                     const float* alpha_scale, hipStream_t s);

// ------------------------------------------------------------------------------ attention
// qkv: (B*T, 3*d); out: (B*T, d); lse: (B, H, T) fp32.
hipError_t launch_attn_fwd(bool is_bf16, int B, int T, int H, int hd, const void* qkv, void* out,
                           float* lse, hipStream_t s);
// dqkv written in full (dq, dk, dv). dsum scratch: (B, H, T) fp32.
hipError_t launch_attn_bwd(bool is_bf16, int B, int T, int H, int hd, const void* qkv,
                           const void* out, const float* lse, const void* dout, void* dqkv,
                           float* dsum, hipStream_t s);

// ------------------------------------------------------------------------------ layernorm
// y(T) = LN(x) * g + b; mean, rstd (M).
hipError_t launch_ln_fwd(bool is_bf16, int M, int d, const float* x, const float* g,
                         const float* b, void* y, float* mean, float* rstd, hipStream_t s);
// dres (fp32, M x d) = (has_dres ? dres : 0) + LN_bwd(dy), dy (T); dres_t (T) = copy of the new
// dres. Column partials per row block into part[blk][3][d]: sum dy*xhat, sum dy, sum new dres.
hipError_t launch_ln_bwd(bool is_bf16, int M, int d, const void* dy, const float* x,
                         const float* mean, const float* rstd, const float* g, float* dres,
                         int has_dres, void* dres_t, float* part, int rows_per_block,
                         hipStream_t s,
                         hipEvent_t done = nullptr);
int ln_bwd_blocks(int M, int rows_per_block);
// Column partial sums of a (M, N) matrix (T or fp32) per block of rows: part[blk][N].
hipError_t launch_colsum_partial(bool src_bf16, int M, int N, const void* src, int64_t ld,
                                 float* part, int rows_per_block, hipStream_t s);
// One column reduction of a batch: columns [0, n) of the partial rows part[p * stride + j],
// p < nparts, column j going to out[j / seg][j % seg] (a NULL output drops its columns). block0
// is the task's first block in the batched launch (64 columns per block, tasks in order).
struct ColTask {
  const float* part;
  int64_t stride;
  int nparts, n, seg, block0;
  float* out[3];
};
// Every task of d_tasks (device memory) in one launch of nblocks blocks, each column summed in
// the same fixed order as launch_colsum_reduce3.
hipError_t launch_colsum_reduce_batch(const ColTask* d_tasks, int ntasks, int nblocks,
                                      int accumulate, hipStream_t s);
// out[j] = (accumulate ? out[j] : 0) + sum_p part[p * stride + j], fixed p order, j < n.
hipError_t launch_colsum_reduce(const float* part, int nparts, int64_t stride, int n, float* out,
                                int accumulate, hipStream_t s);
// The same over columns [0, k*seg) of the partial rows, column j going to out_{j/seg}[j%seg]
// (k = number of non-null outputs among out0, out1, out2, given in that order).
hipError_t launch_colsum_reduce3(const float* part, int nparts, int64_t stride, int seg,
                                 float* out0, float* out1, float* out2, int accumulate,
                                 hipStream_t s);

// ------------------------------------------------------------------------------ loss
// Target id of a position that is not trained (no loss, zero gradient).
constexpr int32_t TARGET_IGNORE = -1;
// logits (M, Vp) T, overwritten by softmax - onehot (pad columns 0); row_loss (M). Rows whose
// target is TARGET_IGNORE get loss 0 and an all-zero gradient row.
hipError_t launch_xent(bool is_bf16, int M, int V, int Vp, void* logits, const int32_t* targets,
                       float* row_loss, int* err, hipStream_t s);
// With n the number of targets other than TARGET_IGNORE: loss_out[0] = sum(row_loss) / n and
// loss_out[1] = 1 / n (both 0 when n = 0); loss_out[0] is also copied to loss_user if not null.
hipError_t launch_loss_mean(int M, const float* row_loss, const int32_t* targets, float* loss_out,
                            float* loss_user, hipStream_t s);

// ------------------------------------------------------------------------------ embedding
hipError_t launch_embed_fwd(int B, int T, int d, int V, const int32_t* tokens, const float* wte,
                            const float* wpe, float* h0, int* err, hipStream_t s);
// Stable sort of (token, position) pairs within each sort chunk of 16384 positions:
// keys[c * 16384 + i] = token << 16 | (position - c * 16384), ascending within the chunk.
hipError_t launch_token_sort(int M, int V, const int32_t* tokens, uint32_t* keys, hipStream_t s);
// dwte[tok] += sum of dh0 rows with that token (deterministic); dwpe = (acc ? dwpe : 0) + sum_b.
hipError_t launch_embed_bwd(int B, int T, int d, const uint32_t* keys, const float* dh0,
                            float* dwte, float* dwpe, int accumulate, float* seg_part,
                            hipStream_t s);
// 64-entry chunks of the largest sort chunk: seg_part holds 2 * embed_bwd_chunks(M) * d floats.
int embed_bwd_chunks(int M);

// ------------------------------------------------------------------------------ optimizer
struct AdamSeg {
  int64_t begin;  // first element of a run of tensors with the same decay flag
  int decay;
  int pad;
};
// AdamW over elements [begin, begin + n) of the flat arrays (begin and n multiples of 4). segs is a
// host array (sorted, the first run beginning at 0, every begin a multiple of 4); the launcher
// passes the runs that meet the range to the kernel by value.
hipError_t launch_adamw(int64_t begin, int64_t n, float* p, const float* g, float* m, float* v,
                        void* shadow, const AdamSeg* segs, int nseg, float lr, float b1, float b2,
                        float eps, float wd, float bc1, float bc2, hipStream_t s);
// Global-norm clipping of the flat gradient g (n a multiple of 4): norm = ||g||_2,
// g *= min(1, max_norm / (norm + 1e-6)). scratch holds CLIP_PARTS + 2 floats (block sums, then
// the norm and the factor); the norm also goes to user_norm when it is not null.
constexpr int CLIP_PARTS = 1024;
hipError_t launch_clip_grad_norm(int64_t n, float* g, float max_norm, float* scratch,
                                 float* user_norm, hipStream_t s);
hipError_t launch_init_normal(int64_t begin, int64_t count, float* p, uint64_t seed, float std,
                              hipStream_t s);
hipError_t launch_fill(int64_t count, float* p, float value, hipStream_t s);
hipError_t launch_cast_bf16(int64_t count, const float* src, void* dst, hipStream_t s);
